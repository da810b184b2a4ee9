"""Native host code checked on the CPU, no GPU needed.

* The C ABI's argument validation (``csrc/la_api.cpp``) built with AddressSanitizer against
  stand-in launchers (``tests/asan/stub_launchers.cpp``) and driven through every entry point
  (``tests/asan/abi_driver.cpp``).
* The fp64 C oracle (``oracle/la_oracle.c``) built with AddressSanitizer and run on exactly
  sized buffers (``tests/asan/oracle_driver.c``).
* The kernels' ``fold`` helper (``csrc/la_tile.h``), compiled for the host: an exact two-sum for
  any magnitudes (``tests/asan/fold_check.cpp``).

Each program is compiled into a temporary directory and run as a child process.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "asan")
CSRC = os.path.join(ROOT, "causal_linear_attention_chunked_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# the harness may preload a library of its own ahead of the sanitizer runtime
ASAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0:abort_on_error=0")


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)


def _compile(cmd):
    r = _run(cmd)
    assert r.returncode == 0, f"compile failed: {' '.join(cmd)}\n{r.stderr[-3000:]}"


def test_abi_validation_under_asan(tmp_path):
    exe = str(tmp_path / "abi_asan")
    # host code only: every -fsanitize= applies to the host compilation
    _compile([HIPCC, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
              "-Xarch_host", "-fsanitize=address", "-I", INCLUDE, "-I", CSRC,
              os.path.join(CSRC, "la_api.cpp"), os.path.join(HERE, "stub_launchers.cpp"),
              os.path.join(HERE, "abi_driver.cpp"), "-o", exe])
    r = _run([exe], env=ASAN_ENV)
    assert r.returncode == 0 and "ok: 0 failures" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr


def test_oracle_under_asan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _compile(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address", "-fopenmp",
              os.path.join(ROOT, "oracle", "la_oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], env=dict(ASAN_ENV, OMP_NUM_THREADS="2"))
    assert r.returncode == 0 and "ok: 0 failures" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr


def test_fold_is_an_exact_two_sum(tmp_path):
    exe = str(tmp_path / "fold")
    # no contraction: the two-sum's error terms must be computed as written
    _compile([HIPCC, "-x", "hip", "--offload-host-only", "-std=c++17", "-O2", "-ffp-contract=off", "-I", CSRC,
              os.path.join(HERE, "fold_check.cpp"), "-o", exe])
    r = _run([exe])
    assert r.returncode == 0 and r.stdout.startswith("ok:"), r.stdout[-2000:] + r.stderr[-2000:]
