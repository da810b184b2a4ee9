"""Throughput of chunked causal linear attention, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is the whole path over one batch of seeded synthetic inputs already
resident in device memory: the forward over each chunk of the sequence in order,
carrying (S, z), then the backward over the chunks in reverse, carrying (dS, dz).
The default workload (G=160 groups, one 128-token chunk, D=64, bf16) is one
forward and one backward launch; `--workload` names the chained ones.  Steps
rotate over enough buffer sets (>= 640 MB) that the 256 MB last-level cache
cannot serve the traffic.  Two timed regions, each bracketed by device
synchronisation:
  1. K steps in up to five consecutive runs of at least 40 steps, each run replayed from one
     HIP graph of its steps (kernel nodes only; `--no-graph` to skip): the median run's time
     per step gives `value` and `ms_per_step`.  The same K steps as plain
     library calls from Python are timed too (`config.plain_loop_*`): there the host's launch
     rate, not the device, can set the pace.  Before timing, replays of one set's graph are
     checked bit for bit against an eager step (`config.graph_replays_match_eager`);
  2. K more steps in which every launch carries a pair of HIP events recorded
     on its kernel dispatch (la_time_next_launch): the per-kernel durations
     behind the roofline.  Those events cost host time per launch, which is why
     they stay out of region 1.
Then, for context only: K steps on a single buffer set (its inputs warm in the cache,
`config.warm_single_set_ms_per_step`) and a 1 GiB device copy (`roofline.copy_GBs_measured`,
the practical ceiling beside the 8 TB/s peak).  Prints one JSON line.

    python bench.py --floors             # launch floors: empty and streaming kernels (no arithmetic)
                                         # of the headline launches' sizes, timed the same ways
    python bench.py --copy-calibration   # one plain device copy of known size, for counter scaling
    python bench.py --counters-summary DIR
        # HBM bytes per launch of each kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE passes
        # (DIR/fetch_bench, DIR/write_bench over this benchmark; DIR/fetch_copy, DIR/write_copy
        # over --copy-calibration), written to profiles/ for the `traffic` field
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens·groups/s for linear-attn fwd+bwd at G=160,C=128,D=64; % roofline"
HEADLINE = "g160_c128_d64_bf16_fwdbwd"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, MI355X
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def algorithmic_bytes(G, C, D, esz, carry, upstream):
    """Bytes each kernel must move at minimum (inputs read once, outputs written once)."""
    tok = G * C * D * esz
    st = G * D * D * 4
    z = G * D * 4
    carry_b = st + z
    fwd = 3 * tok + tok + (carry_b if carry else 0) + carry_b            # q,k,v,[S_in,z_in] -> o,S_out,z_out
    bwd = 4 * tok + 3 * tok + (carry_b if carry else 0) + (carry_b if upstream else 0) + carry_b
    return fwd, bwd


def plan_seq_launches(G, T, D, esz, carry, upstream=False):
    """The two launches of a step through the sequence entry points, as the autograd layer makes
    them: one forward over all the chunks (carry in only if given; the final carry and its
    remainders out) and one backward (the final carry and its remainders in, the upstream
    gradient if given, the carry gradient out); no carry between chunks moves."""
    tok = G * T * D * esz
    carry_b = G * (D * D + D) * 4
    fwd = 4 * tok + (carry_b if carry else 0) + 2 * carry_b
    bwd = 7 * tok + 2 * carry_b + (carry_b if upstream else 0) + carry_b
    return [("seqfwd", T, fwd, 0), ("seqbwd", T, bwd, 0)]


def plan_launches(G, chunks, D, esz, carry):
    """One step's launches as (kind, chunk length, algorithmic bytes, chunk index): the forward
    over chunks 0..n-1 carrying (S, z), then the backward over chunks n-1..0 carrying (dS, dz).
    A chunk after the first always has a carry in; every backward but the last chunk's has an
    upstream (dS_out, dz_out)."""
    n = len(chunks)
    out = []
    for i, C in enumerate(chunks):
        out.append(("fwd", C, algorithmic_bytes(G, C, D, esz, carry or i > 0, False)[0], i))
    for i in range(n - 1, -1, -1):
        out.append(("bwd", chunks[i], algorithmic_bytes(G, chunks[i], D, esz, carry or i > 0, i < n - 1)[1], i))
    return out


# The sources each kernel is built from (beside the shared headers): counter-measured traffic is
# reported only for the build it was taken on, and an edit elsewhere does not void it.
KERNEL_SOURCES = {
    "la_fwd_c128": "la_fwd2.hip", "la_seq_fwd_c128": "la_fwd2.hip",
    "la_bwd_c128w16": "la_bwd4.hip", "la_seq_bwd_c128w16": "la_bwd4.hip",
    "la_seq_fwd_d128": "la_fwd_seq128.hip",
    "la_seq_bwd_d128": "la_bwd_seq128.hip", "la_bwd_d128": "la_bwd_seq128.hip",
    "la_fwd": "la_fwd.hip", "la_bwd": "la_bwd.hip",
    "la_cumsum_fwd": "la_cumsum.hip", "la_cumsum_bwd": "la_cumsum.hip",
}
SHARED_HEADERS = ("la_common.h", "la_tile.h")


def kernel_source_hash(kernel):
    """Hash of the sources `kernel` is built from: its own file and the shared headers (every
    attention source when the kernel is not in KERNEL_SOURCES)."""
    import glob
    csrc = os.path.join(ROOT, "causal_linear_attention_chunked_amd", "csrc")
    base = kernel[:-len("_kernel")] if kernel.endswith("_kernel") else kernel
    base = base[:-len("_elu1")] if base.endswith("_elu1") else base
    if base in KERNEL_SOURCES:
        files = [os.path.join(csrc, f) for f in (*SHARED_HEADERS, KERNEL_SOURCES[base])]
    else:
        files = [f for f in sorted(glob.glob(os.path.join(csrc, "*")))
                 if os.path.basename(f) not in ("la_ce.hip", "la_floor.hip")]
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload):
    return os.path.join(TRAFFIC_DIR, f"traffic_{workload}.json")


def measured_traffic(workload, kernel):
    """Counter-measured HBM bytes per launch of `kernel`, if taken on the current kernel source."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(kernel)
    if k is None or k.get("source_hash") != kernel_source_hash(kernel):
        return None
    return k.get("bytes_per_launch")


def counter_rows(d, counter):
    """(kernel name, value) for every dispatch in a rocprofv3 counter-collection output directory."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {d}")
    return rows


def counters_summary(d, workload, kernels):
    """Per-launch HBM bytes of each kernel: FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by
    what the same counters read for plain 256 MiB device copies (bench.py --copy-calibration)."""
    cal = 256 * 1024  # KiB moved each way by one calibration copy
    fc = max(v for _, v in counter_rows(os.path.join(d, "fetch_copy"), "FETCH_SIZE"))
    wc = max(v for _, v in counter_rows(os.path.join(d, "write_copy"), "WRITE_SIZE"))
    scale_f, scale_w = cal / fc, cal / wc
    out = {"workload": workload,
           "calibration": {"copy_KiB": cal, "fetch_KiB_read": fc, "write_KiB_read": wc,
                           "fetch_scale": scale_f, "write_scale": scale_w},
           "kernels": {}}
    fetch = counter_rows(os.path.join(d, "fetch_bench"), "FETCH_SIZE")
    write = counter_rows(os.path.join(d, "write_bench"), "WRITE_SIZE")
    for k in kernels:
        fv = [v for n, v in fetch if k in n]
        wv = [v for n, v in write if k in n]
        if not fv or not wv:
            continue
        fb = sum(fv) / len(fv) * scale_f * 1024
        wb = sum(wv) / len(wv) * scale_w * 1024
        out["kernels"][k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb,
                             "dispatches": [len(fv), len(wv)], "source_hash": kernel_source_hash(k)}
    with open(traffic_file(workload), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(I, w, min_seconds=10.0, mac_budget=2e9, feature=None, single_seconds=5.0):
    """The fp64 oracle as it stands, on this host's cores, over the workload's first groups
    (all of them when the workload is small), repeated; one call covers all the chunks.  Also
    timed on one thread, over at most `single_seconds`."""
    import oracle
    if feature == "elu1":
        ofwd = lambda *a, nthreads: oracle.features.fwd(*a, dtype=w.dtype, nthreads=nthreads)
        obwd = lambda *a, nthreads: oracle.features.bwd(*a, dtype=w.dtype, nthreads=nthreads)
    else:
        ofwd, obwd = oracle.fwd, oracle.bwd
    per_group = w.T * w.D * w.D
    g = w.G if w.G * per_group <= mac_budget else max(1, int(mac_budget // per_group))
    threads = min(os.cpu_count() or 1, g)
    sl = lambda x: None if x is None else x[:g]
    args = [sl(I[n]) for n in ("q", "k", "v", "S_in", "z_in")]
    dO = sl(I["dO"])
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        ofwd(*args, nthreads=threads)
        obwd(*args, dO, nthreads=threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= min_seconds and len(times) >= 3:
            break
    times.sort()
    med = times[len(times) // 2]
    # one thread: the first groups only, scaled to tokens.groups/s
    g1 = max(1, min(g, int(g * single_seconds / max(med * threads, 1e-9))))
    a1 = [None if x is None else x[:g1] for x in args]
    t0 = time.perf_counter()
    ofwd(*a1, nthreads=1)
    obwd(*a1, None if dO is None else dO[:g1], nthreads=1)
    t1 = time.perf_counter() - t0
    what = f"full {w.name} workload" if g == w.G else f"first {g} of the {w.G} groups of {w.name}"
    return {"value": g * w.T / med, "unit": "tokens·groups/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} (G={g}, {w.T} tokens, D={w.D}), forward+backward in fp64, "
                      f"median of {len(times)} repeats ({sum(times):.1f} s of CPU work)",
            "single_thread_value": g1 * w.T / t1, "single_thread_sample": f"first {g1} groups, one run",
            "cpu_model": cpu_model(), "host_threads": os.cpu_count()}


def copy_bandwidth(torch, gib=1, reps=5):
    """HBM bandwidth of a plain device-to-device copy of `gib` GiB (bytes read + written per
    second), the best of `reps`: the practical ceiling beside the 8 TB/s peak."""
    n = gib * (1 << 30) // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del src, dst
    return 2 * n * 4 / (best / 1e3) / 1e9


def copy_calibration(torch, mib=256, reps=5):
    """Plain copies of a known byte count: what FETCH_SIZE / WRITE_SIZE read for them scales the
    counters taken on the kernels to bytes."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n * 4, "bytes_written": n * 4, "launches": reps}}),
          flush=True)


def timed_runs(torch, fn, K):
    """K calls of fn() in up to five consecutive runs bracketed by device events: the per-call
    times of the runs, sorted, and the host seconds spent enqueuing."""
    per_run, host_s, _ = timed_block_runs(torch, lambda i0, n: [fn(i) for i in range(i0, i0 + n)], K)
    return per_run, host_s


def run_sizes(K, runs=5, min_steps=0):
    """Steps of each of up to `runs` consecutive timed runs (at least `min_steps` each where K allows)."""
    R = max(1, min(runs, K, K // min_steps if min_steps else K))
    return [K // R + (1 if r < K % R else 0) for r in range(R)]


def timed_block_runs(torch, run, K, sizes=None):
    """K steps in consecutive runs of `sizes` steps (default: up to five) bracketed by device
    events (synchronised before and after), `run(i0, n)` enqueuing steps i0 .. i0 + n - 1: the
    per-step times of the runs in ms, sorted, the host seconds spent enqueuing, and the total
    device ms."""
    sizes = sizes or run_sizes(K)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in sizes]
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    i = 0
    for (a, b), nsteps in zip(evs, sizes):
        a.record()
        run(i, nsteps)
        i += nsteps
        b.record()
    host_s = time.perf_counter() - h0
    torch.cuda.synchronize()
    total = sum(a.elapsed_time(b) for a, b in evs)
    return sorted(a.elapsed_time(b) / nsteps for (a, b), nsteps in zip(evs, sizes)), host_s, total


GRAPH_MIN_STEPS = 40  # steps per captured run: one replay's launch cost spread over at least these


def graph_matches_eager(torch, step, sets, outputs_of, replays=3):
    """Whether replays of a graph of one step on the first set give the bits of an eager step: the
    outputs are poisoned with NaN (eager work) before every replay and compared after it."""
    s = sets[0]
    step(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs_of(s)]
    g = RunGraphs(torch, lambda j: step(sets[j]), len(sets), [1])
    for _ in range(replays):
        for t in outputs_of(s):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.run(0, 1)
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(ref, outputs_of(s))):
            return False
    return True


class RunGraphs:
    """The timed runs of a benchmark captured in HIP graphs, one graph per run (kernel nodes only:
    the library's calls record no memset or copy), so that each run is one host call and the
    device, not the host's launch rate, sets the pace.  Run r's graph holds its steps i0 .. i0 +
    n - 1 on the buffer sets i mod nsets, the order of the plain loop.  One graph per run because a
    replay has a fixed cost of its own (over 10 us on this platform, measured): replaying a graph
    per step would add it to every step."""

    def __init__(self, torch, step_on_set, nsets, sizes):
        self.graphs = {}
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        i0 = 0
        for n in sizes:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(i0, i0 + n):
                    step_on_set(i % nsets)
            self.graphs[(i0, n)] = g
            i0 += n
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()

    def run(self, i0, n):
        self.graphs[(i0, n)].replay()

    def warm(self, torch, min_ms=50.0, max_rounds=2000):
        """Untimed replays of every graph, in order, for at least `min_ms` of wall time: the first
        replays upload the graphs, and the device reaches its working clocks whatever the number
        of timed steps (a short timed region would otherwise start from an idle device)."""
        t0 = time.perf_counter()
        for _ in range(max_rounds):
            for i0, n in self.graphs:
                self.run(i0, n)
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= min_ms:
                break


def bench_ce(args, w, torch, lac, inp):
    """The tied head's cross-entropy (Bottleneck #3 / Opt 3 of the pages): one step is la_ce_fwd
    and la_ce_bwd over the N tokens, inputs resident on the device.  Bound by MFMA: four products
    of 2 N V d flops each (the forward's logits; the backward's recomputed logits, dh and dW)."""
    N, d, V = w.N, w.d, w.V
    ce_chunk = args.ce_chunk or N  # tokens per backward chunk (0: all N at once)
    I = inp.ce_workload_inputs(w)
    ws_bytes = lac.ce_workspace_bytes(N, d, V, ce_chunk)
    set_bytes = V * d * 2 + V * d * 4 + 2 * N * d * 2 + ws_bytes  # W, dW, h, dh, workspace
    nsets = max(1, math.ceil(args.footprint_mb * 1e6 / set_bytes))
    dev = "cuda:0"
    sets = []
    for _ in range(nsets):
        s = {n: I[n].to(dev).contiguous() for n in ("h", "W", "targets")}
        s["fout"] = (torch.empty((), dtype=torch.float32, device=dev), torch.empty(N, dtype=torch.float32, device=dev))
        s["bout"] = (torch.empty_like(s["h"]), torch.empty((V, d), dtype=torch.float32, device=dev))
        s["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        sets.append(s)

    def fwd(s):
        lac.ce_fwd(s["h"], s["W"], s["targets"], workspace=s["ws"], out=s["fout"])

    def bwd(s):
        lac.ce_bwd(s["h"], s["W"], s["targets"], s["fout"][1], ce_chunk=ce_chunk, workspace=s["ws"], out=s["bout"])

    def step(i):
        fwd(sets[i % nsets])
        bwd(sets[i % nsets])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    per_run, host_s = timed_runs(torch, step, K)
    ms_per_step = per_run[len(per_run) // 2]
    # per entry point: events recorded on its first and last kernel dispatch
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2)]
          for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        s = sets[i % nsets]
        lac.time_next_launch(*ev[i][0])
        fwd(s)
        lac.time_next_launch(*ev[i][1])
        bwd(s)
    torch.cuda.synchronize()
    gemm = 2.0 * N * V * d
    entry = {}
    for j, (name, flops, kern) in enumerate((
            ("la_ce_fwd", gemm, "la_ce_fwd_kernel + la_ce_lse_kernel + la_ce_mean_kernel"),
            ("la_ce_bwd", 3 * gemm, "la_ce_p_kernel + la_ce_dh_kernel + la_ce_dh_reduce_kernel + la_ce_dw_kernel"))):
        us = sum(e[j][0].elapsed_time(e[j][1]) for e in ev) * 1e3 / K
        tf = flops / (us * 1e-6) / 1e12
        entry[name] = {"avg_us": us, "kernels": kern, "algorithmic_flops": flops, "TFLOP/s": tf,
                       "frac": tf / MFMA_BF16_PEAK_TFLOPS}
    top = "la_ce_bwd"
    kt = entry[top]
    out = {
        "metric": f"tokens/s for the tied-head cross-entropy fwd+bwd, {w.name}"
                  + (f", backward in chunks of {ce_chunk}" if ce_chunk != N else ""),
        "value": N / (ms_per_step / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "N": N, "d": d, "V": V, "ce_chunk": ce_chunk, "buffer_sets": nsets,
                   "footprint_mb": round(nsets * set_bytes / 1e6, 1), "workspace_bytes": ws_bytes,
                   "timed_runs": len(per_run), "ms_per_step_runs": per_run, "graph_captured": False,
                   "host_enqueue_us_per_step": host_s * 1e6 / K,
                   "kernel_timing": "HIP events on the first and last kernel dispatch of each entry point, "
                                    "separate timed loop"},
        "roofline": {"bound": "mfma", "kernel": f"{top} ({kt['kernels']})", "achieved": kt["TFLOP/s"],
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": kt["frac"], "traffic": None,
                     "algorithmic_flops": kt["algorithmic_flops"], "avg_us": kt["avg_us"]},
        "kernels": entry,
        "step_roofline_frac": 4 * gemm / (ms_per_step / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
    }
    if args.library_gemms:
        out["library_gemms"] = library_gemms(torch, N, d, V)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_ce(I, w)
    print(json.dumps(out), flush=True)


def library_gemms(torch, N, d, V, reps=20, runs=5):
    """The cross-entropy's four products as plain library GEMMs (torch.mm, hipBLASLt on ROCm) on
    the same shapes, bf16 in and out, each replayed `reps` times from a HIP graph: the vendor
    library's time for the bare products, beside which the fused kernels' times are read."""
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(0)
    h = torch.randn(N, d, device=dev, dtype=torch.bfloat16, generator=g)
    W = torch.randn(V, d, device=dev, dtype=torch.bfloat16, generator=g)
    P = torch.randn(N, V, device=dev, dtype=torch.bfloat16, generator=g)
    cases = {
        "logits W h^T (V x N)": lambda: torch.mm(W, h.t()),
        "logits h W^T (N x V)": lambda: torch.mm(h, W.t()),
        "dW = P^T h (V x d, k = N)": lambda: torch.mm(P.t(), h),
        "dh = P W (N x d, k = V)": lambda: torch.mm(P, W),
    }
    out = {}
    for name, f in cases.items():
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(3):
                f()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for _ in range(reps):
                f()
        gr.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(runs):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            gr.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / reps)
        us = sorted(ts)[len(ts) // 2]
        tf = 2.0 * N * V * d / (us * 1e-6) / 1e12
        out[name] = {"us": us, "TFLOP/s": tf, "frac": tf / MFMA_BF16_PEAK_TFLOPS}
    return out


def bench_floors(args, torch, lac, nwg=160):
    """Launch floors at the headline launches' sizes: an empty kernel, and streaming kernels (no
    arithmetic, every load issued up front) moving the forward's and the backward's bytes in
    `nwg` workgroups, on buffers rotated over the same footprint as the benchmark.  Each is timed
    as the attention kernels are: back to back from Python, replayed from HIP graphs, and one
    launch at a time between dispatch-bound events; and the two streaming kernels back to back
    as a step, the floor of a step of the two attention launches.  The same bytes again over four
    times the workgroups (128 threads each instead of 512): whether more workgroups lower it."""
    ib, ob = 81920 * nwg, 65536 * nwg  # the larger (backward) shape's bytes; the forward uses less
    nsets = max(2, math.ceil(args.footprint_mb * 1e6 / (ib + ob)))
    dev = "cuda:0"
    sets = [(torch.empty(ib, dtype=torch.uint8, device=dev).fill_(1), torch.empty(ob, dtype=torch.uint8, device=dev))
            for _ in range(nsets)]
    algo = {"empty": 0, "fwd": (65536 + 32768) * nwg, "bwd": (81920 + 65536) * nwg}
    algo.update(fwd_small=algo["fwd"], bwd_small=algo["bwd"])
    wgs = {"empty": nwg, "fwd": nwg, "bwd": nwg, "fwd_small": 4 * nwg, "bwd_small": 4 * nwg}  # same bytes
    K = args.steps
    out = {"floors": {}, "nwg": nwg, "threads": 512, "buffer_sets": nsets,
           "footprint_mb": round(nsets * (ib + ob) / 1e6, 1), "steps": K,
           "kernels": {k: lac.FLOOR_NAMES[lac.FLOOR_KINDS[k]] for k in lac.FLOOR_KINDS}}
    cases = [("empty", ["empty"]), ("fwd", ["fwd"]), ("bwd", ["bwd"]), ("fwd+bwd step", ["fwd", "bwd"]),
             ("fwd, 4x workgroups", ["fwd_small"]), ("bwd, 4x workgroups", ["bwd_small"]),
             ("fwd+bwd step, 4x workgroups", ["fwd_small", "bwd_small"])]
    for label, kinds in cases:
        def step_on(j, kinds=kinds):
            for kd in kinds:
                lac.floor_launch(kd, wgs[kd], sets[j][0], sets[j][1])
        for i in range(args.warmup):
            step_on(i % nsets)
        plain, _, _ = timed_block_runs(torch, lambda i0, n: [step_on(i % nsets) for i in range(i0, i0 + n)], K)
        sizes = run_sizes(K, min_steps=GRAPH_MIN_STEPS)
        graphs = RunGraphs(torch, step_on, nsets, sizes)
        graphs.warm(torch)
        graph, _, _ = timed_block_runs(torch, graphs.run, K, sizes)
        r = {"plain_us": plain[len(plain) // 2] * 1e3, "graph_us": graph[len(graph) // 2] * 1e3}
        if len(kinds) == 1:
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
            torch.cuda.synchronize()
            for i, (a, b) in enumerate(ev):
                lac.time_next_launch(a, b)
                step_on(i % nsets)
            torch.cuda.synchronize()
            d = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
            r.update({"dispatch_events_avg_us": sum(d) / K, "dispatch_events_median_us": d[K // 2],
                      "bytes": algo[kinds[0]]})
        else:
            r["bytes"] = sum(algo[kd] for kd in kinds)
        r["workgroups"] = [wgs[kd] for kd in kinds]
        if r["bytes"]:
            r["graph_frac_of_8TBs"] = r["bytes"] / (r["graph_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS
        out["floors"][label] = r
    print(json.dumps(out), flush=True)


def cpu_baseline_ce(I, w, min_seconds=10.0):
    """The fp64 oracle of the cross-entropy (numpy, its BLAS on every host thread), forward and
    backward over the full workload, repeated; and once on one BLAS thread."""
    from oracle import ce
    from threadpoolctl import threadpool_limits
    h, W, t = (I[n] for n in ("h", "W", "targets"))
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        ce.forward(h, W, t)
        ce.backward(h, W, t)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= min_seconds and len(times) >= 3:
            break
    times.sort()
    med = times[len(times) // 2]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        ce.forward(h, W, t)
        ce.backward(h, W, t)
        t1 = time.perf_counter() - t0
    return {"value": w.N / med, "unit": "tokens/s", "cores": os.cpu_count(), "kind": "oracle",
            "sample": f"full {w.name} workload (N={w.N}, d={w.d}, V={w.V}), forward+backward in fp64 "
                      f"(numpy BLAS), median of {len(times)} repeats ({sum(times):.1f} s of CPU work)",
            "single_thread_value": w.N / t1, "single_thread_sample": "full workload, one run, one BLAS thread",
            "cpu_model": cpu_model(), "host_threads": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seq", action="store_true",
                    help="run the workload through the sequence entry points (one launch per direction)")
    ap.add_argument("--block", type=int, choices=[1, 64], default=None,
                    help="chunk entry points: 64, the blocked (chunked) form; 1, the cumsum form "
                         "(the per-token recurrence); default the workload's")
    ap.add_argument("--feature", choices=["elu1"], default=None,
                    help="with --seq: raw q, k in, the feature map elu(x)+1 fused into the kernels")
    ap.add_argument("--footprint-mb", type=float, default=640.0)
    ap.add_argument("--no-graph", action="store_true",
                    help="time the plain loop of library calls only (no HIP graph capture)")
    ap.add_argument("--floors", action="store_true",
                    help="time the launch-floor kernels (no arithmetic) of the headline launches' sizes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only plain 256 MiB device-to-device copies (HBM counter calibration)")
    ap.add_argument("--ce-chunk", type=int, default=0,
                    help="cross-entropy workloads: tokens per backward chunk (default: all N at once)")
    ap.add_argument("--library-gemms", action="store_true",
                    help="cross-entropy workloads: also time the four products as plain torch.mm GEMMs")
    ap.add_argument("--counters-summary", metavar="DIR",
                    help="turn rocprofv3 FETCH_SIZE/WRITE_SIZE passes under DIR into per-launch HBM bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(groups shard across GPUs with no communication, so one GPU's share is the measurement)",
              file=sys.stderr)
        sys.exit(2)

    if args.counters_summary:
        import causal_linear_attention_chunked_amd as lac
        from causal_linear_attention_chunked_amd import inputs as inp
        w = inp.workload(args.workload)
        names = {lac.kernel_name(b, w.dtype, C, w.D, blk, f) for b in (False, True) for C in set(w.chunks)
                 for blk in (1, 64) for f in (None, "elu1")} - {None}
        names |= {lac.seq_kernel_name(b, w.dtype, max(w.chunks), w.D, f) for b in (False, True)
                  for f in (None, "elu1")} - {None}
        counters_summary(args.counters_summary, w.name + ("_seq" if args.seq else "")
                         + (f"_{args.feature}" if args.feature else "")
                         + ("_block1" if args.block == 1 else ""), sorted(names))
        return
    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import causal_linear_attention_chunked_amd as lac
    from causal_linear_attention_chunked_amd import inputs as inp

    lac.load_library()
    if args.floors:
        return bench_floors(args, torch, lac)
    if args.workload in inp.CE_WORKLOADS:
        return bench_ce(args, inp.ce_workload(args.workload), torch, lac, inp)
    w = inp.workload(args.workload)
    if not w.backward:
        raise SystemExit("bench.py times forward+backward workloads")
    block = w.block if args.block is None else args.block
    if args.seq and block != 64:
        raise SystemExit("--seq runs the blocked form (block 64) only")
    I = inp.make_inputs(G=w.G, T=w.T, D=w.D, dtype=w.dtype, carry=w.carry, backward=w.backward, seed=w.seed,
                        prior_len=w.prior_len, features="raw" if args.feature else "mapped")
    dev = torch.device("cuda:0")
    esz = 2 if w.dtype == "bf16" else 4
    G, D = w.G, w.D
    bounds = inp.chunk_bounds(w.chunks)
    n = len(bounds)
    carry = I["S_in"] is not None

    tname = (w.name + ("_seq" if args.seq else "") + (f"_{args.feature}" if args.feature else "")
             + ("_block1" if block == 1 else ""))  # and the traffic file
    if args.seq:
        # equal chunks but for a shorter last one
        regular = len(set(w.chunks[:-1])) <= 1 and w.chunks[-1] <= w.chunks[0]
        if not regular or not lac.seq_supported(w.dtype, w.T, D, w.chunks[0], args.feature):
            raise SystemExit(f"{w.name}: the sequence entry points do not take this workload")
        launches = plan_seq_launches(G, w.T, D, esz, carry)
    else:
        launches = plan_launches(G, w.chunks, D, esz, carry)
    set_bytes = sum(b for _, _, b, _ in launches)
    nsets = max(1, math.ceil(args.footprint_mb * 1e6 / set_bytes))

    def new_set():
        s = {"chunks": []}
        if args.seq:
            s["seq"] = {x: I[x].to(dev).contiguous() for x in ("q", "k", "v", "dO")}
            q = s["seq"]["q"]
            s["seq"]["fout"] = (torch.empty_like(q), torch.empty((G, D, D), device=dev),
                                torch.empty((G, D), device=dev), torch.empty((G, D, D), device=dev),
                                torch.empty((G, D), device=dev))
            s["seq"]["bout"] = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q),
                                torch.empty((G, D, D), device=dev), torch.empty((G, D), device=dev))
            s["S_in"] = None if I["S_in"] is None else I["S_in"].to(dev).contiguous()
            s["z_in"] = None if I["z_in"] is None else I["z_in"].to(dev).contiguous()
            return s
        for t0, t1 in bounds:
            c = {x: I[x][:, t0:t1].to(dev).contiguous() for x in ("q", "k", "v", "dO")}
            C = t1 - t0
            c["fout"] = (torch.empty_like(c["q"]), torch.empty((G, D, D), device=dev),
                         torch.empty((G, D), device=dev))
            c["bout"] = (torch.empty_like(c["q"]), torch.empty_like(c["q"]), torch.empty_like(c["q"]),
                         torch.empty((G, D, D), device=dev), torch.empty((G, D), device=dev))
            s["chunks"].append(c)
        s["S_in"] = None if I["S_in"] is None else I["S_in"].to(dev).contiguous()
        s["z_in"] = None if I["z_in"] is None else I["z_in"].to(dev).contiguous()
        return s

    sets = [new_set() for _ in range(nsets)]

    def carry_in(s, i):
        if i == 0:
            return s["S_in"], s["z_in"]
        prev = s["chunks"][i - 1]["fout"]
        return prev[1], prev[2]

    def launch(s, kind, i):
        if kind == "seqfwd":
            x = s["seq"]
            lac.seq_fwd(x["q"], x["k"], x["v"], s["S_in"], s["z_in"], out=x["fout"], feature=args.feature,
                        residual=True)
            return
        if kind == "seqbwd":
            x = s["seq"]
            lac.seq_bwd(x["q"], x["k"], x["v"], x["fout"][1], x["fout"][2], x["dO"], out=x["bout"],
                        feature=args.feature, S_res=x["fout"][3], z_res=x["fout"][4])
            return
        c = s["chunks"][i]
        S, z = carry_in(s, i)
        if kind == "fwd":
            lac.fwd(c["q"], c["k"], c["v"], S, z, block=block, out=c["fout"], feature=args.feature)
        else:
            up = s["chunks"][i + 1]["bout"] if i + 1 < n else None
            lac.bwd(c["q"], c["k"], c["v"], S, z, c["dO"], None if up is None else up[3],
                    None if up is None else up[4], block=block, out=c["bout"], feature=args.feature)

    def step(s):
        for kind, _, _, i in launches:
            launch(s, kind, i)

    def outputs_of(s):
        if args.seq:
            return [t for t in (*s["seq"]["fout"], *s["seq"]["bout"]) if t is not None]
        return [t for c in s["chunks"] for t in (*c["fout"], *c["bout"])]

    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()

    K = args.steps
    # region 1: K steps in up to five consecutive runs (the median run's per-step time is the
    # result; the mean over all K is reported beside it), replayed from HIP graphs so that the
    # device, not the host's launch rate, sets the pace; the same K steps as plain library calls
    # from Python are timed beside them
    plain_runs, plain_host_s, plain_total = timed_block_runs(
        torch, lambda i0, nst: [step(sets[i % nsets]) for i in range(i0, i0 + nst)], K)
    graphs, graph_error, graph_check = None, None, None
    sizes = run_sizes(K, min_steps=GRAPH_MIN_STEPS)
    if not args.no_graph:
        try:
            graph_check = graph_matches_eager(torch, step, sets, outputs_of)
            graphs = RunGraphs(torch, lambda j: step(sets[j]), nsets, sizes)
            graphs.warm(torch)
        except Exception as e:  # reported; the plain loop then gives the result
            graphs, graph_error = None, repr(e)
    if graphs is not None:
        per_run, host_s, total_ms = timed_block_runs(torch, graphs.run, K, sizes)
    else:
        per_run, host_s, total_ms = plain_runs, plain_host_s, plain_total
    ms_per_step = per_run[len(per_run) // 2]
    ms_per_step_mean = total_ms / K
    value = G * w.T / (ms_per_step / 1e3)

    # region 2: the same steps with dispatch-bound events on every launch
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in launches]
          for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        s = sets[i % nsets]
        for (kind, _, _, c), e in zip(launches, ev[i]):
            lac.time_next_launch(e[0], e[1])
            launch(s, kind, c)
    torch.cuda.synchronize()

    # warm: the same steps on one buffer set, whose inputs then sit in the last-level cache
    # (labelled; not the measurement)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(K):
        step(sets[0])
    b.record()
    torch.cuda.synchronize()
    warm_ms = a.elapsed_time(b) / K
    copy_gbs = copy_bandwidth(torch)

    # per kernel: launches, total bytes and total time over the K steps
    per = {}
    for i in range(K):
        for (kind, C, b, _), e in zip(launches, ev[i]):
            name = (lac.seq_kernel_name(kind == "seqbwd", w.dtype, max(w.chunks), D, args.feature)
                    if kind.startswith("seq")
                    else lac.kernel_name(kind == "bwd", w.dtype, C, D, block, args.feature))
            p = per.setdefault(name, {"launches": 0, "bytes": 0, "ms": 0.0})
            p["launches"] += 1
            p["bytes"] += b
            p["ms"] += e[0].elapsed_time(e[1])
    kernels = {}
    for name, p in per.items():
        gbs = p["bytes"] / (p["ms"] / 1e3) / 1e9
        kernels[name] = {"avg_us": p["ms"] * 1e3 / p["launches"], "launches_per_step": p["launches"] // K,
                         "algorithmic_bytes": p["bytes"] / p["launches"], "GB/s": gbs, "frac": gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic(tname, name)}
    # the roofline names the kernel with the most time per step
    top = max(per, key=lambda k: per[k]["ms"])
    kt = kernels[top]
    out = {
        "metric": (METRIC if tname == HEADLINE
                   else f"tokens·groups/s for linear-attn fwd+bwd, {tname}"),
        "value": value, "unit": "tokens·groups/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "G": G, "T": w.T, "chunks": n, "C": max(w.chunks), "D": D,
                   "block": block, "carry": w.carry, "launches_per_step": len(launches),
                   "buffer_sets": nsets, "footprint_mb": round(nsets * set_bytes / 1e6, 1),
                   "entry_points": "la_seq_fwd/la_seq_bwd" if args.seq else "la_chunk_fwd/la_chunk_bwd",
                   "timed_runs": len(per_run), "ms_per_step_runs": per_run, "ms_per_step_mean": ms_per_step_mean,
                   "warm_single_set_ms_per_step": warm_ms,
                   "feature_map": args.feature or "applied by the caller",
                   "graph_captured": graphs is not None, "graph_error": graph_error,
                   "graph_replays_match_eager": graph_check,
                   "host_enqueue_us_per_step": host_s * 1e6 / K,
                   "plain_loop_ms_per_step": plain_runs[len(plain_runs) // 2],
                   "plain_loop_ms_per_step_runs": plain_runs,
                   "plain_loop_host_enqueue_us_per_step": plain_host_s * 1e6 / K,
                   "kernel_timing": "HIP events recorded on each kernel dispatch, separate timed loop"},
        "roofline": {"bound": "hbm", "kernel": top, "achieved": kt["GB/s"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": kt["frac"], "traffic": kt["traffic"],
                     "algorithmic_bytes": kt["algorithmic_bytes"], "avg_us": kt["avg_us"],
                     "copy_GBs_measured": copy_gbs, "frac_of_copy": kt["GB/s"] / copy_gbs},
        "kernels": kernels,
        "step_roofline_frac": set_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS,
    }
    if tname == HEADLINE:
        # the pages' own figure for this shape (context, another machine, not the target): their
        # CPU micro-benchmark of the chunked form, fp32, forward+backward 72.4 ms at G=160, C=128, D=64
        out["context"] = {"pages_cpu_fwdbwd_tokens_groups_per_s": 160 * 128 / 72.4e-3,
                          "source": "Fractus-1B training optimization, CPU benchmark of the chunked form "
                                    "(fp32 PyTorch, CPU model not stated)"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(I, w, feature=args.feature)
    print(json.dumps(out), flush=True)

if __name__ == "__main__":
    main()
