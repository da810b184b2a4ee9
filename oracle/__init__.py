"""CPU oracle for causal linear attention with a carried state.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import anything from this package.  It shares
no code with the GPU library and never imports it.

* :mod:`oracle.core`   -- ctypes front end of ``la_oracle.c``: the per-token fp64
  recurrence (forward) and reverse scan (backward), OpenMP over groups.
* :mod:`oracle.forms`  -- independent numpy fp64 forms used to cross-check it: the
  masked-einsum form, the blocked form at any block size, and the whole-chunk
  matrix backward.
* :mod:`oracle.exact`  -- exact rational brute force (fractions + dual numbers)
  for tiny shapes; writes the stored golden values.
* :mod:`oracle.features` -- the positive feature map elu(x) + 1 in front of the op
  (raw inputs in, gradients with respect to them out), by the chain rule.
* :mod:`oracle.ce` -- the cross-entropy over the tied output head (the pages' third
  bottleneck and its chunked, checkpointed form), fp64.

Every function cites the passage of "Fractus-1B training optimization" it
follows.  Which pins cover which function is listed in the test suite.
"""
from .core import build, fwd, bwd, lib_path, max_threads  # noqa: F401
from . import features  # noqa: F401
from . import ce  # noqa: F401
