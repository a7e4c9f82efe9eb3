"""CPU oracle for exact softmax attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 numpy code that evaluates the definition of attention directly
(scores, mask, softmax, dropout, weighted sum of values) and materialises the
N x N score and probability matrices, plus an independent Philox4x32-10
generator for the dropout keep-mask.

Only the test-suite, the package smoke check and the CPU-baseline leg of the
benchmark may import this package. The GPU library never calls it, links it or
falls back to it; it shares no code with the HIP kernels.

Modules
  philox         Philox4x32-10 block function and the dropout keep rule.
  attention      forward / backward of attention by definition (fp64).
  online_softmax fp64 model of the tiled online-softmax recurrence, used to
                 show that tiling reproduces the definition exactly.

Every function is pinned by CPU tests in ``tests/test_oracle_*.py`` against
closed forms, invariants, brute force and library routines; none is
"parity unpinned".
"""
from . import philox, attention, online_softmax  # noqa: F401
