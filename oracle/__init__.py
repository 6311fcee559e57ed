"""Oracle for the chunk-wise test-time-training fast-weight layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 NumPy
statement of what the layer computes, written from the pages' equations.
Only the test suite, the smoke check and the bench's CPU-baseline leg may
import it; the product path (the HIP library and its Python binding) never
does, and shares no code, table or constant with it.

Modules:
  inplace  -- the In-Place TTT layer: gated-MLP producer, causal conv target,
              apply-then-update over chunks (dot-product and MSE objectives),
              and the three-step prefix-sum form of the dot-product update.
  lact     -- the LaCT SwiGLU fast weight: full-chunk MSE gradient, plain GD,
              update-then-apply (or apply-then-update) over chunks.

Every function is pinned by the CPU tests against something other than
itself (library routines, closed forms, brute force, finite differences,
autograd).  Nothing here is "parity unpinned".
"""
from . import inplace, lact  # noqa: F401
