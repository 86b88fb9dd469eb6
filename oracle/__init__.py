"""CPU oracle for segment-causal attention over a lifelong INT8 KV cache.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow definition that the
GPU library is checked against.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path (the HIP
library and its Python binding) never does, and this package imports nothing
from it.  The two share no code, tables or constants; only the seeded input
generator in ``synth`` feeds both.

Modules
  nomas_ref  numpy float64 definitions (token layout, 3D RoPE, INT8
             quantiser, segment-causal attention and its gradients for
             packed training sequences, decoder window attention, the
             INT8-weight linear layer, camera tokens and camera
             cross-attention), chunked only over independent (head, query
             block) pieces.
  brute      pure-Python loops with math.fsum / fractions.Fraction, for tiny
             inputs; written separately so that it pins nomas_ref.

Parity status: every function is pinned by the not-gpu tests (brute force,
closed forms, invariants, special cases; the gradients by finite differences
of the pinned forward and by torch autograd).  The match to the released Hy-Nomas
model itself (RoPE pair convention, text-token positions, scale layout) is
"parity unpinned": the pages give no code, weights or worked example.
"""
from . import nomas_ref, brute  # noqa: F401
from .nomas_ref import *  # noqa: F401,F403
