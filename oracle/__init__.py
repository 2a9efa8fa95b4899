"""CPU oracle of the grouped-linear hot path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct float64 numpy code written from the pages that
define the method (TransformerEngine's GroupedLinear and the pull requests
around it).  It shares no code with the HIP library in ``grouped_gemm_gl_amd``
and never imports it; the library never imports this package.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import, call or run anything here.  The product path must not.

Modules
  grouped_linear  split offsets, grouped forward, dgrad, wgrad, bias grad
  mxfp8           OCP MX E4M3 block quantizer (E8M0 scales), rowwise and columnwise
                  (per group, stored transposed), its decoder, and the MXFP8 forward,
                  dgrad and wgrad on dequantized operands
  grouped_mlp     FC1 -> SwiGLU -> FC2 over the same splits, forward and backward

Every function here is pinned by ``tests/test_oracle_*.py`` against something
other than itself (library identities, autograd, closed forms, hand-worked
examples, exhaustive library cross-checks).
"""
from . import grouped_linear, grouped_mlp, mxfp8  # noqa: F401
from .grouped_linear import offsets, forward, dgrad, wgrad, bgrad, group_of_rows  # noqa: F401
from .mxfp8 import (  # noqa: F401
    e4m3_round, e4m3_encode, e4m3_decode, quantize_mxfp8, dequantize_mxfp8, forward_mxfp8,
    COLWISE_ALIGN, colwise_offsets, quantize_mxfp8_colwise, quantize_mxfp8_colwise_weights, dgrad_mxfp8,
    wgrad_mxfp8,
)
from .grouped_mlp import silu, swiglu, swiglu_backward, mlp_forward, mlp_backward, store  # noqa: F401
