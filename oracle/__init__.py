"""CPU oracle for the dual-phase policy step -- TEST INFRASTRUCTURE, NOT PRODUCT.

A plain, slow, readable numpy implementation of what the policy step computes,
in float64 unless the method itself fixes a precision (the ternary quantizer of
Eq. 4 works in float32 and rounds its outputs to bfloat16).  It exists to prove
the HIP library right.  Only the test suite, the smoke check of the build entry
point and the CPU-baseline leg of the benchmark may import or run anything in
this package; the library and its Python binding never do, and the oracle never
imports them.  It shares no code with the GPU path: inputs come from the seeded
generator module, which holds no arithmetic of the method.

Sources ("the paper" below is *vla.cpp: A Unified Inference Runtime for
Vision-Language-Action Models*, arXiv 2606.08094; "the reading notes" are the
paper.gecl.asia notes on the same paper):

  * Euler flow-matching solver ............ the paper, §III-A, Eq. 1
  * cross-attention over cached K/V ....... the paper, §III-B, Eq. 2
  * bidirectional prefix, hidden states
    taken before the LM output projection .. the reading notes, Method points 1-3
  * ternary W2A8 linear ................... the paper, §III-D, Eq. 4
  * action-space error metrics ............ the paper, §III-E, Eq. 5

Pieces the pages do not specify (RMSNorm placement and form, the GeGLU MLP, the
sinusoidal time embedding, the expert's self-attention over chunk tokens, the
weight layout) follow the plainest reading; each function says which.

Pins: every function here is checked in tests/ against something other than
itself (brute force on tiny inputs, closed forms, invariants, library routines,
hand-computed fixtures under tests/golden/).  The whole-model composition at the
large workload sizes has no printed output on the pages to compare with; it is
pinned only through its parts and through structural invariants (token
permutation equivariance, zero-weight identities, cached == recompute), and a
float32-vs-float64 self-consistency check.
"""
from .policy import (  # noqa: F401
    rms_norm, gelu, attention, time_embedding, linear, uniform_schedule,
    euler_integrate, prefix_layer, encode_prefix, cache_project, velocity,
    denoise, denoise_recompute, run_policy, Oracle,
)
from .ternary import (  # noqa: F401
    bf16_round, quantize_rows, w2a8_accumulate, w2a8_linear, w2a8_linear_grouped, pack_ternary,
    unpack_ternary,
)
from .metrics import e_inf, e_rel  # noqa: F401
