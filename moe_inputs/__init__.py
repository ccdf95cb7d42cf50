"""Seeded synthetic inputs for the sparse MoE FFN layer forward.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark. It holds input *construction* only (random draws, the bf16
round-to-nearest-even cast, the weight layouts); none of the layer's own
arithmetic (routing, selection, gating, expert FFN, combine) lives here.

Layouts (row-major, the shapes of "Tutorial 11: Mixture of Experts (MoE)",
section 4 "The Complete MoE Layer"):
    x         [T, d]
    w_router  [E, d]
    w_gate    [E, h, d]      w_up [E, h, d]      w_down [E, d, h]
    b_router  [E]   float32  (optional)
    ws_gate   [hs, d], ws_up [hs, d], ws_down [d, hs]  (optional shared expert)
    w_shared_gate [d]                                   (optional sigmoid gate)

bf16 tensors are returned as ``numpy.uint16`` arrays holding the bf16 bit
patterns; fp32 tensors as ``numpy.float32``.
"""

from .spec import (  # noqa: F401
    MoESpec,
    SPECS,
    spec_by_name,
    small_spec,
)
from .generate import (  # noqa: F401
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    generate,
)
