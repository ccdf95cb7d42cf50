"""CPU oracle for the sparse MoE FFN layer forward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. It shares no code with the HIP path.
"""

from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (  # noqa: F401
    combine, dispatch, down, expert_ffn, gate_up, gate_weights, layer_forward,
    near_ties, route, router_logits, shared_expert, sigmoid, silu, softmax,
    swiglu, to_f64, token_forward, topk_select,
)
