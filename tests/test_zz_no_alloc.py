"""moe_layer_forward_noalloc (the entry point for callers that cannot
allocate: its workspace is the library's static device array) against
moe_layer_forward on the same inputs with a caller workspace: the same
kernels in the same order, so the outputs and the routing must be equal bit
for bit. Two calls in a row, the second with a smaller batch, so the second
runs on the first call's leftover scratch contents; each is also checked
against the CPU oracle within the bf16 bound."""

import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_sparse_amd.binding as B
from gpu_helpers import check_out, check_routing, device_inputs, oracle_logits_scores, say
import oracle.moe_oracle as O
from moe_inputs import generate, small_spec, spec_by_name

pytestmark = pytest.mark.gpu


def _weights(d):
    return {n: d.get(n) for n in ("w_router", "b_router", "w_gate", "w_up", "w_down", "ws_gate",
                                  "ws_up", "ws_down", "w_shared_gate", "w_gate_sb", "w_up_sb",
                                  "w_down_sb")}


def _both(inp, d, T):
    spec = inp["spec"]
    cfg = B.config_from_spec(spec, T)
    x = d["x"][:T]
    outs = {}
    for how in ("noalloc", "workspace"):
        ids = torch.full((T, spec.k), -1, dtype=torch.int32, device="cuda")
        gates = torch.full((T, spec.k), -1.0, dtype=torch.float32, device="cuda")
        counts = torch.full((spec.E,), -1, dtype=torch.int32, device="cuda")
        if how == "noalloc":
            out = B.layer_forward_noalloc(cfg, _weights(d), x, ids=ids, gates=gates, counts=counts)
        else:
            out = B.layer_forward(cfg, _weights(d), x, ids=ids, gates=gates, counts=counts)
        torch.cuda.synchronize()
        outs[how] = (out, ids, gates, counts)
    a, b = outs["noalloc"], outs["workspace"]
    for n, u, v in zip(("out", "ids", "gates", "counts"), a, b):
        assert torch.equal(u, v), f"{n} differs between the no-alloc and workspace calls"
    # and the oracle, on the same batch
    sub_spec = spec.with_T(T) if spec.x_rows else dataclasses.replace(spec, T=T)
    sub = dict(inp, spec=sub_spec, x=inp["x"][:T])
    L, S = oracle_logits_scores(sub)
    gids = a[1].cpu().numpy().astype(np.int64)
    _, mism = check_routing(S, gids, spec.k)
    ref = O.layer_forward(sub, ids_override={int(t): gids[t] for t in mism})
    check_out(a[0].float().cpu().numpy().astype(np.float64), ref["out"], spec.dtype,
              f"no-alloc out T={T}")


@pytest.mark.parametrize("name,T1,T2", [
    ("decode", 64, 16),          # full decode shape, then a smaller batch
    ("decode", 4, 1),            # the few-token and one-token launch sequences
    ("shared_small", 700, 300),  # several route blocks and tiled GEMMs, shared expert
])
def test_noalloc_matches_workspace_entry(name, T1, T2):
    if name == "decode":
        inp = generate(spec_by_name("decode@T64"))
    else:
        inp = generate(small_spec("shared_routed", T=T1, d=264, E=12, h=96, k=4, shared_h=376))
    d = device_inputs(inp)
    for T in (T1, T2):
        say(f"[no-alloc] {name}: T={T}")
        _both(inp, d, T)


def test_noalloc_rejects_oversize_on_gpu():
    spec = spec_by_name("skewed_prefill")
    cfg = B.config_from_spec(spec)
    assert B.workspace_size(cfg) > B.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((16, spec.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.layer_forward_noalloc(cfg, {"w_router": x, "w_gate": x, "w_up": x, "w_down": x}, x)
    assert ei.value.status == B.MOE_ERR_SCRATCH_LIMIT
