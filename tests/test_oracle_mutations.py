"""Plant plausible mistakes in the oracle (on the CPU) and check that at
least one pin fails for each. This shows the pins constrain every step:
selection, gating, dispatch, expert FFN, combine, shared expert, bias, and
the backward (SwiGLU derivative, gate-to-logit derivative, weight grads)."""

import numpy as np
import pytest

import oracle.moe_oracle as O
import oracle_pins as pins


def _topk_ties_high(L, k):
    E = L.shape[1]
    rev = np.argsort(-L[:, ::-1], axis=1, kind="stable")[:, :k]
    return (E - 1 - rev).astype(np.int64)


def _gates_no_renorm(L, ids, mode, renormalize):
    return _ORIG["gate_weights"](L, ids, mode, False)


def _gates_selected_as_all(L, ids, mode, renormalize):
    if mode == O.SOFTMAX_SELECTED:
        mode = O.SOFTMAX_ALL
    return _ORIG["gate_weights"](L, ids, mode, renormalize)


def _dispatch_unstable(ids, E):
    counts, offsets, perm, inv = _ORIG["dispatch"](ids, E)
    perm = perm.copy()
    for e in range(E):
        perm[offsets[e]:offsets[e + 1]] = perm[offsets[e]:offsets[e + 1]][::-1]
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    return counts, offsets, perm, inv


def _combine_wrong_index(y_sorted, inv, gates, shared=None):
    T, k = gates.shape
    perm = np.empty_like(inv)
    perm[inv] = np.arange(inv.size)
    return _ORIG["combine"](y_sorted, perm, gates, shared)


def _silu_dropped_z(z):
    return 1.0 / (1.0 + np.exp(-z))


def _gate_up_swapped(x, perm, offsets, k, w_gate, w_up):
    return _ORIG["gate_up"](x, perm, offsets, k, w_up, w_gate)


def _gate_up_token_mod(x, perm, offsets, k, w_gate, w_up):
    # wrong token index: pair % k instead of pair // k
    X = O.to_f64(x)
    E, h, _ = w_gate.shape
    act = np.zeros((perm.size, h))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r0 == r1:
            continue
        Xe = X[perm[r0:r1] % k]
        act[r0:r1] = O.silu(Xe @ O.to_f64(w_gate[e]).T) * (Xe @ O.to_f64(w_up[e]).T)
    return act


def _down_transposed(act, offsets, w_down):
    return _ORIG["down"](act, offsets, np.swapaxes(w_down, 1, 2))


def _shared_ungated(x, ws_gate, ws_up, ws_down, w_shared_gate=None):
    return _ORIG["shared_expert"](x, ws_gate, ws_up, ws_down, None)


def _logits_no_bias(x, w_router, b_router=None):
    return _ORIG["router_logits"](x, w_router, None)


def _combine_drop_last_slot(y_sorted, inv, gates, shared=None):
    g = gates.copy()
    g[:, -1] = 0.0
    return _ORIG["combine"](y_sorted, inv, g, shared)


def _sigmoid_gates_biased(L, ids, mode, renormalize):
    # the selection bias leaking into the gates: gate with a softmax of the
    # selected logits instead of the raw affinities
    if mode == O.SIGMOID:
        mode = O.SOFTMAX_SELECTED
    return _ORIG["gate_weights"](L, ids, mode, renormalize)


def _selection_ignores_bias(L, mode, sel_bias=None):
    return _ORIG["selection_scores"](L, mode, None)


def _selection_bias_inside_sigmoid(L, mode, sel_bias=None):
    if mode == O.SIGMOID and sel_bias is not None:
        return O.sigmoid(L + O.to_f64(sel_bias)[None, :])
    return _ORIG["selection_scores"](L, mode, sel_bias)


def _stats_share_over_T(L, counts, k, mode, alpha):
    share, P, H, aux = _ORIG["routing_stats"](L, counts, k, mode, alpha)
    return share * k, P, H, aux


def _stats_entropy_sign(L, counts, k, mode, alpha):
    share, P, H, aux = _ORIG["routing_stats"](L, counts, k, mode, alpha)
    return share, P, -H, aux


def _stats_aux_without_N(L, counts, k, mode, alpha):
    share, P, H, aux = _ORIG["routing_stats"](L, counts, k, mode, alpha)
    return share, P, H, aux / L.shape[1]


def _q4_nibbles_swapped(packed, sb):
    p = np.asarray(packed, dtype=np.uint8)
    return _ORIG["dequantize_q4"](((p & 15) << 4) | (p >> 4), sb)


def _q4_scale_bias_swapped(packed, sb):
    sb = np.asarray(sb, dtype=np.uint32)
    return _ORIG["dequantize_q4"](packed, (sb >> 16) | ((sb & 0xFFFF) << 16))


def _q4_group_of_32(packed, sb):
    # scales indexed per 32 positions instead of 64
    sb = np.asarray(sb, dtype=np.uint32)
    half = np.repeat(sb, 2, axis=-1)[..., : sb.shape[-1]]
    return _ORIG["dequantize_q4"](packed, half)


def _silu_grad_no_curvature(z):
    # d silu / dz taken as sigmoid(z) alone
    return O.sigmoid(z)


def _logit_grad_sign(L, ids, g, dG, mode, renormalize):
    return -_ORIG["gate_logit_grad"](L, ids, g, dG, mode, renormalize)


def _logit_grad_renorm_ignored(L, ids, g, dG, mode, renormalize):
    return _ORIG["gate_logit_grad"](L, ids, g, dG, mode, False)


def _swiglu_bwd_up_uses_z(X, Wg, Wu, Wd, dY):
    # the up-projection gradient scaled by z_g instead of silu(z_g)
    zg, zu = X @ Wg.T, X @ Wu.T
    a = O.silu(zg) * zu
    da = dY @ Wd
    dzg = da * zu * O.silu_grad(zg)
    dzu = da * zg
    return dzg @ Wg + dzu @ Wu, dzg.T @ X, dzu.T @ X, dY.T @ a


def _swiglu_bwd_down_from_preactivation(X, Wg, Wu, Wd, dY):
    dX, dWg, dWu, _ = _ORIG["swiglu_backward"](X, Wg, Wu, Wd, dY)
    return dX, dWg, dWu, dY.T @ (X @ Wu.T)


def _bf16_shift8(a):
    # bf16 bits placed 8 bits too low in the float32 word
    if a is not None and np.asarray(a).dtype == np.uint16:
        return (np.asarray(a).astype(np.uint32) << np.uint32(8)).view(np.float32).astype(np.float64)
    return _ORIG["to_f64"](a)


def _q4_up_with_gate_scales(inp):
    # the up projection's codes paired with the gate projection's scale words
    if inp.get("w_gate_sb") is not None:
        return (O.dequantize_q4(inp["w_gate"], inp["w_gate_sb"]),
                O.dequantize_q4(inp["w_up"], inp["w_gate_sb"]),
                O.dequantize_q4(inp["w_down"], inp["w_down_sb"]))
    return _ORIG["expert_weights"](inp)


_ORIG = {n: getattr(O, n) for n in ("to_f64", "expert_weights", "gate_weights", "dispatch", "combine", "gate_up",
                                    "down", "shared_expert", "router_logits", "topk_select",
                                    "silu", "selection_scores", "routing_stats",
                                    "dequantize_q4", "gate_logit_grad", "swiglu_backward")}

MUTATIONS = [
    ("topk_select", _topk_ties_high),
    ("gate_weights", _gates_no_renorm),
    ("gate_weights", _gates_selected_as_all),
    ("dispatch", _dispatch_unstable),
    ("combine", _combine_wrong_index),
    ("combine", _combine_drop_last_slot),
    ("silu", _silu_dropped_z),
    ("gate_up", _gate_up_swapped),
    ("gate_up", _gate_up_token_mod),
    ("down", _down_transposed),
    ("shared_expert", _shared_ungated),
    ("router_logits", _logits_no_bias),
    ("gate_weights", _sigmoid_gates_biased),
    ("selection_scores", _selection_ignores_bias),
    ("selection_scores", _selection_bias_inside_sigmoid),
    ("routing_stats", _stats_share_over_T),
    ("routing_stats", _stats_entropy_sign),
    ("routing_stats", _stats_aux_without_N),
    ("dequantize_q4", _q4_nibbles_swapped),
    ("dequantize_q4", _q4_scale_bias_swapped),
    ("dequantize_q4", _q4_group_of_32),
    ("silu_grad", _silu_grad_no_curvature),
    ("gate_logit_grad", _logit_grad_sign),
    ("gate_logit_grad", _logit_grad_renorm_ignored),
    ("swiglu_backward", _swiglu_bwd_up_uses_z),
    ("swiglu_backward", _swiglu_bwd_down_from_preactivation),
    ("to_f64", _bf16_shift8),
    ("expert_weights", _q4_up_with_gate_scales),
]


def _any_pin_fails():
    for check in pins.ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            return check.__name__
    return None


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    failed = _any_pin_fails()
    assert failed is not None, f"no pin caught the planted mistake {fn.__name__}"
