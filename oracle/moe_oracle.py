"""CPU oracle for the sparse mixture-of-experts FFN layer forward.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module; only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg use it. It shares no code with the HIP path:
it receives the generated input arrays (bf16 bit patterns or float32) and
converts them exactly to float64; every step below runs in float64 with no
intermediate rounding.

Steps, in the order the pages give them:

1. router logits  L = x W_r^T (+ b)
   ("Tutorial 11: Mixture of Experts (MoE)", section 2 "The Router": a plain
   linear map from hidden states to one score per expert; the router of
   "Mixture-of-Experts -- more capacity per byte of weight", section "What's
   wired today", is bias-free. The bias is an extra input of the skewed
   workload only.)
2. top-k selection on L, ties to the lower expert index, slots in descending
   logit order (Tutorial 11, section 2, step 3 picks the k largest; "Small MoE
   Architecture, in depth", section "A small MoE layer in PyTorch", uses topk).
3. gates: softmax over all experts, gathered at the selection and optionally
   renormalised to sum 1 (Tutorial 11, section 2, steps 2, 4 and 5), or a
   softmax over the k selected logits ("Small models, sparse experts",
   section "How it works", step 3).
4. dispatch: counts per expert, exclusive offsets and a stable sort of the
   flattened (token, slot) pairs by expert (Tutorial 11, section 3, step 1;
   the per-expert load is the bincount of "Small MoE Architecture, in depth",
   section "A small MoE layer in PyTorch").
5. expert FFN, looping over experts and running each expert's SwiGLU
   W_d (silu(W_g x) * (W_u x)) on its own rows only (Tutorial 11, section 3,
   step 2; "Small MoE Architecture, in depth", class Expert and the
   loop-over-experts of SmallMoE.forward).
6. combine: out[t] = sum_j g[t, j] y[t, j], an additive weighted sum in slot
   order (Tutorial 11, section 3, step 3 and section 4, step 5).
7. shared expert: an always-on SwiGLU added to the routed output ("Small MoE
   Architecture, in depth", section "A small MoE layer in PyTorch"); the
   sigmoid(w_s . x) scale on it is an input option of the shared-plus-routed
   workload, not a formula on the pages.

Sigmoid scoring ("Small MoE Architecture, in depth", sections "A small MoE
layer in PyTorch" and "Balancing without fighting the loss"): affinities
s = sigmoid(L) of the bias-free logits; the top-k is taken on s + b, where b
is a balance bias that only steers the choice; the gates are the raw s of
the chosen experts divided by their sum. Steps 4-7 are unchanged.

Quantised routed experts (``dequantize_q4``): the routed experts' weights
may arrive as 4-bit affine groups, about half a byte per weight ("Small MoE
Architecture, in depth", sections "Worked example: the batch-1 budget on a
device" and "Quantisation fits MoE unusually well", where routed experts are
quantised and the shared expert stays at higher precision). The format is a
reading: groups of 64 consecutive weights along the reduction axis, each
with a bf16 scale s and bias b, w = s * q + b for the 4-bit code q in
[0, 15]; two codes per byte, the even position in the low nibble. The
oracle dequantises exactly (float64) and runs the same layer.

Backward (``layer_backward``): the gradients of the scalar sum(out * dO)
for an upstream gradient dO, as a training step takes them ("Small models,
sparse experts", section "Tuning the training loop": the whole step,
forward, backward and optimiser, is compiled together, and activations are
recomputed in the backward pass rather than stored). The pages print no
backward formula; this is the derivative of steps 1-7 with the selection
held fixed (top-k is piecewise constant in the logits): through the gates
into the router logits and weights, through each expert's SwiGLU into its
weights and the token rows, and through the shared expert and its gate. The
router bias and the balance bias are constants (no gradient is returned for
them).

Routing statistics (``routing_stats``): the per-expert token share, the mean
router probability per expert, the mean router entropy and the Switch
load-balance term alpha * N * sum_e f_e P_e ("Mixture-of-Experts -- more
capacity per byte of weight", section "What's wired today"; "Small MoE
Architecture, in depth", section "Fine-tuning a small MoE", which asks for
token share and router entropy to be logged).
"""

from __future__ import annotations

import numpy as np

SOFTMAX_ALL = 0
SOFTMAX_SELECTED = 1
SIGMOID = 2

NEAR_TIE_EPS = 1e-5


# ----------------------------------------------------------------------------
# exact input conversion
# ----------------------------------------------------------------------------

def to_f64(a):
    """bf16 bit patterns (uint16) or float32 -> float64, exactly."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported input dtype {a.dtype}")


# ----------------------------------------------------------------------------
# textbook building blocks
# ----------------------------------------------------------------------------

def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def softmax(z, axis=-1):
    """Max-subtracted softmax (the numerically careful form)."""
    m = np.max(z, axis=axis, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def swiglu(X, Wg, Wu, Wd):
    """The SwiGLU FFN W_d (silu(W_g x) * (W_u x)) on the rows of X.

    "Small MoE Architecture, in depth", section "A small MoE layer in
    PyTorch", class Expert; Tutorial 11, section 4, step 4.
    """
    return (silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T


# ----------------------------------------------------------------------------
# quantised expert weights
# ----------------------------------------------------------------------------

Q4_GROUP = 64


def dequantize_q4(packed, sb):
    """packed [..., K/2] uint8 (code of position 2i in the low nibble of byte
    i, 2i+1 in the high nibble), sb [..., K/64] uint32 (bf16 scale in the low
    half, bf16 bias in the high half) -> float64 [..., K] with
    w[..., k] = s[..., k // 64] * q[..., k] + b[..., k // 64]."""
    packed = np.asarray(packed, dtype=np.uint8)
    sb = np.asarray(sb, dtype=np.uint32)
    K = packed.shape[-1] * 2
    q = np.empty(packed.shape[:-1] + (K,), dtype=np.float64)
    q[..., 0::2] = packed & 0x0F
    q[..., 1::2] = packed >> 4
    scale = ((sb & 0xFFFF) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    bias = ((sb >> 16) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    if scale.shape[-1] * Q4_GROUP != K:
        raise ValueError("scale groups do not cover K")
    return q * np.repeat(scale, Q4_GROUP, axis=-1) + np.repeat(bias, Q4_GROUP, axis=-1)


def expert_weights(inp):
    """The routed experts' weights (gate, up, down) as float64, dequantised
    when they arrive quantised."""
    if inp.get("w_gate_sb") is not None:
        return (dequantize_q4(inp["w_gate"], inp["w_gate_sb"]),
                dequantize_q4(inp["w_up"], inp["w_up_sb"]),
                dequantize_q4(inp["w_down"], inp["w_down_sb"]))
    return to_f64(inp["w_gate"]), to_f64(inp["w_up"]), to_f64(inp["w_down"])


# ----------------------------------------------------------------------------
# step 1-3: route
# ----------------------------------------------------------------------------

def router_logits(x, w_router, b_router=None):
    """L[t, e] = sum_i x[t, i] W_r[e, i] (+ b[e])."""
    L = to_f64(x) @ to_f64(w_router).T
    if b_router is not None:
        L = L + to_f64(b_router)[None, :]
    return L


def topk_select(L, k):
    """The k largest logits per row: ties go to the lower expert index, and
    slots are ordered by descending logit (lower index first among equals).

    A stable ascending sort of -L keeps equal keys in index order, which is
    exactly that order.
    """
    E = L.shape[1]
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    return np.argsort(-L, axis=1, kind="stable")[:, :k].astype(np.int64)


def selection_scores(L, mode, sel_bias=None):
    """The scores the top-k is taken on. Softmax modes: the logits (any bias is
    already inside L, it moves the softmax too). SIGMOID: sigmoid(L) + b, the
    balance bias b steering the choice only ("Small MoE Architecture, in
    depth", section "A small MoE layer in PyTorch": topk of scores plus the
    balance bias)."""
    if mode != SIGMOID:
        return L
    S = sigmoid(L)
    if sel_bias is not None:
        S = S + to_f64(sel_bias)[None, :]
    return S


def gate_weights(L, ids, mode, renormalize):
    """Gate weights for the selected experts.

    SOFTMAX_ALL: p = softmax(L) over all E experts; g[t, j] = p[t, ids[t, j]];
    optionally g /= sum_j g (Tutorial 11, section 2, steps 2, 4, 5).
    SOFTMAX_SELECTED: g = softmax over the k selected logits ("Small models,
    sparse experts", section "How it works", step 3).
    Returns (g, p) where p is the full softmax (None for SOFTMAX_SELECTED).
    """
    if mode == SOFTMAX_ALL:
        p = softmax(L, axis=1)
        g = np.take_along_axis(p, ids, axis=1)
        if renormalize:
            g = g / np.sum(g, axis=1, keepdims=True)
        return g, p
    if mode == SOFTMAX_SELECTED:
        g = softmax(np.take_along_axis(L, ids, axis=1), axis=1)
        if renormalize:
            g = g / np.sum(g, axis=1, keepdims=True)
        return g, None
    if mode == SIGMOID:
        # the raw affinities of the chosen experts weight the outputs; the
        # balance bias is not part of them ("Small MoE Architecture, in
        # depth", sections "A small MoE layer in PyTorch" and "Balancing
        # without fighting the loss")
        g = np.take_along_axis(sigmoid(L), ids, axis=1)
        if renormalize:
            g = g / np.sum(g, axis=1, keepdims=True)
        return g, None
    raise ValueError(f"unknown gate mode {mode}")


def router_probs(L, mode):
    """The router's distribution over all E experts: softmax(L) in the softmax
    modes; in the sigmoid mode the affinities normalised to sum 1 (a reading:
    the pages log "router entropy" without defining the distribution for
    sigmoid scores)."""
    if mode == SIGMOID:
        s = sigmoid(L)
        return s / np.sum(s, axis=1, keepdims=True)
    return softmax(L, axis=1)


def routing_stats(L, counts, k, mode, alpha):
    """Per-expert token share f_e = counts_e / (T k) (the fraction of the T k
    token-to-expert assignments; a balanced 8-expert layer gives each 12.5%,
    "Mini-MoE", section "Results"), mean router
    probability P_e = mean_t p[t, e], mean router entropy
    H = mean_t (-sum_e p[t, e] ln p[t, e]) in nats, and the Switch load-balance
    term alpha * N * sum_e f_e P_e with N = E experts ("Mixture-of-Experts --
    more capacity per byte of weight", section "What's wired today").
    Returns (share [E], mean_prob [E], entropy, aux)."""
    L = np.asarray(L, dtype=np.float64)
    T, E = L.shape
    counts = np.asarray(counts, dtype=np.float64)
    share = counts / float(T * k) if T > 0 else np.zeros(E)
    p = router_probs(L, mode) if T > 0 else np.zeros((0, E))
    mean_prob = p.mean(axis=0) if T > 0 else np.zeros(E)
    plogp = np.where(p > 0.0, p * np.log(np.where(p > 0.0, p, 1.0)), 0.0)
    entropy = float(-plogp.sum(axis=1).mean()) if T > 0 else 0.0
    aux = float(alpha * E * np.sum(share * mean_prob))
    return share, mean_prob, entropy, aux


def near_ties(L, k, eps=NEAR_TIE_EPS):
    """Tokens whose routing is decided by a score gap below ``eps`` (L: the
    selection scores, the logits in the softmax modes).

    Returns (select, order): ``select`` marks tokens where the k-th and
    (k+1)-th largest logits differ by less than eps (the selected *set* is
    then ambiguous at fp32 precision); ``order`` marks tokens where two
    adjacent selected logits differ by less than eps (the slot *order* is then
    ambiguous). Both are empty when k == E for ``select``.
    """
    s = -np.sort(-L, axis=1)
    T, E = L.shape
    if k < E:
        select = (s[:, k - 1] - s[:, k]) < eps
    else:
        select = np.zeros(T, dtype=bool)
    if k > 1:
        order = np.any((s[:, : k - 1] - s[:, 1:k]) < eps, axis=1)
    else:
        order = np.zeros(T, dtype=bool)
    return select, order


# ----------------------------------------------------------------------------
# step 4: dispatch
# ----------------------------------------------------------------------------

def dispatch(ids, E):
    """Counting sort of the T*k (token, slot) pairs by expert.

    Pair p = t*k + j has expert ids[t, j]. Returns counts[E], offsets[E+1]
    (exclusive prefix sum, offsets[E] = T*k), perm[P] (sorted row -> pair,
    stable: rows of one expert keep ascending p) and inv[P] = perm^-1.
    """
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int64)
    return counts, offsets, perm, inv


# ----------------------------------------------------------------------------
# step 5: grouped expert FFN
# ----------------------------------------------------------------------------

def gate_up(x, perm, offsets, k, w_gate, w_up):
    """act[r] = silu(W_g[e] x_t) * (W_u[e] x_t) for sorted row r of expert e,
    t = perm[r] // k. Loops over experts, not tokens."""
    X = to_f64(x)
    E, h, _ = w_gate.shape
    P = perm.size
    act = np.zeros((P, h))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r0 == r1:
            continue
        Xe = X[perm[r0:r1] // k]
        act[r0:r1] = silu(Xe @ to_f64(w_gate[e]).T) * (Xe @ to_f64(w_up[e]).T)
    return act


def down(act, offsets, w_down):
    """y[r] = W_d[e] act[r] for sorted row r of expert e."""
    E, d, _ = w_down.shape
    y = np.zeros((act.shape[0], d))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r0 == r1:
            continue
        y[r0:r1] = act[r0:r1] @ to_f64(w_down[e]).T
    return y


def expert_ffn(x, perm, offsets, k, w_gate, w_up, w_down):
    """y[P, d] in sorted order, un-gated: each expert's SwiGLU on its rows."""
    return down(gate_up(x, perm, offsets, k, w_gate, w_up), offsets, w_down)


# ----------------------------------------------------------------------------
# step 6-7: combine and shared expert
# ----------------------------------------------------------------------------

def combine(y_sorted, inv, gates, shared=None):
    """out[t] = sum_{j<k} g[t, j] y[inv[t*k + j]] (+ shared[t]), summed in
    slot order j = 0..k-1."""
    T, k = gates.shape
    d = y_sorted.shape[1]
    Y = y_sorted[np.asarray(inv).reshape(T, k)]  # [T, k, d]
    out = np.zeros((T, d))
    for j in range(k):
        out += gates[:, j, None] * Y[:, j, :]
    if shared is not None:
        out += shared
    return out


def shared_expert(x, ws_gate, ws_up, ws_down, w_shared_gate=None):
    """s[t] = (sigmoid(w_s . x_t) if gated else 1) * SwiGLU_shared(x_t)."""
    X = to_f64(x)
    s = swiglu(X, to_f64(ws_gate), to_f64(ws_up), to_f64(ws_down))
    if w_shared_gate is not None:
        s = s * sigmoid(X @ to_f64(w_shared_gate))[:, None]
    return s


# ----------------------------------------------------------------------------
# the whole layer
# ----------------------------------------------------------------------------

def _spec_fields(spec):
    return spec.E, spec.k, spec.mode, bool(spec.renormalize)


def route(inp, ids_override=None):
    """Steps 1-3. ``ids_override`` (dict token -> k expert ids) replaces the
    selection of those tokens; their gates are still computed by step 3 from
    the float64 logits (used for tokens whose selection is a near tie)."""
    spec = inp["spec"]
    E, k, mode, renorm = _spec_fields(spec)
    if mode == SIGMOID:
        # bias-free logits; the bias only steers the selection
        L = router_logits(inp["x"], inp["w_router"], None)
        S = selection_scores(L, mode, inp.get("b_router"))
    else:
        L = router_logits(inp["x"], inp["w_router"], inp.get("b_router"))
        S = L
    ids = topk_select(S, k)
    if ids_override:
        for t, sel in ids_override.items():
            ids[t] = np.asarray(sel, dtype=np.int64)
    g, p = gate_weights(L, ids, mode, renorm)
    return L, ids, g, p


def layer_forward(inp, ids_override=None):
    """Steps 1-7 on the whole batch. Returns a dict with out [T, d] (float64),
    logits, ids, gates, counts, offsets, perm, inv, y (sorted, un-gated),
    shared (or None) and the near-tie masks."""
    spec = inp["spec"]
    E, k = spec.E, spec.k
    L, ids, g, p = route(inp, ids_override)
    counts, offsets, perm, inv = dispatch(ids, E)
    Wg, Wu, Wd = expert_weights(inp)
    y = expert_ffn(inp["x"], perm, offsets, k, Wg, Wu, Wd)
    shared = None
    if inp.get("ws_gate") is not None:
        shared = shared_expert(inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"],
                               inp.get("w_shared_gate"))
    out = combine(y, inv, g, shared)
    S = selection_scores(L, spec.mode, inp.get("b_router") if spec.mode == SIGMOID else None)
    sel_tie, ord_tie = near_ties(S, k)
    return {"out": out, "logits": L, "scores": S, "probs": p, "ids": ids, "gates": g,
            "counts": counts, "offsets": offsets, "perm": perm, "inv": inv,
            "y": y, "shared": shared, "near_tie_select": sel_tie,
            "near_tie_order": ord_tie}


def token_forward(inp, tokens, ids, gates):
    """Output rows for a few tokens, one token at a time, from a given
    selection and gates: out[t] = sum_j g[t, j] SwiGLU_{ids[t, j]}(x_t)
    (+ shared). This is the per-token statement of the same layer, used to
    check sampled rows of full-size runs."""
    X = to_f64(inp["x"])
    has_shared = inp.get("ws_gate") is not None
    if has_shared:
        Sg, Su, Sd = (to_f64(inp[n]) for n in ("ws_gate", "ws_up", "ws_down"))
        wsg = to_f64(inp.get("w_shared_gate")) if inp.get("w_shared_gate") is not None else None
    Wg, Wu, Wd = expert_weights(inp)
    rows = []
    for t, sel, g in zip(tokens, ids, gates):
        xt = X[t:t + 1]
        o = np.zeros(X.shape[1])
        for e, ge in zip(sel, g):
            o += ge * swiglu(xt, Wg[e], Wu[e], Wd[e])[0]
        if has_shared:
            s = swiglu(xt, Sg, Su, Sd)[0]
            if wsg is not None:
                s = s * sigmoid(float(xt[0] @ wsg))
            o += s
        rows.append(o)
    return np.stack(rows) if rows else np.zeros((0, X.shape[1]))


# ----------------------------------------------------------------------------
# backward: the derivative of steps 1-7 with the selection held fixed
# ----------------------------------------------------------------------------

def silu_grad(z):
    """d silu / dz = sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def gate_logit_grad(L, ids, g, dG, mode, renormalize):
    """dL [T, E] from the gate gradient dG [T, k] (step 3 differentiated).

    SOFTMAX_ALL without renormalisation: g_j = p[ids_j] with p = softmax(L),
    so dL_i = p_i (v_i - sum_j dG_j g_j) where v_i sums dG_j over the slots
    that chose i. Renormalised, and SOFTMAX_SELECTED, the gates are the
    softmax of the k selected logits: dL[ids_m] = g_m (dG_m - sum_j dG_j g_j),
    zero elsewhere. SIGMOID: s = sigmoid(L); the gates are s[ids] (divided by
    their sum when renormalised), and ds/dL = s (1 - s).
    """
    T, E = L.shape
    k = ids.shape[1]
    dL = np.zeros((T, E))
    rows = np.arange(T)[:, None]
    inner = np.sum(dG * g, axis=1, keepdims=True)       # sum_j dG_j g_j
    if mode == SOFTMAX_ALL and not renormalize:
        p = softmax(L, axis=1)
        v = np.zeros((T, E))
        np.add.at(v, (np.repeat(np.arange(T), k), ids.reshape(-1)), dG.reshape(-1))
        return p * (v - inner)
    if mode in (SOFTMAX_ALL, SOFTMAX_SELECTED):
        np.add.at(dL, (np.broadcast_to(rows, ids.shape), ids), g * (dG - inner))
        return dL
    if mode == SIGMOID:
        s = sigmoid(np.take_along_axis(L, ids, axis=1))
        if renormalize:
            ds = (dG - inner) / np.sum(s, axis=1, keepdims=True)
        else:
            ds = dG
        np.add.at(dL, (np.broadcast_to(rows, ids.shape), ids), ds * s * (1.0 - s))
        return dL
    raise ValueError(f"unknown gate mode {mode}")


def swiglu_backward(X, Wg, Wu, Wd, dY):
    """Gradients of sum(SwiGLU(X) * dY) for one expert on its rows X:
    returns (dX, dWg, dWu, dWd). z_g = X Wg^T, z_u = X Wu^T,
    a = silu(z_g) z_u, Y = a Wd^T."""
    zg = X @ Wg.T
    zu = X @ Wu.T
    a = silu(zg) * zu
    dWd = dY.T @ a
    da = dY @ Wd
    dzg = da * zu * silu_grad(zg)
    dzu = da * silu(zg)
    return dzg @ Wg + dzu @ Wu, dzg.T @ X, dzu.T @ X, dWd


def layer_backward(inp, dout, ids_override=None):
    """Gradients of sum(out * dout) for the layer of ``layer_forward``.

    Returns a dict of float64 arrays: dx [T, d], dw_router [E, d],
    dw_gate / dw_up [E, h, d], dw_down [E, d, h] (zero for experts no token
    chose), the gate and logit gradients dgates [T, k] and dlogits [T, E],
    and, with a shared expert, dws_gate / dws_up [hs, d], dws_down [d, hs]
    and dw_shared_gate [d] (None when ungated). Quantised experts are not
    differentiated (their weights are not parameters here)."""
    spec = inp["spec"]
    if getattr(spec, "expert_quant", None):
        raise ValueError("backward of quantised experts is not defined")
    E, k, mode, renorm = _spec_fields(spec)
    fwd = layer_forward(inp, ids_override)
    X = to_f64(inp["x"])
    dO = to_f64(dout)
    T, d = X.shape
    ids, g, perm, offsets = fwd["ids"], fwd["gates"], fwd["perm"], fwd["offsets"]
    Wg, Wu, Wd = expert_weights(inp)
    h = Wg.shape[1]
    dX = np.zeros((T, d))
    dWg = np.zeros((E, h, d))
    dWu = np.zeros((E, h, d))
    dWd = np.zeros((E, d, h))
    dG = np.zeros((T, k))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r0 == r1:
            continue
        pairs = perm[r0:r1]
        toks, slots = pairs // k, pairs % k
        Xe = X[toks]
        ye = swiglu(Xe, Wg[e], Wu[e], Wd[e])                 # un-gated expert rows
        dG[toks, slots] = np.sum(dO[toks] * ye, axis=1)
        dXe, dWg[e], dWu[e], dWd[e] = swiglu_backward(Xe, Wg[e], Wu[e], Wd[e],
                                                      g[toks, slots][:, None] * dO[toks])
        np.add.at(dX, toks, dXe)
    dL = gate_logit_grad(fwd["logits"], ids, g, dG, mode, renorm)
    Wr = to_f64(inp["w_router"])
    dX += dL @ Wr
    res = {"dx": dX, "dw_router": dL.T @ X, "dw_gate": dWg, "dw_up": dWu, "dw_down": dWd,
           "dgates": dG, "dlogits": dL, "ids": ids, "gates": g,
           "dws_gate": None, "dws_up": None, "dws_down": None, "dw_shared_gate": None}
    if inp.get("ws_gate") is not None:
        Sg, Su, Sd = (to_f64(inp[n]) for n in ("ws_gate", "ws_up", "ws_down"))
        dOs = dO
        if inp.get("w_shared_gate") is not None:
            ws = to_f64(inp["w_shared_gate"])
            c = sigmoid(X @ ws)
            f = swiglu(X, Sg, Su, Sd)
            dpre = np.sum(dO * f, axis=1) * c * (1.0 - c)
            res["dw_shared_gate"] = X.T @ dpre
            dX += dpre[:, None] * ws[None, :]
            dOs = c[:, None] * dO
        dXs, res["dws_gate"], res["dws_up"], res["dws_down"] = swiglu_backward(X, Sg, Su, Sd, dOs)
        dX += dXs
    return res
