"""Pins of the CPU oracle to facts outside itself.

Each ``check_*`` function raises AssertionError when the oracle disagrees
with what the pages or the mathematics fix. ``test_oracle_pins.py`` runs
them as they are; ``test_oracle_mutations.py`` plants plausible mistakes in
the oracle and confirms that at least one of them fails.

The pins:
  worked example  - the renormalisation example of "Tutorial 11: Mixture of
                    Experts (MoE)", section 2 (tests/golden)
  brute force     - top-k by a rank-count definition and by maximising the
                    sum of selected logits over all subsets (tiny E)
  dense mask      - running every expert on every token and masking with the
                    gate scattered to [T, E] ("Small models, sparse experts",
                    section "Dispatch decides everything"; "Mixture-of-Experts
                    -- more capacity per byte of weight", section "What's NOT
                    shipped yet") gives the same output as sparse dispatch
  invariants      - conservation of pairs, permutation, monotone offsets,
                    stable groups, gate sums
  special cases   - k=1 with renorm is the argmax expert; k=E is the full
                    softmax mixture; identical experts give the plain FFN;
                    x = 0 gives 0; hidden-slice concatenation
  textbook        - silu / sigmoid / softmax values and scipy
  sigmoid router  - selection on sigmoid(L) + balance bias, gates from the
                    raw sigmoid ("Small MoE Architecture, in depth", sections
                    "A small MoE layer in PyTorch" and "Balancing without
                    fighting the loss"): zero bias reduces to the logit top-k,
                    a large bias forces an expert in without entering its
                    gate, rank-count brute force on the biased scores, and the
                    dense-mask equivalence above
  4-bit experts   - the dequantisation against the error bound of an affine
                    4-bit code (at most half a step), exact recovery of
                    weights built from known codes (distinct per position, so
                    a nibble-order or group-index slip shows), the bytes
                    per weight against the page's "about half a byte"
                    ("Small MoE Architecture, in depth", section "Worked
                    example: the batch-1 budget on a device"), and the whole
                    layer on quantised experts against the layer on the
                    weights the codes stand for, decoded position by position
  bf16 decode     - every finite bf16 bit pattern against the format's
                    definition (sign, biased exponent, fraction, subnormals),
                    and a whole layer on bf16 bits against the same layer on
                    their float64 values
  routing stats   - the 12.5% ideal share of a balanced 8-expert top-2 layer
                    ("Mini-MoE", section "Results"; tests/golden), entropy ln E
                    for a flat router and 0 in the one-hot limit, the Switch
                    term equal to alpha at perfect balance, a two-expert closed
                    form, Gibbs' bound
"""

from __future__ import annotations

import dataclasses
import itertools
import json
import math
import os

import numpy as np

import oracle.moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(T, d, E, h, k, mode, renorm, seed=0, shared_h=0, gated=False, bias=False,
            scale=1.0, bias_scale=0.5):
    """A small float32 input dict in the generator's layout (drawn here so the
    pins do not depend on the generator)."""
    from moe_inputs.spec import MoESpec, F32
    r = _rng(seed)
    spec = MoESpec(name="pin", T=T, d=d, E=E, h=h, k=k, dtype=F32, mode=mode,
                   renormalize=renorm, shared_h=shared_h, shared_gate=gated,
                   router_bias="zipf" if bias else None)
    inp = {
        "spec": spec,
        "x": r.standard_normal((T, d)).astype(np.float32),
        "w_router": (r.standard_normal((E, d)) * 0.3 * scale).astype(np.float32),
        "b_router": (r.standard_normal(E) * bias_scale).astype(np.float32) if bias else None,
        "w_gate": (r.standard_normal((E, h, d)) * 0.2).astype(np.float32),
        "w_up": (r.standard_normal((E, h, d)) * 0.2).astype(np.float32),
        "w_down": (r.standard_normal((E, d, h)) * 0.2).astype(np.float32),
    }
    if shared_h:
        inp["ws_gate"] = (r.standard_normal((shared_h, d)) * 0.2).astype(np.float32)
        inp["ws_up"] = (r.standard_normal((shared_h, d)) * 0.2).astype(np.float32)
        inp["ws_down"] = (r.standard_normal((d, shared_h)) * 0.2).astype(np.float32)
        inp["w_shared_gate"] = (r.standard_normal(d) * 0.3).astype(np.float32) if gated else None
    else:
        inp["ws_gate"] = inp["ws_up"] = inp["ws_down"] = inp["w_shared_gate"] = None
    return inp


# ---------------------------------------------------------------------------
# worked example
# ---------------------------------------------------------------------------

def check_worked_example():
    with open(os.path.join(GOLDEN, "renorm_worked_example.json")) as f:
        g = json.load(f)
    probs = np.array(g["probs"], dtype=np.float64)
    L = np.log(probs)[None, :]
    k = g["top_k"]
    ids = O.topk_select(L, k)
    assert ids[0].tolist() == g["expected_ids"], ids
    raw, p = O.gate_weights(L, ids, O.SOFTMAX_ALL, False)
    np.testing.assert_allclose(p[0], probs, rtol=1e-12, atol=0)
    np.testing.assert_allclose(raw[0], g["expected_scores_raw"], rtol=1e-12, atol=0)
    assert abs(raw[0].sum() - g["expected_raw_sum"]) < 1e-12
    half = 0.5 * 10.0 ** (-g["printed_decimals"])
    for mode in (O.SOFTMAX_ALL, O.SOFTMAX_SELECTED):
        ren, _ = O.gate_weights(L, ids, mode, mode == O.SOFTMAX_ALL)
        got = ren[0]
        assert np.all(np.abs(got - np.array(g["expected_scores_renorm_printed"])) <= half), got
        # exact values behind the printed ones: 0.3/0.55 = 6/11, 0.25/0.55 = 5/11
        np.testing.assert_allclose(got, [6 / 11, 5 / 11], rtol=1e-12, atol=0)
        assert abs(got.sum() - g["expected_renorm_sum"]) < 1e-12


# ---------------------------------------------------------------------------
# brute-force top-k
# ---------------------------------------------------------------------------

def _rank_count_topk(Lrow, k):
    """e is selected iff fewer than k experts beat it, where e' beats e if its
    logit is larger, or equal with a lower index. Slot = that count."""
    E = Lrow.size
    out = [None] * k
    for e in range(E):
        beats = sum(1 for f in range(E)
                    if Lrow[f] > Lrow[e] or (Lrow[f] == Lrow[e] and f < e))
        if beats < k:
            out[beats] = e
    return out


def _subset_max(Lrow, k):
    best = None
    for sub in itertools.combinations(range(Lrow.size), k):
        s = sum(Lrow[i] for i in sub)
        if best is None or s > best[0]:
            best = (s, sub)
    return best


def check_brute_force_topk():
    r = _rng(1)
    for trial in range(300):
        E = int(r.integers(1, 9))
        k = int(r.integers(1, E + 1))
        if trial % 3 == 0:
            Lrow = r.integers(-2, 3, size=E).astype(np.float64)  # many exact ties
        else:
            Lrow = r.standard_normal(E)
        ids = O.topk_select(Lrow[None, :], k)[0].tolist()
        assert ids == _rank_count_topk(Lrow, k), (Lrow, k, ids)
        assert len(set(ids)) == k
        s, _ = _subset_max(Lrow, k)
        assert abs(sum(Lrow[i] for i in ids) - s) <= 1e-12 * max(1.0, abs(s))
    # all-equal logits: ids are the first k experts in index order
    for E in (1, 5, 8):
        for k in range(1, E + 1):
            ids = O.topk_select(np.zeros((3, E)), k)
            assert (ids == np.arange(k)[None, :]).all()


# ---------------------------------------------------------------------------
# sparse dispatch == dense all-experts-then-mask
# ---------------------------------------------------------------------------

def dense_mask_forward(inp):
    """Every expert on every token, weighted by a gate that is zero outside
    the top-k. Computed without the oracle's dispatch, combine or top-k."""
    spec = inp["spec"]
    X = inp["x"].astype(np.float64)
    Wr = inp["w_router"].astype(np.float64)
    L = X @ Wr.T
    if inp.get("b_router") is not None:
        L = L + inp["b_router"].astype(np.float64)[None, :]
    T, E = L.shape
    k = spec.k
    mask = np.zeros((T, E))
    if spec.mode == O.SIGMOID:
        # bias-free affinities; the bias only moves the choice
        L = X @ Wr.T
        aff = 1.0 / (1.0 + np.exp(-L))
        sel = aff + (inp["b_router"].astype(np.float64)[None, :]
                     if inp.get("b_router") is not None else 0.0)
    else:
        sel = L
    for t in range(T):
        for e in _rank_count_topk(sel[t], k):
            mask[t, e] = 1.0
    if spec.mode == O.SIGMOID:
        G = aff * mask
        if spec.renormalize:
            G = G / G.sum(axis=1, keepdims=True)
    elif spec.mode == O.SOFTMAX_ALL:
        z = np.exp(L - L.max(axis=1, keepdims=True))
        G = z / z.sum(axis=1, keepdims=True) * mask
        if spec.renormalize:
            G = G / G.sum(axis=1, keepdims=True)
    else:
        z = np.exp(L - L.max(axis=1, keepdims=True)) * mask
        G = z / z.sum(axis=1, keepdims=True)
    out = np.zeros((T, X.shape[1]))
    for e in range(E):
        Wg = inp["w_gate"][e].astype(np.float64)
        Wu = inp["w_up"][e].astype(np.float64)
        Wd = inp["w_down"][e].astype(np.float64)
        a = X @ Wg.T
        ye = ((a / (1.0 + np.exp(-a))) * (X @ Wu.T)) @ Wd.T
        out += G[:, e:e + 1] * ye
    if inp.get("ws_gate") is not None:
        a = X @ inp["ws_gate"].astype(np.float64).T
        s = ((a / (1.0 + np.exp(-a))) * (X @ inp["ws_up"].astype(np.float64).T)) \
            @ inp["ws_down"].astype(np.float64).T
        if inp.get("w_shared_gate") is not None:
            s = s / (1.0 + np.exp(-(X @ inp["w_shared_gate"].astype(np.float64))))[:, None]
        out += s
    return out


def check_dense_mask_equivalence():
    cases = [
        dict(T=37, d=24, E=8, h=16, k=2, mode=O.SOFTMAX_ALL, renorm=True),
        dict(T=29, d=16, E=6, h=12, k=3, mode=O.SOFTMAX_ALL, renorm=False),
        dict(T=31, d=16, E=7, h=8, k=4, mode=O.SOFTMAX_SELECTED, renorm=False),
        dict(T=23, d=16, E=5, h=8, k=2, mode=O.SOFTMAX_ALL, renorm=True, bias=True),
        dict(T=19, d=16, E=6, h=8, k=2, mode=O.SOFTMAX_ALL, renorm=False,
             shared_h=20, gated=True),
        dict(T=17, d=16, E=4, h=8, k=4, mode=O.SOFTMAX_ALL, renorm=False),
        dict(T=27, d=16, E=9, h=8, k=3, mode=O.SIGMOID, renorm=True, bias=True,
             bias_scale=0.05),
        dict(T=21, d=16, E=6, h=8, k=2, mode=O.SIGMOID, renorm=False, bias=True,
             bias_scale=0.05, shared_h=12),
    ]
    for i, c in enumerate(cases):
        inp = _inputs(seed=10 + i, **c)
        got = O.layer_forward(inp)["out"]
        ref = dense_mask_forward(inp)
        err = np.max(np.abs(got - ref))
        assert err <= 1e-12 * max(1.0, np.max(np.abs(ref))), (c, err)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def check_dispatch_invariants():
    r = _rng(2)
    for trial in range(50):
        E = int(r.integers(1, 40))
        k = int(r.integers(1, min(E, 8) + 1))
        T = int(r.integers(0, 60))
        ids = np.stack([r.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), int)
        counts, offsets, perm, inv = O.dispatch(ids, E)
        P = T * k
        assert counts.sum() == P
        assert offsets[0] == 0 and offsets[-1] == P
        assert np.all(np.diff(offsets) == counts)
        assert sorted(perm.tolist()) == list(range(P))
        assert np.all(inv[perm] == np.arange(P))
        flat = ids.reshape(-1)
        for e in range(E):
            grp = perm[offsets[e]:offsets[e + 1]]
            assert np.all(flat[grp] == e)
            assert np.all(np.diff(grp) > 0)  # stable: ascending pair index
            assert counts[e] == int(np.sum(flat == e))


def check_gate_sums():
    r = _rng(3)
    for trial in range(40):
        E = int(r.integers(2, 20))
        k = int(r.integers(1, E + 1))
        L = r.standard_normal((11, E)) * 3
        ids = O.topk_select(L, k)
        g, p = O.gate_weights(L, ids, O.SOFTMAX_ALL, True)
        assert np.allclose(g.sum(1), 1.0, rtol=0, atol=1e-12)
        g, p = O.gate_weights(L, ids, O.SOFTMAX_SELECTED, False)
        assert np.allclose(g.sum(1), 1.0, rtol=0, atol=1e-12)
        g2, _ = O.gate_weights(L, ids, O.SOFTMAX_ALL, True)
        assert np.allclose(g, g2, rtol=0, atol=1e-12)  # the two modes agree
        g, p = O.gate_weights(L, ids, O.SOFTMAX_ALL, False)
        assert np.all(g.sum(1) <= 1.0 + 1e-12)
        assert np.all(np.diff(g, axis=1) <= 1e-15)  # slot order = descending score
        # full softmax is scipy's
        from scipy.special import softmax as sp_softmax
        np.testing.assert_allclose(p, sp_softmax(L, axis=1), rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# special cases and closed forms
# ---------------------------------------------------------------------------

def _ffn(x, Wg, Wu, Wd):
    a = x @ Wg.T
    return ((a / (1.0 + np.exp(-a))) * (x @ Wu.T)) @ Wd.T


def check_k1_is_argmax_expert():
    inp = _inputs(T=25, d=16, E=6, h=10, k=1, mode=O.SOFTMAX_ALL, renorm=True, seed=4)
    res = O.layer_forward(inp)
    assert np.all(res["gates"] == 1.0)
    X = inp["x"].astype(np.float64)
    L = X @ inp["w_router"].astype(np.float64).T
    for t in range(25):
        e = int(np.argmax(L[t]))
        ref = _ffn(X[t:t + 1], inp["w_gate"][e].astype(np.float64),
                   inp["w_up"][e].astype(np.float64), inp["w_down"][e].astype(np.float64))[0]
        np.testing.assert_allclose(res["out"][t], ref, rtol=1e-12, atol=1e-12)


def check_k_equals_E_is_soft_mixture():
    for renorm in (False, True):
        inp = _inputs(T=13, d=12, E=5, h=6, k=5, mode=O.SOFTMAX_ALL, renorm=renorm, seed=5)
        res = O.layer_forward(inp)
        X = inp["x"].astype(np.float64)
        L = X @ inp["w_router"].astype(np.float64).T
        from scipy.special import softmax as sp_softmax
        p = sp_softmax(L, axis=1)
        ref = np.zeros_like(res["out"])
        for e in range(5):
            ref += p[:, e:e + 1] * _ffn(X, inp["w_gate"][e].astype(np.float64),
                                        inp["w_up"][e].astype(np.float64),
                                        inp["w_down"][e].astype(np.float64))
        np.testing.assert_allclose(res["out"], ref, rtol=1e-11, atol=1e-12)
        assert not res["near_tie_select"].any()


def check_identical_experts():
    for mode, renorm in ((O.SOFTMAX_ALL, True), (O.SOFTMAX_SELECTED, False)):
        inp = _inputs(T=21, d=16, E=6, h=10, k=3, mode=mode, renorm=renorm, seed=6)
        for n in ("w_gate", "w_up", "w_down"):
            inp[n] = np.repeat(inp[n][:1], 6, axis=0)
        res = O.layer_forward(inp)
        X = inp["x"].astype(np.float64)
        ref = _ffn(X, inp["w_gate"][0].astype(np.float64), inp["w_up"][0].astype(np.float64),
                   inp["w_down"][0].astype(np.float64))
        np.testing.assert_allclose(res["out"], ref, rtol=1e-11, atol=1e-12)


def check_zero_input():
    inp = _inputs(T=9, d=16, E=5, h=8, k=2, mode=O.SOFTMAX_ALL, renorm=False, seed=7,
                  bias=True, shared_h=8, gated=True)
    inp["x"] = np.zeros_like(inp["x"])
    res = O.layer_forward(inp)
    assert np.all(res["out"] == 0.0)
    # all logits equal the bias: selection follows the bias order
    order = np.argsort(-inp["b_router"].astype(np.float64), kind="stable")[:2]
    assert np.all(res["ids"] == order[None, :])


def check_hidden_slice_concatenation():
    """A SwiGLU of hidden H is the sum of the SwiGLUs on a partition of its
    hidden units: four slices of a dense FFN routed with a zero router (all
    logits tie, so ids = 0..3 and softmax-all gates are 1/4) give FFN/4; the
    shared expert of hidden 4*h equals the sum of four hidden-h pieces."""
    r = _rng(8)
    T, d, h = 15, 16, 6
    G = r.standard_normal((4 * h, d)) * 0.3
    U = r.standard_normal((4 * h, d)) * 0.3
    D = r.standard_normal((d, 4 * h)) * 0.3
    X = r.standard_normal((T, d))
    from moe_inputs.spec import MoESpec, F32
    spec = MoESpec(name="slices", T=T, d=d, E=4, h=h, k=4, dtype=F32,
                   mode=O.SOFTMAX_ALL, renormalize=False)
    inp = {"spec": spec, "x": X, "w_router": np.zeros((4, d)), "b_router": None,
           "w_gate": np.stack([G[s * h:(s + 1) * h] for s in range(4)]),
           "w_up": np.stack([U[s * h:(s + 1) * h] for s in range(4)]),
           "w_down": np.stack([D[:, s * h:(s + 1) * h] for s in range(4)]),
           "ws_gate": None, "ws_up": None, "ws_down": None, "w_shared_gate": None}
    res = O.layer_forward(inp)
    assert np.all(res["ids"] == np.arange(4)[None, :])
    np.testing.assert_allclose(res["gates"], 0.25, rtol=0, atol=1e-15)
    dense = _ffn(X, G, U, D)
    np.testing.assert_allclose(res["out"], dense / 4, rtol=1e-11, atol=1e-12)
    s = O.shared_expert(X, G, U, D)
    parts = sum(_ffn(X, G[i * h:(i + 1) * h], U[i * h:(i + 1) * h], D[:, i * h:(i + 1) * h])
                for i in range(4))
    np.testing.assert_allclose(s, parts, rtol=1e-11, atol=1e-12)


def check_textbook_functions():
    from scipy.special import expit
    z = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(O.sigmoid(z), expit(z), rtol=1e-14, atol=0)
    np.testing.assert_allclose(O.silu(z), z * expit(z), rtol=1e-13, atol=1e-300)
    assert O.silu(np.array(0.0)) == 0.0
    assert O.sigmoid(np.array(0.0)) == 0.5
    assert abs(float(O.silu(np.array(1.0))) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    # softmax of logs of a distribution returns it
    q = np.array([[1.0, 2.0, 3.0, 4.0]]) / 10.0
    np.testing.assert_allclose(O.softmax(np.log(q)), q, rtol=1e-14)
    # shift invariance (the max subtraction must not change values)
    a = np.array([[1000.0, 1001.0, 999.0]])
    np.testing.assert_allclose(O.softmax(a), O.softmax(a - 1000.0), rtol=1e-14)


def check_combine_gather_vs_loop():
    """The combine against the per-token statement of the layer: for each
    token, the weighted sum of its selected experts' SwiGLU outputs."""
    inp = _inputs(T=14, d=12, E=5, h=7, k=3, mode=O.SOFTMAX_ALL, renorm=False, seed=9,
                  shared_h=9, gated=True)
    res = O.layer_forward(inp)
    rows = O.token_forward(inp, list(range(14)), res["ids"], res["gates"])
    np.testing.assert_allclose(res["out"], rows, rtol=1e-12, atol=1e-13)


def check_near_tie_detection():
    L = np.array([[1.0, 0.5, 0.5 - 5e-6, -1.0],    # k=2: 2nd vs 3rd within eps
                  [2.0, 2.0 - 3e-6, 0.0, -1.0],     # order tie among selected
                  [3.0, 2.0, 1.0, 0.0]])            # clean
    sel, order = O.near_ties(L, 2)
    assert sel.tolist() == [True, False, False]
    assert order.tolist() == [False, True, False]
    sel, order = O.near_ties(L, 4)
    assert not sel.any()


# ---------------------------------------------------------------------------
# sigmoid scoring with a selection-only balance bias
# ---------------------------------------------------------------------------

def check_sigmoid_zero_bias_is_logit_topk():
    """sigmoid is strictly increasing, so with no bias the choice is the
    logit top-k; renormalised gates sum to 1 and follow the slot order."""
    for seed, (E, k) in enumerate([(8, 2), (13, 5), (6, 6)]):
        inp = _inputs(T=40, d=12, E=E, h=4, k=k, mode=O.SIGMOID, renorm=True, seed=30 + seed)
        L, ids, g, _ = O.route(inp)
        assert np.array_equal(ids, O.topk_select(L, k))
        assert np.allclose(g.sum(1), 1.0, rtol=0, atol=1e-12)
        assert np.all(np.diff(g, axis=1) <= 1e-15)
        # unnormalised gates are affinities: strictly inside (0, 1)
        inp2 = dict(inp, spec=inp["spec"].__class__(**{**inp["spec"].__dict__, "renormalize": False}))
        _, _, g2, _ = O.route(inp2)
        assert np.all((g2 > 0) & (g2 < 1))
        # and renormalising them gives the renormalised gates
        assert np.allclose(g2 / g2.sum(1, keepdims=True), g, rtol=0, atol=1e-12)


def check_sigmoid_bias_steers_choice_not_gates():
    """A bias far above any affinity gap forces its expert into slot 0 of every
    token; the gates still come from the unbiased affinities, so a second bias
    vector that leads to the same choice leaves the gates unchanged."""
    inp = _inputs(T=50, d=12, E=10, h=4, k=3, mode=O.SIGMOID, renorm=True, seed=41)
    b = np.zeros(10, np.float32)
    b[7] = 3.0  # affinities lie in (0, 1): +3 always wins
    L, ids, g, _ = O.route(dict(inp, b_router=b))
    assert np.all(ids[:, 0] == 7)
    aff = 1.0 / (1.0 + np.exp(-L))
    np.testing.assert_allclose(g[:, 0], aff[:, 7] / np.take_along_axis(aff, ids, 1).sum(1),
                               rtol=1e-12, atol=0)
    b2 = b.copy()
    b2[7] = 5.0  # same choice, larger bias
    _, ids2, g2, _ = O.route(dict(inp, b_router=b2))
    assert np.array_equal(ids, ids2) and np.array_equal(g, g2)


def check_sigmoid_brute_force_topk():
    """Small biases comparable to the affinity gaps: the oracle's choice is the
    rank-count top-k of sigmoid(L) + b (computed here independently)."""
    for seed in range(6):
        inp = _inputs(T=60, d=10, E=7, h=4, k=3, mode=O.SIGMOID, renorm=True, seed=50 + seed,
                      bias=True, bias_scale=0.05)
        L, ids, _, _ = O.route(inp)
        X = inp["x"].astype(np.float64)
        aff = 1.0 / (1.0 + np.exp(-(X @ inp["w_router"].astype(np.float64).T)))
        S = aff + inp["b_router"].astype(np.float64)[None, :]
        for t in range(S.shape[0]):
            assert list(ids[t]) == _rank_count_topk(S[t], 3), t


# ---------------------------------------------------------------------------
# routing statistics
# ---------------------------------------------------------------------------

def check_routing_stats_printed_share():
    with open(os.path.join(GOLDEN, "mini_moe_share.json")) as f:
        g = json.load(f)
    E, k = g["experts"], g["top_k"]
    T = 96
    # perfectly balanced top-2 routing over 8 experts
    ids = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)])
    counts, _, _, _ = O.dispatch(ids, E)
    share, _, _, _ = O.routing_stats(np.zeros((T, E)), counts, k, O.SOFTMAX_ALL, 0.01)
    assert np.allclose(share, g["ideal_share"], rtol=0, atol=1e-15)
    lo, hi = g["observed_share_range"]
    assert lo < g["ideal_share"] < hi


def check_routing_stats_closed_forms():
    alpha = 0.01
    for E, k in [(8, 2), (5, 1), (16, 4)]:
        T = 4 * E
        ids = np.array([[(k * t + j) % E for j in range(k)] for t in range(T)])
        counts, _, _, _ = O.dispatch(ids, E)
        for mode in (O.SOFTMAX_ALL, O.SOFTMAX_SELECTED, O.SIGMOID):
            # a flat router: p = 1/E everywhere, entropy ln E, and at perfect
            # balance the Switch term is exactly alpha
            share, P, H, aux = O.routing_stats(np.zeros((T, E)), counts, k, mode, alpha)
            assert np.allclose(P, 1.0 / E, rtol=0, atol=1e-15)
            assert abs(H - math.log(E)) < 1e-12
            assert abs(aux - alpha) < 1e-15
    # one-hot limit: entropy -> 0
    L = np.zeros((3, 6))
    L[:, 2] = 60.0
    _, P, H, _ = O.routing_stats(L, np.array([3, 0, 0, 0, 0, 0]), 1, O.SOFTMAX_ALL, 0.01)
    assert H < 1e-20 and abs(P[2] - 1.0) < 1e-20
    # two experts, softmax: p = (1/(1+e^-a), 1/(1+e^a)) and
    # H = ln(1 + e^a) - a e^a / (1 + e^a)
    for a in (-3.0, -0.4, 0.0, 1.7, 5.0):
        _, _, H, _ = O.routing_stats(np.array([[a, 0.0]]), np.array([1, 0]), 1, O.SOFTMAX_ALL, 0.0)
        assert abs(H - (math.log1p(math.exp(a)) - a * math.exp(a) / (1.0 + math.exp(a)))) < 1e-13
    # Gibbs: 0 <= H <= ln E; shares and mean probabilities sum to 1
    r = _rng(9)
    for mode in (O.SOFTMAX_ALL, O.SIGMOID):
        L = r.standard_normal((30, 9)) * 2
        ids = O.topk_select(L, 3)
        counts, _, _, _ = O.dispatch(ids, 9)
        share, P, H, aux = O.routing_stats(L, counts, 3, mode, 0.01)
        assert 0.0 <= H <= math.log(9) + 1e-12
        assert abs(share.sum() - 1.0) < 1e-12 and abs(P.sum() - 1.0) < 1e-12
        assert aux >= 0.0


# ---------------------------------------------------------------------------
# 4-bit routed-expert weights
# ---------------------------------------------------------------------------

def check_q4_roundtrip_error_bound():
    from moe_inputs.generate import quantize_q4_g64
    r = _rng(21)
    w = (r.standard_normal((5, 7, 256)) * 0.05).astype(np.float32)
    w[0, 0, :64] = 0.0  # a constant group
    packed, sb = quantize_q4_g64(w)
    dq = O.dequantize_q4(packed, sb)
    scale = ((sb & 0xFFFF).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    step = np.repeat(scale, 64, axis=-1)
    err = np.abs(dq - w.astype(np.float64))
    assert np.all(err <= step / 2 * (1 + 1e-6)), float(np.max(err / step))
    # the codes use the range: every non-constant group reaches 0 and 15
    q = np.empty(w.shape, np.int64)
    q[..., 0::2] = packed & 15
    q[..., 1::2] = packed >> 4
    g = q.reshape(5, 7, 4, 64)
    live = np.ptp(w.reshape(5, 7, 4, 64), axis=-1) > 0
    assert np.all(g.min(-1)[live] == 0) and np.all(g.max(-1)[live] >= 14)


def check_q4_known_codes():
    """Weights built exactly as s * q + b from known codes: quantising them
    gives those codes back and dequantising gives the weights exactly."""
    from moe_inputs.generate import quantize_q4_g64
    K = 192
    k = np.arange(K)
    codes = (k * 7 + 3 + k // 64) % 16
    for g0 in range(3):  # every group holds a 0 and a 15
        codes[g0 * 64] = 0
        codes[g0 * 64 + 1] = 15
    s = np.array([2.0 ** -7, 2.0 ** -5, 2.0 ** -9])
    b = np.array([-2.0 ** -4, 0.25, -1.0])
    w = (s[k // 64] * codes + b[k // 64]).astype(np.float32)[None, :]
    packed, sb = quantize_q4_g64(w)
    assert np.array_equal(packed[0] & 15, codes[0::2]) and np.array_equal(packed[0] >> 4, codes[1::2])
    np.testing.assert_array_equal(O.dequantize_q4(packed, sb), w.astype(np.float64))


def check_q4_bytes_per_weight():
    """Codes plus one bf16 scale and bias per 64 weights: 0.5625 bytes per
    weight, the page's "about half a byte per parameter"."""
    from moe_inputs.generate import quantize_q4_g64
    w = np.zeros((3, 128), np.float32)
    packed, sb = quantize_q4_g64(w)
    per = (packed.nbytes + sb.nbytes) / w.size
    assert per == 0.5625 and abs(per - 0.5) < 0.1


# ---------------------------------------------------------------------------
# exact bf16 input decode
# ---------------------------------------------------------------------------

def _bf16_value(bits):
    """A bf16 bit pattern's value from the format's definition: sign bit 15,
    8 exponent bits (bias 127), 7 fraction bits; exponent 0 holds zero and
    the subnormals 2^-126 * m/128. Python integer and ldexp arithmetic,
    exact."""
    sign = -1.0 if (bits >> 15) & 1 else 1.0
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return sign * math.ldexp(m, -126 - 7)
    return sign * math.ldexp(128 + m, e - 127 - 7)


def check_bf16_decode():
    """The oracle reads bf16 inputs exactly: every finite bit pattern (both
    zeros, all subnormals and normals up to +-max) decodes to the value the
    format defines, and a whole layer given bf16 bits equals the same layer
    given those values as float64."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    bits = bits[finite].astype(np.uint16)
    got = O.to_f64(bits)
    assert got.dtype == np.float64
    want = np.array([_bf16_value(int(b)) for b in bits], dtype=np.float64)
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:5]
    # landmarks: +-0, the smallest subnormal, 1, -2, +-max
    marks = {0x0000: 0.0, 0x8000: -0.0, 0x0001: 2.0 ** -133, 0x3F80: 1.0, 0xC000: -2.0,
             0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0xFF7F: -(2 - 2 ** -7) * 2.0 ** 127}
    for b, v in marks.items():
        assert O.to_f64(np.array([b], np.uint16))[0] == v, hex(b)
    assert math.copysign(1.0, O.to_f64(np.array([0x8000], np.uint16))[0]) == -1.0

    # a layer with every input in bf16 bits against the same layer on float64
    from moe_inputs.spec import MoESpec, BF16
    r = _rng(91)
    T, d, E, h, k, hs = 9, 16, 6, 8, 2, 8
    spec = MoESpec(name="pin_bf16", T=T, d=d, E=E, h=h, k=k, dtype=BF16, mode=O.SOFTMAX_ALL,
                   renormalize=True, shared_h=hs, shared_gate=True)

    def bits_of(shape, std):
        f = (r.standard_normal(shape) * std).astype(np.float32)
        return (f.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 bits do

    shapes = {"x": ((T, d), 1.0), "w_router": ((E, d), 0.5), "w_gate": ((E, h, d), 0.3),
              "w_up": ((E, h, d), 0.3), "w_down": ((E, d, h), 0.3), "ws_gate": ((hs, d), 0.3),
              "ws_up": ((hs, d), 0.3), "ws_down": ((d, hs), 0.3), "w_shared_gate": ((d,), 0.3)}
    b_inp = {n: bits_of(*sv) for n, sv in shapes.items()}
    f_inp = {n: np.vectorize(_bf16_value, otypes=[np.float64])(v.astype(np.int64))
             for n, v in b_inp.items()}
    for dct in (b_inp, f_inp):
        dct.update(spec=spec, b_router=None, w_gate_sb=None, w_up_sb=None, w_down_sb=None)
    rb, rf = O.layer_forward(b_inp), O.layer_forward(f_inp)
    assert np.array_equal(rb["ids"], rf["ids"])
    assert np.array_equal(rb["out"], rf["out"])
    assert np.max(np.abs(rf["out"])) > 0


# ---------------------------------------------------------------------------
# the layer on 4-bit routed experts
# ---------------------------------------------------------------------------

def _q4_decode(packed, sb):
    """The 4-bit format read back element by element: byte i of a row holds
    position 2i in its low nibble and 2i+1 in its high nibble; word g holds
    the bf16 scale of positions 64g..64g+63 in its low half and the bf16 bias
    in its high half."""
    packed = np.asarray(packed)
    sb = np.asarray(sb)
    rows = packed.reshape(-1, packed.shape[-1])
    words = sb.reshape(-1, sb.shape[-1])
    K = rows.shape[1] * 2
    out = np.empty((rows.shape[0], K))
    for r in range(rows.shape[0]):
        for pos in range(K):
            byte = int(rows[r, pos // 2])
            q = (byte >> 4) if pos % 2 else (byte & 15)
            w = int(words[r, pos // 64])
            out[r, pos] = _bf16_value(w & 0xFFFF) * q + _bf16_value(w >> 16)
    return out.reshape(packed.shape[:-1] + (K,))


def check_q4_layer_forward():
    """The layer on quantised routed experts equals the layer on the float64
    weights those codes stand for (decoded here, position by position), with
    a bf16 shared expert beside them. Each matrix has its own scale words, so
    a pairing of one matrix's codes with another's scales shows."""
    from moe_inputs.generate import quantize_q4_g64
    from moe_inputs.spec import MoESpec, BF16
    r = _rng(93)
    T, d, E, h, k, hs = 10, 128, 4, 64, 2, 64
    spec = MoESpec(name="pin_q4", T=T, d=d, E=E, h=h, k=k, dtype=BF16, mode=O.SOFTMAX_ALL,
                   renormalize=False, shared_h=hs, expert_quant="q4_g64")

    def bits(shape, std):
        return ((r.standard_normal(shape) * std).astype(np.float32).view(np.uint32)
                >> 16).astype(np.uint16)

    q_inp = {"spec": spec, "x": bits((T, d), 1.0), "w_router": bits((E, d), 0.3),
             "b_router": None, "ws_gate": bits((hs, d), 0.1), "ws_up": bits((hs, d), 0.1),
             "ws_down": bits((d, hs), 0.1), "w_shared_gate": None}
    f_inp = dict(q_inp, spec=dataclasses.replace(spec, expert_quant=None),
                 w_gate_sb=None, w_up_sb=None, w_down_sb=None)
    for name, shape, std in (("w_gate", (E, h, d), 0.1), ("w_up", (E, h, d), 0.05),
                             ("w_down", (E, d, h), 0.2)):
        w = (r.standard_normal(shape) * std).astype(np.float32)
        q_inp[name], q_inp[name + "_sb"] = quantize_q4_g64(w)
        f_inp[name] = _q4_decode(q_inp[name], q_inp[name + "_sb"])
    rq, rf = O.layer_forward(q_inp), O.layer_forward(f_inp)
    assert np.array_equal(rq["ids"], rf["ids"])
    scale = float(np.max(np.abs(rf["out"])))
    assert scale > 0
    np.testing.assert_allclose(rq["out"], rf["out"], rtol=0, atol=1e-12 * scale)


# ---------------------------------------------------------------------------
# backward: pinned by automatic differentiation of the dense formulation and
# by finite differences of the forward
# ---------------------------------------------------------------------------

def _dense_mask_torch(tensors, spec, mask, has_bias_in_logits, sel_bias):
    """The dense all-experts forward of ``dense_mask_forward`` written in torch
    (float64) so autograd can differentiate it; the 0/1 selection mask is an
    input (top-k is piecewise constant)."""
    import torch
    X, Wr, Wg, Wu, Wd = (tensors[n] for n in ("x", "w_router", "w_gate", "w_up", "w_down"))
    L = X @ Wr.T
    if spec.mode == O.SIGMOID:
        aff = torch.sigmoid(L)
        G = aff * mask
        if spec.renormalize:
            G = G / G.sum(dim=1, keepdim=True)
    else:
        if has_bias_in_logits is not None:
            L = L + has_bias_in_logits[None, :]
        if spec.mode == O.SOFTMAX_ALL:
            G = torch.softmax(L, dim=1) * mask
            if spec.renormalize:
                G = G / G.sum(dim=1, keepdim=True)
        else:
            z = torch.exp(L - L.max(dim=1, keepdim=True).values) * mask
            G = z / z.sum(dim=1, keepdim=True)
    out = torch.zeros_like(X)
    for e in range(Wg.shape[0]):
        a = X @ Wg[e].T
        ye = (torch.nn.functional.silu(a) * (X @ Wu[e].T)) @ Wd[e].T
        out = out + G[:, e:e + 1] * ye
    if "ws_gate" in tensors:
        a = X @ tensors["ws_gate"].T
        sh = (torch.nn.functional.silu(a) * (X @ tensors["ws_up"].T)) @ tensors["ws_down"].T
        if "w_shared_gate" in tensors:
            sh = sh * torch.sigmoid(X @ tensors["w_shared_gate"])[:, None]
        out = out + sh
    return out


def _autograd_grads(inp, dO):
    import torch
    spec = inp["spec"]
    names = ["x", "w_router", "w_gate", "w_up", "w_down"]
    if inp.get("ws_gate") is not None:
        names += ["ws_gate", "ws_up", "ws_down"]
        if inp.get("w_shared_gate") is not None:
            names.append("w_shared_gate")
    tensors = {n: torch.tensor(inp[n].astype(np.float64), requires_grad=True) for n in names}
    # the selection, from this file's own rank-count top-k on float64 scores
    X = inp["x"].astype(np.float64)
    Lnp = X @ inp["w_router"].astype(np.float64).T
    b = inp.get("b_router")
    if spec.mode == O.SIGMOID:
        sel = 1.0 / (1.0 + np.exp(-Lnp)) + (b.astype(np.float64)[None, :] if b is not None else 0.0)
    else:
        sel = Lnp + (b.astype(np.float64)[None, :] if b is not None else 0.0)
    mask = np.zeros_like(Lnp)
    for t in range(Lnp.shape[0]):
        mask[t, _rank_count_topk(sel[t], spec.k)] = 1.0
    bias_t = torch.tensor(b.astype(np.float64)) if (b is not None and spec.mode != O.SIGMOID) else None
    out = _dense_mask_torch(tensors, spec, torch.tensor(mask), bias_t, None)
    (out * torch.tensor(dO)).sum().backward()
    return {n: tensors[n].grad.numpy() for n in names}


_GRAD_KEYS = {"x": "dx", "w_router": "dw_router", "w_gate": "dw_gate", "w_up": "dw_up",
              "w_down": "dw_down", "ws_gate": "dws_gate", "ws_up": "dws_up",
              "ws_down": "dws_down", "w_shared_gate": "dw_shared_gate"}


def check_backward_autograd_dense():
    """The oracle's sparse backward equals torch autograd (float64) through
    the dense run-every-expert-then-mask forward, in every gate mode, with a
    logit bias, a balance bias and a gated or ungated shared expert."""
    cases = [
        dict(T=9, d=8, E=5, h=6, k=2, mode=O.SOFTMAX_ALL, renorm=False),
        dict(T=9, d=8, E=5, h=6, k=2, mode=O.SOFTMAX_ALL, renorm=True, bias=True),
        dict(T=9, d=8, E=5, h=6, k=3, mode=O.SOFTMAX_SELECTED, renorm=False),
        dict(T=7, d=6, E=6, h=4, k=2, mode=O.SIGMOID, renorm=True, bias=True),
        dict(T=7, d=6, E=6, h=4, k=2, mode=O.SIGMOID, renorm=False),
        dict(T=8, d=8, E=4, h=5, k=2, mode=O.SOFTMAX_ALL, renorm=False, shared_h=7, gated=True),
        dict(T=8, d=8, E=4, h=5, k=1, mode=O.SOFTMAX_SELECTED, renorm=False, shared_h=3),
        dict(T=6, d=5, E=3, h=4, k=3, mode=O.SOFTMAX_ALL, renorm=False),  # k = E
    ]
    for i, c in enumerate(cases):
        inp = _inputs(c["T"], c["d"], c["E"], c["h"], c["k"], c["mode"], c["renorm"], seed=40 + i,
                      shared_h=c.get("shared_h", 0), gated=c.get("gated", False),
                      bias=c.get("bias", False))
        dO = _rng(90 + i).standard_normal((c["T"], c["d"]))
        ref = _autograd_grads(inp, dO)
        got = O.layer_backward(inp, dO)
        for n, g in ref.items():
            o = got[_GRAD_KEYS[n]]
            assert o is not None and o.shape == g.shape, (i, n)
            err = np.max(np.abs(o - g))
            assert err <= 1e-10 * max(1.0, np.max(np.abs(g))), (i, n, err)


def check_backward_finite_differences():
    """Central differences of sum(out * dO) through the oracle's own forward
    (float64 inputs) match the oracle's backward entry by entry."""
    inp = _inputs(7, 6, 4, 5, 2, O.SOFTMAX_ALL, True, seed=61, shared_h=4, gated=True)
    for n in ("x", "w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down",
              "w_shared_gate"):
        inp[n] = inp[n].astype(np.float64)
    dO = _rng(62).standard_normal((7, 6))
    got = O.layer_backward(inp, dO)
    base_ids = got["ids"]
    r = _rng(63)
    step = 1e-6
    for n in ("x", "w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down",
              "w_shared_gate"):
        a = inp[n]
        for _ in range(4):
            idx = tuple(int(r.integers(0, s)) for s in a.shape)
            keep = a[idx]
            vals = []
            for sgn in (1.0, -1.0):
                a[idx] = keep + sgn * step
                f = O.layer_forward(inp)
                assert np.array_equal(f["ids"], base_ids)  # the selection must not move
                vals.append(np.sum(f["out"] * dO))
            a[idx] = keep
            fd = (vals[0] - vals[1]) / (2 * step)
            an = got[_GRAD_KEYS[n]][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (n, idx, fd, an)


def check_backward_softmax_logit_grads_sum_to_zero():
    """Adding one constant to all of a token's logits leaves softmax gates
    unchanged, so each row of dL sums to zero in both softmax modes; in the
    sigmoid mode without renormalisation dL vanishes outside the selection."""
    for mode, renorm in ((O.SOFTMAX_ALL, False), (O.SOFTMAX_ALL, True), (O.SOFTMAX_SELECTED, False)):
        inp = _inputs(10, 6, 5, 4, 2, mode, renorm, seed=71)
        dO = _rng(72).standard_normal((10, 6))
        dL = O.layer_backward(inp, dO)["dlogits"]
        assert np.max(np.abs(dL.sum(axis=1))) <= 1e-12 * max(1.0, np.max(np.abs(dL)))
        assert np.max(np.abs(dL)) > 1e-6
    inp = _inputs(10, 6, 5, 4, 2, O.SIGMOID, False, seed=73)
    res = O.layer_backward(inp, _rng(74).standard_normal((10, 6)))
    off = np.ones_like(res["dlogits"], dtype=bool)
    np.put_along_axis(off, res["ids"], False, axis=1)
    assert np.all(res["dlogits"][off] == 0.0)


def check_backward_untouched_experts_have_zero_grads():
    """An expert no token chose gets exactly zero weight gradients."""
    inp = _inputs(6, 6, 6, 4, 1, O.SOFTMAX_ALL, False, seed=81)
    inp["b_router"] = np.array([0, 0, 0, -40, -40, -40], dtype=np.float32)
    from moe_inputs.spec import MoESpec, F32
    inp["spec"] = MoESpec(name="pin", T=6, d=6, E=6, h=4, k=1, dtype=F32, mode=O.SOFTMAX_ALL,
                          renormalize=False, router_bias="zipf")
    res = O.layer_backward(inp, _rng(82).standard_normal((6, 6)))
    assert set(np.unique(res["ids"])) <= {0, 1, 2}
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert np.all(res[n][3:] == 0.0) and np.max(np.abs(res[n][:3])) > 0


ALL_CHECKS = [
    check_worked_example,
    check_brute_force_topk,
    check_dense_mask_equivalence,
    check_dispatch_invariants,
    check_gate_sums,
    check_k1_is_argmax_expert,
    check_k_equals_E_is_soft_mixture,
    check_identical_experts,
    check_zero_input,
    check_hidden_slice_concatenation,
    check_textbook_functions,
    check_combine_gather_vs_loop,
    check_near_tie_detection,
    check_sigmoid_zero_bias_is_logit_topk,
    check_sigmoid_bias_steers_choice_not_gates,
    check_sigmoid_brute_force_topk,
    check_routing_stats_printed_share,
    check_routing_stats_closed_forms,
    check_q4_roundtrip_error_bound,
    check_q4_known_codes,
    check_q4_bytes_per_weight,
    check_q4_layer_forward,
    check_bf16_decode,
    check_backward_autograd_dense,
    check_backward_finite_differences,
    check_backward_softmax_logit_grads_sum_to_zero,
    check_backward_untouched_experts_have_zero_grads,
]
