"""GPU parity of the layer backward (moe_layer_backward through the C ABI)
against the oracle's float64 layer_backward.

Every gradient the library returns (dx, the router, every expert's three
weight matrices, the shared expert's and its gate's, and the intermediate
gate and logit gradients) is compared over all of its entries with the bf16
bound of the forward: max|gpu - oracle| <= 2e-2 * max|oracle|. The selection
is held fixed by the derivative; tokens whose selection is a near tie are
re-derived by the oracle with the GPU's own selection (taken from the forward
on the same inputs), as in the forward parity protocol. Cases span several
128-row tiles with ragged tails, one route block (the split router), 256
experts, E not a multiple of 8, every gate mode, logit and balance biases,
gated and ungated shared experts, experts of 256 rows and more, and
per-expert weights larger than one XCD's L2 (the straight tile order of the
row products); the gemma-shaped and skewed-prefill workloads are checked
whole at full size.
"""

import numpy as np
import pytest
import torch

import mixture_experts_sparse_amd.binding as B
import oracle.moe_oracle as O
from gpu_helpers import check_routing, dev, device_inputs, oracle_logits_scores, run_layer, say
from moe_inputs import generate, small_spec, spec_by_name
from moe_inputs.generate import bf16_bits_from_f32
from moe_inputs.spec import SOFTMAX_SELECTED, MoESpec

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    B.lib()


CASES = {
    # softmax over the selected (gemma's mode), K and N tails (d = 200, h = 136)
    "gemma_small": small_spec("gemma_upcycled", T=300, d=200, E=16, h=136, k=4),
    # softmax over all, renormalised, Zipf logit bias: most rows on a few experts
    "skewed_small": small_spec("skewed_prefill", T=700, d=256, E=32, h=200, k=8),
    # softmax over all without renormalisation, sigmoid-gated shared expert, E = 12
    "shared_small": small_spec("shared_routed", T=520, d=264, E=12, h=96, k=4, shared_h=376),
    # sigmoid affinities, renormalised, balance bias, ungated shared expert
    "sigmoid_small": small_spec("small_moe_sigmoid", T=300, d=136, E=16, h=72, k=4, shared_h=200),
    # one route block (split router and inline dispatch)
    "one_block": small_spec("decode", T=37, d=264, E=64, h=96, k=8),
    # 256 experts, most with one or two rows, many with none
    "e256": MoESpec(name="e256_bwd", T=150, d=64, E=256, h=32, k=6, mode=SOFTMAX_SELECTED),
    # E not a multiple of 8 (padded logit rows), k = 3, T just past one route block
    "e12_k3": small_spec("shared_routed", T=77, d=72, E=12, h=40, k=3, shared_h=0,
                         shared_gate=False),
    # at least 256 rows per expert (several row tiles per expert), with K and N
    # tails, the shared expert, and sigmoid gates
    "big_tiles": small_spec("skewed_prefill", T=700, d=264, E=4, h=200, k=2),
    "big_tiles_shared": small_spec("shared_routed", T=600, d=136, E=3, h=96, k=2, shared_h=200),
    "big_tiles_sigmoid": small_spec("small_moe_sigmoid", T=520, d=128, E=4, h=64, k=2,
                                    shared_h=128),
    # 20 slots per token without renormalisation (the dx rows summed in batches
    # of 8 with a tail of 4; the slot gradients spread over lanes)
    "sigmoid_k20": small_spec("small_moe_sigmoid", T=90, d=128, E=64, h=32, k=20, shared_h=0,
                              renormalize=False),
    # an expert's weight operand above one XCD's 4 MB L2 (2*d*2h and 2*d*h
    # bytes > 4 MiB): the row products take the straight tile order, as at the
    # prefill shapes; h = 2056 leaves an N tail
    "wide_expert": small_spec("skewed_prefill", T=300, d=1024, E=2, h=2056, k=1),
    # the same for the shared expert's row products (2*d*2*shared_h > 4 MiB)
    "wide_shared": small_spec("shared_routed", T=260, d=1024, E=4, h=64, k=2, shared_h=2056),
    # 256-row tiles with an N tail of 8 hidden units (2056 = 16 * 128 + 8) and
    # a weight operand above 4 MiB
    "wide_expert_tile256": small_spec("skewed_prefill", T=600, d=1024, E=2, h=2056, k=1),
}

GRADS = ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up", "dws_down",
         "dw_shared_gate", "dgates", "dlogits")


def _dout(spec, seed):
    r = np.random.default_rng(seed)
    return bf16_bits_from_f32(r.standard_normal((spec.T, spec.d)).astype(np.float32))


def _weights(d_inp):
    return {n: d_inp[n] for n in ("w_router", "b_router", "w_gate", "w_up", "w_down", "ws_gate",
                                  "ws_up", "ws_down", "w_shared_gate")}


def _compare(name, got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    say(f"    {name}: max|gpu-oracle| = {err:.3e}, max|oracle| = {scale:.3e}, "
        f"ratio = {err / max(scale, 1e-300):.3e} (bound {TOL_BF16:g})")
    assert err <= TOL_BF16 * scale, f"{name}: {err} > {TOL_BF16} * {scale}"


def backward_parity(inp, seed=7):
    spec = inp["spec"]
    d_inp = device_inputs(inp)
    dO = _dout(spec, seed)
    # the GPU's selection (the backward recomputes the same route)
    g = run_layer(inp, d_inp)
    L, S = oracle_logits_scores(inp)
    near, mism = check_routing(S, g["ids"], spec.k)
    override = {int(t): g["ids"][t] for t in mism}
    ref = O.layer_backward(inp, dO, ids_override=override)
    cfg = B.config_from_spec(spec)
    got = B.layer_backward(cfg, _weights(d_inp), d_inp["x"], dev(dO), want_intermediates=True)
    torch.cuda.synchronize()
    for n in GRADS:
        if ref.get(n) is None:
            assert n not in got, n
            continue
        _compare(n, got[n].cpu().numpy(), ref[n])
    say(f"    near-tie tokens {near}, rerouted {len(mism)}")
    return got, ref


@pytest.mark.parametrize("name", list(CASES))
def test_backward_small(name):
    spec = CASES[name]
    say(f"[backward] {name}: T={spec.T} d={spec.d} E={spec.E} h={spec.h} k={spec.k} "
        f"mode={spec.mode} shared_h={spec.shared_h}")
    backward_parity(generate(spec))


def test_backward_repeat_is_deterministic():
    """Two calls on the same inputs give bit-identical gradients."""
    spec = CASES["shared_small"]
    inp = generate(spec)
    d_inp = device_inputs(inp)
    dO = dev(_dout(spec, 3))
    cfg = B.config_from_spec(spec)
    a = B.layer_backward(cfg, _weights(d_inp), d_inp["x"], dO)
    b = B.layer_backward(cfg, _weights(d_inp), d_inp["x"], dO)
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_backward_no_tokens_zero_weight_grads():
    spec = CASES["shared_small"]
    inp = generate(spec)
    d_inp = device_inputs(inp)
    cfg = B.config_from_spec(spec, 0)
    got = B.layer_backward(cfg, _weights(d_inp), d_inp["x"][:0], dev(_dout(spec, 1))[:0])
    torch.cuda.synchronize()
    for n in ("dw_router", "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up", "dws_down",
              "dw_shared_gate"):
        assert torch.count_nonzero(got[n]).item() == 0, n


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["gemma_upcycled", "skewed_prefill", "shared_routed",
                                  "small_moe_sigmoid"])
def test_backward_full(name):
    """A workload at full size, every gradient entry checked."""
    spec = spec_by_name(name)
    say(f"[backward] {name} full: T={spec.T}")
    backward_parity(generate(spec), seed=11)
