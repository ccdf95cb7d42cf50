"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small shapes run the whole-batch oracle and span several tiles with ragged
tails (T not a multiple of the 64-token route block or the 128-row M tile,
d not a multiple of the 64-deep K chunk, h not a multiple of the N tile).
Full-size workloads run the whole-batch oracle too: routing and counts for
every token, every output entry, and the fused call's dispatch tables (read
back from its workspace) bit for bit against the oracle's stable sort of the
GPU's ids. Every comparison follows the protocol in gpu_helpers.
"""

import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_sparse_amd.binding as B
import oracle.moe_oracle as O
from gpu_helpers import (EPS_TIE, check_gates, check_out, check_routing, dev, device_inputs,
                         full_parity, host, oracle_logits_scores, run_layer, say)
from moe_inputs import generate, small_spec, spec_by_name
from moe_inputs.spec import BF16, F32, SOFTMAX_ALL, SOFTMAX_SELECTED, SPECS, MoESpec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    B.lib()


SMALL = {
    "tiny_fp32": SPECS["tiny_fp32"],
    "tiny_fp32_ragged": small_spec("tiny_fp32", T=203, d=72, E=8, h=40, k=2),
    "gemma_small": small_spec("gemma_upcycled", T=300, d=200, E=16, h=136, k=4),
    "decode_small": small_spec("decode", T=37, d=264, E=64, h=96, k=8),
    "skewed_small": small_spec("skewed_prefill", T=700, d=256, E=32, h=200, k=8),
    "shared_small": small_spec("shared_routed", T=520, d=264, E=12, h=96, k=4, shared_h=376),
    # at least 256 rows per expert: the 256-row tiles; d and h leave K and N tails
    "big_tile_small": small_spec("skewed_prefill", T=600, d=200, E=4, h=136, k=2),
    "big_tile_shared_small": small_spec("shared_routed", T=700, d=264, E=3, h=96, k=2, shared_h=200),
    # 256-row tiles: a column tail (d = 200); the shared group with a longer
    # reduction than the routed one; more tiles than the GPU has CUs
    "tile256_col_tail": small_spec("skewed_prefill", T=600, d=200, E=4, h=128, k=2),
    "tile256_shared_longer_k": small_spec("shared_routed", T=700, d=264, E=3, h=128, k=2,
                                          shared_h=256),
    "tile256_many_tiles": small_spec("skewed_prefill", T=8192, d=2048, E=4, h=128, k=2),
    "shared_fp32_small": small_spec("shared_routed", T=130, d=48, E=6, h=24, k=2, shared_h=40,
                                    dtype=F32),
    "e256_small": MoESpec(name="e256", T=150, d=64, E=256, h=32, k=6, mode=SOFTMAX_SELECTED),
    # at most 16 rows per expert on average: the weight-stationary small-batch
    # GEMMs. Skewed k=1 routing puts most of the 64 tokens on expert 0 (several
    # 16-row blocks); h and d leave column tails and K tails
    "small_rowblocks": small_spec("skewed_prefill", T=64, d=264, E=8, h=40, k=1),
    "small_tails": small_spec("decode", T=20, d=136, E=32, h=72, k=4),
    # reduction longer than 2048: eight waves per workgroup
    "small_k2560": small_spec("decode", T=16, d=2560, E=16, h=64, k=2),
    # at least 4 down items per CU: the persistent down kernel, with K and
    # column tails, and (skewed routing) experts of several 16-row blocks
    "small_pers_tails": small_spec("decode", T=64, d=2056, E=64, h=200, k=4),
    "small_pers_rowblocks": small_spec("skewed_prefill", T=64, d=2056, E=16, h=72, k=4),
    # one route block with the split router: shared-gate column, 256 experts
    "split_route_shared": small_spec("shared_routed", T=40, d=264, E=12, h=96, k=4, shared_h=200),
    "split_route_e256": MoESpec(name="e256_t64", T=64, d=640, E=256, h=64, k=4,
                                mode=SOFTMAX_SELECTED),
    "split_route_e256_shared": small_spec("shared_routed", T=8, d=64, E=256, h=32, k=8,
                                          shared_h=64),
    # sigmoid affinities, selection-only balance bias, renormalised raw gates:
    # several route blocks with the shared expert; one route block with the
    # small-batch GEMMs; more than 16 slots per token without renormalisation
    "sigmoid_small": small_spec("small_moe_sigmoid", T=300, d=256, E=64, h=64, k=8, shared_h=128),
    "sigmoid_one_block": small_spec("small_moe_sigmoid", T=16, d=256, E=64, h=64, k=8, shared_h=0),
    "sigmoid_k20": small_spec("small_moe_sigmoid", T=90, d=128, E=64, h=32, k=20, shared_h=0,
                              renormalize=False),
    # gemma's d = 640 with at least 32 rows per expert (the persistent gate/up
    # kernel): a column tail (h = 136), experts of two 128-row tiles, and the
    # shared expert's tiles in the same persistent walk
    "pers_d640": small_spec("gemma_upcycled", T=300, d=640, E=16, h=136, k=4),
    "pers_d640_two_mtiles": small_spec("gemma_upcycled", T=700, d=640, E=8, h=64, k=2),
    "pers_d640_shared": small_spec("shared_routed", T=260, d=640, E=8, h=96, k=2, shared_h=200),
    # dispatch: the one-launch scan and scatter at eight route blocks per
    # workgroup (500 blocks of 32 tokens, 128 experts), and the two-launch
    # path once the block histogram passes 65536 entries (282 blocks x 256)
    "dispatch_fused_8_blocks": small_spec("skewed_prefill", T=16000, d=64, E=128, h=32, k=2),
    "dispatch_split_e256": MoESpec(name="e256_t9000", T=9000, d=64, E=256, h=32, k=2,
                                   mode=SOFTMAX_SELECTED),
    # exactly at the one-launch limits: 512 route blocks of 32 tokens x 128
    # experts = 65536 histogram entries, eight blocks per workgroup
    "dispatch_fused_at_limit": small_spec("skewed_prefill", T=16383, d=64, E=128, h=32, k=2),
    # the two-launch path past 512 route blocks (625 blocks of 64 tokens, 8 experts)
    "dispatch_split_625_blocks": small_spec("decode", T=40000, d=64, E=8, h=32, k=2),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small(name):
    spec = SMALL[name]
    say(f"[gpu] layer_forward {name}: T={spec.T} d={spec.d} E={spec.E} h={spec.h} k={spec.k}")
    inp = generate(spec)
    full_parity(inp)


@pytest.mark.parametrize("name", list(SMALL))
def test_entry_points_small(name):
    """route -> dispatch -> gate_up -> down -> (shared) -> combine, each entry
    point checked against the matching oracle step, then the chain against the
    fused call (bitwise: same kernels, same order)."""
    spec = SMALL[name]
    say(f"[gpu] entry points {name}")
    inp = generate(spec)
    d = device_inputs(inp)
    cfg = B.config_from_spec(spec)
    T, k, E = spec.T, spec.k, spec.E
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids, gates = B.route(cfg, d["x"], d["w_router"], d["b_router"], logits=logits)
    torch.cuda.synchronize()
    L, S = oracle_logits_scores(inp)
    lerr = float(np.max(np.abs(host(logits) - L)))
    say(f"    logits max err {lerr:.2e}")
    assert lerr <= (1e-5 if spec.dtype == F32 else 1e-4) * max(1.0, float(np.max(np.abs(L))))
    gids = ids.cpu().numpy().astype(np.int64)
    near, mism = check_routing(S, gids, k)
    ref_ids = O.topk_select(S, k)
    ref_ids[mism] = gids[mism]
    ref_g, _ = O.gate_weights(L, ref_ids, spec.mode, spec.renormalize)
    check_gates(gates.cpu().numpy().astype(np.float64), ref_g)

    counts, offsets, perm, inv = B.dispatch(cfg, ids)
    torch.cuda.synchronize()
    rc, ro, rp, ri = O.dispatch(gids, E)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(perm.cpu().numpy(), rp)
    assert np.array_equal(inv.cpu().numpy(), ri)

    act = B.gate_up(cfg, d["x"], perm, offsets, d["w_gate"], d["w_up"])
    y = B.down(cfg, act, offsets, d["w_down"])
    y2 = B.expert_ffn(cfg, d["x"], perm, offsets, d["w_gate"], d["w_up"], d["w_down"])
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    ref_act = O.gate_up(inp["x"], rp, ro, k, inp["w_gate"], inp["w_up"])
    check_out(host(act), ref_act, spec.dtype, "act")
    ref_y = O.down(ref_act, ro, inp["w_down"])
    check_out(host(y), ref_y, spec.dtype, "y")

    shared = None
    ref_s = None
    if spec.shared_h:
        shared = B.shared_expert(cfg, d["x"], d["ws_gate"], d["ws_up"], d["ws_down"],
                                 d["w_shared_gate"])
        torch.cuda.synchronize()
        ref_s = O.shared_expert(inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"],
                                inp.get("w_shared_gate"))
        check_out(host(shared), ref_s, spec.dtype, "shared")
    out = B.combine(cfg, y, inv, gates, shared)
    torch.cuda.synchronize()
    ref_out = O.combine(ref_y, ri, ref_g, ref_s)
    check_out(host(out), ref_out, spec.dtype, "combine")

    fused = run_layer(inp, d)
    if spec.T > 64:
        assert np.array_equal(fused["ids"], gids)
        if spec.shared_h == 0:
            # same kernels in the same order: bitwise equal
            assert torch.equal(fused["out_t"], out)
    else:
        # one route block: the fused layer splits the router GEMM over K
        # (another fp32 summation order than moe_route's single workgroup),
        # so ids agree outside near-ties and outputs to the bf16 tolerance
        tie = np.logical_or(*O.near_ties(S, k, EPS_TIE))
        assert np.array_equal(fused["ids"][~tie], gids[~tie])
        check_out(host(fused["out_t"]), host(out).astype(np.float64), spec.dtype, "fused vs chain")


# 4-bit routed experts (the fused layer only: the standalone expert entry
# points take activation-dtype weights). Scale-group K tails, skewed routing
# with several 16-row blocks per expert, a bf16 shared expert beside them,
# and a reduction of 4096 (eight waves)
SMALL_Q4 = {
    "q4_small": small_spec("decode_q4", T=20, d=256, E=32, h=128, k=4),
    "q4_group_tails": small_spec("decode_q4", T=37, d=192, E=16, h=320, k=3),
    "q4_rowblocks": small_spec("decode_q4", T=64, d=128, E=8, h=64, k=1, router_bias="zipf",
                               renormalize=True),
    "q4_shared": small_spec("decode_q4", T=24, d=256, E=16, h=64, k=4, shared_h=128,
                            shared_gate=True),
    "q4_k4096": small_spec("decode_q4", T=8, d=4096, E=8, h=64, k=2),
    # more than four 16-column workgroups per CU: the 32-column gate/up shape
    # whose partial sums reuse the code buffer, with Zipf-skewed routing so
    # that experts of several 16-row blocks stage their codes again
    "q4_wide_rowblocks": small_spec("decode_q4", T=64, d=256, E=64, h=512, k=4,
                                    router_bias="zipf", renormalize=True),
    # the same for the 128-column down shape (reduction h = 256)
    "q4_wide_down": small_spec("decode_q4", T=48, d=1024, E=64, h=256, k=4,
                               router_bias="zipf", renormalize=True),
    # the wide shapes at a gate/up reduction short of the 8-wave span
    # (d = 1536: the last two waves' groups are past K) and a down reduction
    # of 384 (the last of four waves partly past K)
    "q4_wide_k1536": small_spec("decode_q4", T=32, d=1536, E=64, h=384, k=8),
    # a column tail in the 128-column down slices (d = 576 = 4.5 slices)
    "q4_wide_coltail": small_spec("decode_q4", T=24, d=576, E=64, h=320, k=4,
                                  router_bias="zipf"),
    # more than one route block (T > 64): the dispatch tables from the scan
    # and scatter launches
    "q4_multiblock": small_spec("decode_q4", T=128, d=576, E=64, h=320, k=8,
                                router_bias="zipf", renormalize=True),
    # every token on the same few experts (k = 1, strong skew): most
    # workgroups of the wide grid find their slot empty
    "q4_wide_few_experts": small_spec("decode_q4", T=64, d=576, E=64, h=320, k=1,
                                      router_bias="zipf"),
    # at most four tokens: the gate/up launch makes the selection and the
    # dispatch tables itself (16- and 32-column shapes, a gated shared
    # expert beside it, one expert)
    "q4_tiny_T1": small_spec("decode_q4", T=1, d=256, E=32, h=128, k=4),
    "q4_tiny_T3_sel": small_spec("decode_q4", T=3, d=512, E=64, h=192, k=8,
                                 mode=SOFTMAX_SELECTED),
    "q4_tiny_T4_wide": small_spec("decode_q4", T=4, d=512, E=64, h=640, k=8,
                                  router_bias="zipf", renormalize=True),
    "q4_tiny_T2_shared": small_spec("decode_q4", T=2, d=256, E=16, h=64, k=2, shared_h=128,
                                    shared_gate=True),
    "q4_tiny_T1_E1": small_spec("decode_q4", T=1, d=128, E=1, h=64, k=1),
    # one token, down and combine in one launch: six 32-code chunks per
    # column (lanes 6 and 7 of each column idle), three rows
    "q4_tiny_T1_h192": small_spec("decode_q4", T=1, d=320, E=16, h=192, k=3),
}


@pytest.mark.parametrize("name", list(SMALL_Q4))
def test_layer_q4_small(name):
    spec = SMALL_Q4[name]
    say(f"[gpu] layer_forward q4 {name}: T={spec.T} d={spec.d} E={spec.E} h={spec.h} k={spec.k}")
    if spec.T <= 4:
        cfg = B.config_from_spec(spec)
        ws = B.alloc_workspace(cfg)
        g, _, _ = full_parity(generate(spec), ws=ws)
        _check_tables(cfg, ws, g["ids"], spec.E, name)
        say("    dispatch tables bit-exact")
    else:
        full_parity(generate(spec))


FULL = ["tiny_fp32", "gemma_upcycled", "skewed_prefill", "shared_routed",
        "decode@T1", "decode@T4", "decode@T16", "decode@T64", "small_moe_sigmoid",
        "decode_q4@T1", "decode_q4@T4", "decode_q4@T16", "decode_q4@T64"]

_cache = {}


def _full_inputs(name):
    """Full-size inputs; the decode batch sizes share one draw (x rows are a
    prefix of the same 64 drawn tokens)."""
    base = name.split("@")[0]
    key = f"{base}@T64" if base in ("decode", "decode_q4") else name
    if key not in _cache:
        _cache.clear()
        _cache[key] = generate(spec_by_name(key))
    inp = _cache[key]
    if key != name:
        spec = spec_by_name(name)
        inp = dict(inp, spec=spec, x=inp["x"][:spec.T])
    return inp


def _check_tables(cfg, ws, gids, E, what):
    """The dispatch tables in a workspace against the oracle's counting sort
    of the GPU's ids, bit for bit."""
    offs, perm, inv = (t.cpu().numpy().astype(np.int64) for t in B.workspace_tables(cfg, ws))
    _, ro, rp, ri = O.dispatch(gids, E)
    assert np.array_equal(offs, ro), f"{what}: offsets differ"
    assert np.array_equal(perm, rp), f"{what}: perm differs"
    assert np.array_equal(inv, ri), f"{what}: inv differs"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_layer_full_size(name):
    """The whole batch against the whole-batch oracle: every one of the T*d
    output entries within the bound, and the fused call's offsets, perm and
    inv equal to the oracle's stable sort of the GPU's ids."""
    spec = spec_by_name(name)
    say(f"[gpu] full-size {name}: T={spec.T} d={spec.d} E={spec.E} h={spec.h} k={spec.k}")
    inp = _full_inputs(name)
    cfg = B.config_from_spec(spec)
    ws = B.alloc_workspace(cfg)
    g, ref, _ = full_parity(inp, ws=ws)
    _check_tables(cfg, ws, g["ids"], spec.E, "fused call")
    counts = g["counts"]
    say(f"    touched experts {int((counts > 0).sum())}, max/mean load "
        f"{counts.max() / max(counts.mean(), 1e-9):.2f}, dispatch tables bit-exact")
    if name in ("gemma_upcycled", "skewed_prefill"):
        # the standalone dispatch entry point on the fused call's ids
        d_ids = torch.from_numpy(g["ids"].astype(np.int32)).cuda()
        c2, o2, p2, i2 = B.dispatch(cfg, d_ids)
        torch.cuda.synchronize()
        rc, ro, rp, ri = O.dispatch(g["ids"], spec.E)
        assert np.array_equal(c2.cpu().numpy(), rc)
        assert np.array_equal(o2.cpu().numpy(), ro)
        assert np.array_equal(p2.cpu().numpy(), rp)
        assert np.array_equal(i2.cpu().numpy(), ri)
        say("    moe_dispatch on the same ids: bit-exact")


def test_determinism():
    spec = small_spec("skewed_prefill", T=333, d=128, E=32, h=64, k=8)
    say("[gpu] determinism")
    inp = generate(spec)
    d = device_inputs(inp)
    a = run_layer(inp, d)
    b = run_layer(inp, d)
    assert np.array_equal(a["ids"], b["ids"])
    assert np.array_equal(a["counts"], b["counts"])
    assert torch.equal(a["out_t"], b["out_t"])


EDGE = {
    "T1_bf16": small_spec("decode", T=1, d=128, E=16, h=64, k=4),
    "T1_fp32": small_spec("tiny_fp32", T=1),
    "T65": small_spec("skewed_prefill", T=65, d=128, E=16, h=64, k=3),
    "T129": small_spec("gemma_upcycled", T=129, d=64, E=8, h=64, k=2),
    "k1": small_spec("skewed_prefill", T=200, d=128, E=16, h=64, k=1),
    "k_eq_E": small_spec("decode", T=90, d=64, E=8, h=32, k=8),
    "k_eq_E_renorm": small_spec("skewed_prefill", T=70, d=64, E=6, h=32, k=6),
    "E1": small_spec("decode", T=50, d=64, E=1, h=32, k=1),
    "d8": small_spec("decode", T=70, d=8, E=4, h=8, k=2),
    "big_k": MoESpec(name="big_k", T=40, d=64, E=200, h=16, k=130),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases(name):
    spec = EDGE[name]
    say(f"[gpu] edge {name}: T={spec.T} d={spec.d} E={spec.E} h={spec.h} k={spec.k}")
    full_parity(generate(spec))


# At most 4 tokens and 64 experts: the split router's one-wave finish
# (selection by rank, gates, dispatch tables) in every gating mode, with and
# without the router bias and the shared-expert gate, k = 1 and k = E.
TINY_ROUTE = {
    "T1_softmax_all": small_spec("decode", T=1, d=264, E=64, h=64, k=8),
    "T2_softmax_all_renorm_bias": small_spec("skewed_prefill", T=2, d=264, E=60, h=64, k=8),
    "T3_softmax_selected": MoESpec(name="t3_sel", T=3, d=200, E=37, h=40, k=5,
                                   mode=SOFTMAX_SELECTED),
    "T4_shared_gate": small_spec("shared_routed", T=4, d=264, E=60, h=64, k=4, shared_h=96),
    "T4_sigmoid_renorm": small_spec("small_moe_sigmoid", T=4, d=256, E=64, h=64, k=8,
                                    shared_h=64),
    "T3_sigmoid_raw_k20": small_spec("small_moe_sigmoid", T=3, d=128, E=64, h=32, k=20,
                                     shared_h=0, renormalize=False),
    "T4_k1": small_spec("skewed_prefill", T=4, d=128, E=16, h=64, k=1),
    "T2_k_eq_E": small_spec("decode", T=2, d=64, E=8, h=32, k=8),
    "T1_E1": small_spec("decode", T=1, d=64, E=1, h=32, k=1),
    "T4_fp32": small_spec("tiny_fp32", T=4),
    # one token: the selection and the tables come from the gate/up launch,
    # in every gate mode, with a logit bias and a gated shared expert
    "T1_softmax_all_renorm_bias": small_spec("skewed_prefill", T=1, d=264, E=60, h=64, k=8),
    "T1_softmax_selected": MoESpec(name="t1_sel", T=1, d=200, E=37, h=40, k=5,
                                   mode=SOFTMAX_SELECTED),
    "T1_shared_gate": small_spec("shared_routed", T=1, d=264, E=60, h=64, k=4, shared_h=96),
    "T1_sigmoid_renorm": small_spec("small_moe_sigmoid", T=1, d=256, E=64, h=64, k=8,
                                    shared_h=64),
    "T1_sigmoid_raw_k20": small_spec("small_moe_sigmoid", T=1, d=128, E=64, h=32, k=20,
                                     shared_h=0, renormalize=False),
    "T1_d4096_eight_waves": small_spec("decode", T=1, d=4096, E=16, h=128, k=4),
    # one token, down and combine in one launch: three rows, a reduction of
    # three 64-wide loads, a width of 40 eight-column slices
    "T1_k3_h192": small_spec("decode", T=1, d=320, E=16, h=192, k=3),
    # a few tokens, down and combine in one launch: experts holding several
    # rows (4 tokens, 4 experts, top-2), and 15 rows over a 9-slice width
    "T4_E4_multirow": small_spec("decode", T=4, d=256, E=4, h=128, k=2),
    "T3_k5_h128": small_spec("decode", T=3, d=72, E=16, h=128, k=5),
}


# One route block of up to 16 tokens at d from 128 to 2048: the split router
# (every gating mode, bias, shared gate, k = 1, k = E, E = 1, T = 16), the
# dispatch tables compared bit for bit.
SHORT_ROUTE = {
    "T1_d2048_softmax_all": small_spec("decode", T=1, d=2048, E=64, h=64, k=8),
    "T16_d1024_renorm_bias": small_spec("skewed_prefill", T=16, d=1024, E=64, h=64, k=8),
    "T9_d512_selected": MoESpec(name="t9_sel", T=9, d=512, E=40, h=40, k=5,
                                mode=SOFTMAX_SELECTED),
    "T7_d256_shared_gate": small_spec("shared_routed", T=7, d=256, E=60, h=64, k=4, shared_h=96),
    "T16_d256_sigmoid_bias": small_spec("small_moe_sigmoid", T=16, d=256, E=64, h=64, k=8,
                                        shared_h=64),
    "T12_d128_sigmoid_raw_k20": small_spec("small_moe_sigmoid", T=12, d=128, E=64, h=32, k=20,
                                           shared_h=0, renormalize=False),
    "T5_d512_k1": small_spec("skewed_prefill", T=5, d=512, E=16, h=64, k=1),
    "T3_d128_k_eq_E": small_spec("decode", T=3, d=128, E=8, h=32, k=8),
    "T2_d256_E1": small_spec("decode", T=2, d=256, E=1, h=32, k=1),
}


@pytest.mark.parametrize("name", list(SHORT_ROUTE))
def test_short_batch_router(name):
    spec = SHORT_ROUTE[name]
    say(f"[gpu] short-batch router {name}: T={spec.T} d={spec.d} E={spec.E} k={spec.k} "
        f"mode={spec.mode}")
    inp = generate(spec)
    cfg = B.config_from_spec(spec)
    ws = B.alloc_workspace(cfg)
    g, ref, _ = full_parity(inp, ws=ws)
    _check_tables(cfg, ws, g["ids"], spec.E, name)
    say("    dispatch tables bit-exact")


@pytest.mark.parametrize("name", list(TINY_ROUTE))
def test_tiny_batch_routing(name):
    spec = TINY_ROUTE[name]
    say(f"[gpu] tiny route {name}: T={spec.T} d={spec.d} E={spec.E} k={spec.k} mode={spec.mode}")
    inp = generate(spec)
    cfg = B.config_from_spec(spec)
    ws = B.alloc_workspace(cfg)
    g, ref, _ = full_parity(inp, ws=ws)
    _check_tables(cfg, ws, g["ids"], spec.E, name)
    say("    dispatch tables bit-exact")


def test_tiny_batch_ties():
    """All-zero router on three tokens: every score ties, so the ids are
    0..k-1 and the softmax-all gates 1/E."""
    spec = small_spec("decode", T=3, d=64, E=12, h=32, k=3)
    inp = generate(spec)
    inp["w_router"] = np.zeros_like(inp["w_router"])
    g = run_layer(inp)
    assert np.all(g["ids"] == np.arange(3)[None, :])
    assert np.allclose(g["gates"], 1.0 / 12, rtol=0, atol=1e-7)
    assert np.array_equal(g["counts"], np.r_[np.full(3, 3), np.zeros(9)].astype(np.int64))


def test_all_tokens_one_expert_and_empty_experts():
    """Router weights zero plus a bias that favours expert 5: every token
    picks 5 first (then the next-largest biases), most experts stay empty,
    and one expert's group spans many M tiles."""
    spec = small_spec("skewed_prefill", T=600, d=128, E=16, h=64, k=2)
    inp = generate(spec)
    inp["w_router"] = np.zeros_like(inp["w_router"])
    b = np.full(spec.E, -5.0, dtype=np.float32)
    b[5], b[9] = 3.0, 2.0
    inp["b_router"] = b
    say("[gpu] all tokens on experts 5 and 9")
    g, ref, _ = full_parity(inp)
    assert g["counts"][5] == 600 and g["counts"][9] == 600 and g["counts"].sum() == 1200


def test_tie_break_lower_index():
    """All-zero router: every logit ties, so the ids are 0..k-1 in order and
    softmax-all gates are 1/E (a pin of the selection rule, with exact ties)."""
    spec = small_spec("decode", T=77, d=64, E=12, h=32, k=3)
    inp = generate(spec)
    inp["w_router"] = np.zeros_like(inp["w_router"])
    g = run_layer(inp)
    assert np.all(g["ids"] == np.arange(3)[None, :])
    assert np.allclose(g["gates"], 1.0 / 12, rtol=0, atol=1e-7)


def test_hidden_slice_identity():
    """Four experts holding the four hidden slices of one dense SwiGLU, zero
    router, k=4, softmax-all: out = FFN_dense(x) / 4."""
    T, d, h = 150, 128, 64
    rng = np.random.default_rng(5)
    from moe_inputs import bf16_bits_from_f32
    G = bf16_bits_from_f32(rng.standard_normal((4 * h, d)).astype(np.float32) * 0.05)
    U = bf16_bits_from_f32(rng.standard_normal((4 * h, d)).astype(np.float32) * 0.05)
    D = bf16_bits_from_f32(rng.standard_normal((d, 4 * h)).astype(np.float32) * 0.05)
    X = bf16_bits_from_f32(rng.standard_normal((T, d)).astype(np.float32))
    spec = MoESpec(name="slices", T=T, d=d, E=4, h=h, k=4, dtype=BF16, mode=SOFTMAX_ALL)
    inp = {"spec": spec, "x": X, "w_router": np.zeros((4, d), np.uint16), "b_router": None,
           "w_gate": np.ascontiguousarray(np.stack([G[s * h:(s + 1) * h] for s in range(4)])),
           "w_up": np.ascontiguousarray(np.stack([U[s * h:(s + 1) * h] for s in range(4)])),
           "w_down": np.ascontiguousarray(np.stack([D[:, s * h:(s + 1) * h] for s in range(4)])),
           "ws_gate": None, "ws_up": None, "ws_down": None, "w_shared_gate": None}
    g = run_layer(inp)
    dense = O.swiglu(O.to_f64(X), O.to_f64(G), O.to_f64(U), O.to_f64(D)) / 4
    check_out(g["out"], dense, BF16, "slices vs dense/4")


def test_zero_tokens_is_noop():
    spec = small_spec("decode", T=0, d=64, E=8, h=32, k=2)
    cfg = B.config_from_spec(spec)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    wg = torch.zeros((8, 32, 64), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((8, 64, 32), dtype=torch.bfloat16, device="cuda")
    B.layer_forward(cfg, {"w_router": w, "w_gate": wg, "w_up": wg, "w_down": wd}, x, out=out,
                    ws=ws)
    torch.cuda.synchronize()


def test_workspace_too_small_is_rejected_on_gpu():
    spec = small_spec("decode", T=10, d=64, E=8, h=32, k=2)
    inp = generate(spec)
    d = device_inputs(inp)
    cfg = B.config_from_spec(spec)
    ws = torch.empty(B.workspace_size(cfg) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.layer_forward(cfg, {n: d[n] for n in ("w_router", "w_gate", "w_up", "w_down")},
                        d["x"], ws=ws)
    assert ei.value.status == B.MOE_ERR_WORKSPACE


STATS = {
    "stats_softmax_all": small_spec("decode", T=300, d=128, E=64, h=32, k=8),
    "stats_selected_e256": MoESpec(name="st_e256", T=1000, d=64, E=256, h=16, k=4,
                                   mode=SOFTMAX_SELECTED),
    "stats_biased": small_spec("skewed_prefill", T=700, d=128, E=32, h=32, k=8),
    "stats_sigmoid": small_spec("small_moe_sigmoid", T=513, d=128, E=64, h=32, k=8, shared_h=0),
    "stats_fp32_tiny": SPECS["tiny_fp32"],
    "stats_T1": small_spec("decode", T=1, d=128, E=64, h=32, k=8),
    # full token counts and expert counts of the layer workloads (the
    # statistics read only the router): 256 blocks of 32 and of 64 tokens
    "stats_gemma_full": small_spec("gemma_upcycled", h=16),
    "stats_skewed_full": small_spec("skewed_prefill", d=256, h=16),
    # 141 blocks of 64 tokens, the last one ragged inside a wave
    "stats_ragged_9000": small_spec("skewed_prefill", T=9000, d=128, h=16),
}


@pytest.mark.parametrize("name", list(STATS))
def test_routing_stats(name):
    """moe_routing_stats on moe_route's logits and moe_dispatch's counts
    against the oracle's statistics on its float64 logits and the same
    counts."""
    spec = STATS[name]
    say(f"[gpu] routing stats {name}: T={spec.T} E={spec.E} k={spec.k} mode={spec.mode}")
    inp = generate(spec)
    d = device_inputs(inp)
    cfg = B.config_from_spec(spec)
    logits = torch.empty((spec.T, spec.E), dtype=torch.float32, device="cuda")
    ids, _ = B.route(cfg, d["x"], d["w_router"], d["b_router"], logits=logits)
    counts, _, _, _ = B.dispatch(cfg, ids)
    share, mean_prob, scalars = B.routing_stats(cfg, logits, counts, alpha=0.01)
    torch.cuda.synchronize()
    L, _ = oracle_logits_scores(inp)
    rs, rp, rh, ra = O.routing_stats(L, counts.cpu().numpy(), spec.k, spec.mode, 0.01)
    gs, gp, (gh, ga) = share.cpu().numpy(), mean_prob.cpu().numpy(), scalars.cpu().numpy()
    say(f"    share err {np.max(np.abs(gs - rs)):.2e}, mean prob err {np.max(np.abs(gp - rp)):.2e}, "
        f"entropy {gh:.6f} vs {rh:.6f}, aux {ga:.6e} vs {ra:.6e}")
    assert np.max(np.abs(gs - rs)) <= 1e-6
    assert np.max(np.abs(gp - rp)) <= 1e-5 * max(1.0, float(np.max(rp)))
    assert abs(gh - rh) <= 1e-5 * max(1.0, rh)
    assert abs(ga - ra) <= 1e-5 * max(ra, 1e-3)
    assert abs(float(gs.sum()) - 1.0) < 1e-5 and abs(float(gp.sum()) - 1.0) < 1e-4
