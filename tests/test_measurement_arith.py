"""The roofline arithmetic against the figures the pages print."""

import json
import os

from mixture_experts_sparse_amd import roofline as R

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _fig():
    with open(os.path.join(GOLDEN, "measurement_figures.json")) as f:
        return json.load(f)


def test_gathered_weight_bytes_matches_printed():
    g = _fig()["gathered_weights"]
    b = R.gathered_weight_bytes(g["T"], g["h"], g["d"], g["elem_bytes"])
    assert b == 2_684_354_560
    assert round(b / 1e9, g["printed_decimals"]) == g["printed_gb"]


def test_dense_waste_ratio_matches_printed():
    g = _fig()["dense_expert_waste"]
    assert R.dense_to_sparse_flop_ratio(g["E"], g["k"]) == g["printed_ratio"]
    # the same ratio falls out of the FLOP counter: all-E experts vs top-k
    T, d, h = 100, 640, 512
    routed = R.layer_flops(T, d, g["E"], h, g["k"]) - 2.0 * T * d * g["E"]
    dense = R.layer_flops(T, d, g["E"], h, g["E"]) - 2.0 * T * d * g["E"]
    assert dense / routed == g["printed_ratio"]


def test_decode_ceilings_match_printed():
    """The page's worked decode budget: a model's resident footprint is its
    total parameter count times the bytes per parameter, and its batch-1 rate
    is bounded by the memory bandwidth over the bytes of the parameters one
    token activates. The bound is the product's own stream_bound_tokens_per_s."""
    g = _fig()["decode_ceilings"]
    bw = g["mem_gb_s"] * 1e9
    for row in g["rows"]:
        footprint_gb = row["total"] * g["bytes_per_param"] / 1e9
        assert round(footprint_gb, 2) == row["footprint_gb"], row
        per_token = row["active"] * g["bytes_per_param"]
        assert round(R.stream_bound_tokens_per_s(per_token, bw)) == row["ceiling_tok_s"], row


def test_decode_bound_uses_layer_bytes():
    """The decode HBM bound the bench reports: the layer's algorithmic bytes
    at T = 1 (8 touched experts of 12,582,912 bytes, router, x and out) at
    8 TB/s, about 79.3 k tokens/s; 4-bit experts move 0.5625 / 2 of the
    expert bytes."""
    b = 8 * 12_582_912 + 64 * 2048 * 2 + 2 * 2048 * 2
    assert R.layer_bytes(1, 2048, 64, 1024, 8, 2) == b
    assert abs(R.decode_bound_tokens_per_s(1, 2048, 64, 1024, 8, 2) - 8e12 / b) < 1e-6
    assert abs(R.decode_bound_tokens_per_s(1, 2048, 64, 1024, 8, 2) - 79.3e3) < 0.1e3
    q = R.decode_bound_tokens_per_s(1, 2048, 64, 1024, 8, 2, R.Q4_BYTES_PER_WEIGHT)
    assert q == 8e12 / (8 * 3 * 2048 * 1024 * 0.5625 + 64 * 2048 * 2 + 2 * 2048 * 2)


def test_workload_counts():
    # gemma_upcycled: T=8192, d=640, E=256, h=512, k=4, all experts touched
    f = R.layer_flops(8192, 640, 256, 512, 4)
    assert abs(f - 6.711e10) / 6.711e10 < 1e-3
    b = R.layer_bytes(8192, 640, 256, 512, 256, 2)
    assert abs(b - 5.246e8) / 5.246e8 < 1e-3
    # shared_routed: half routed, half shared
    f5 = R.layer_flops(8192, 2048, 60, 1408, 4, hs=5632, shared_gate=True)
    assert abs(f5 - 1.13592e12) / 1.13592e12 < 1e-3
    # skewed_prefill
    f4 = R.layer_flops(16384, 2048, 128, 768, 8)
    assert abs(f4 - 1.2455e12) / 1.2455e12 < 1e-3
    # decode: 12,582,912 bytes per expert
    assert 3 * 2048 * 1024 * 2 == 12_582_912
    assert abs(R.ridge_flop_per_byte() - 312.5) < 1e-9


def test_backward_stage_flops_add_up():
    """The backward's products: the recomputed gate/up pre-activations (the
    forward's gate/up FLOPs), then twice the forward's expert FLOPs (the
    gradients into the inputs and into the weights), and the router's two
    products; counted independently of the per-stage split."""
    T, d, E, h, k, hs = 300, 200, 16, 136, 4, 96
    P = T * k
    st = R.backward_stage_flops(T, d, E, h, k, hs, True)
    fwd_experts = 6.0 * P * d * h + 6.0 * T * d * hs
    recompute = R.gate_up_flops(P, d, h, T, hs)
    expect = 2.0 * T * d * E + recompute + 2.0 * fwd_experts + 2 * (2.0 * T * d * E) + 4.0 * T * d
    assert abs(sum(st.values()) - expect) <= 1e-9 * expect
    assert st["router_grad"] == 0.0


def test_backward_stage_bytes_terms():
    """The backward's byte model, term by term for the weight gradients (the
    float32 outputs dominate at the gemma shape: dW_gate|up is HBM-bound
    there and MFMA-bound at the skewed-prefill shape)."""
    T, d, E, h, k = 8192, 640, 256, 512, 4
    P = T * k
    b = R.backward_stage_bytes(T, d, E, h, k)
    assert b["dw_gate_up"] == 2 * P * h * 2 + T * d * 2 + 2 * E * h * d * 4
    assert b["dw_down"] == T * d * 2 + P * h * 2 + E * d * h * 4
    # the routed dx rows are stored in bf16 (the shared expert's in float32)
    assert b["dx_rows"] == 2 * P * h * 2 + 2 * E * h * d * 2 + P * d * 2
    f = R.backward_stage_flops(T, d, E, h, k)
    assert f["dw_gate_up"] / R.PEAK_BF16_MFMA_FLOPS < b["dw_gate_up"] / R.PEAK_HBM_BYTES
    T, d, E, h, k = 16384, 2048, 128, 768, 8
    b = R.backward_stage_bytes(T, d, E, h, k)
    f = R.backward_stage_flops(T, d, E, h, k)
    assert f["dw_gate_up"] / R.PEAK_BF16_MFMA_FLOPS > b["dw_gate_up"] / R.PEAK_HBM_BYTES
    # the shared expert adds its own rows and weights
    bs = R.backward_stage_bytes(300, 64, 8, 32, 2, hs=96)
    bn = R.backward_stage_bytes(300, 64, 8, 32, 2)
    assert bs["dw_gate_up"] - bn["dw_gate_up"] == 2 * 300 * 96 * 2 + 2 * 96 * 64 * 4


def test_routing_stats_bytes():
    # the float32 logits dominate: T*E*4, plus counts in and share,
    # mean probability and the two scalars out
    assert R.routing_stats_bytes(8192, 256) == 8192 * 256 * 4 + 256 * 4 + 2 * 256 * 4 + 8
    assert R.routing_stats_bytes(1, 8) == 32 + 32 + 64 + 8
