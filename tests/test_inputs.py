"""The seeded generator: determinism, bf16 rounding, shapes, structure."""

import numpy as np
import pytest
import torch

from moe_inputs import bf16_bits_from_f32, f32_from_bf16_bits, generate, small_spec, spec_by_name
from moe_inputs.generate import zipf_router_bias
from moe_inputs.spec import BF16, F32, SPECS


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    a = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875, 3.0e-39],
                                 dtype=np.float32)])
    mine = bf16_bits_from_f32(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    back = f32_from_bf16_bits(mine)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_ties_to_even():
    # 1 + 2^-8 is exactly halfway between two bf16 values: rounds to even (1.0)
    a = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)
    b = f32_from_bf16_bits(bf16_bits_from_f32(a))
    assert b[0] == 1.0 and b[1] == 1.0 + 4 * 2.0 ** -8


def test_deterministic_and_shapes():
    s = small_spec("shared_routed", T=33, d=64, E=6, h=32, k=2, shared_h=48)
    a, b = generate(s), generate(s)
    for n in ("x", "w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down",
              "w_shared_gate"):
        assert np.array_equal(a[n], b[n]), n
        assert a[n].dtype == np.uint16
    assert a["x"].shape == (33, 64)
    assert a["w_gate"].shape == (6, 32, 64) and a["w_down"].shape == (6, 64, 32)
    assert a["ws_gate"].shape == (48, 64) and a["ws_down"].shape == (64, 48)
    assert a["w_shared_gate"].shape == (64,)


def test_fp32_spec():
    a = generate(SPECS["tiny_fp32"])
    assert a["x"].dtype == np.float32 and a["x"].shape == (64, 64)
    assert a["w_gate"].shape == (8, 128, 64)
    assert abs(float(np.std(a["x"])) - 1.0) < 0.05
    assert abs(float(np.std(a["w_gate"])) - 0.02) < 0.002


def test_zipf_bias():
    b = zipf_router_bias(128)
    assert b.dtype == np.float32
    assert b[0] == 0.0
    np.testing.assert_allclose(b, -2.2 * np.log(np.arange(1, 129)), rtol=1e-6)


def test_upcycled_structure():
    s = small_spec("gemma_upcycled", T=16, d=32, E=8, h=16, k=2)
    assert s.upcycle_copies == 2
    a = generate(s)
    wg = f32_from_bf16_bits(a["w_gate"])
    # copy 0 of each slice is the scaled base; copy 1 differs in ~10% of entries
    frac = np.mean(wg[0] != wg[1])
    assert 0.05 < frac < 0.15, frac
    # scaled entries are ~N(0, 0.08)
    assert abs(float(np.std(wg[0])) - 0.08) < 0.015


def test_decode_prefix():
    a1 = generate(spec_by_name("decode@T1").__class__(**{**spec_by_name("decode@T1").__dict__,
                                                         "d": 64, "h": 32, "E": 8}))
    s4 = spec_by_name("decode@T4")
    assert s4.T == 4 and s4.x_rows == 64
    small = dict(d=64, h=32, E=8)
    import dataclasses
    x1 = generate(dataclasses.replace(spec_by_name("decode@T1"), **small))["x"]
    x4 = generate(dataclasses.replace(spec_by_name("decode@T4"), **small))["x"]
    assert np.array_equal(x1[0], x4[0])
    assert a1["x"].shape == (1, 64)


def test_named_specs():
    assert SPECS["gemma_upcycled"].upcycle_copies * SPECS["gemma_upcycled"].upcycle_slices == 256
    assert SPECS["skewed_prefill"].dtype == BF16 and SPECS["tiny_fp32"].dtype == F32
    with pytest.raises(ValueError):
        spec_by_name("decode@T65")


def test_balance_bias_is_whole_bias_steps():
    from moe_inputs.generate import balance_router_bias
    b = balance_router_bias(64)
    steps = b.astype(np.float64) / 1e-3
    assert np.allclose(steps, np.round(steps), atol=1e-4)
    assert np.max(np.abs(steps)) <= 20 + 1e-6
    assert len(set(np.round(steps).astype(int).tolist())) > 30  # a spread, not a constant
    assert np.array_equal(b, balance_router_bias(64))


def test_small_moe_sigmoid_spec_matches_page_defaults():
    from moe_inputs.spec import SIGMOID
    s = SPECS["small_moe_sigmoid"]
    # SmallMoE(d=1024, n_experts=64, k=8, expert_hidden=256, shared_hidden=1024)
    assert (s.d, s.E, s.k, s.h, s.shared_h) == (1024, 64, 8, 256, 1024)
    assert s.mode == SIGMOID and s.renormalize and not s.shared_gate
