"""Seeded generator for the sparse MoE FFN layer inputs.

Draw order (one ``numpy.random.default_rng(seed)`` stream, PCG64, float32
standard normals scaled by the spec's std):

    x [x_rows or T, d], w_router [E, d], (bias: deterministic, no draw),
    w_gate [E, h, d], w_up [E, h, d], w_down [E, d, h],
    then, if there is a shared expert: ws_gate [hs, d], ws_up [hs, d],
    ws_down [d, hs], w_shared_gate [d].

Drop-upcycled experts (``spec.upcycle``) replace the three expert draws by:
base dense SwiGLU G, U [slices*h, d] and D [d, slices*h] (in that order), then
for every copy c >= 1 of every slice, in expert order, a Bernoulli(redraw)
mask and fresh N(0, std) values for gate, up and down (mask then values, per
matrix). Expert e = slice*copies + c copies hidden rows [h*slice, h*(slice+1))
of G and U (and the same columns of D), multiplied by ``upcycle_scale``; the
masked entries take the fresh, unscaled values. This follows the construction
described in "Small models, sparse experts", section "How it works" (split
into four 512-wide slices, 64 copies, scale 64**(1/3), redraw 10% in every
copy except the first).

bf16 tensors are rounded from the float32 draws with round-to-nearest-even
and returned as uint16 bit patterns.
"""

from __future__ import annotations

import math

import numpy as np

from .spec import BF16, MoESpec


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _cast(spec: MoESpec, a: np.ndarray) -> np.ndarray:
    return bf16_bits_from_f32(a) if spec.dtype == BF16 else np.ascontiguousarray(a, np.float32)


def zipf_router_bias(E: int) -> np.ndarray:
    """b_e = 2*ln(1/(e+1)**1.1) = -2.2*ln(e+1), e zero-based, float32."""
    e = np.arange(E, dtype=np.float64)
    return (2.0 * np.log(1.0 / np.power(e + 1.0, 1.1))).astype(np.float32)


def _bf16_round_toward(a: np.ndarray, up: bool) -> np.ndarray:
    """float32 -> the nearest bf16 value at or above (up) / at or below a, as
    float32 (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    t = (a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)  # toward zero
    step_away = ((t.view(np.uint32) + np.uint32(0x10000)).view(np.float32))  # next away from 0
    need = (t < a) if up else (t > a)
    return np.where(need, step_away, t).astype(np.float32)


def quantize_q4_g64(w: np.ndarray):
    """Input construction for the quantised-expert workloads: float32
    weights [..., K] -> (packed [..., K/2] uint8, sb [..., K/64] uint32) in the
    4-bit affine format the layer reads (groups of 64 along the last axis;
    bf16 scale s in the low half of sb, bf16 bias b in the high half; code of
    position 2i in the low nibble of byte i). b is the group minimum rounded
    down to bf16 and s = (max - b) / 15 rounded up to bf16, so every weight
    of the group lies in [b, b + 15 s] and q = round((w - b) / s) dequantises
    within s / 2 of it."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K = w.shape[-1]
    if K % 64 != 0:
        raise ValueError("K must be a multiple of 64")
    g = w.reshape(w.shape[:-1] + (K // 64, 64))
    lo = g.min(axis=-1)
    hi = g.max(axis=-1)
    b = _bf16_round_toward(lo, up=False)
    s = _bf16_round_toward(np.maximum((hi.astype(np.float64) - b) / 15.0, 1e-30).astype(np.float32),
                           up=True)
    q = np.rint((g.astype(np.float64) - b[..., None]) / s[..., None])
    q = np.clip(q, 0, 15).astype(np.uint8).reshape(w.shape)
    packed = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
    sb = (bf16_bits_from_f32(s).astype(np.uint32) |
          (bf16_bits_from_f32(b).astype(np.uint32) << np.uint32(16)))
    return packed, sb


def balance_router_bias(E: int, step: float = 1e-3) -> np.ndarray:
    """A selection-only balance bias as the update rule of "Small MoE
    Architecture, in depth" leaves it: whole multiples of the bias step
    (default 1e-3), here b_e = step * (((7 e + 3) mod 41) - 20), at most 20
    steps either way; deterministic (no draw), float32."""
    e = np.arange(E, dtype=np.int64)
    return (step * (((7 * e + 3) % 41) - 20)).astype(np.float32)


def _upcycled_experts(spec: MoESpec, rng: np.random.Generator):
    S, C, h, d = spec.upcycle_slices, spec.upcycle_copies, spec.h, spec.d
    if S * C != spec.E:
        raise ValueError(f"upcycle: slices*copies={S * C} != E={spec.E}")
    H = S * h
    G = _normal(rng, (H, d), spec.expert_std)
    U = _normal(rng, (H, d), spec.expert_std)
    D = _normal(rng, (d, H), spec.expert_std)
    lam = np.float32(spec.upcycle_scale)
    wg = np.empty((spec.E, h, d), np.float32)
    wu = np.empty((spec.E, h, d), np.float32)
    wd = np.empty((spec.E, d, h), np.float32)
    for s in range(S):
        gs = G[s * h:(s + 1) * h] * lam
        us = U[s * h:(s + 1) * h] * lam
        ds = D[:, s * h:(s + 1) * h] * lam
        for c in range(C):
            e = s * C + c
            wg[e], wu[e], wd[e] = gs, us, ds
            if c == 0:
                continue
            for w in (wg[e], wu[e], wd[e]):
                mask = rng.random(size=w.shape, dtype=np.float32) < np.float32(spec.upcycle_redraw)
                fresh = _normal(rng, w.shape, spec.expert_std)
                w[mask] = fresh[mask]
    return wg, wu, wd


def generate(spec: MoESpec) -> dict:
    """Returns a dict of numpy arrays plus ``spec``. See the module docstring."""
    rng = np.random.default_rng(spec.seed)
    rows = spec.x_rows if spec.x_rows is not None else spec.T
    if spec.T > rows:
        raise ValueError("T exceeds the drawn x rows")
    x = _normal(rng, (rows, spec.d), spec.x_std)[: spec.T]
    w_router = _normal(rng, (spec.E, spec.d), spec.router_std)
    out = {"spec": spec, "x": _cast(spec, x), "w_router": _cast(spec, w_router)}
    if spec.router_bias == "zipf":
        out["b_router"] = zipf_router_bias(spec.E)
    elif spec.router_bias == "balance":
        out["b_router"] = balance_router_bias(spec.E)
    elif spec.router_bias is not None:
        raise ValueError(f"unknown router bias {spec.router_bias!r}")
    else:
        out["b_router"] = None
    if spec.upcycle:
        wg, wu, wd = _upcycled_experts(spec, rng)
    else:
        wg = _normal(rng, (spec.E, spec.h, spec.d), spec.expert_std)
        wu = _normal(rng, (spec.E, spec.h, spec.d), spec.expert_std)
        wd = _normal(rng, (spec.E, spec.d, spec.h), spec.expert_std)
    if spec.expert_quant == "q4_g64":
        # routed experts quantised from the same draws; the shared expert
        # below stays in the activation dtype
        for name, w in (("w_gate", wg), ("w_up", wu), ("w_down", wd)):
            out[name], out[name + "_sb"] = quantize_q4_g64(w)
    elif spec.expert_quant is not None:
        raise ValueError(f"unknown expert quantisation {spec.expert_quant!r}")
    else:
        out["w_gate"], out["w_up"], out["w_down"] = _cast(spec, wg), _cast(spec, wu), _cast(spec, wd)
        out["w_gate_sb"] = out["w_up_sb"] = out["w_down_sb"] = None
    del wg, wu, wd
    if spec.shared_h > 0:
        hs = spec.shared_h
        out["ws_gate"] = _cast(spec, _normal(rng, (hs, spec.d), spec.expert_std))
        out["ws_up"] = _cast(spec, _normal(rng, (hs, spec.d), spec.expert_std))
        out["ws_down"] = _cast(spec, _normal(rng, (spec.d, hs), spec.expert_std))
        if spec.shared_gate:
            out["w_shared_gate"] = _cast(spec, _normal(rng, (spec.d,), spec.expert_std))
        else:
            out["w_shared_gate"] = None
    else:
        out["ws_gate"] = out["ws_up"] = out["ws_down"] = out["w_shared_gate"] = None
    return out


def rotation_x(spec: MoESpec, i: int) -> np.ndarray:
    """x for rotation copy i >= 1 of a timed loop (copy 0 is the workload's
    own x): [T, d] N(0, x_std) float32 normals from
    ``numpy.random.default_rng((seed, i))``, cast like x (bf16 RNE or
    float32). Distinct draws so the routing changes from copy to copy."""
    if i < 1:
        raise ValueError("copy 0 is the workload's own x")
    rng = np.random.default_rng((spec.seed, i))
    return _cast(spec, _normal(rng, (spec.T, spec.d), spec.x_std))


def lambda_upcycle(copies: int) -> float:
    """The drop-upcycling scale copies**(1/3) (64 copies -> 4.0)."""
    return round(math.pow(copies, 1.0 / 3.0), 12)
