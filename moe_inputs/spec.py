"""Workload specifications for the sparse MoE FFN layer forward.

A spec fixes the shapes, the activation dtype, the gating mode and the
distributions the generator draws from. The five named workloads are:

* ``tiny_fp32``       T=64, d=64, E=8, h=128, k=2, fp32; softmax over all 8
                      logits, top-2, renormalised. Everything ~N(0, 0.02) except
                      x ~ N(0, 1).
* ``gemma_upcycled``  T=8192 (16 sequences of 512), d=640, E=256, h=512, k=4,
                      bf16; gates = softmax over the 4 selected logits (the
                      router of "Small models, sparse experts", section "How it
                      works"). Router ~N(0, 0.01). Experts drop-upcycled from a
                      640->2048 SwiGLU: 4 slices of 512 hidden units, each
                      copied 64 times, scaled by 64**(1/3) = 4, with 10% of the
                      entries redrawn in every copy but the first.
* ``decode``          d=2048, E=64, h=1024, k=8, bf16, softmax over all 64,
                      top-8, no renormalisation; T in {1, 4, 16, 64}.
* ``skewed_prefill``  T=16384, d=2048, E=128, h=768, k=8, bf16; softmax over
                      all then renormalised over the 8; fp32 router bias
                      b_e = 2*ln(1/(e+1)**1.1) for a Zipf-like expert load.
* ``shared_routed``   T=8192, d=2048, E=60, h=1408, k=4, bf16, softmax over all
                      60 without renormalisation; plus one always-on shared
                      SwiGLU of hidden 5632 scaled by sigmoid(w_s . x).
* ``decode_q4``       the decode workload with its routed experts in 4-bit affine
                      groups of 64 (``generate.quantize_q4_g64`` of the same
                      draws); T in {1, 4, 16, 64}.
* ``small_moe_sigmoid`` the defaults of the SmallMoE module of "Small MoE
                      Architecture, in depth" (d=1024, 64 experts, top-8,
                      expert hidden 256, one ungated shared expert of hidden
                      1024) on T=4096 tokens, bf16: sigmoid affinities, top-8
                      on affinity + balance bias, gates = affinities of the
                      chosen experts renormalised. The balance bias is a fixed
                      pattern of multiples of the page's bias step 1e-3, at
                      most 20 steps either way (``balance_router_bias``).

Standard deviations are given as std (not variance). ``small_spec`` builds
reduced shapes with the same structure for tests that the CPU oracle must
finish in seconds.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

# Gate modes. Values match the C ABI enum ``moe_score_mode``.
SOFTMAX_ALL = 0
SOFTMAX_SELECTED = 1
SIGMOID = 2

# Activation dtypes. Values match the C ABI enum ``moe_dtype``.
F32 = 0
BF16 = 1


@dataclasses.dataclass(frozen=True)
class MoESpec:
    name: str
    T: int
    d: int
    E: int
    h: int
    k: int
    dtype: int = BF16
    mode: int = SOFTMAX_ALL
    renormalize: bool = False
    x_std: float = 1.0
    router_std: float = 0.02
    expert_std: float = 0.02
    # "zipf": b_e = 2*ln(1/(e+1)**1.1) added to the logits; "balance": a
    # selection-only balance bias (SIGMOID mode); None: no bias vector
    router_bias: Optional[str] = None
    # 0: no shared expert
    shared_h: int = 0
    # routed-expert weight format: None (activation dtype) or "q4_g64"
    # (4-bit affine groups of 64 along the reduction axis, bf16 scale + bias)
    expert_quant: Optional[str] = None
    # sigmoid(w_s . x) gate on the shared expert (only meaningful if shared_h > 0)
    shared_gate: bool = False
    # drop-upcycled expert construction (gemma_upcycled)
    upcycle: bool = False
    upcycle_slices: int = 4
    upcycle_copies: int = 64
    upcycle_scale: float = 4.0  # 64 ** (1/3)
    upcycle_redraw: float = 0.10
    # token budget drawn for x; T <= x_rows (decode draws 64 rows once and
    # uses a prefix, so every T sees the same first tokens)
    x_rows: Optional[int] = None
    seed: int = 0

    @property
    def P(self) -> int:
        return self.T * self.k

    @property
    def has_bias(self) -> bool:
        return self.router_bias is not None

    @property
    def act_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    def with_T(self, T: int) -> "MoESpec":
        rows = self.x_rows if self.x_rows is not None else None
        if rows is not None and T > rows:
            raise ValueError(f"T={T} exceeds the x rows drawn for {self.name} ({rows})")
        return dataclasses.replace(self, T=T, name=f"{self.name.split('@')[0]}@T{T}")


SPECS = {
    "tiny_fp32": MoESpec(
        name="tiny_fp32", T=64, d=64, E=8, h=128, k=2, dtype=F32,
        mode=SOFTMAX_ALL, renormalize=True, router_std=0.02, expert_std=0.02),
    "gemma_upcycled": MoESpec(
        name="gemma_upcycled", T=8192, d=640, E=256, h=512, k=4, dtype=BF16,
        mode=SOFTMAX_SELECTED, renormalize=False, router_std=0.01,
        expert_std=0.02, upcycle=True),
    "decode": MoESpec(
        name="decode@T1", T=1, d=2048, E=64, h=1024, k=8, dtype=BF16,
        mode=SOFTMAX_ALL, renormalize=False, router_std=0.02, expert_std=0.02,
        x_rows=64),
    "skewed_prefill": MoESpec(
        name="skewed_prefill", T=16384, d=2048, E=128, h=768, k=8, dtype=BF16,
        mode=SOFTMAX_ALL, renormalize=True, router_std=0.02, expert_std=0.02,
        router_bias="zipf"),
    "shared_routed": MoESpec(
        name="shared_routed", T=8192, d=2048, E=60, h=1408, k=4, dtype=BF16,
        mode=SOFTMAX_ALL, renormalize=False, router_std=0.02, expert_std=0.02,
        shared_h=5632, shared_gate=True),
    "decode_q4": MoESpec(
        name="decode_q4@T1", T=1, d=2048, E=64, h=1024, k=8, dtype=BF16,
        mode=SOFTMAX_ALL, renormalize=False, router_std=0.02, expert_std=0.02,
        x_rows=64, expert_quant="q4_g64"),
    "small_moe_sigmoid": MoESpec(
        name="small_moe_sigmoid", T=4096, d=1024, E=64, h=256, k=8, dtype=BF16,
        mode=SIGMOID, renormalize=True, router_std=0.02, expert_std=0.02,
        router_bias="balance", shared_h=1024, shared_gate=False),
}

DECODE_TOKENS = (1, 4, 16, 64)


def spec_by_name(name: str) -> MoESpec:
    """``decode@T16`` style names select a decode batch size."""
    if "@T" in name:
        base, t = name.split("@T")
        return SPECS[base].with_T(int(t))
    return SPECS[name]


def small_spec(base: str, **overrides) -> MoESpec:
    """A reduced-shape copy of a named workload (same modes and distributions)."""
    s = SPECS[base]
    fields = dict(overrides)
    fields.setdefault("name", f"{base}-small")
    if s.upcycle and "upcycle_copies" not in fields:
        E = fields.get("E", s.E)
        slices = fields.get("upcycle_slices", s.upcycle_slices)
        fields["upcycle_copies"] = max(1, E // slices)
    if s.x_rows is not None and "x_rows" not in fields:
        fields["x_rows"] = None
    return dataclasses.replace(s, **fields)
