"""Algorithmic work counts and roofline arithmetic for the MoE layer forward.

These are the figures the benchmark divides by measured time. They count
what the method must do, not what an implementation adds:

* FLOPs = 2*T*d*E (router) + 2*P*3*d*h (routed SwiGLU experts, P = T*k)
          + 2*T*3*d*hs + 2*T*d (shared expert and its sigmoid gate).
  Softmax, top-k, dispatch and combine are not counted (well under 0.1%).
* bytes = U*3*d*h*b (the weights of the U experts that received at least one
          token) + E*d*b (router) + T*d*b (x) + T*d*b (out)
          + 3*d*hs*b + d*b (shared expert) + 4*E (fp32 router bias),
  with b the bytes per activation/weight element; routed experts in the
  4-bit format count Q4_BYTES_PER_WEIGHT (codes plus one bf16 scale and
  bias per 64 weights) instead of b. Intermediates (act, y, dispatch
  tables) are implementation traffic and are not counted.

Two formulas from the pages pin this module's arithmetic:
* the gathered-weight tensor a naive dispatch builds, T*h*d*bytes
  ("Small models, sparse experts", section "Dispatch decides everything":
  one projection, one layer, 2,048 tokens, [2048, 512, 640] fp32 = 2.68 GB);
* the memory-bound decode limit: a step that must stream B bytes per
  token from memory of bandwidth W runs at most W / B tokens per second
  ("Small MoE Architecture, in depth", section "Worked example: the batch-1
  budget on a device").
"""

from __future__ import annotations

# MI355X published peaks.
PEAK_BF16_MFMA_FLOPS = 2.5e15       # dense bf16 MFMA
PEAK_FP32_VALU_FLOPS = 157.3e12     # fp32 vector
PEAK_HBM_BYTES = 8.0e12             # HBM3E

# 4-bit routed-expert weights: half a byte per code plus 2 + 2 bytes of
# scale and bias per group of 64 weights
Q4_BYTES_PER_WEIGHT = 0.5 + 4.0 / 64


def layer_flops(T, d, E, h, k, hs=0, shared_gate=False):
    f = 2.0 * T * d * E + 2.0 * T * k * 3 * d * h
    if hs:
        f += 2.0 * T * 3 * d * hs
        if shared_gate:
            f += 2.0 * T * d
    return f


def layer_bytes(T, d, E, h, U, elem_bytes, hs=0, shared_gate=False, has_bias=False,
                expert_bytes=None):
    b = elem_bytes
    eb = b if expert_bytes is None else expert_bytes
    n = U * 3.0 * d * h * eb + E * d * b + 2.0 * T * d * b
    if hs:
        n += 3.0 * d * hs * b
        if shared_gate:
            n += d * b
    if has_bias:
        n += 4.0 * E
    return n


def gate_up_flops(P, d, h, T=0, hs=0):
    """Gate and up projections of the routed rows (+ the shared expert's)."""
    return 2.0 * P * 2 * d * h + 2.0 * T * 2 * d * hs


def gate_up_bytes(T, d, h, U, elem_bytes, hs=0, expert_bytes=None):
    """Gate and up weights of the touched experts (+ shared) and x, once."""
    eb = elem_bytes if expert_bytes is None else expert_bytes
    return U * 2.0 * d * h * eb + (2.0 * d * hs + T * d) * elem_bytes


def down_flops(P, d, h, T=0, hs=0):
    return 2.0 * P * d * h + 2.0 * T * d * hs


def down_bytes(d, h, U, elem_bytes, hs=0, expert_bytes=None):
    eb = elem_bytes if expert_bytes is None else expert_bytes
    return U * d * h * eb + d * hs * elem_bytes


def gathered_weight_bytes(T, h, d, elem_bytes):
    """Bytes of one projection's per-token gathered weights [T, h, d]."""
    return T * h * d * elem_bytes


def dense_to_sparse_flop_ratio(E, k):
    """Running all E experts instead of the k selected multiplies expert
    arithmetic by E/k."""
    return E / k


def stream_bound_tokens_per_s(bytes_per_token, bandwidth_bytes_per_s=PEAK_HBM_BYTES):
    """Tokens per second a memory-bound step cannot exceed when each token
    must stream ``bytes_per_token`` from memory at the given bandwidth."""
    return bandwidth_bytes_per_s / bytes_per_token


def decode_bound_tokens_per_s(T, d, E, h, U, elem_bytes, expert_bytes=None,
                              bandwidth_bytes_per_s=PEAK_HBM_BYTES):
    """The HBM bound of one decode-shaped layer call: the call's algorithmic
    bytes (``layer_bytes``, U touched experts) streamed once at the given
    bandwidth, for T tokens."""
    per_call = layer_bytes(T, d, E, h, U, elem_bytes, expert_bytes=expert_bytes)
    return T * stream_bound_tokens_per_s(per_call, bandwidth_bytes_per_s)


def ridge_flop_per_byte(peak_flops=PEAK_BF16_MFMA_FLOPS, peak_bytes=PEAK_HBM_BYTES):
    return peak_flops / peak_bytes


def backward_stage_bytes(T, d, E, h, k, hs=0, U=None):
    """Bytes each stage of the layer backward must move through HBM at least
    once (bf16 activations, weights, da' and routed dx rows, float32
    gradients and the shared expert's dx rows),
    the shared expert's included; U: experts touched (all of E by default).
    route: x and W_r in, logits out; d_hidden: dO and W_d in, da' out; z: x,
    W_g|u and da' in, g a and dz out; router_grad: the gate-gradient partials
    and logits in, dL out; dW_down: dO and g a in, dW_d out; dW_gate|up: dz
    and x in, dW_g|u out; dx rows: dz and W_g|u in, the rows out; dx_router:
    dL, W_r, x and the rows in, dx and dW_r out."""
    P = T * k
    U = min(E, P) if U is None else U
    a, f = 2.0, 4.0  # bf16, float32
    gp = -(-h // 32) + (-(-hs // 32) if hs else 0)
    return {"route": (E * d + T * d) * a + T * E * f,
            "d_hidden": T * d * a + (U * d * h + d * hs) * a + (P * h + T * hs) * a,
            "z": T * d * a + 2.0 * (U * h * d + hs * d) * a + 4.0 * (P * h + T * hs) * a,
            "router_grad": P * gp * f + T * E * f + T * E * a,
            "dw_down": T * d * a + (P * h + T * hs) * a + (E * d * h + d * hs) * f,
            "dw_gate_up": 2.0 * (P * h + T * hs) * a + T * d * a + 2.0 * (E * h * d + hs * d) * f,
            "dx_rows": 2.0 * (P * h + T * hs) * a + 2.0 * (U * h * d + hs * d) * a
                       + P * d * a + (T * d if hs else 0) * f,
            "dx_router": T * E * a + E * d * a + T * d * a + P * d * a + (T * d if hs else 0) * f
                         + T * d * f + E * d * f}


def backward_stage_flops(T, d, E, h, k, hs=0, shared_gate=False):
    """FLOPs of each stage of the layer backward (the products it runs,
    the recomputed gate/up pre-activations included): z = 4 P d h, the
    hidden-unit gradient 2 P d h, dW_down 2 P d h, dW_gate|up 4 P d h, the dx
    rows 4 P d h (each + the shared expert's on T rows), the router's two
    products 4 T d E."""
    P = T * k
    return {"route": 2.0 * T * d * E, "z": 4.0 * P * d * h + 4.0 * T * d * hs,
            "d_hidden": 2.0 * P * d * h + 2.0 * T * d * hs, "router_grad": 0.0,
            "dw_down": 2.0 * P * d * h + 2.0 * T * d * hs,
            "dw_gate_up": 4.0 * P * d * h + 4.0 * T * d * hs,
            "dx_rows": 4.0 * P * d * h + 4.0 * T * d * hs,
            "dx_router": 4.0 * T * d * E + (4.0 * T * d if shared_gate else 0.0)}


def routing_stats_bytes(T, E):
    """Algorithmic HBM bytes of one routing-statistics call: the float32
    logits [T, E] and int32 counts [E] read once, share and mean probability
    [E] and the two scalars written (the partial table stays in cache)."""
    return 4.0 * T * E + 4.0 * E + 8.0 * E + 8.0
