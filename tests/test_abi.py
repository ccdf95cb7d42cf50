"""The C ABI on a machine without a GPU: the library loads, exports every
function include/moe.h declares, and rejects bad arguments on the host before
any HIP call (only null or fake pointers are passed here, and every call is
one that must fail validation, so nothing reaches the device)."""

import ctypes

import pytest

import mixture_experts_sparse_amd.binding as B
from mixture_experts_sparse_amd import build as build_mod


def test_library_exports_every_header_function():
    L = B.lib()
    names = B.header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert L.moe_abi_version() == 4


def test_noalloc_rejects_calls_beyond_its_scratch():
    """The no-alloc entry point refuses a configuration whose workspace is
    larger than its static array, on the host, before any HIP call; T = 0
    is a no-op and a bad configuration is an argument error."""
    big = B.make_config(16384, 2048, 128, 768, 8)
    assert B.workspace_size(big) > B.MOE_NOALLOC_SCRATCH_BYTES
    w = B.MoeWeights()
    st = B.lib().moe_layer_forward_noalloc(ctypes.byref(big), ctypes.byref(w), None, None,
                                           None, None, None, None)
    assert st == B.MOE_ERR_SCRATCH_LIMIT
    assert "MOE_ERR_SCRATCH_LIMIT" in B.status_string(st)
    zero = B.make_config(0, 2048, 64, 1024, 8)
    assert B.lib().moe_layer_forward_noalloc(ctypes.byref(zero), ctypes.byref(w), None, None,
                                             None, None, None, None) == B.MOE_OK
    bad = B.make_config(10, 64, 8, 32, 9)
    assert B.lib().moe_layer_forward_noalloc(ctypes.byref(bad), ctypes.byref(w), None, None,
                                             None, None, None, None) == B.MOE_ERR_INVALID_ARG
    # decode-shaped calls fit
    assert B.workspace_size(B.make_config(64, 2048, 64, 1024, 8)) <= B.MOE_NOALLOC_SCRATCH_BYTES


def test_workspace_table_offsets():
    """The dispatch tables a fused call leaves in its workspace lie inside the
    layer-forward workspace, 256-byte aligned and disjoint; bad arguments
    give SIZE_MAX (raised by the binding)."""
    c = B.make_config(8192, 640, 256, 512, 4)
    ws = B.workspace_size(c)
    P = 8192 * 4
    spans = []
    for t, n in ((B.MOE_TABLE_OFFSETS, 257), (B.MOE_TABLE_PERM, P), (B.MOE_TABLE_INV, P)):
        off = B.workspace_table_offset(c, t)
        assert off % 256 == 0 and off + 4 * n <= ws
        spans.append((off, off + 4 * n))
    spans.sort()
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    with pytest.raises(B.MoeError):
        B.workspace_table_offset(c, 3)
    with pytest.raises(B.MoeError):
        B.workspace_table_offset(B.make_config(1, 64, 8, 32, 9), B.MOE_TABLE_PERM)


def test_status_strings():
    for s in range(6):
        assert B.status_string(s).startswith("MOE_")
    assert "UNKNOWN" in B.status_string(99)


def _cfg(**kw):
    base = dict(T=100, d=64, E=8, h=32, top_k=2)
    base.update(kw)
    return B.make_config(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), B.MOE_OK),
    (dict(T=0), B.MOE_OK),
    (dict(T=-1), B.MOE_ERR_INVALID_ARG),
    (dict(d=0), B.MOE_ERR_INVALID_ARG),
    (dict(E=0), B.MOE_ERR_INVALID_ARG),
    (dict(h=-8), B.MOE_ERR_INVALID_ARG),
    (dict(top_k=0), B.MOE_ERR_INVALID_ARG),
    (dict(top_k=9), B.MOE_ERR_INVALID_ARG),     # k > E is rejected, not capped
    (dict(top_k=8), B.MOE_OK),                  # k = E is legal
    (dict(dtype=7), B.MOE_ERR_INVALID_ARG),
    (dict(mode=3), B.MOE_ERR_INVALID_ARG),
    (dict(mode=B.MOE_SIGMOID, has_router_bias=True), B.MOE_OK),
    (dict(expert_quant=B.MOE_QUANT_Q4_G64), B.MOE_OK),
    (dict(expert_quant=2), B.MOE_ERR_INVALID_ARG),
    (dict(shared_gate=True), B.MOE_ERR_INVALID_ARG),  # gate without a shared expert
    (dict(d=60), B.MOE_ERR_UNSUPPORTED),
    (dict(h=36), B.MOE_ERR_UNSUPPORTED),
    (dict(shared_h=12), B.MOE_ERR_UNSUPPORTED),
    (dict(E=257, top_k=2), B.MOE_ERR_UNSUPPORTED),
    (dict(E=256, top_k=256), B.MOE_OK),
])
def test_config_validation(kw, status):
    assert B.validate_config(_cfg(**kw)) == status


def test_workspace_sizes_are_bounded():
    # the skewed prefill shape: workspace is O(P*(d+h)), never O(T*h*d)
    c = B.make_config(16384, 2048, 128, 768, 8)
    ws = B.workspace_size(c)
    P = 16384 * 8
    assert ws >= P * (2048 + 768) * 2
    assert ws < 1.1 * P * (2048 + 768) * 2 + 16 * 2**20
    gathered = 16384 * 768 * 2048 * 2
    assert ws < gathered / 10
    for e in range(7):
        assert B.workspace_size(c, e) <= ws
    # routing statistics: one row of E + 1 floats per block of at least 32
    # tokens, at most 256 blocks
    assert B.workspace_size(c, B.MOE_ENTRY_ROUTING_STATS) == 256 * 129 * 4
    small = B.make_config(1000, 64, 64, 32, 8)
    assert B.workspace_size(small, B.MOE_ENTRY_ROUTING_STATS) == (-(-1000 // 32) * 65 * 4 + 255) // 256 * 256
    huge = B.make_config(1 << 20, 64, 256, 32, 8)
    assert B.workspace_size(huge, B.MOE_ENTRY_ROUTING_STATS) == 256 * 257 * 4
    assert B.workspace_size(c, B.MOE_ENTRY_DISPATCH) < 8 * 2**20
    assert B.workspace_size(B.make_config(1, 64, 8, 32, 9)) == 0  # invalid cfg


FAKE = 0x1000  # 16-byte aligned, never dereferenced: every call below fails validation


def test_entry_points_reject_bad_args_without_gpu():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("fake-pointer validation checks run only where no GPU is present")
    L = B.lib()
    c = _cfg()
    bad = _cfg(top_k=0)
    cp, bp = ctypes.byref(c), ctypes.byref(bad)
    # null required pointers
    assert L.moe_route(cp, None, FAKE, None, FAKE, FAKE, None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_route(cp, FAKE, FAKE, None, None, FAKE, None, None) == B.MOE_ERR_INVALID_ARG
    # misaligned pointer
    assert L.moe_route(cp, FAKE + 2, FAKE, None, FAKE, FAKE, None, None) == B.MOE_ERR_UNSUPPORTED
    # bias required when has_router_bias
    cb = _cfg(has_router_bias=True)
    assert L.moe_route(ctypes.byref(cb), FAKE, FAKE, None, FAKE, FAKE, None, None) == B.MOE_ERR_INVALID_ARG
    # bad config
    assert L.moe_route(bp, FAKE, FAKE, None, FAKE, FAKE, None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_route(None, FAKE, FAKE, None, FAKE, FAKE, None, None) == B.MOE_ERR_INVALID_ARG
    # workspace too small / misaligned
    need = B.workspace_size(c, B.MOE_ENTRY_DISPATCH)
    assert L.moe_dispatch(cp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == B.MOE_ERR_WORKSPACE
    assert L.moe_dispatch(cp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16, need, None) == B.MOE_ERR_WORKSPACE
    assert L.moe_dispatch(cp, FAKE, FAKE, FAKE, FAKE, FAKE, None, need, None) == B.MOE_ERR_WORKSPACE
    assert L.moe_gate_up(cp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == B.MOE_ERR_WORKSPACE
    assert L.moe_down(cp, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn(cp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, None) == B.MOE_ERR_WORKSPACE
    # shared expert without shared_h
    assert L.moe_shared_expert(cp, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_combine(cp, FAKE, FAKE, None, None, FAKE, None) == B.MOE_ERR_INVALID_ARG
    # layer forward: null weights struct, missing shared weights, tiny workspace
    assert L.moe_layer_forward(cp, None, FAKE, FAKE, None, None, None, FAKE, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    w = B.MoeWeights(FAKE, None, FAKE, FAKE, FAKE, None, None, None, None)
    assert L.moe_layer_forward(cp, ctypes.byref(w), FAKE, FAKE, None, None, None, FAKE, 16, None) == B.MOE_ERR_WORKSPACE
    cs = _cfg(shared_h=16, shared_gate=True)
    assert L.moe_layer_forward(ctypes.byref(cs), ctypes.byref(w), FAKE, FAKE, None, None, None, FAKE,
                               1 << 40, None) == B.MOE_ERR_INVALID_ARG
    w2 = B.MoeWeights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert L.moe_layer_forward(ctypes.byref(cs), ctypes.byref(w2), FAKE, FAKE, None, None, None, FAKE,
                               1 << 40, None) == B.MOE_ERR_INVALID_ARG
    # misaligned optional output
    assert L.moe_layer_forward(cp, ctypes.byref(w), FAKE, FAKE, FAKE + 4, None, None, FAKE,
                               1 << 40, None) == B.MOE_ERR_UNSUPPORTED
    # 4-bit routed experts: scale words required; only small-batch shapes;
    # the standalone expert entry points take activation-dtype weights only
    cq = _cfg(T=16, d=128, h=64, expert_quant=B.MOE_QUANT_Q4_G64)
    wq = B.MoeWeights(FAKE, None, FAKE, FAKE, FAKE, None, None, None, None, FAKE, None, FAKE)
    assert L.moe_layer_forward(ctypes.byref(cq), ctypes.byref(wq), FAKE, FAKE, None, None, None,
                               FAKE, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    cq_big = _cfg(T=100, d=128, h=64, expert_quant=B.MOE_QUANT_Q4_G64)  # P = 200 > 16 * 8
    wq2 = B.MoeWeights(FAKE, None, FAKE, FAKE, FAKE, None, None, None, None, FAKE, FAKE, FAKE)
    assert L.moe_layer_forward(ctypes.byref(cq_big), ctypes.byref(wq2), FAKE, FAKE, None, None,
                               None, FAKE, 1 << 40, None) == B.MOE_ERR_UNSUPPORTED
    cq_odd = _cfg(T=16, d=96, h=64, expert_quant=B.MOE_QUANT_Q4_G64)  # d not whole groups
    assert L.moe_layer_forward(ctypes.byref(cq_odd), ctypes.byref(wq2), FAKE, FAKE, None, None,
                               None, FAKE, 1 << 40, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_gate_up(ctypes.byref(cq), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                         None) == B.MOE_ERR_UNSUPPORTED
    # routing statistics: required pointers, alpha range, workspace
    f32 = ctypes.c_float
    assert L.moe_routing_stats(cp, None, FAKE, f32(0.01), FAKE, FAKE, FAKE, FAKE, 1 << 30,
                               None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_routing_stats(cp, FAKE, FAKE, f32(0.01), FAKE, None, FAKE, FAKE, 1 << 30,
                               None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_routing_stats(cp, FAKE, FAKE, f32(-1.0), FAKE, FAKE, FAKE, FAKE, 1 << 30,
                               None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_routing_stats(cp, FAKE, FAKE, f32(float("nan")), FAKE, FAKE, FAKE, FAKE, 1 << 30,
                               None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_routing_stats(cp, FAKE, FAKE, f32(0.01), FAKE, FAKE, FAKE, FAKE, 8,
                               None) == B.MOE_ERR_WORKSPACE
    assert L.moe_routing_stats(bp, FAKE, FAKE, f32(0.01), FAKE, FAKE, FAKE, FAKE, 1 << 30,
                               None) == B.MOE_ERR_INVALID_ARG


def test_build_script_lists_existing_sources():
    import os
    for s in build_mod.SOURCES:
        assert os.path.exists(os.path.join(build_mod.CSRC, s)), s


def _fake(n=1):
    # 16-byte aligned addresses that are never dereferenced (every call below
    # fails host validation first)
    return [ctypes.c_void_p(0x10000 + 256 * i) for i in range(n)]


def _backward(cfg, grads_fields=None, ws_bytes=0, weights_null=False):
    w = B.MoeWeights(*[None] * len(B.MoeWeights._fields_)) if weights_null else \
        B.MoeWeights(*_fake(len(B.MoeWeights._fields_)))
    gf = grads_fields if grads_fields is not None else _fake(len(B.MoeGrads._fields_))
    g = B.MoeGrads(*gf)
    x, dout, ws = _fake(3)
    return B.lib().moe_layer_backward(ctypes.byref(cfg), ctypes.byref(w), x, dout,
                                      ctypes.byref(g), ws, ws_bytes, None)


def test_backward_workspace_size():
    c = _cfg()
    n = B.workspace_size(c, B.MOE_ENTRY_LAYER_BACKWARD)
    P = 100 * 2
    # at least the bf16 da' [P, h], the bf16 pre-activation gradients
    # [P, 2h] and the bf16 dx rows [P, d] (h = 32, d = 64)
    assert n >= P * 32 * 2 + P * 2 * 32 * 2 + P * 64 * 2
    assert n % 256 == 0
    assert B.workspace_size(_cfg(d=60), B.MOE_ENTRY_LAYER_BACKWARD) == 0


def test_backward_host_validation():
    c = _cfg()
    assert _backward(_cfg(dtype=B.MOE_F32)) == B.MOE_ERR_UNSUPPORTED
    assert _backward(_cfg(expert_quant=B.MOE_QUANT_Q4_G64)) == B.MOE_ERR_UNSUPPORTED
    assert _backward(c, weights_null=True) == B.MOE_ERR_INVALID_ARG
    assert _backward(c, grads_fields=[None] * len(B.MoeGrads._fields_)) == B.MOE_ERR_INVALID_ARG
    assert _backward(c, ws_bytes=0) == B.MOE_ERR_WORKSPACE
    assert _backward(_cfg(T=-1)) == B.MOE_ERR_INVALID_ARG
    # a shared expert needs its gradient buffers
    gf = _fake(len(B.MoeGrads._fields_))
    gf[B.MoeGrads._fields_.index(("dws_gate", ctypes.c_void_p))] = None
    assert _backward(_cfg(shared_h=64), grads_fields=gf) == B.MOE_ERR_INVALID_ARG
