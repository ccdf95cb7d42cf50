"""ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the layer runs in the library's kernels.
There is no fallback: if libmoe.so is missing or a call fails, this module
raises.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libmoe.so")
HEADER = os.path.join(ROOT, "include", "moe.h")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4
MOE_ERR_SCRATCH_LIMIT = 5
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

MOE_F32 = 0
MOE_BF16 = 1
MOE_SOFTMAX_ALL = 0
MOE_SOFTMAX_SELECTED = 1
MOE_SIGMOID = 2
MOE_QUANT_NONE = 0
MOE_QUANT_Q4_G64 = 1

MOE_ENTRY_LAYER_FORWARD = 0
MOE_ENTRY_DISPATCH = 1
MOE_ENTRY_GATE_UP = 2
MOE_ENTRY_DOWN = 3
MOE_ENTRY_EXPERT_FFN = 4
MOE_ENTRY_SHARED_EXPERT = 5
MOE_ENTRY_ROUTING_STATS = 6
MOE_ENTRY_LAYER_BACKWARD = 7

MOE_TABLE_OFFSETS = 0
MOE_TABLE_PERM = 1
MOE_TABLE_INV = 2

MOE_NUM_STAGES = 5
STAGE_NAMES = ("route", "dispatch", "gate_up", "down", "combine")
MOE_NUM_BWD_STAGES = 8
BWD_STAGE_NAMES = ("route", "d_hidden", "z", "router_grad", "dw_down", "dw_gate_up", "dx_rows",
                   "dx_router")


class MoeConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T", "d", "E", "h", "top_k", "dtype", "mode", "renormalize", "has_router_bias",
        "shared_h", "shared_gate", "expert_quant")]


class MoeWeights(ctypes.Structure):
    _fields_ = [
        ("w_router", ctypes.c_void_p), ("b_router", ctypes.c_void_p),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("ws_gate", ctypes.c_void_p), ("ws_up", ctypes.c_void_p), ("ws_down", ctypes.c_void_p),
        ("w_shared_gate", ctypes.c_void_p),
        ("w_gate_sb", ctypes.c_void_p), ("w_up_sb", ctypes.c_void_p),
        ("w_down_sb", ctypes.c_void_p),
    ]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up", "dws_down",
        "dw_shared_gate", "dgates", "dlogits")]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


_lib = None

_P = ctypes.c_void_p
_SIG = {
    "moe_abi_version": ([], ctypes.c_int32),
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_validate_config": ([_P], ctypes.c_int),
    "moe_workspace_size_entry": ([_P, ctypes.c_int32], ctypes.c_size_t),
    "moe_workspace_size": ([_P], ctypes.c_size_t),
    "moe_workspace_table_offset": ([_P, ctypes.c_int32], ctypes.c_size_t),
    "moe_route": ([_P] * 8, ctypes.c_int),
    "moe_dispatch": ([_P] * 7 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_gate_up": ([_P] * 8 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_down": ([_P] * 6 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_expert_ffn": ([_P] * 9 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_shared_expert": ([_P] * 8 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_combine": ([_P] * 7, ctypes.c_int),
    "moe_routing_stats": ([_P] * 3 + [ctypes.c_float] + [_P] * 4 + [ctypes.c_size_t, _P],
                          ctypes.c_int),
    "moe_layer_forward": ([_P] * 8 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_layer_forward_traced": ([_P] * 8 + [ctypes.c_size_t, _P, _P], ctypes.c_int),
    "moe_layer_forward_noalloc": ([_P] * 8, ctypes.c_int),
    "moe_layer_backward": ([_P] * 6 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_layer_backward_traced": ([_P] * 6 + [ctypes.c_size_t, _P, _P], ctypes.c_int),
}


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with "
                "`python -m mixture_experts_sparse_amd.build` (there is no fallback path)")
        # torch first: its bundled HIP runtime carries the same SONAME
        # (libamdhip64.so.7), so libmoe binds to the runtime torch's streams
        # and allocations belong to instead of loading a second copy.
        import torch  # noqa: F401
        L = ctypes.CDLL(path)
        for name, (args, res) in _SIG.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/moe.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


# ----------------------------------------------------------------------------
# config helpers
# ----------------------------------------------------------------------------

def make_config(T, d, E, h, top_k, dtype=MOE_BF16, mode=MOE_SOFTMAX_ALL, renormalize=False,
                has_router_bias=False, shared_h=0, shared_gate=False,
                expert_quant=MOE_QUANT_NONE) -> MoeConfig:
    return MoeConfig(int(T), int(d), int(E), int(h), int(top_k), int(dtype), int(mode),
                     int(bool(renormalize)), int(bool(has_router_bias)), int(shared_h),
                     int(bool(shared_gate)), int(expert_quant))


def config_from_spec(spec, T: Optional[int] = None) -> MoeConfig:
    """Config from a moe_inputs.MoESpec-like object (duck-typed)."""
    return make_config(spec.T if T is None else T, spec.d, spec.E, spec.h, spec.k,
                       dtype=spec.dtype, mode=spec.mode, renormalize=spec.renormalize,
                       has_router_bias=spec.router_bias is not None, shared_h=spec.shared_h,
                       shared_gate=spec.shared_gate and spec.shared_h > 0,
                       expert_quant=MOE_QUANT_Q4_G64 if getattr(spec, "expert_quant", None)
                       else MOE_QUANT_NONE)


def validate_config(cfg: MoeConfig) -> int:
    return lib().moe_validate_config(ctypes.byref(cfg))


def workspace_size(cfg: MoeConfig, entry: int = MOE_ENTRY_LAYER_FORWARD) -> int:
    return int(lib().moe_workspace_size_entry(ctypes.byref(cfg), int(entry)))


def workspace_table_offset(cfg: MoeConfig, table: int) -> int:
    off = int(lib().moe_workspace_table_offset(ctypes.byref(cfg), int(table)))
    if off == 2**64 - 1:
        raise MoeError(MOE_ERR_INVALID_ARG, "moe_workspace_table_offset")
    return off


def workspace_tables(cfg: MoeConfig, ws):
    """(offsets [E+1], perm [P], inv [P]) int32 views into a layer-forward
    workspace ``ws`` (a uint8 tensor): the dispatch of the last
    moe_layer_forward that used it, once that call has completed."""
    import torch
    P = cfg.T * cfg.top_k
    out = []
    for table, n in ((MOE_TABLE_OFFSETS, cfg.E + 1), (MOE_TABLE_PERM, P), (MOE_TABLE_INV, P)):
        off = workspace_table_offset(cfg, table)
        out.append(ws[off:off + 4 * n].view(torch.int32))
    return tuple(out)


# ----------------------------------------------------------------------------
# tensor marshalling
# ----------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _torch_dtype(cfg: MoeConfig):
    import torch
    return torch.bfloat16 if cfg.dtype == MOE_BF16 else torch.float32


def alloc_workspace(cfg: MoeConfig, entry: int = MOE_ENTRY_LAYER_FORWARD, device="cuda"):
    import torch
    n = workspace_size(cfg, entry)
    if n == 0 and validate_config(cfg) != MOE_OK:
        _check(validate_config(cfg), "workspace_size")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def route(cfg, x, w_router, b_router=None, ids=None, gates=None, logits=None, stream=None):
    import torch
    dev = x.device
    if ids is None:
        ids = torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device=dev)
    if gates is None:
        gates = torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device=dev)
    _check(lib().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(b_router),
                           _ptr(ids), _ptr(gates), _ptr(logits), _stream(stream)), "moe_route")
    return ids, gates


def dispatch(cfg, ids, ws=None, stream=None):
    import torch
    dev = ids.device
    P = cfg.T * cfg.top_k
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
    if ws is None:
        ws = alloc_workspace(cfg, MOE_ENTRY_DISPATCH, dev)
    _check(lib().moe_dispatch(ctypes.byref(cfg), _ptr(ids), _ptr(counts), _ptr(offsets),
                              _ptr(perm), _ptr(inv), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_dispatch")
    return counts, offsets, perm[:P], inv[:P]


def gate_up(cfg, x, perm, offsets, w_gate, w_up, act=None, ws=None, stream=None):
    import torch
    if act is None:
        act = torch.empty((cfg.T * cfg.top_k, cfg.h), dtype=_torch_dtype(cfg), device=x.device)
    if ws is None:
        ws = alloc_workspace(cfg, MOE_ENTRY_GATE_UP, x.device)
    _check(lib().moe_gate_up(ctypes.byref(cfg), _ptr(x), _ptr(perm), _ptr(offsets),
                             _ptr(w_gate), _ptr(w_up), _ptr(act), _ptr(ws), ws.numel(),
                             _stream(stream)), "moe_gate_up")
    return act


def down(cfg, act, offsets, w_down, y=None, ws=None, stream=None):
    import torch
    if y is None:
        y = torch.empty((cfg.T * cfg.top_k, cfg.d), dtype=_torch_dtype(cfg), device=act.device)
    if ws is None:
        ws = alloc_workspace(cfg, MOE_ENTRY_DOWN, act.device)
    _check(lib().moe_down(ctypes.byref(cfg), _ptr(act), _ptr(offsets), _ptr(w_down), _ptr(y),
                          _ptr(ws), ws.numel(), _stream(stream)), "moe_down")
    return y


def expert_ffn(cfg, x, perm, offsets, w_gate, w_up, w_down, y=None, ws=None, stream=None):
    import torch
    if y is None:
        y = torch.empty((cfg.T * cfg.top_k, cfg.d), dtype=_torch_dtype(cfg), device=x.device)
    if ws is None:
        ws = alloc_workspace(cfg, MOE_ENTRY_EXPERT_FFN, x.device)
    _check(lib().moe_expert_ffn(ctypes.byref(cfg), _ptr(x), _ptr(perm), _ptr(offsets),
                                _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y), _ptr(ws),
                                ws.numel(), _stream(stream)), "moe_expert_ffn")
    return y


def shared_expert(cfg, x, ws_gate, ws_up, ws_down, w_shared_gate=None, out=None, ws=None,
                  stream=None):
    import torch
    if out is None:
        out = torch.empty((cfg.T, cfg.d), dtype=_torch_dtype(cfg), device=x.device)
    if ws is None:
        ws = alloc_workspace(cfg, MOE_ENTRY_SHARED_EXPERT, x.device)
    _check(lib().moe_shared_expert(ctypes.byref(cfg), _ptr(x), _ptr(ws_gate), _ptr(ws_up),
                                   _ptr(ws_down), _ptr(w_shared_gate), _ptr(out), _ptr(ws),
                                   ws.numel(), _stream(stream)), "moe_shared_expert")
    return out


def combine(cfg, y, inv, gates, shared=None, out=None, stream=None):
    import torch
    if out is None:
        out = torch.empty((cfg.T, cfg.d), dtype=_torch_dtype(cfg), device=y.device)
    _check(lib().moe_combine(ctypes.byref(cfg), _ptr(y), _ptr(inv), _ptr(gates), _ptr(shared),
                             _ptr(out), _stream(stream)), "moe_combine")
    return out


def routing_stats(cfg, logits, counts, alpha=0.01, ws=None, stream=None, outs=None):
    """(share [E], mean_prob [E], scalars [2] = (entropy, aux)) as device
    tensors, from router logits [T, E] f32 and counts [E] int32. ``outs``:
    optional preallocated (share [E], mean_prob [E], scalars [>= 2]) f32."""
    import torch
    dev = logits.device
    if outs is not None:
        share, mean_prob, scalars = outs
    else:
        share = torch.empty(cfg.E, dtype=torch.float32, device=dev)
        mean_prob = torch.empty(cfg.E, dtype=torch.float32, device=dev)
        scalars = torch.empty(4, dtype=torch.float32, device=dev)
    if ws is None:
        ws = alloc_workspace(cfg, MOE_ENTRY_ROUTING_STATS, dev)
    _check(lib().moe_routing_stats(ctypes.byref(cfg), _ptr(logits), _ptr(counts),
                                   ctypes.c_float(alpha), _ptr(share), _ptr(mean_prob),
                                   _ptr(scalars), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_routing_stats")
    return share, mean_prob, scalars[:2]


def weights_struct(w: dict) -> MoeWeights:
    """w: dict of device tensors keyed like moe_weights' fields."""
    return MoeWeights(*[_ptr(w.get(n)) for n, _ in MoeWeights._fields_])


def layer_forward(cfg, weights, x, out=None, ids=None, gates=None, counts=None, ws=None,
                  stage_events=None, stream=None):
    """The whole layer. ``weights`` is a MoeWeights or a dict of tensors.
    ``stage_events``: a ctypes array of MOE_NUM_STAGES + 1 hipEvent_t, or None."""
    import torch
    if out is None:
        out = torch.empty((cfg.T, cfg.d), dtype=_torch_dtype(cfg), device=x.device)
    if ws is None:
        ws = alloc_workspace(cfg, MOE_ENTRY_LAYER_FORWARD, x.device)
    wst = weights if isinstance(weights, MoeWeights) else weights_struct(weights)
    args = (ctypes.byref(cfg), ctypes.byref(wst), _ptr(x), _ptr(out), _ptr(ids), _ptr(gates),
            _ptr(counts), _ptr(ws), ws.numel())
    if stage_events is None:
        st = lib().moe_layer_forward(*args, _stream(stream))
    else:
        st = lib().moe_layer_forward_traced(*args, ctypes.cast(stage_events, ctypes.c_void_p),
                                            _stream(stream))
    _check(st, "moe_layer_forward")
    return out


def layer_forward_noalloc(cfg, weights, x, out=None, ids=None, gates=None, counts=None,
                          stream=None):
    """The whole layer with the library's static device workspace
    (moe_layer_forward_noalloc): no workspace argument, nothing allocated by
    the library."""
    import torch
    if out is None:
        out = torch.empty((cfg.T, cfg.d), dtype=_torch_dtype(cfg), device=x.device)
    wst = weights if isinstance(weights, MoeWeights) else weights_struct(weights)
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(cfg), ctypes.byref(wst), _ptr(x),
                                           _ptr(out), _ptr(ids), _ptr(gates), _ptr(counts),
                                           _stream(stream)), "moe_layer_forward_noalloc")
    return out


def layer_backward(cfg, weights, x, dout, grads=None, ws=None, want_intermediates=False,
                   stage_events=None, stream=None):
    """Gradients of sum(out * dout) for the layer (moe_layer_backward). Returns
    a dict of float32 device tensors keyed like moe_grads' fields (the shared
    expert's only when the layer has one; dgates / dlogits only when
    ``want_intermediates``). ``grads``: a dict of preallocated outputs."""
    import torch
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(grads or {})
    shapes = {"dx": (cfg.T, cfg.d), "dw_router": (cfg.E, cfg.d),
              "dw_gate": (cfg.E, cfg.h, cfg.d), "dw_up": (cfg.E, cfg.h, cfg.d),
              "dw_down": (cfg.E, cfg.d, cfg.h)}
    if cfg.shared_h > 0:
        shapes.update(dws_gate=(cfg.shared_h, cfg.d), dws_up=(cfg.shared_h, cfg.d),
                      dws_down=(cfg.d, cfg.shared_h))
        if cfg.shared_gate:
            shapes["dw_shared_gate"] = (cfg.d,)
    if want_intermediates:
        shapes.update(dgates=(cfg.T, cfg.top_k), dlogits=(cfg.T, cfg.E))
    for n, shp in shapes.items():
        if n not in g:
            g[n] = torch.empty(shp, **f32)
    if ws is None:
        ws = alloc_workspace(cfg, MOE_ENTRY_LAYER_BACKWARD, dev)
    wst = weights if isinstance(weights, MoeWeights) else weights_struct(weights)
    gs = MoeGrads(*[_ptr(g.get(n)) for n, _ in MoeGrads._fields_])
    args = (ctypes.byref(cfg), ctypes.byref(wst), _ptr(x), _ptr(dout), ctypes.byref(gs), _ptr(ws),
            ws.numel())
    if stage_events is None:
        st = lib().moe_layer_backward(*args, _stream(stream))
    else:
        st = lib().moe_layer_backward_traced(*args, ctypes.cast(stage_events, ctypes.c_void_p),
                                             _stream(stream))
    _check(st, "moe_layer_backward")
    return g
