"""Python binding of libmoe.so, the MI355X (gfx950) sparse-MoE layer forward.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Functions carry the C entry points' names (see include/moe.h for
the full contract) and take torch tensors that live on the current HIP
device; PyTorch provides the device memory and the stream, nothing else.

The library must have been built (``__graft_entry__.build()`` or
``python -m sparse_moe_layer_fp32_amd._build``); importing fails loudly
otherwise -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
STAGES = ("router_gemm", "topk", "rank", "scan", "scatter", "gateup", "down", "combine")
MOE_NUM_STAGES = len(STAGES)
(MOE_WS_TOPK_IDS, MOE_WS_TOPK_W, MOE_WS_EXPERT_OFFSETS, MOE_WS_SORTED_PAIRS, MOE_WS_PAIR_POS,
 MOE_WS_H, MOE_WS_O, MOE_WS_FUSED_CTL, MOE_WS_FUSED_STATUS) = range(9)
FUSED_MAX_TOKENS, FUSED_MAX_PAIRS = 256, 2048


class MoeError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"moe status {status}: {text}")
        self.status = status


class moe_config(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("inter_shared", ctypes.c_int32),
                ("routed_scaling", ctypes.c_float), ("renormalize", ctypes.c_int32),
                ("swiglu_limit", ctypes.c_float), ("swiglu_limit_shared", ctypes.c_float)]


def make_config(tokens, hidden=4096, num_experts=288, top_k=8, inter=1280, inter_shared=1280,
                routed_scaling=3.0, renormalize=True, swiglu_limit=0.0,
                swiglu_limit_shared=0.0) -> moe_config:
    return moe_config(int(tokens), int(hidden), int(num_experts), int(top_k), int(inter),
                      int(inter_shared), float(routed_scaling), int(bool(renormalize)),
                      float(swiglu_limit), float(swiglu_limit_shared))


class moe_dense_config(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("swiglu_limit", ctypes.c_float), ("reserved", ctypes.c_int32)]


def make_dense_config(tokens, hidden=4096, inter=11264, swiglu_limit=0.0) -> moe_dense_config:
    return moe_dense_config(int(tokens), int(hidden), int(inter), float(swiglu_limit), 0)


_lib = None


def load_library():
    """Load libmoe.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first "
                          "(python -m sparse_moe_layer_fp32_amd._build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, cp = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(moe_config)
    lib.moe_workspace_size.argtypes = [cp]
    lib.moe_workspace_size.restype = sz
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_route.argtypes = [cp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_permute.argtypes = [cp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_forward.argtypes = [cp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_forward_timed.argtypes = lib.moe_forward.argtypes + [ctypes.POINTER(vp), ctypes.c_int]
    lib.moe_forward_noalloc.argtypes = [cp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_workspace_view.argtypes = [cp, ctypes.c_int, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.moe_forward_fp8.argtypes = [cp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    vp, sz, vp]
    dp = ctypes.POINTER(moe_dense_config)
    lib.moe_dense_workspace_size.argtypes = [dp]
    lib.moe_dense_workspace_size.restype = sz
    lib.moe_dense_forward.argtypes = [dp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_forward_fused.argtypes = lib.moe_forward.argtypes
    for f in ("moe_route", "moe_permute", "moe_forward", "moe_forward_timed",
              "moe_workspace_view", "moe_dense_forward", "moe_forward_fp8", "moe_forward_fused"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


EXPORTED = ("moe_workspace_size", "moe_last_error", "moe_route", "moe_permute", "moe_forward",
            "moe_forward_timed", "moe_workspace_view", "moe_dense_workspace_size",
            "moe_dense_forward", "moe_forward_fp8", "moe_forward_fused",
            "moe_forward_noalloc")
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES


# ------------------------------------------------------------------ helpers

def _torch():
    import torch
    return torch


def _ptr(t, dtype=None, name="tensor", optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtype}")
    return t.data_ptr()


def _bf16():
    torch = _torch()
    return (torch.bfloat16, torch.uint16, torch.int16)


def _f32():
    return (_torch().float32,)


def _i32():
    return (_torch().int32,)


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, load_library().moe_last_error().decode())


def moe_last_error() -> str:
    return load_library().moe_last_error().decode()


def moe_workspace_size(cfg: moe_config) -> int:
    n = load_library().moe_workspace_size(ctypes.byref(cfg))
    if n == 0:
        raise MoeError(MOE_ERR_INVALID_ARG, moe_last_error())
    return int(n)


def alloc_workspace(cfg: moe_config, device=None):
    """A zero-filled uint8 device tensor of moe_workspace_size(cfg) bytes
    (zero-filled once, as moe_forward_fused requires of its control words)."""
    torch = _torch()
    return torch.zeros(moe_workspace_size(cfg), dtype=torch.uint8,
                       device=device or torch.device("cuda"))


def moe_route(cfg, x, router_w, router_bias, topk_ids, topk_w, ws, stream=None):
    lib = load_library()
    _check(lib.moe_route(ctypes.byref(cfg), _ptr(x, _bf16(), "x"), _ptr(router_w, _f32(), "router_w"),
                         _ptr(router_bias, _f32(), "router_bias", True),
                         _ptr(topk_ids, _i32(), "topk_ids"), _ptr(topk_w, _f32(), "topk_w"),
                         _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)))


def moe_permute(cfg, topk_ids, expert_offsets, sorted_pairs, pair_pos, ws, stream=None):
    lib = load_library()
    _check(lib.moe_permute(ctypes.byref(cfg), _ptr(topk_ids, _i32(), "topk_ids"),
                           _ptr(expert_offsets, _i32(), "expert_offsets"),
                           _ptr(sorted_pairs, _i32(), "sorted_pairs"),
                           _ptr(pair_pos, _i32(), "pair_pos"), _ptr(ws, None, "ws"),
                           ws.numel() * ws.element_size(), _stream(stream)))


def _forward_args(cfg, x, router_w, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                  y, topk_ids_out, topk_w_out, ws, stream, no_ws=False):
    bf = _bf16()
    args = [ctypes.byref(cfg), _ptr(x, bf, "x"), _ptr(router_w, _f32(), "router_w"),
            _ptr(router_bias, _f32(), "router_bias", True), _ptr(w_gate, bf, "w_gate"),
            _ptr(w_up, bf, "w_up"), _ptr(w_down, bf, "w_down"),
            _ptr(ws_gate, bf, "ws_gate", True), _ptr(ws_up, bf, "ws_up", True),
            _ptr(ws_down, bf, "ws_down", True), _ptr(y, bf, "y"),
            _ptr(topk_ids_out, _i32(), "topk_ids_out", True),
            _ptr(topk_w_out, _f32(), "topk_w_out", True)]
    if not no_ws:
        args += [_ptr(ws, None, "ws"), ws.numel() * ws.element_size()]
    return args + [_stream(stream)]


def moe_forward(cfg, x, router_w, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y,
                topk_ids_out=None, topk_w_out=None, ws=None, stream=None):
    lib = load_library()
    _check(lib.moe_forward(*_forward_args(cfg, x, router_w, router_bias, w_gate, w_up, w_down,
                                          ws_gate, ws_up, ws_down, y, topk_ids_out, topk_w_out,
                                          ws, stream)))


def moe_forward_fused(cfg, x, router_w, router_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                      ws_down, y, topk_ids_out=None, topk_w_out=None, ws=None, stream=None):
    """moe_forward in a single launch (tokens <= 256, tokens * top_k <= 2048)."""
    lib = load_library()
    _check(lib.moe_forward_fused(*_forward_args(cfg, x, router_w, router_bias, w_gate, w_up,
                                                w_down, ws_gate, ws_up, ws_down, y, topk_ids_out,
                                                topk_w_out, ws, stream)))


def moe_forward_noalloc(cfg, x, router_w, router_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                        ws_down, y, topk_ids_out=None, topk_w_out=None, stream=None):
    """moe_forward with the library's fixed scratch as its workspace (no
    workspace argument, nothing allocated)."""
    lib = load_library()
    args = _forward_args(cfg, x, router_w, router_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                         ws_down, y, topk_ids_out, topk_w_out, None, stream, no_ws=True)
    _check(lib.moe_forward_noalloc(*args))


def moe_forward_timed(cfg, x, router_w, router_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                      ws_down, y, topk_ids_out=None, topk_w_out=None, ws=None, stream=None,
                      events=None):
    """`events`: MOE_NUM_STAGES + 1 torch.cuda.Event(enable_timing=True)."""
    lib = load_library()
    if events is None or len(events) != MOE_NUM_STAGES + 1:
        raise ValueError(f"need {MOE_NUM_STAGES + 1} events")
    handles = []
    for ev in events:
        if ev.cuda_event == 0:  # torch creates the HIP event lazily
            ev.record(_torch().cuda.current_stream())
        handles.append(ev.cuda_event)
    arr = (ctypes.c_void_p * len(handles))(*handles)
    _check(lib.moe_forward_timed(*_forward_args(cfg, x, router_w, router_bias, w_gate, w_up,
                                                w_down, ws_gate, ws_up, ws_down, y, topk_ids_out,
                                                topk_w_out, ws, stream), arr, len(handles)))


def moe_workspace_view(cfg, which: int):
    """(byte offset, byte size) of an intermediate inside the workspace."""
    lib = load_library()
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.moe_workspace_view(ctypes.byref(cfg), int(which), ctypes.byref(off),
                                  ctypes.byref(nb)))
    return int(off.value), int(nb.value)


# --------------------------------------------------------- layer wrapper

@dataclasses.dataclass
class MoeWeights:
    """Device tensors of one MoE layer (bf16 tensors may be torch.bfloat16 or
    raw-bit uint16/int16)."""
    router_w: object
    router_b: object
    w_gate: object
    w_up: object
    w_down: object
    ws_gate: object = None
    ws_up: object = None
    ws_down: object = None


def forward(cfg: moe_config, x, weights: MoeWeights, y=None, ws=None, topk_ids=None,
            topk_w=None, stream=None):
    """Allocate what is missing (output, workspace) and run moe_forward."""
    torch = _torch()
    if y is None:
        y = torch.empty((cfg.tokens, cfg.hidden), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = alloc_workspace(cfg, x.device)
    sh = cfg.inter_shared > 0
    moe_forward(cfg, x, weights.router_w, weights.router_b, weights.w_gate, weights.w_up,
                weights.w_down, weights.ws_gate if sh else None, weights.ws_up if sh else None,
                weights.ws_down if sh else None, y, topk_ids, topk_w, ws, stream)
    return y


# ------------------------------------------------------------------ dense FFN

def moe_dense_workspace_size(cfg: moe_dense_config) -> int:
    n = load_library().moe_dense_workspace_size(ctypes.byref(cfg))
    if n == 0:
        raise MoeError(MOE_ERR_INVALID_ARG, moe_last_error())
    return int(n)


def alloc_dense_workspace(cfg: moe_dense_config, device=None):
    torch = _torch()
    return torch.empty(moe_dense_workspace_size(cfg), dtype=torch.uint8,
                       device=device or torch.device("cuda"))


def moe_dense_forward(cfg, x, w_gate, w_up, w_down, y, ws, stream=None):
    lib = load_library()
    _check(lib.moe_dense_forward(ctypes.byref(cfg), _ptr(x, _bf16(), "x", cfg.tokens == 0),
                                 _ptr(w_gate, _bf16(), "w_gate"), _ptr(w_up, _bf16(), "w_up"),
                                 _ptr(w_down, _bf16(), "w_down"),
                                 _ptr(y, _bf16(), "y", cfg.tokens == 0),
                                 _ptr(ws, None, "ws"), ws.numel() * ws.element_size(),
                                 _stream(stream)))


# ------------------------------------------------------------------ FP8 experts

def _u8():
    return (_torch().uint8, _torch().float8_e4m3fn)


def moe_forward_fp8(cfg, x, router_w, router_bias, w8_gate, w8_up, w8_down, scale_gate, scale_up,
                    scale_down, ws_gate, ws_up, ws_down, y, topk_ids_out, topk_w_out, ws,
                    stream=None):
    lib = load_library()
    empty = cfg.tokens == 0
    _check(lib.moe_forward_fp8(
        ctypes.byref(cfg), _ptr(x, _bf16(), "x", empty), _ptr(router_w, _f32(), "router_w"),
        _ptr(router_bias, _f32(), "router_bias", True), _ptr(w8_gate, _u8(), "w8_gate"),
        _ptr(w8_up, _u8(), "w8_up"), _ptr(w8_down, _u8(), "w8_down"),
        _ptr(scale_gate, _f32(), "scale_gate"), _ptr(scale_up, _f32(), "scale_up"),
        _ptr(scale_down, _f32(), "scale_down"), _ptr(ws_gate, _bf16(), "ws_gate", True),
        _ptr(ws_up, _bf16(), "ws_up", True), _ptr(ws_down, _bf16(), "ws_down", True),
        _ptr(y, _bf16(), "y", empty), _ptr(topk_ids_out, _i32(), "topk_ids_out", True),
        _ptr(topk_w_out, _f32(), "topk_w_out", True), _ptr(ws, None, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)))
