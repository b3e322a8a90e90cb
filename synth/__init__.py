"""Seeded synthetic inputs for the sparse-MoE layer (shared by the GPU path's
tests and benchmark and by the CPU oracle; holds none of the layer's math).

The generator itself is plain C (``synth.c``): counter-based SplitMix64 words,
Box-Muller normals, float32 values rounded to bf16 where a tensor is bf16.
Every element depends only on (seed, tensor id, index).

Workload recipes follow the layer's configuration as published for
Step-3.5-Flash (model cards' raw config fields: hidden_size 4096,
moe_num_experts 288, moe_top_k 8, moe_intermediate_size 1280,
share_expert_dim 1280, moe_router_scaling_factor 3, norm_expert_weight true)
plus the five synthetic layer workloads (tiny, decode, prefill, skewed,
long).  ``N(0, v)`` in a recipe means variance ``v``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "synth.c")

# Tensor ids of the per-tensor streams.
T_X, T_WG, T_B, T_WGATE, T_WUP, T_WDOWN, T_WSGATE, T_WSUP, T_WSDOWN, T_HOT, T_SCALE = range(1, 12)


def build() -> str:
    """Compile libsynth.so with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", _SRC, "-o", _SO + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_double, ctypes.c_void_p)
        lib.synth_normal_f32.argtypes = [u64, u64, dbl, dbl, vp, i64, ctypes.c_int]
        lib.synth_normal_bf16.argtypes = [u64, u64, dbl, dbl, vp, i64, ctypes.c_int]
        lib.synth_scaled_normal_bf16.argtypes = [u64, u64, u64, dbl, dbl, dbl, dbl, vp, i64, i64,
                                                 ctypes.c_int]
        lib.synth_uniform_f32.argtypes = [u64, u64, dbl, dbl, vp, i64, ctypes.c_int]
        lib.synth_choose.argtypes = [u64, u64, i32, i32, vp]
        lib.synth_words.argtypes = [u64, u64, vp, i64]
        lib.synth_words.restype = None
        lib.synth_normal_e4m3_rows.argtypes = [u64, u64, dbl, dbl, vp, vp, i64, i64, ctypes.c_int]
        lib.synth_e4m3_encode.argtypes = [vp, i64, vp]
        lib.synth_e4m3_encode.restype = None
        lib.synth_splitmix64_next.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
        lib.synth_splitmix64_next.restype = ctypes.c_uint64
        _lib = lib
    return _lib


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_f32(seed, tensor, n, std, mean=0.0) -> np.ndarray:
    out = np.empty(int(n), dtype=np.float32)
    _load().synth_normal_f32(seed, tensor, mean, std, out.ctypes.data, out.size, threads())
    return out


def normal_bf16(seed, tensor, n, std, mean=0.0) -> np.ndarray:
    """bf16 values as raw uint16 bits."""
    out = np.empty(int(n), dtype=np.uint16)
    _load().synth_normal_bf16(seed, tensor, mean, std, out.ctypes.data, out.size, threads())
    return out


def scaled_normal_bf16(seed, tensor, row_tensor, rows, row_len, std, lo, hi) -> np.ndarray:
    out = np.empty(int(rows) * int(row_len), dtype=np.uint16)
    _load().synth_scaled_normal_bf16(seed, tensor, row_tensor, 0.0, std, lo, hi, out.ctypes.data,
                                     rows, row_len, threads())
    return out


def uniform_f32(seed, tensor, n, lo, hi) -> np.ndarray:
    out = np.empty(int(n), dtype=np.float32)
    _load().synth_uniform_f32(seed, tensor, lo, hi, out.ctypes.data, out.size, threads())
    return out


def choose(seed, tensor, n, m) -> np.ndarray:
    out = np.empty(int(m), dtype=np.int32)
    rc = _load().synth_choose(seed, tensor, n, m, out.ctypes.data)
    if rc:
        raise ValueError(f"synth_choose failed ({rc})")
    return out


def words(seed, tensor, n) -> np.ndarray:
    out = np.empty(int(n), dtype=np.uint64)
    _load().synth_words(seed, tensor, out.ctypes.data, out.size)
    return out


def splitmix64_sequence(state: int, n: int) -> list[int]:
    s = ctypes.c_uint64(state)
    return [int(_load().synth_splitmix64_next(ctypes.byref(s))) for _ in range(n)]


def normal_e4m3_rows(seed, tensor, rows, row_len, std, mean=0.0):
    """rows x row_len normals (the stream normal_bf16 draws) stored as OCP
    e4m3 codes with a per-row fp32 scale max|row| / 448."""
    codes = np.empty((int(rows), int(row_len)), dtype=np.uint8)
    scales = np.empty(int(rows), dtype=np.float32)
    _load().synth_normal_e4m3_rows(seed, tensor, mean, std, codes.ctypes.data, scales.ctypes.data,
                                   rows, row_len, threads())
    return codes, scales


def e4m3_encode(values) -> np.ndarray:
    """Codes of values with |v| <= 448 (round to nearest even), for tests."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().synth_e4m3_encode(v.ctypes.data, v.size, out.ctypes.data)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- workloads

@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic MoE-layer workload: sizes plus the input recipe."""
    name: str
    T: int
    H: int = 4096
    E: int = 288
    k: int = 8
    I: int = 1280
    Is: int = 1280
    routed_scaling: float = 3.0
    renormalize: bool = True
    limit: float = 0.0           # routed SwiGLU clamp, 0 = none
    limit_shared: float = 0.0    # shared-expert clamp, 0 = none
    bias_var: float = 0.1        # router bias ~ N(0, bias_var)
    hot_experts: int = 0         # this many experts get bias == hot_bias
    hot_bias: float = 2.0
    x_scale: tuple | None = None  # per-token factor ~ U(lo, hi) on x
    use_bias: bool = True        # False: no router bias (NULL pointer)
    seed: int = 0

    @property
    def P(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", T=16, H=256, E=16, k=4, I=64, Is=64, bias_var=0.5),
    "decode": Workload("decode", T=64),
    "prefill": Workload("prefill", T=8192),
    "skewed": Workload("skewed", T=4096, hot_experts=16, hot_bias=2.0, limit=7.0, limit_shared=0.0),
    "long": Workload("long", T=32768, bias_var=0.3, x_scale=(0.5, 2.0)),
    # The predecessor Step-3's MoE shape (model card comparison table): H 7168, 48 experts,
    # top-3, I = shared 5120, norm_expert_weight false; no router bias or scaling is listed
    # for it, so none (scaling 1.0).
    "step3": Workload("step3", T=4096, H=7168, E=48, k=3, I=5120, Is=5120, routed_scaling=1.0,
                      renormalize=False, use_bias=False),
    # The dense SwiGLU FFN of Step-3.5-Flash's first layers (intermediate_size 11264): no
    # router and no routed experts (E = k = I = 0); the MLP's weights are the "shared" ones.
    "dense": Workload("dense", T=8192, E=0, k=0, I=0, Is=11264),
}


@dataclasses.dataclass
class Inputs:
    """Host arrays of one workload.  bf16 tensors are raw uint16 bits."""
    wl: Workload
    x: np.ndarray          # [T][H] bf16
    router_w: np.ndarray   # [E][H] f32
    router_b: np.ndarray   # [E]    f32
    w_gate: np.ndarray     # [E][I][H] bf16
    w_up: np.ndarray       # [E][I][H] bf16
    w_down: np.ndarray     # [E][H][I] bf16
    ws_gate: np.ndarray    # [Is][H] bf16
    ws_up: np.ndarray      # [Is][H] bf16
    ws_down: np.ndarray    # [H][Is] bf16
    hot: np.ndarray | None = None


def gen_x(wl: Workload) -> np.ndarray:
    if wl.x_scale is None:
        x = normal_bf16(wl.seed, T_X, wl.T * wl.H, 1.0)
    else:
        x = scaled_normal_bf16(wl.seed, T_X, T_SCALE, wl.T, wl.H, 1.0, *wl.x_scale)
    return x.reshape(wl.T, wl.H)


def gen_router(wl: Workload):
    if wl.E == 0:
        return np.zeros((0, wl.H), np.float32), None, None
    wg = normal_f32(wl.seed, T_WG, wl.E * wl.H, math.sqrt(1.0 / wl.H)).reshape(wl.E, wl.H)
    b = normal_f32(wl.seed, T_B, wl.E, math.sqrt(wl.bias_var))
    hot = None
    if wl.hot_experts:
        hot = np.sort(choose(wl.seed, T_HOT, wl.E, wl.hot_experts))
        b[hot] = np.float32(wl.hot_bias)
    return wg, b, hot


def gen_experts(wl: Workload):
    E, I, H, Is = wl.E, wl.I, wl.H, wl.Is
    wg = normal_bf16(wl.seed, T_WGATE, E * I * H, math.sqrt(1.0 / H)).reshape(E, I, H)
    wu = normal_bf16(wl.seed, T_WUP, E * I * H, math.sqrt(1.0 / H)).reshape(E, I, H)
    wd = normal_bf16(wl.seed, T_WDOWN, E * H * I, math.sqrt(1.0 / max(I, 1))).reshape(E, H, I)
    if Is > 0:
        sg = normal_bf16(wl.seed, T_WSGATE, Is * H, math.sqrt(1.0 / H)).reshape(Is, H)
        su = normal_bf16(wl.seed, T_WSUP, Is * H, math.sqrt(1.0 / H)).reshape(Is, H)
        sd = normal_bf16(wl.seed, T_WSDOWN, H * Is, math.sqrt(1.0 / Is)).reshape(H, Is)
    else:
        sg = np.zeros((0, H), np.uint16)
        su = np.zeros((0, H), np.uint16)
        sd = np.zeros((H, 0), np.uint16)
    return wg, wu, wd, sg, su, sd


@dataclasses.dataclass
class Fp8Experts:
    """Routed-expert weights as OCP e4m3 codes with one fp32 scale per output
    row (weight = decode(code) * scale): the same normal draws as
    gen_experts, quantised row by row."""
    w8_gate: np.ndarray    # [E][I][H] uint8
    s_gate: np.ndarray     # [E][I] f32
    w8_up: np.ndarray      # [E][I][H] uint8
    s_up: np.ndarray       # [E][I] f32
    w8_down: np.ndarray    # [E][H][I] uint8
    s_down: np.ndarray     # [E][H] f32


def gen_experts_fp8(wl: Workload) -> Fp8Experts:
    E, I, H = wl.E, wl.I, wl.H
    g, sg = normal_e4m3_rows(wl.seed, T_WGATE, E * I, H, math.sqrt(1.0 / H))
    u, su = normal_e4m3_rows(wl.seed, T_WUP, E * I, H, math.sqrt(1.0 / H))
    d, sd = normal_e4m3_rows(wl.seed, T_WDOWN, E * H, I, math.sqrt(1.0 / max(I, 1)))
    return Fp8Experts(g.reshape(E, I, H), sg.reshape(E, I), u.reshape(E, I, H), su.reshape(E, I),
                      d.reshape(E, H, I), sd.reshape(E, H))


def make_inputs(wl: Workload, experts=None) -> Inputs:
    """All inputs of a workload.  `experts` may pass a tuple from gen_experts
    for the same (H, E, I, Is, seed) to avoid regenerating 9 GB of weights."""
    x = gen_x(wl)
    wg, b, hot = gen_router(wl)
    if not wl.use_bias:
        b = None
    if experts is None:
        experts = gen_experts(wl)
    return Inputs(wl, x, wg, b, *experts, hot=hot)
