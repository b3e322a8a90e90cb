"""CPU oracle of the Step-3.5-Flash sparse-MoE FFN layer forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of ``bench.py``.  The GPU product path never imports it.

The arithmetic lives in ``oracle.cpp`` (plain C++, double precision, built
with g++); this module only marshals numpy arrays.  What each function
follows on the pages is stated in ``oracle.cpp``.

Parity status of each function (pins live in ``tests/test_oracle.py``):
  route    pinned: brute-force top-k, all-tied, bias-only, hand-computed
           worked examples, weights sum to the routed scaling, bias-only-
           selects invariant.
  forward  pinned: hand-computed layout examples (golden files), closed forms
           (identical experts, zero routed scaling = dense SwiGLU MLP via a
           library matmul), scalar SwiGLU and clamp values.
  expert   pinned: scalar SwiGLU closed forms, dense MLP via library matmul.
  permute  pinned: agrees with a library stable argsort and with invariants.
  e4m3_decode  pinned: all 256 codes against torch's float8_e4m3fn and the
           format's named values (max 448, smallest normal 2^-6, smallest
           subnormal 2^-9, NaN codes).
  forward_fp8  pinned: with codes and scales that represent bf16 weights
           exactly it equals forward on those weights; scales factor out of
           each expert (scaling a row's scale scales that output unit).
  The reading "bias added after the sigmoid" and the reading of N(0, v) as a
  variance are not fixed by the pages' numbers: parity unpinned for those
  two readings (no page prints a worked routing example).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.cpp")


class Cfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("I", ctypes.c_int32), ("Is", ctypes.c_int32),
                ("routed_scaling", ctypes.c_double), ("renormalize", ctypes.c_int32),
                ("limit", ctypes.c_double), ("limit_shared", ctypes.c_double)]


def build() -> str:
    """Compile liboracle.so with g++ (always recompiles)."""
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", _SRC, "-o", _SO + ".tmp"]
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
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        cp = ctypes.POINTER(Cfg)
        lib.oracle_route.argtypes = [cp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int]
        lib.oracle_forward.argtypes = [cp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp,
                                       vp, vp, ctypes.c_int]
        lib.oracle_expert.argtypes = [i32, i32, dbl, vp, i64, vp, vp, vp, vp, vp, ctypes.c_int]
        lib.oracle_forward_fp8.argtypes = [cp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           i64, vp, vp, vp, vp, ctypes.c_int]
        lib.oracle_e4m3_decode.argtypes = [vp, i64, vp]
        lib.oracle_permute.argtypes = [i64, i32, i32, vp, vp, vp, vp]
        lib.oracle_hardware_threads.argtypes = []
        _lib = lib
    return _lib


def hardware_threads() -> int:
    return int(_load().oracle_hardware_threads())


def default_threads() -> int:
    """Threads for the oracle: the CPUs this process may run on, at most 16
    (the host CPU share that goes with one GPU on the machines this runs
    on); MOE_ORACLE_THREADS overrides."""
    env = os.environ.get("MOE_ORACLE_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, hardware_threads(), len(os.sched_getaffinity(0))))


def make_cfg(T, H, E, k, I, Is, routed_scaling=3.0, renormalize=True, limit=0.0,
             limit_shared=0.0) -> Cfg:
    return Cfg(int(T), int(H), int(E), int(k), int(I), int(Is), float(routed_scaling),
               int(bool(renormalize)), float(limit), float(limit_shared))


def cfg_of(wl, T=None) -> Cfg:
    """Oracle config of a synth.Workload (optionally with another T)."""
    return make_cfg(wl.T if T is None else T, wl.H, wl.E, wl.k, wl.I, wl.Is, wl.routed_scaling,
                    wl.renormalize, wl.limit, wl.limit_shared)


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def route(cfg: Cfg, x, router_w, router_b=None, want_keys=False, threads=None):
    """-> dict(ids [T,k] int32, w [T,k] f64, gap [T] f64, keys/scores [T,E] f64 optional)."""
    x = _c(x, np.uint16)
    router_w = _c(router_w, np.float32)
    router_b = _c(router_b, np.float32)
    T, k, E = cfg.T, cfg.k, cfg.E
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    gap = np.empty(T, np.float64)
    keys = np.empty((T, E), np.float64) if want_keys else None
    scores = np.empty((T, E), np.float64) if want_keys else None
    rc = _load().oracle_route(ctypes.byref(cfg), _p(x), _p(router_w), _p(router_b), _p(ids),
                              _p(w), _p(gap), _p(keys), _p(scores), threads or default_threads())
    if rc:
        raise ValueError(f"oracle_route failed ({rc})")
    out = dict(ids=ids, w=w, gap=gap)
    if want_keys:
        out.update(keys=keys, scores=scores)
    return out


def forward(cfg: Cfg, inp, tokens=None, forced_ids=None, threads=None):
    """Layer output for all tokens (tokens=None) or a list of token ids.
    `inp` has the fields of synth.Inputs.  -> dict(y [n,H] f64, ids, w)."""
    x = _c(inp.x, np.uint16)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    n = cfg.T if tok is None else tok.size
    fid = None if forced_ids is None else _c(np.asarray(forced_ids, np.int32), np.int32)
    y = np.empty((n, cfg.H), np.float64)
    ids = np.empty((n, cfg.k), np.int32)
    w = np.empty((n, cfg.k), np.float64)
    args = [_c(inp.router_w, np.float32), _c(inp.router_b, np.float32),
            _c(inp.w_gate, np.uint16), _c(inp.w_up, np.uint16), _c(inp.w_down, np.uint16),
            _c(inp.ws_gate, np.uint16), _c(inp.ws_up, np.uint16), _c(inp.ws_down, np.uint16)]
    rc = _load().oracle_forward(ctypes.byref(cfg), _p(x), *[_p(a) for a in args], _p(tok), n,
                                _p(fid), _p(y), _p(ids), _p(w), threads or default_threads())
    if rc:
        raise ValueError(f"oracle_forward failed ({rc})")
    return dict(y=y, ids=ids, w=w)


def forward_fp8(cfg: Cfg, inp, fp8, tokens=None, forced_ids=None, threads=None):
    """forward with the routed experts' weights from `fp8` (synth.Fp8Experts:
    e4m3 codes and per-row scales); the shared expert from `inp`.
    -> dict(y [n,H] f64, ids, w)."""
    x = _c(inp.x, np.uint16)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    n = cfg.T if tok is None else tok.size
    fid = None if forced_ids is None else _c(np.asarray(forced_ids, np.int32), np.int32)
    y = np.empty((n, cfg.H), np.float64)
    ids = np.empty((n, cfg.k), np.int32)
    w = np.empty((n, cfg.k), np.float64)
    args = [_c(inp.router_w, np.float32), _c(inp.router_b, np.float32),
            _c(fp8.w8_gate, np.uint8), _c(fp8.w8_up, np.uint8), _c(fp8.w8_down, np.uint8),
            _c(fp8.s_gate, np.float32), _c(fp8.s_up, np.float32), _c(fp8.s_down, np.float32),
            _c(inp.ws_gate, np.uint16), _c(inp.ws_up, np.uint16), _c(inp.ws_down, np.uint16)]
    rc = _load().oracle_forward_fp8(ctypes.byref(cfg), _p(x), *[_p(a) for a in args], _p(tok), n,
                                    _p(fid), _p(y), _p(ids), _p(w), threads or default_threads())
    if rc:
        raise ValueError(f"oracle_forward_fp8 failed ({rc})")
    return dict(y=y, ids=ids, w=w)


def e4m3_decode(codes) -> np.ndarray:
    """OCP e4m3 codes -> float64 values."""
    c = _c(np.asarray(codes, np.uint8), np.uint8)
    out = np.empty(c.shape, np.float64)
    rc = _load().oracle_e4m3_decode(_p(c), c.size, _p(out))
    if rc:
        raise ValueError("oracle_e4m3_decode failed")
    return out


def expert(rows, gate, up, down, limit=0.0, threads=None):
    """One SwiGLU expert on rows [n,H] (bf16 bits) -> (h [n,I] f64, o [n,H] f64)."""
    rows = _c(rows, np.uint16)
    gate, up, down = _c(gate, np.uint16), _c(up, np.uint16), _c(down, np.uint16)
    n, H = rows.shape
    I = gate.shape[0]
    h = np.empty((n, I), np.float64)
    o = np.empty((n, H), np.float64)
    rc = _load().oracle_expert(H, I, float(limit), _p(rows), n, _p(gate), _p(up), _p(down),
                               _p(h), _p(o), threads or default_threads())
    if rc:
        raise ValueError(f"oracle_expert failed ({rc})")
    return h, o


def permute(ids, E):
    """Stable expert-sorted order of pairs -> (offsets [E+1], sorted [P], pos [P])."""
    ids = _c(np.asarray(ids, np.int32), np.int32)
    T, k = ids.shape
    offsets = np.empty(E + 1, np.int32)
    sorted_ = np.empty(T * k, np.int32)
    pos = np.empty(T * k, np.int32)
    rc = _load().oracle_permute(T, k, E, _p(ids), _p(offsets), _p(sorted_), _p(pos))
    if rc:
        raise ValueError(f"oracle_permute failed ({rc})")
    return offsets, sorted_, pos
