"""Small helpers shared by the tests (no layer arithmetic here)."""
from __future__ import annotations

import json
import os
import types

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32_to_bf16_bits(a) -> np.ndarray:
    """bf16 bits of float values that must be exactly representable in bf16."""
    f = np.asarray(a, dtype=np.float32)
    bits = f.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("value not exactly representable in bf16")
    return (bits >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def inputs(x, router_w, router_b, w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None):
    """A synth.Inputs-like namespace from plain arrays (bf16 tensors given as bits)."""
    H = x.shape[1]
    if ws_gate is None:
        ws_gate = np.zeros((0, H), np.uint16)
        ws_up = np.zeros((0, H), np.uint16)
        ws_down = np.zeros((H, 0), np.uint16)
    return types.SimpleNamespace(x=x, router_w=np.ascontiguousarray(router_w, np.float32),
                                 router_b=None if router_b is None else
                                 np.ascontiguousarray(router_b, np.float32),
                                 w_gate=w_gate, w_up=w_up, w_down=w_down, ws_gate=ws_gate,
                                 ws_up=ws_up, ws_down=ws_down)
