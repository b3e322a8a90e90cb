"""GPU-side helpers for the parity tests: upload seeded inputs, run the C ABI
through the Python binding, and compare with the oracle by the parity
protocol (ids bit-exact except near-ties, weights within 1e-5, outputs within
1e-2 * max|oracle| + 1e-3)."""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
import synth

GAP_TOL = 1e-5       # near-tie threshold on the oracle's k-th vs (k+1)-th key
W_TOL = 1e-5         # gating weights
Y_RTOL_M = 1e-2      # y: |gpu - oracle| <= Y_RTOL_M * max|oracle| + Y_ATOL
Y_ATOL = 1e-3


def note(msg: str):
    """Name the case before a GPU step (visible with pytest -s; pytest -v
    already prints each test id before it runs)."""
    print(msg, flush=True)


def torch_mod():
    import torch
    return torch


def to_dev(a: np.ndarray):
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def bf16_dev_to_f32(t) -> np.ndarray:
    torch = torch_mod()
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else \
        synth.bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))


def cfg_of(wl, T=None):
    import sparse_moe_layer_fp32_amd as moe
    return moe.make_config(wl.T if T is None else T, wl.H, wl.E, wl.k, wl.I, wl.Is,
                           wl.routed_scaling, wl.renormalize, wl.limit, wl.limit_shared)


@dataclasses.dataclass
class DevInputs:
    x: object
    router_w: object
    router_b: object
    w_gate: object
    w_up: object
    w_down: object
    ws_gate: object
    ws_up: object
    ws_down: object


def upload(inp, experts_dev=None) -> DevInputs:
    ex = experts_dev or tuple(to_dev(a) if a.size else None for a in
                              (inp.w_gate, inp.w_up, inp.w_down, inp.ws_gate, inp.ws_up,
                               inp.ws_down))
    return DevInputs(to_dev(inp.x), to_dev(inp.router_w),
                     None if inp.router_b is None else to_dev(inp.router_b), *ex)


@dataclasses.dataclass
class GpuOut:
    y: np.ndarray      # float32 [T][H] (bf16 values)
    ids: np.ndarray    # int32 [T][k]
    w: np.ndarray      # float32 [T][k]
    ws: object         # device workspace (for views)


def run_forward(wl, d: DevInputs, ws=None, use_bias=True) -> GpuOut:
    import sparse_moe_layer_fp32_amd as moe
    torch = torch_mod()
    cfg = cfg_of(wl)
    if ws is None:
        ws = moe.alloc_workspace(cfg)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
    sh = wl.Is > 0
    moe.moe_forward(cfg, d.x, d.router_w, d.router_b if use_bias else None, d.w_gate, d.w_up,
                    d.w_down, d.ws_gate if sh else None, d.ws_up if sh else None,
                    d.ws_down if sh else None, y, ids, w, ws)
    torch.cuda.synchronize()
    return GpuOut(y.float().cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(), ws)


def ws_view(cfg, ws, which, dtype, shape=None):
    import sparse_moe_layer_fp32_amd as moe
    torch = torch_mod()
    off, nb = moe.moe_workspace_view(cfg, which)
    raw = ws[off:off + nb]
    if dtype == "bf16":
        arr = raw.view(torch.bfloat16).float().cpu().numpy()
    else:
        arr = raw.view(dtype).cpu().numpy()
    return arr if shape is None else arr.reshape(shape)


# ----------------------------------------------------------- comparisons

@dataclasses.dataclass
class RouteReport:
    n_tokens: int
    near_tie: list        # tokens whose oracle k-th/(k+1)-th key gap is in (0, GAP_TOL)
    mismatched: list      # tokens whose id sets differ (all near-ties if ok)
    max_w_err: float
    order_swaps: int = 0  # tokens with the same set whose rank order differs (near-equal keys)
    exact_ties: int = 0   # tokens with two equal oracle keys among the selected or at the cut


def compare_route(wl, gpu_ids, gpu_w, ref) -> RouteReport:
    """Ids and gating weights of the GPU against ref = oracle.route(...,
    want_keys=True), token by token.

    * Set: equal to the oracle's, unless the token is a near-tie: an expert
      in the oracle's set and one outside it have keys that differ by a
      nonzero amount below GAP_TOL, which fp32 may order either way (the
      oracle's k-th and (k+1)-th keys closer than GAP_TOL but not equal, or
      equal with another expert within GAP_TOL of them).  Then the GPU's set
      must still be a valid top-k within GAP_TOL.  Equal keys rank the lower
      expert index first on both sides, so an exact tie at the cut with no
      such neighbour is not exempt: the ids must match.
    * Rank order: slot by slot the GPU's id equals the oracle's, unless the
      two experts' oracle keys differ by a nonzero amount below GAP_TOL.
      Along the GPU's slots the oracle keys never increase by GAP_TOL or
      more, and two exactly equal keys are listed lower index first.
    * Weights: matched by expert id, within W_TOL.
    """
    T, k = gpu_ids.shape
    gpu_ids = np.asarray(gpu_ids)
    oids = np.asarray(ref["ids"])
    keys = ref["keys"]
    gap = ref["gap"]
    assert np.all((gpu_ids >= 0) & (gpu_ids < keys.shape[1])), "expert id out of range"
    kth = np.take_along_axis(keys, oids[:, -1:].astype(np.int64), 1)[:, 0]  # oracle's cut key
    near_mask = (gap > 0) & (gap < GAP_TOL)
    if np.any(gap == 0):
        # exact tie at the cut: a near-tie only if another key lies within
        # GAP_TOL of the cut key without being equal to it
        close = (np.abs(keys - kth[:, None]) < GAP_TOL) & (keys != kth[:, None])
        near_mask |= (gap == 0) & np.any(close, 1)
    near = np.nonzero(near_mask)[0]
    mism = np.nonzero(np.any(np.sort(gpu_ids, 1) != np.sort(oids, 1), 1))[0]
    bad = np.setdiff1d(mism, near)
    assert bad.size == 0, f"expert ids differ on tokens that are not near-ties {bad[:10].tolist()}"
    for t in mism.tolist():  # a near-tie may pick either side; the pick must still be valid
        kth = np.sort(keys[t])[::-1][k - 1]
        assert np.all(keys[t][gpu_ids[t]] >= kth - GAP_TOL), f"token {t}: invalid near-tie choice"
        assert len(set(gpu_ids[t].tolist())) == k, f"token {t}: repeated expert"
    kg = np.take_along_axis(keys, gpu_ids.astype(np.int64), 1)  # oracle keys of the GPU's ids
    ko = np.take_along_axis(keys, oids.astype(np.int64), 1)
    same = np.ones(T, bool)
    same[mism] = False
    dk = np.abs(kg - ko)
    bad_slot = (gpu_ids != oids) & ~((dk > 0) & (dk < GAP_TOL)) & same[:, None]
    rows = np.nonzero(bad_slot.any(1))[0]
    assert rows.size == 0, (f"rank order differs from the oracle on token {rows[0]}: gpu "
                            f"{gpu_ids[rows[0]].tolist()} oracle {oids[rows[0]].tolist()}")
    if k > 1:
        d = kg[:, :-1] - kg[:, 1:]
        assert np.all(d > -GAP_TOL), "GPU ids not in descending key order"
        tied = d == 0
        assert np.all(gpu_ids[:, :-1][tied] < gpu_ids[:, 1:][tied]), \
            "exactly equal keys not listed lower index first"
    swaps = int(np.count_nonzero(np.any(gpu_ids != oids, 1) & same))
    tied = gap == 0  # an exact tie at the cut, or between two selected experts
    if k > 1:
        tied |= np.any(ko[:, :-1] == ko[:, 1:], 1)
    ties = int(np.count_nonzero(tied))
    # weights matched by expert id on tokens with identical sets
    og = np.argsort(gpu_ids[same], 1)
    oo = np.argsort(oids[same], 1)
    wg = np.take_along_axis(np.asarray(gpu_w)[same].astype(np.float64), og, 1)
    wo = np.take_along_axis(ref["w"][same], oo, 1)
    err = float(np.max(np.abs(wg - wo))) if wg.size else 0.0
    assert err <= W_TOL, f"gating weight error {err}"
    return RouteReport(T, near.tolist(), mism.tolist(), err, swaps, ties)


def per_token_rel_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    """Largest over tokens of max_d |gpu - oracle| / max_d |oracle| (a
    diagnostic: tokens with small outputs, such as the long workload's
    small-scale tokens, show their own relative error here)."""
    den = np.max(np.abs(y_ref), axis=1)
    num = np.max(np.abs(y_gpu.astype(np.float64) - y_ref), axis=1)
    ok = den > 0
    return float(np.max(num[ok] / den[ok])) if np.any(ok) else 0.0


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, what=""):
    M = float(np.max(np.abs(y_ref)))
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bound = Y_RTOL_M * M + Y_ATOL
    worst = float(err.max()) if err.size else 0.0
    assert worst <= bound, f"{what}: max |gpu - oracle| = {worst:.3e} > {bound:.3e} (M = {M:.3e})"
    return worst, M


def oracle_y_for(wl, inp, tokens, gpu_ids, near_mismatch):
    """Oracle outputs for `tokens`; where the GPU took the other side of a
    near-tie, the oracle is rerun with the GPU's ids (weights recomputed from
    the bias-free scores over that set)."""
    cfg = oracle.cfg_of(wl)
    tokens = np.asarray(tokens, np.int64)
    ref = oracle.forward(cfg, inp, tokens=tokens)["y"]
    swapped = set(int(t) for t in near_mismatch)
    forced = [i for i, t in enumerate(tokens.tolist()) if t in swapped]
    if forced:
        sub = tokens[forced]
        ref[forced] = oracle.forward(cfg, inp, tokens=sub, forced_ids=gpu_ids[sub])["y"]
    return ref
