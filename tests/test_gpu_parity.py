"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Protocol: expert ids bit-exact as sets except on tokens whose oracle
k-th/(k+1)-th key gap is < 1e-5 (counted; the GPU's pick must still be a
valid top-k there, and y is then checked against the oracle rerun with the
GPU's ids); gating weights within 1e-5; outputs within
1e-2 * max|oracle| + 1e-3 elementwise; the permutation bit-exact.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_case(request):
    gu.note(f"[gpu-test] {request.node.nodeid}")
    yield


@pytest.fixture(scope="module")
def moe():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_moe_layer_fp32_amd as m
    m.load_library()
    return m


def _full_parity(moe, wl, inp=None, use_bias=True, tokens=None):
    """Run the GPU forward and compare route, permutation and y."""
    inp = inp or synth.make_inputs(wl)
    if not use_bias:
        inp.router_b = None
    d = gu.upload(inp)
    gu.note(f"  forward {wl}")
    out = gu.run_forward(wl, d)
    ref = oracle.route(oracle.cfg_of(wl), inp.x, inp.router_w, inp.router_b, want_keys=True)
    rep = gu.compare_route(wl, out.ids, out.w, ref)
    # permutation, from the forward's own workspace
    cfg = gu.cfg_of(wl)
    off = gu.ws_view(cfg, out.ws, moe.MOE_WS_EXPERT_OFFSETS, moe_i32())
    srt = gu.ws_view(cfg, out.ws, moe.MOE_WS_SORTED_PAIRS, moe_i32())
    pos = gu.ws_view(cfg, out.ws, moe.MOE_WS_PAIR_POS, moe_i32())
    o_off, o_srt, o_pos = oracle.permute(out.ids, wl.E)
    assert np.array_equal(off, o_off) and np.array_equal(srt, o_srt) and np.array_equal(pos, o_pos)
    toks = np.arange(wl.T) if tokens is None else np.asarray(tokens)
    y_ref = gu.oracle_y_for(wl, inp, toks, out.ids, rep.mismatched)
    err, M = gu.check_y(out.y[toks], y_ref, wl.name)
    return out, rep, err, M, inp, d


def moe_i32():
    import torch
    return torch.int32


# ------------------------------------------------------------ small shapes

def test_tiny_full_parity(moe):
    wl = synth.WORKLOADS["tiny"]
    out, rep, err, M, inp, d = _full_parity(moe, wl)
    gu.note(f"  tiny: max err {err:.3e} M {M:.3e} near-ties {len(rep.near_tie)}")
    # deterministic: a second run is bit-identical
    out2 = gu.run_forward(wl, d)
    assert np.array_equal(out.y, out2.y) and np.array_equal(out.ids, out2.ids)
    assert np.array_equal(out.w, out2.w)
    # weights sum to the routed scaling
    assert np.max(np.abs(out.w.astype(np.float64).sum(1) - 3.0)) <= 1e-5


SMALL = {
    # several row tiles per hot expert with a ragged tail, split-K router
    "ragged": dict(T=333, H=512, E=24, k=6, I=192, Is=128, hot_experts=4, bias_var=0.1),
    "no_shared": dict(T=77, H=256, E=16, k=4, I=64, Is=0, bias_var=0.5),
    "k_equals_E": dict(T=50, H=256, E=8, k=8, I=64, Is=64),
    "single_token": dict(T=1, H=128, E=4, k=2, I=64, Is=64),
    "no_renorm": dict(T=40, H=256, E=16, k=4, I=64, Is=64, renormalize=False),
    "clamped": dict(T=96, H=256, E=16, k=4, I=128, Is=64, limit=0.05, limit_shared=0.1),
    "zero_scaling": dict(T=40, H=256, E=16, k=4, I=64, Is=64, routed_scaling=0.0),
    "full_router": dict(T=40, H=4096, E=288, k=8, I=64, Is=64),
    "wide_inter": dict(T=130, H=384, E=10, k=3, I=320, Is=192, bias_var=0.3),
    # small tiles 256 weight rows wide (I and Is multiples of 128), ragged expert rows
    "wide_small": dict(T=150, H=512, E=12, k=4, I=256, Is=128, bias_var=0.3),
    # enough rows per expert for the 256 x 256 tile shape, ragged last tiles
    "big_tile": dict(T=1100, H=512, E=8, k=4, I=256, Is=128, bias_var=0.5),
    "big_tile_no_shared": dict(T=1500, H=768, E=6, k=3, I=384, Is=0, bias_var=0.2),
    # enough tokens for the wave-per-token top-k
    "many_tokens": dict(T=2500, H=256, E=40, k=6, I=64, Is=64, bias_var=0.2),
    # the ABI's limits, E = 1024 and k = 32, on both top-k paths (a block per
    # token below 2048 tokens, a wave per token from there)
    "max_experts": dict(T=100, H=256, E=1024, k=32, I=64, Is=64, bias_var=0.2),
    "max_experts_wave": dict(T=2100, H=256, E=1024, k=32, I=64, Is=64, bias_var=0.2),
    # degenerate routing: one expert per token (every weight is the scaling
    # factor), and a single expert that takes every token
    "top1": dict(T=300, H=256, E=16, k=1, I=64, Is=64, bias_var=0.3),
    "single_expert": dict(T=200, H=256, E=1, k=1, I=128, Is=0),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_parity(moe, name):
    wl = synth.WORKLOADS["tiny"].with_(name=name, **SMALL[name])
    out, rep, err, M, *_ = _full_parity(moe, wl)
    gu.note(f"  {name}: max err {err:.3e} M {M:.3e} near-ties {len(rep.near_tie)}")


def test_workspace_reused_across_batch_sizes(moe):
    """One workspace, filled with garbage once, for calls of alternating
    batch sizes that take the big tiles (persistent grid, work queues in the
    workspace) and the small ones: every call equals the same call on a
    fresh workspace, bit for bit."""
    import dataclasses
    torch = gu.torch_mod()
    big = synth.WORKLOADS["tiny"].with_(name="reuse", **SMALL["big_tile"])
    d = gu.upload(synth.make_inputs(big))
    sizes = (big.T, 48, big.T, 300, 1, big.T)
    nbytes = max(moe.moe_workspace_size(gu.cfg_of(big, T=T)) for T in sizes)
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    for T in sizes:
        wl = big.with_(T=T)
        dT = dataclasses.replace(d, x=d.x[:T])
        gu.note(f"  T={T}")
        ref = gu.run_forward(wl, dT)
        got = gu.run_forward(wl, dT, ws=ws)
        assert np.array_equal(ref.ids, got.ids), f"T={T}: ids differ"
        assert np.array_equal(ref.w.view(np.uint32), got.w.view(np.uint32)), f"T={T}: weights"
        assert np.array_equal(ref.y.view(np.uint32), got.y.view(np.uint32)), f"T={T}: y differs"


def test_topk_paths_agree(moe):
    """Below 2048 tokens the top-k runs one block per token, from 2048 one
    wave per token.  2047 and 2048 tokens give the same router tiling, so
    the shared tokens must get bit-identical ids and weights."""
    torch = gu.torch_mod()
    wl = synth.WORKLOADS["tiny"].with_(name="topk_paths", T=2048, H=256, E=288, k=8, I=64, Is=64)
    inp = synth.make_inputs(wl)
    x = gu.to_dev(inp.x)
    rw = gu.to_dev(inp.router_w)
    rb = gu.to_dev(inp.router_b)
    res = {}
    for T in (2047, 2048):
        gu.note(f"  moe_route T={T} E=288 k=8")
        cfg = gu.cfg_of(wl, T=T)
        ws = moe.alloc_workspace(cfg)
        ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")
        moe.moe_route(cfg, x[:T], rw, rb, ids, w, ws)
        torch.cuda.synchronize()
        res[T] = (ids.cpu().numpy(), w.cpu().numpy())
    assert np.array_equal(res[2047][0], res[2048][0][:2047])
    assert np.array_equal(res[2047][1].view(np.uint32), res[2048][1][:2047].view(np.uint32))


def test_no_bias(moe):
    wl = synth.WORKLOADS["tiny"].with_(name="no_bias", T=48)
    _full_parity(moe, wl, use_bias=False)


def test_route_and_permute_entry_points(moe):
    import torch
    wl = synth.WORKLOADS["tiny"].with_(name="entry", **SMALL["ragged"])
    inp = synth.make_inputs(wl)
    d = gu.upload(inp)
    cfg = gu.cfg_of(wl)
    ws = moe.alloc_workspace(cfg)
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
    gu.note("  moe_route")
    moe.moe_route(cfg, d.x, d.router_w, d.router_b, ids, w, ws)
    torch.cuda.synchronize()
    ref = oracle.route(oracle.cfg_of(wl), inp.x, inp.router_w, inp.router_b, want_keys=True)
    gids, gw = ids.cpu().numpy(), w.cpu().numpy()
    gu.compare_route(wl, gids, gw, ref)
    # ids come in rank order: keys non-increasing along the slots
    keys = np.take_along_axis(ref["keys"], gids.astype(np.int64), 1)
    assert np.all(np.diff(keys, axis=1) <= 1e-5)
    off = torch.empty(wl.E + 1, dtype=torch.int32, device="cuda")
    srt = torch.empty(wl.T * wl.k, dtype=torch.int32, device="cuda")
    pos = torch.empty(wl.T * wl.k, dtype=torch.int32, device="cuda")
    gu.note("  moe_permute")
    moe.moe_permute(cfg, ids, off, srt, pos, ws)
    torch.cuda.synchronize()
    o_off, o_srt, o_pos = oracle.permute(gids, wl.E)
    assert np.array_equal(off.cpu().numpy(), o_off)
    assert np.array_equal(srt.cpu().numpy(), o_srt)
    assert np.array_equal(pos.cpu().numpy(), o_pos)

@pytest.mark.parametrize("T2,E2,k2", [(5000, 40, 5), (70000, 300, 4), (3, 1024, 32), (1000, 7, 1)])
def test_permute_arbitrary_ids(moe, T2, E2, k2):
    """moe_permute on ids not made by the router: several chunks, chunks
    ranked in several LDS passes, the largest expert count, k = 1."""
    import torch
    rng = np.random.default_rng(T2 + E2)
    ids2 = np.argsort(rng.random((T2, E2)), axis=1)[:, :k2].astype(np.int32)
    ids2[: T2 // 3] = np.sort(ids2[: T2 // 3], 1)  # a skewed stretch
    cfg2 = moe.make_config(T2, 256, E2, k2, 64, 0)
    ws2 = moe.alloc_workspace(cfg2)
    ids2_d = torch.from_numpy(ids2).cuda()
    off2 = torch.empty(E2 + 1, dtype=torch.int32, device="cuda")
    srt2 = torch.empty(T2 * k2, dtype=torch.int32, device="cuda")
    pos2 = torch.empty(T2 * k2, dtype=torch.int32, device="cuda")
    gu.note(f"  moe_permute T={T2} E={E2} k={k2}")
    moe.moe_permute(cfg2, ids2_d, off2, srt2, pos2, ws2)
    torch.cuda.synchronize()
    e_off, e_srt, e_pos = oracle.permute(ids2, E2)
    assert np.array_equal(off2.cpu().numpy(), e_off)
    assert np.array_equal(srt2.cpu().numpy(), e_srt)
    assert np.array_equal(pos2.cpu().numpy(), e_pos)


def test_grouped_gemm_equals_per_expert_loop(moe):
    """The grouped gate/up GEMM's rows of expert e equal the per-expert loop
    on those rows (sglang-jax issue, Implementation strategy)."""
    wl = synth.WORKLOADS["tiny"].with_(name="gmm", **SMALL["ragged"])
    inp = synth.make_inputs(wl)
    d = gu.upload(inp)
    out = gu.run_forward(wl, d)
    cfg = gu.cfg_of(wl)
    off = gu.ws_view(cfg, out.ws, moe.MOE_WS_EXPERT_OFFSETS, moe_i32())
    srt = gu.ws_view(cfg, out.ws, moe.MOE_WS_SORTED_PAIRS, moe_i32())
    h = gu.ws_view(cfg, out.ws, moe.MOE_WS_H, "bf16")
    P = wl.T * wl.k
    h_routed = h[: P * wl.I].reshape(P, wl.I)
    h_shared = h[P * wl.I:].reshape(wl.T, wl.Is)
    counts = np.diff(off)
    experts = [int(e) for e in np.argsort(-counts)[:3]] + \
              [int(e) for e in np.nonzero((counts > 0) & (counts < 20))[0][:2]]
    for e in experts:
        rows = srt[off[e]:off[e + 1]] // wl.k
        href, _ = oracle.expert(inp.x[rows], inp.w_gate[e], inp.w_up[e], inp.w_down[e], wl.limit)
        hg = h_routed[off[e]:off[e + 1]]
        M = np.max(np.abs(href))
        assert np.all(np.abs(hg - href) <= 8e-3 * np.abs(href) + 1e-3 * M), f"expert {e}"
    href, _ = oracle.expert(inp.x, inp.ws_gate, inp.ws_up, inp.ws_down, wl.limit_shared)
    M = np.max(np.abs(href))
    assert np.all(np.abs(h_shared - href) <= 8e-3 * np.abs(href) + 1e-3 * M)


def test_empty_batch(moe):
    import torch
    wl = synth.WORKLOADS["tiny"].with_(T=0)
    cfg = gu.cfg_of(wl)
    ws = moe.alloc_workspace(cfg)
    x = torch.empty((0, wl.H), dtype=torch.bfloat16, device="cuda")
    rw = torch.zeros((wl.E, wl.H), dtype=torch.float32, device="cuda")
    we = torch.zeros((wl.E, wl.I, wl.H), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((wl.E, wl.H, wl.I), dtype=torch.bfloat16, device="cuda")
    sg = torch.zeros((wl.Is, wl.H), dtype=torch.bfloat16, device="cuda")
    sd = torch.zeros((wl.H, wl.Is), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((0, wl.H), dtype=torch.bfloat16, device="cuda")
    moe.moe_forward(cfg, x, rw, None, we, we, wd, sg, sg, sd, y, None, None, ws)
    off = torch.full((wl.E + 1,), 7, dtype=torch.int32, device="cuda")
    ids = torch.empty((0, wl.k), dtype=torch.int32, device="cuda")
    e0 = torch.empty(16, dtype=torch.int32, device="cuda")  # never written for T = 0
    moe.moe_permute(cfg, ids, off, e0, e0, ws)
    torch.cuda.synchronize()
    assert off.cpu().numpy().tolist() == [0] * (wl.E + 1)


def test_errors_enqueue_nothing(moe):
    import torch
    wl = synth.WORKLOADS["tiny"]
    cfg = gu.cfg_of(wl)
    inp = synth.make_inputs(wl)
    d = gu.upload(inp)
    ws = moe.alloc_workspace(cfg)
    y = torch.full((wl.T, wl.H), 1.5, dtype=torch.bfloat16, device="cuda")
    small = ws[: ws.numel() // 2]
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward(cfg, d.x, d.router_w, d.router_b, d.w_gate, d.w_up, d.w_down, d.ws_gate,
                        d.ws_up, d.ws_down, y, None, None, small)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y.float() == 1.5)


# ------------------------------------------------------------- exact ties
# Equal selection keys rank the lower expert index first.  These inputs make
# the keys equal in fp32 and in double alike, so the GPU's ids must equal the
# oracle's bit for bit, in rank order, with no near-tie exemption.  The batch
# sizes take each router form and each top-k kernel: 40 (split-k partials,
# one top-k block per token), 1500 (weight-plane GEMM, block top-k), 2500
# (plane GEMM, one top-k wave per token), 8192 (plane GEMM with 256-row
# tiles, wave top-k).

TIE_T = [40, 1500, 2500, 8192]


@pytest.fixture(scope="module")
def tie_inputs():
    """Full router width (H 4096, 288 experts, top 8), small experts (I 64)."""
    wl = synth.WORKLOADS["tiny"].with_(name="ties", T=max(TIE_T), H=4096, E=288, k=8, I=64,
                                       Is=64)
    return wl, synth.make_inputs(wl)


def _tie_case(wl, inp, T, router_w, router_b):
    import dataclasses
    sub = dataclasses.replace(inp, x=inp.x[:T], router_w=router_w, router_b=router_b)
    return wl.with_(T=T), sub


def _run_ties(moe, wl, inp):
    d = gu.upload(inp)
    gu.note(f"  forward {wl.name} T={wl.T}")
    out = gu.run_forward(wl, d)
    ref = oracle.route(oracle.cfg_of(wl), inp.x, inp.router_w, inp.router_b, want_keys=True)
    rep = gu.compare_route(wl, out.ids, out.w, ref)
    y_ref = gu.oracle_y_for(wl, inp, np.arange(wl.T), out.ids, rep.mismatched)
    err, M = gu.check_y(out.y, y_ref, wl.name)
    return out, ref, rep


@pytest.mark.parametrize("T", TIE_T)
def test_ties_all_keys_equal(moe, tie_inputs, T):
    """Wg = 0 and b = 0: every logit is 0, every score sigmoid(0) = 1/2 and
    every key 1/2, so the top 8 are experts 0..7 in that order and each
    weight is 3 * 0.5 / 4.0 = 0.375 exactly."""
    wl, inp = tie_inputs
    E, H = wl.E, wl.H
    wlT, sub = _tie_case(wl, inp, T, np.zeros((E, H), np.float32), np.zeros(E, np.float32))
    out, ref, rep = _run_ties(moe, wlT, sub)
    assert not rep.near_tie  # every key is exactly 1/2
    assert np.all(out.ids == np.arange(wl.k, dtype=np.int32)), "ties not broken by lower index"
    assert np.all(out.w == np.float32(0.375)), "weights of equal scores are not 3/k"
    assert rep.exact_ties == T


@pytest.mark.parametrize("T", TIE_T)
def test_ties_coarse_bias(moe, tie_inputs, T):
    """Wg = 0 and a bias of five exactly representable levels: keys 1/2 + b
    tie within each level; the top 8 are the eight lowest-numbered experts of
    the highest level, in index order, each weighted 0.375."""
    wl, inp = tie_inputs
    E, H = wl.E, wl.H
    rng = np.random.default_rng(11)
    b = rng.choice(np.array([-0.5, -0.25, 0.0, 0.25, 0.5], np.float32), E)
    b[:5] = -0.5  # the lowest indices are not the winners
    wlT, sub = _tie_case(wl, inp, T, np.zeros((E, H), np.float32), b)
    out, ref, rep = _run_ties(moe, wlT, sub)
    assert not rep.near_tie  # keys take five exact values
    want = np.nonzero(b == np.float32(0.5))[0][: wl.k].astype(np.int32)
    assert np.all(out.ids == want)
    assert np.all(out.w == np.float32(0.375))


@pytest.mark.parametrize("T", TIE_T)
def test_ties_twin_experts(moe, tie_inputs, T):
    """Experts in twins: expert 2i+1 has the router row and bias of expert 2i,
    so their logits, scores and keys are equal (the GPU computes both with
    the same arithmetic, as the oracle does).  With top 7 every token takes
    three whole pairs, each listed lower index first, and the lower member
    of a fourth pair whose twin ties with it exactly at the cut."""
    wl, inp = tie_inputs
    rw = inp.router_w.copy()
    rw[1::2] = rw[0::2]
    b = inp.router_b.copy()
    b[1::2] = b[0::2]
    wlT, sub = _tie_case(wl.with_(k=7), inp, T, rw, b)
    out, ref, rep = _run_ties(moe, wlT, sub)
    assert np.all(ref["gap"] == 0), "a twin pair does not straddle the cut"
    # where no other key comes within 1e-5 of the cut, the ids are the oracle's
    strict = np.setdiff1d(np.arange(T), rep.near_tie)
    assert np.array_equal(out.ids[strict], ref["ids"][strict])
    gu.note(f"  twins T={T}: {len(rep.near_tie)} near-ties, {len(rep.mismatched)} of them "
            "resolved the other way")
    assert np.all(out.ids % 2 == np.array([0, 1, 0, 1, 0, 1, 0]))
    assert np.all(out.ids[:, 1:6:2] == out.ids[:, 0:6:2] + 1), "a pair's upper twin is missing"


def test_route_entry_point_ties(moe, tie_inputs):
    """moe_route alone on all-equal keys: ids 0..k-1, weights 3/k."""
    import torch
    wl, inp = tie_inputs
    wlT = wl.with_(T=300)
    cfg = gu.cfg_of(wlT)
    ws = moe.alloc_workspace(cfg)
    ids = torch.empty((wlT.T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((wlT.T, wl.k), dtype=torch.float32, device="cuda")
    zero_w = torch.zeros((wl.E, wl.H), dtype=torch.float32, device="cuda")
    moe.moe_route(cfg, gu.to_dev(inp.x[:wlT.T]), zero_w, None, ids, w, ws)
    torch.cuda.synchronize()
    assert np.all(ids.cpu().numpy() == np.arange(wl.k))
    assert np.all(w.cpu().numpy() == np.float32(0.375))


# ------------------------------------------------------------- full shapes
# Every token of the four full-shape workloads is compared with the oracle.
# The GPU forward runs once per workload; its outputs are checked in chunks
# of FULL_CHUNK tokens (one test each), so that no test holds the CPU oracle
# for minutes.  M is taken over the chunk (never larger than over the whole
# output, so the bound is at least as strict).

FULL_CHUNK = 4096
FULL_CASES = [("decode", 0), ("prefill", 0), ("prefill", 1), ("skewed", 0)] + \
    [("long", c) for c in range(8)]
_full_cache = {}


def _full_run(moe, full_experts, name):
    """GPU forward of a full-shape workload, its routing and permutation
    checked on every token; cached for the chunk tests of that workload."""
    if name in _full_cache:
        return _full_cache[name]
    _full_cache.clear()
    wl = synth.WORKLOADS[name]
    host, dev = full_experts
    inp = synth.make_inputs(wl, experts=host)
    d = gu.upload(inp, experts_dev=dev)
    gu.note(f"  forward {name} T={wl.T}")
    out = gu.run_forward(wl, d)
    ref = oracle.route(oracle.cfg_of(wl), inp.x, inp.router_w, inp.router_b, want_keys=True)
    rep = gu.compare_route(wl, out.ids, out.w, ref)
    cfg = gu.cfg_of(wl)
    off = gu.ws_view(cfg, out.ws, moe.MOE_WS_EXPERT_OFFSETS, moe_i32())
    srt = gu.ws_view(cfg, out.ws, moe.MOE_WS_SORTED_PAIRS, moe_i32())
    pos = gu.ws_view(cfg, out.ws, moe.MOE_WS_PAIR_POS, moe_i32())
    o_off, o_srt, o_pos = oracle.permute(out.ids, wl.E)
    assert np.array_equal(off, o_off) and np.array_equal(srt, o_srt) and np.array_equal(pos, o_pos)
    U = int(np.count_nonzero(np.diff(off)))
    if name == "prefill":  # determinism at scale
        out2 = gu.run_forward(wl, d, ws=out.ws)
        assert np.array_equal(out.y, out2.y) and np.array_equal(out.ids, out2.ids)
    gu.note(f"  {name}: U={U} near-ties={len(rep.near_tie)} mismatched={len(rep.mismatched)} "
            f"rank-order swaps={rep.order_swaps} max w err={rep.max_w_err:.2e}")
    out.ws = None
    del d
    _full_cache[name] = (wl, inp, out, rep)
    return _full_cache[name]


@pytest.mark.parametrize("name,chunk", FULL_CASES, ids=[f"{n}-{c}" for n, c in FULL_CASES])
def test_full_shape_parity(moe, full_experts, name, chunk):
    wl, inp, out, rep = _full_run(moe, full_experts, name)
    toks = np.arange(chunk * FULL_CHUNK, min(wl.T, (chunk + 1) * FULL_CHUNK), dtype=np.int64)
    assert toks.size > 0
    gu.note(f"  oracle on tokens {toks[0]}..{toks[-1]}")
    y_ref = gu.oracle_y_for(wl, inp, toks, out.ids, rep.mismatched)
    err, M = gu.check_y(out.y[toks], y_ref, f"{name} tokens {toks[0]}..{toks[-1]}")
    rel = gu.per_token_rel_err(out.y[toks], y_ref)
    gu.note(f"  {name} tokens {toks[0]}..{toks[-1]}: max y err={err:.3e} M={M:.3e} "
            f"err/M={err / M:.2e} worst per-token rel err={rel:.2e}")
    if (chunk + 1) * FULL_CHUNK >= wl.T:
        _full_cache.clear()
