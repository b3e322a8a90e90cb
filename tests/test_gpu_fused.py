"""The single-launch forward, moe_forward_fused.

It runs the same tiles in the same arithmetic order as the multi-launch
moe_forward, so the guard is bit-equality of y, the expert ids and the
gating weights between the two on the same inputs (the equality pattern the
sglang-jax issue asks of the grouped matmul against the per-expert loop,
"Implementation strategy"), plus the oracle parity protocol on the fused
outputs themselves.  Also: the control words are back to zero after every
call and the status word stays zero; repeated calls on one workspace,
interleaved with the multi-launch path; empty batches; the size limits.
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


def _run(moe, wl, d, fused, ws=None, use_bias=True, T=None):
    """One forward (fused or multi-launch) on the first T tokens of d.x.
    Outputs start as NaN / -1 so that anything left unwritten shows."""
    torch = gu.torch_mod()
    T = wl.T if T is None else T
    cfg = gu.cfg_of(wl, T=T)
    if ws is None:
        ws = moe.alloc_workspace(cfg)
    y = torch.full((T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((T, wl.k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, wl.k), float("nan"), dtype=torch.float32, device="cuda")
    sh = wl.Is > 0
    fn = moe.moe_forward_fused if fused else moe.moe_forward
    gu.note(f"  {'fused' if fused else 'multi-launch'} forward {wl.name} T={T}")
    fn(cfg, d.x[:T], d.router_w, d.router_b if use_bias else None, d.w_gate, d.w_up, d.w_down,
       d.ws_gate if sh else None, d.ws_up if sh else None, d.ws_down if sh else None, y, ids, w,
       ws)
    torch.cuda.synchronize()
    return dict(y_bits=y.view(torch.int16).cpu().numpy(), y=y.float().cpu().numpy(),
                ids=ids.cpu().numpy(), w=w.cpu().numpy(), ws=ws, cfg=cfg)


def _check_ctl_clear(moe, r):
    torch = gu.torch_mod()
    ctl = gu.ws_view(r["cfg"], r["ws"], moe.MOE_WS_FUSED_CTL, torch.int32)
    status = gu.ws_view(r["cfg"], r["ws"], moe.MOE_WS_FUSED_STATUS, torch.int32)
    assert int(status[0]) == 0, f"a fused wait gave up (status {int(status[0]):#x})"
    assert not np.any(ctl), f"control words left nonzero at {np.nonzero(ctl)[0][:8]}"


def _assert_identical(a, b, what):
    assert np.array_equal(a["ids"], b["ids"]), f"{what}: expert ids differ"
    assert np.array_equal(a["w"].view(np.uint32), b["w"].view(np.uint32)), f"{what}: weights differ"
    diff = np.nonzero(a["y_bits"] != b["y_bits"])
    assert diff[0].size == 0, f"{what}: y differs at {list(zip(*diff))[:4]}"


SMALL = {
    "tiny": dict(),
    "single_token": dict(T=1, H=128, E=4, k=2, I=64, Is=64),
    # expert count not a multiple of 64, ragged rows
    "ragged": dict(T=37, H=512, E=40, k=6, I=192, Is=128, bias_var=0.3),
    # several 64-row tiles per hot expert and four shared row tiles
    "multi_tile": dict(T=200, H=256, E=16, k=8, I=64, Is=64, bias_var=0.5),
    # the largest batch: tokens * k = 2048, 300 experts (5 router tiles)
    "max_pairs": dict(T=256, H=256, E=300, k=8, I=64, Is=64, bias_var=0.2),
    # the largest expert count and k
    "max_experts": dict(T=8, H=256, E=1024, k=32, I=64, Is=64),
    "no_shared": dict(T=77, H=256, E=16, k=4, I=64, Is=0, bias_var=0.5),
    "clamped_hot": dict(T=64, H=512, E=64, k=8, I=128, Is=128, limit=0.05, limit_shared=0.1,
                        hot_experts=4),
    "no_renorm": dict(T=40, H=256, E=16, k=4, I=64, Is=64, renormalize=False),
    "k_equals_E": dict(T=50, H=256, E=8, k=8, I=64, Is=64),
    # full router width (split-k router tiles, 288 experts)
    "full_router": dict(T=40, H=4096, E=288, k=8, I=64, Is=64),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_equals_multi_launch(moe, name):
    wl = synth.WORKLOADS["tiny"].with_(name=name, **SMALL[name])
    inp = synth.make_inputs(wl)
    d = gu.upload(inp)
    a = _run(moe, wl, d, fused=False)
    b = _run(moe, wl, d, fused=True)
    _assert_identical(a, b, name)
    _check_ctl_clear(moe, b)
    # the fused outputs against the oracle (every token)
    ref = oracle.route(oracle.cfg_of(wl), inp.x, inp.router_w, inp.router_b, want_keys=True)
    rep = gu.compare_route(wl, b["ids"], b["w"], ref)
    y_ref = gu.oracle_y_for(wl, inp, np.arange(wl.T), b["ids"], rep.mismatched)
    err, M = gu.check_y(b["y"], y_ref, name)
    gu.note(f"  {name}: identical to multi-launch; oracle max err {err:.3e} M {M:.3e}")


def test_fused_no_bias(moe):
    wl = synth.WORKLOADS["tiny"].with_(name="no_bias", T=48)
    d = gu.upload(synth.make_inputs(wl))
    _assert_identical(_run(moe, wl, d, False, use_bias=False),
                      _run(moe, wl, d, True, use_bias=False), "no_bias")


def test_fused_repeated_and_interleaved(moe):
    """One workspace: fused, multi-launch, fused, fused on different batch
    sizes; every fused call matches the multi-launch result for its size
    and leaves the control words zero."""
    wl = synth.WORKLOADS["tiny"].with_(name="repeat", **SMALL["multi_tile"])
    inp = synth.make_inputs(wl)
    d = gu.upload(inp)
    ws = _run(moe, wl, d, True)["ws"]  # sized for the largest batch
    for T in (200, 63, 200, 1, 130):
        ref = _run(moe, wl, d, False, T=T)
        got = _run(moe, wl, d, True, ws=ws, T=T)
        _assert_identical(ref, got, f"T={T}")
        _check_ctl_clear(moe, got)
        got2 = _run(moe, wl, d, False, ws=ws, T=T)  # the other path on the same workspace
        _assert_identical(ref, got2, f"multi-launch after fused, T={T}")


def test_fused_empty_batch(moe):
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
    moe.moe_forward_fused(cfg, x, rw, None, we, we, wd, sg, sg, sd, y, None, None, ws)
    torch.cuda.synchronize()
    assert not torch.any(ws)  # nothing was launched


def test_fused_over_limit_enqueues_nothing(moe):
    import torch
    wl = synth.WORKLOADS["tiny"].with_(name="over", T=moe.FUSED_MAX_TOKENS + 1)
    d = gu.upload(synth.make_inputs(wl))
    cfg = gu.cfg_of(wl)
    ws = moe.alloc_workspace(cfg)
    y = torch.full((wl.T, wl.H), 1.5, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_fused(cfg, d.x, d.router_w, d.router_b, d.w_gate, d.w_up, d.w_down,
                              d.ws_gate, d.ws_up, d.ws_down, y, None, None, ws)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(y.float() == 1.5)


@pytest.mark.parametrize("T", [64, 1, 17])
def test_fused_full_shape(moe, full_experts, T):
    """Decoding batches at the full layer shape (4096 -> 1280 -> 4096, 288
    experts, top 8, shared expert): bit-identical to the multi-launch path,
    and the oracle on every token."""
    wl = synth.WORKLOADS["decode"]
    host, dev = full_experts
    inp = synth.make_inputs(wl, experts=host)
    d = gu.upload(inp, experts_dev=dev)
    a = _run(moe, wl, d, False, T=T)
    b = _run(moe, wl, d, True, T=T)
    _assert_identical(a, b, f"decode T={T}")
    _check_ctl_clear(moe, b)
    wlT = wl.with_(T=T)
    x_T = inp.x[:T]
    ref = oracle.route(oracle.cfg_of(wlT), x_T, inp.router_w, inp.router_b, want_keys=True)
    rep = gu.compare_route(wlT, b["ids"], b["w"], ref)
    toks = np.arange(T, dtype=np.int64)
    y_ref = gu.oracle_y_for(wl, inp, toks, b["ids"], rep.mismatched)
    err, M = gu.check_y(b["y"][toks], y_ref, f"decode T={T}")
    gu.note(f"  decode T={T}: identical to multi-launch; oracle max err {err:.3e} M {M:.3e}")


@pytest.mark.parametrize("levels", [False, True])
def test_fused_ties(moe, levels):
    """Router weight 0: all scores 1/2; without a bias every key ties (ids
    0..k-1), with a bias of five exact levels the keys tie within each level
    (the lowest-numbered experts of the top level).  The single launch's own
    top-k body must rank equal keys lower index first, as moe_forward does."""
    wl = synth.WORKLOADS["tiny"].with_(name="fused_ties", T=64, H=512, E=300, k=8, I=64, Is=64)
    inp = synth.make_inputs(wl)
    inp.router_w[:] = 0.0
    if levels:
        rng = np.random.default_rng(5)
        inp.router_b = rng.choice(np.array([-0.5, -0.25, 0.0, 0.25, 0.5], np.float32), wl.E)
        want = np.nonzero(inp.router_b == np.float32(0.5))[0][: wl.k]
    else:
        inp.router_b = np.zeros(wl.E, np.float32)
        want = np.arange(wl.k)
    d = gu.upload(inp)
    a = _run(moe, wl, d, False)
    b = _run(moe, wl, d, True)
    _assert_identical(a, b, "ties")
    _check_ctl_clear(moe, b)
    assert np.all(b["ids"] == want) and np.all(b["w"] == np.float32(0.375))
