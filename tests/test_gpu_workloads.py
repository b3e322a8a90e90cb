"""Second workloads on the same kernels, against the oracle (same protocol as
test_gpu_parity): the dense SwiGLU FFN of the model's first layers
(intermediate 11264) through moe_dense_forward, and the predecessor Step-3's
MoE shape (H 7168, 48 experts, top-3, I 5120, no weight renormalisation)
through moe_forward."""
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


def _dense_inputs(wl):
    inp = synth.make_inputs(wl)
    return inp.x, inp.ws_gate, inp.ws_up, inp.ws_down


def _run_dense(moe, wl, x, wg, wu, wd, limit=0.0):
    torch = gu.torch_mod()
    cfg = moe.make_dense_config(wl.T, wl.H, wl.Is, limit)
    ws = moe.alloc_dense_workspace(cfg)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    dx = gu.to_dev(x) if wl.T else None
    moe.moe_dense_forward(cfg, dx, gu.to_dev(wg), gu.to_dev(wu), gu.to_dev(wd), y if wl.T else None,
                          ws)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


DENSE = {
    # 64 x 128 tiles (fewer than 1024 rows), ragged last tile
    "small": dict(T=300, H=512, Is=384),
    "small_clamped": dict(T=77, H=256, Is=192, limit_shared=0.05),
    # 256 x 256 tiles, ragged
    "big": dict(T=1100, H=512, Is=256),
    "big_clamped": dict(T=1500, H=768, Is=384, limit_shared=0.1),
}


@pytest.mark.parametrize("name", list(DENSE))
def test_dense_parity(moe, name):
    wl = synth.WORKLOADS["dense"].with_(name=name, **DENSE[name])
    x, wg, wu, wd = _dense_inputs(wl)
    gu.note(f"  moe_dense_forward T={wl.T} H={wl.H} I={wl.Is} limit={wl.limit_shared}")
    y = _run_dense(moe, wl, x, wg, wu, wd, wl.limit_shared)
    _, o = oracle.expert(x, wg, wu, wd, wl.limit_shared)
    err, M = gu.check_y(y, o, name)
    gu.note(f"  dense {name}: max err {err:.3e} M {M:.3e}")
    # the MLP is the shared expert of a layer whose routed part contributes 0
    assert np.all(np.isfinite(y))


_dense_cache = {}


@pytest.mark.parametrize("chunk", [0, 1])
def test_dense_full_shape(moe, chunk):
    """Every token of the dense FFN workload (T 8192, I 11264), compared
    with the oracle in two halves (one GPU run)."""
    wl = synth.WORKLOADS["dense"]
    if not _dense_cache:
        x, wg, wu, wd = _dense_inputs(wl)
        gu.note(f"  moe_dense_forward T={wl.T} H={wl.H} I={wl.Is}")
        _dense_cache["run"] = (x, wg, wu, wd, _run_dense(moe, wl, x, wg, wu, wd))
    x, wg, wu, wd, y = _dense_cache["run"]
    half = wl.T // 2
    toks = np.arange(chunk * half, (chunk + 1) * half)
    _, o = oracle.expert(x[toks], wg, wu, wd, 0.0)
    err, M = gu.check_y(y[toks], o, f"dense tokens {toks[0]}..{toks[-1]}")
    gu.note(f"  dense tokens {toks[0]}..{toks[-1]}: max err {err:.3e} M {M:.3e}")
    if chunk == 1:
        _dense_cache.clear()


def test_dense_empty(moe):
    wl = synth.WORKLOADS["dense"].with_(T=0, H=256, Is=128)
    torch = gu.torch_mod()
    cfg = moe.make_dense_config(0, 256, 128)
    ws = moe.alloc_dense_workspace(cfg)
    w = torch.zeros((128, 256), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((256, 128), dtype=torch.bfloat16, device="cuda")
    moe.moe_dense_forward(cfg, None, w, w, wd, None, ws)
    torch.cuda.synchronize()
    assert wl.T == 0


_step3_cache = {}


@pytest.mark.parametrize("chunk", [0, 1, 2, 3])
def test_step3_full_shape(moe, chunk):
    """Step-3's MoE block: 48 experts of I 5120 at H 7168, top-3, weights not
    renormalised, no router bias, routed scaling 1.  One GPU run; every
    token compared with the oracle, a quarter per test."""
    wl = synth.WORKLOADS["step3"]
    if not _step3_cache:
        gu.note("  generating Step-3 shape inputs (10.8 GB of expert weights)")
        inp = synth.make_inputs(wl)
        assert inp.router_b is None
        d = gu.upload(inp)
        gu.note(f"  forward step3 T={wl.T}")
        out = gu.run_forward(wl, d)
        out.ws = None
        del d
        ref = oracle.route(oracle.cfg_of(wl), inp.x, inp.router_w, None, want_keys=True)
        rep = gu.compare_route(wl, out.ids, out.w, ref)
        # without renormalisation the weights are the raw scores (scaling 1)
        assert np.all(out.w > 0) and np.all(out.w < 1)
        _step3_cache["run"] = (inp, out, rep)
    inp, out, rep = _step3_cache["run"]
    part = wl.T // 4
    toks = np.arange(chunk * part, (chunk + 1) * part, dtype=np.int64)
    y_ref = gu.oracle_y_for(wl, inp, toks, out.ids, rep.mismatched)
    err, M = gu.check_y(out.y[toks], y_ref, f"step3 tokens {toks[0]}..{toks[-1]}")
    gu.note(f"  step3 tokens {toks[0]}..{toks[-1]}: near-ties={len(rep.near_tie)} "
            f"mismatched={len(rep.mismatched)} max w err={rep.max_w_err:.2e} "
            f"max y err={err:.3e} M={M:.3e}")
    if chunk == 3:
        _step3_cache.clear()
