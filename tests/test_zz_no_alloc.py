"""moe_forward_noalloc, the layer forward whose workspace is the library's
fixed scratch, against moe_forward with a caller workspace on the same
inputs: y, the expert ids and the gating weights bit for bit, on two calls
in a row, the second with a smaller batch (the scratch keeps the first
call's contents).  A batch too large for the scratch is refused before
anything is enqueued."""
import dataclasses

import numpy as np
import pytest

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


def _noalloc(moe, wl, d):
    torch = gu.torch_mod()
    cfg = gu.cfg_of(wl)
    assert moe.moe_workspace_size(cfg) <= moe.NOALLOC_SCRATCH_BYTES
    y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((wl.T, wl.k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((wl.T, wl.k), float("nan"), dtype=torch.float32, device="cuda")
    sh = wl.Is > 0
    gu.note(f"  moe_forward_noalloc {wl.name} T={wl.T}")
    moe.moe_forward_noalloc(cfg, d.x, d.router_w, d.router_b, d.w_gate, d.w_up, d.w_down,
                            d.ws_gate if sh else None, d.ws_up if sh else None,
                            d.ws_down if sh else None, y, ids, w)
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


def _same(moe, wl, d):
    """One moe_forward (fresh workspace) and one moe_forward_noalloc call."""
    torch = gu.torch_mod()
    gu.note(f"  moe_forward {wl.name} T={wl.T}")
    ref = gu.run_forward(wl, d)
    y_bits = torch.from_numpy(ref.y).to(torch.bfloat16).view(torch.int16).numpy()
    got_y, got_ids, got_w = _noalloc(moe, wl, d)
    assert np.array_equal(got_ids, ref.ids), f"{wl.name} T={wl.T}: ids differ"
    assert np.array_equal(got_w.view(np.uint32), ref.w.view(np.uint32)), \
        f"{wl.name} T={wl.T}: weights differ"
    assert np.array_equal(got_y, y_bits), f"{wl.name} T={wl.T}: y differs"


def test_noalloc_decode_shape(moe, full_experts):
    """The full-shape decode layer (hidden 4096, 288 experts, top 8,
    intermediate 1280): 64 tokens, then 16."""
    wl = synth.WORKLOADS["decode"]
    host, dev = full_experts
    d = gu.upload(synth.make_inputs(wl, experts=host), experts_dev=dev)
    for T in (64, 16):
        _same(moe, wl.with_(T=T), dataclasses.replace(d, x=d.x[:T]))


def test_noalloc_both_tile_shapes(moe):
    """600 tokens over 16 experts take the persistent 256 x 256 tiles (their
    work-queue counters live in the scratch), then 100 tokens the 64-row
    tiles."""
    wl = synth.WORKLOADS["tiny"].with_(name="noalloc_tiles", T=600, H=4096, E=16, k=8, I=256,
                                       Is=256, bias_var=0.2)
    d = gu.upload(synth.make_inputs(wl))
    for T in (600, 100):
        _same(moe, wl.with_(T=T), dataclasses.replace(d, x=d.x[:T]))


def test_noalloc_refuses_batches_beyond_the_scratch(moe):
    torch = gu.torch_mod()
    wl = synth.WORKLOADS["tiny"].with_(name="noalloc_big", T=1024, H=4096, E=16, k=8, I=1280,
                                       Is=1280)
    cfg = gu.cfg_of(wl)
    assert moe.moe_workspace_size(cfg) > moe.NOALLOC_SCRATCH_BYTES
    d = gu.upload(synth.make_inputs(wl))
    y = torch.full((wl.T, wl.H), 1.5, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_noalloc(cfg, d.x, d.router_w, d.router_b, d.w_gate, d.w_up, d.w_down,
                                d.ws_gate, d.ws_up, d.ws_down, y)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(y.float() == 1.5)
