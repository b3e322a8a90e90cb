"""The layer forward inside a captured HIP graph, and on a caller stream that
is not the default one.  Every replay is checked bit for bit against the
eager result, with eager work and synchronisations between replays."""
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


CASES = {
    # few rows per expert (64-row tiles)
    "small": dict(T=48, H=512, E=32, k=4, I=128, Is=128, bias_var=0.3),
    # many rows per expert (256 x 256 tiles)
    "big_tile": dict(T=1100, H=512, E=8, k=4, I=256, Is=128, bias_var=0.5),
}


@pytest.mark.parametrize("name", list(CASES))
def test_forward_graph_replays(moe, name):
    import torch
    wl = synth.WORKLOADS["tiny"].with_(name=name, **CASES[name])
    inp = synth.make_inputs(wl)
    d = gu.upload(inp)
    cfg = gu.cfg_of(wl)
    ws = moe.alloc_workspace(cfg)
    args = (cfg, d.x, d.router_w, d.router_b, d.w_gate, d.w_up, d.w_down, d.ws_gate, d.ws_up,
            d.ws_down)
    y_ref = gu.run_forward(wl, d).y

    s = torch.cuda.Stream()
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(s):  # warm-up on the capture stream
        moe.moe_forward(*args, y, None, None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(y.float().cpu().numpy(), y_ref), "non-default caller stream"

    gu.note(f"  capture {name}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_forward(*args, y, None, None, ws)
    for rep in range(3):
        y.fill_(0.0)
        other = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")
        torch.cuda.synchronize()
        gu.note(f"  replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.float().cpu().numpy(), y_ref), f"replay {rep} differs"
        del other


def test_noalloc_forward_graph_replays(moe):
    """moe_forward_noalloc captured in a graph (its workspace is the library's
    fixed scratch, so the capture holds no allocation): every replay equals
    the eager moe_forward, bit for bit."""
    import torch
    wl = synth.WORKLOADS["tiny"].with_(name="noalloc_graph", **CASES["small"])
    inp = synth.make_inputs(wl)
    d = gu.upload(inp)
    cfg = gu.cfg_of(wl)
    args = (cfg, d.x, d.router_w, d.router_b, d.w_gate, d.w_up, d.w_down, d.ws_gate, d.ws_up,
            d.ws_down)
    y_ref = gu.run_forward(wl, d).y
    s = torch.cuda.Stream()
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(s):  # the scratch address is looked up on this first call
        moe.moe_forward_noalloc(*args, y)
    torch.cuda.synchronize()
    assert np.array_equal(y.float().cpu().numpy(), y_ref)
    gu.note("  capture moe_forward_noalloc")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_forward_noalloc(*args, y)
    for rep in range(3):
        y.fill_(0.0)
        other = gu.run_forward(wl.with_(T=8), dataclasses.replace(d, x=d.x[:8]))
        torch.cuda.synchronize()
        gu.note(f"  replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.float().cpu().numpy(), y_ref), f"replay {rep} differs"
        del other
