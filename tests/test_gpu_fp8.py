"""moe_forward_fp8 (routed experts' weights as OCP e4m3 codes with a scale
per output row) against the oracle on the same codes and scales, with the
protocol of test_gpu_parity: ids as sets (near-ties excepted), weights within
1e-5, y within 1e-2 * max|oracle| + 1e-3."""
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


def _fp8_dev(f8):
    return tuple(gu.to_dev(a) for a in (f8.w8_gate, f8.w8_up, f8.w8_down, f8.s_gate, f8.s_up,
                                        f8.s_down))


def run_fp8(moe, wl, inp, f8dev, shared_dev=None):
    torch = gu.torch_mod()
    cfg = gu.cfg_of(wl)
    ws = moe.alloc_workspace(cfg)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
    sh = wl.Is > 0
    if shared_dev is None:
        shared_dev = tuple(gu.to_dev(a) for a in (inp.ws_gate, inp.ws_up, inp.ws_down)) if sh \
            else (None, None, None)
    rb = None if inp.router_b is None else gu.to_dev(inp.router_b)
    moe.moe_forward_fp8(cfg, gu.to_dev(inp.x), gu.to_dev(inp.router_w), rb, *f8dev, *shared_dev,
                        y, ids, w, ws)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


def _check(wl, inp, f8, y, ids, w, tokens=None, rep=None):
    """Routing (unless rep is given) and y on `tokens` (default all); where
    the GPU took the other side of a near-tie, the oracle reruns that token
    with the GPU's ids."""
    if rep is None:
        ref = oracle.route(oracle.cfg_of(wl), inp.x, inp.router_w, inp.router_b, want_keys=True)
        rep = gu.compare_route(wl, ids, w, ref)
    toks = np.arange(wl.T, dtype=np.int64) if tokens is None else np.asarray(tokens, np.int64)
    cfg = oracle.cfg_of(wl)
    y_ref = oracle.forward_fp8(cfg, inp, f8, tokens=toks)["y"]
    swapped = set(rep.mismatched)
    forced = [i for i, t in enumerate(toks.tolist()) if t in swapped]
    if forced:
        sub = toks[forced]
        y_ref[forced] = oracle.forward_fp8(cfg, inp, f8, tokens=sub, forced_ids=ids[sub])["y"]
    err, M = gu.check_y(y[toks], y_ref, wl.name)
    return rep, err, M


CASES = {
    "tiny": {},
    # several row tiles per hot expert, ragged tails, k-steps not a multiple of 2
    "ragged": dict(T=333, H=512, E=24, k=6, I=192, Is=128, hot_experts=4, bias_var=0.1),
    "no_shared": dict(T=77, H=256, E=16, k=4, I=64, Is=0, bias_var=0.5),
    "clamped": dict(T=96, H=256, E=16, k=4, I=128, Is=64, limit=0.05, limit_shared=0.1),
    # small tiles 256 wide (I and Is multiples of 128, H of 256), ragged expert rows
    "wide_small": dict(T=150, H=512, E=12, k=4, I=256, Is=128, bias_var=0.3),
    # 256 x 256 tiles
    "big_tile": dict(T=1100, H=512, E=8, k=4, I=256, Is=128, bias_var=0.5),
    "big_tile_no_shared": dict(T=1500, H=768, E=6, k=3, I=384, Is=0, bias_var=0.2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_parity(moe, name):
    wl = synth.WORKLOADS["tiny"].with_(name=name, **CASES[name])
    inp = synth.make_inputs(wl)
    f8 = synth.gen_experts_fp8(wl)
    gu.note(f"  moe_forward_fp8 {wl}")
    y, ids, w = run_fp8(moe, wl, inp, _fp8_dev(f8))
    rep, err, M = _check(wl, inp, f8, y, ids, w)
    gu.note(f"  fp8 {name}: max err {err:.3e} M {M:.3e} near-ties {len(rep.near_tie)}")


def test_fp8_matches_bf16_path_on_exact_weights(moe):
    """Codes and power-of-two scales that are exactly representable as bf16
    weights: moe_forward_fp8 and moe_forward on those bf16 weights give the
    same bits (a power-of-two scale commutes with every fp32 rounding)."""
    wl = synth.WORKLOADS["tiny"].with_(name="exact", T=200, H=256, E=8, k=2, I=128, Is=64)
    inp = synth.make_inputs(wl)
    rng = np.random.default_rng(7)
    E, I, H = wl.E, wl.I, wl.H

    def codes(shape):
        return ((rng.integers(0, 2, shape) << 7) | (rng.integers(1, 11, shape) << 3)
                | rng.integers(0, 8, shape)).astype(np.uint8)

    def scales(shape):
        return np.ldexp(1.0, rng.integers(-12, -4, size=shape)).astype(np.float32)

    f8 = synth.Fp8Experts(codes((E, I, H)), scales((E, I)), codes((E, I, H)), scales((E, I)),
                          codes((E, H, I)), scales((E, H)))

    def as_bf16(c, s):
        v = oracle.e4m3_decode(c) * s[..., None].astype(np.float64)
        return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)

    inp_bf = inp.__class__(**{**inp.__dict__, "w_gate": as_bf16(f8.w8_gate, f8.s_gate),
                              "w_up": as_bf16(f8.w8_up, f8.s_up),
                              "w_down": as_bf16(f8.w8_down, f8.s_down)})
    y8, ids8, w8 = run_fp8(moe, wl, inp, _fp8_dev(f8))
    out = gu.run_forward(wl, gu.upload(inp_bf))
    assert np.array_equal(ids8, out.ids)
    assert np.array_equal(y8, out.y), float(np.max(np.abs(y8 - out.y)))


@pytest.fixture(scope="module")
def full_fp8():
    wl = synth.WORKLOADS["decode"]
    gu.note("  generating full-shape e4m3 expert weights (4.5 GB)")
    f8 = synth.gen_experts_fp8(wl)
    return f8, _fp8_dev(f8)


_fp8_cache = {}
FP8_CASES = [("decode", 0), ("prefill", 0), ("prefill", 1), ("skewed", 0)]
FP8_CHUNK = 4096


@pytest.mark.parametrize("name,chunk", FP8_CASES, ids=[f"{n}-{c}" for n, c in FP8_CASES])
def test_fp8_full_shape(moe, full_fp8, name, chunk):
    """Every token of the full-shape decode, prefill and skewed (clamped)
    workloads (one GPU run each; the oracle on chunks of FP8_CHUNK tokens)."""
    wl = synth.WORKLOADS[name]
    f8, f8dev = full_fp8
    if name not in _fp8_cache:
        _fp8_cache.clear()
        inp = synth.make_inputs(wl, experts=(np.zeros((0,), np.uint16),) * 3 +
                                tuple(synth.gen_experts(wl.with_(E=0, I=0))[3:]))
        gu.note(f"  moe_forward_fp8 {name} T={wl.T}")
        y, ids, w = run_fp8(moe, wl, inp, f8dev)
        ref = oracle.route(oracle.cfg_of(wl), inp.x, inp.router_w, inp.router_b, want_keys=True)
        rep = gu.compare_route(wl, ids, w, ref)
        _fp8_cache[name] = (inp, y, ids, w, rep)
    inp, y, ids, w, rep = _fp8_cache[name]
    toks = np.arange(chunk * FP8_CHUNK, min(wl.T, (chunk + 1) * FP8_CHUNK), dtype=np.int64)
    rep, err, M = _check(wl, inp, f8, y, ids, w, toks, rep)
    gu.note(f"  fp8 {name} tokens {toks[0]}..{toks[-1]}: near-ties={len(rep.near_tie)} "
            f"mismatched={len(rep.mismatched)} max w err={rep.max_w_err:.2e} "
            f"max y err={err:.3e} M={M:.3e}")
    if (chunk + 1) * FP8_CHUNK >= wl.T:
        _fp8_cache.clear()


def test_fp8_ties(moe):
    """Router weight 0 and no bias: all keys equal, ids 0..k-1 in order and
    weights 3/k exactly, as on the bf16 path (same routing kernels)."""
    wl = synth.WORKLOADS["tiny"].with_(name="fp8_ties", T=100, H=512, E=40, k=8, I=128, Is=64)
    inp = synth.make_inputs(wl)
    inp.router_w[:] = 0.0
    inp.router_b = None
    f8 = synth.gen_experts_fp8(wl)
    y, ids, w = run_fp8(moe, wl, inp, _fp8_dev(f8))
    assert np.all(ids == np.arange(wl.k)) and np.all(w == np.float32(0.375))
    _check(wl, inp, f8, y, ids, w)
