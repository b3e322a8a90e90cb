"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values
derived by hand (golden files), closed forms, brute force, invariants stated
on the pages, and special cases that reduce to a library routine.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import synth
from tests.helpers import bf16_bits_to_f32, f32_to_bf16_bits, golden, inputs

TINY = synth.WORKLOADS["tiny"]


def tiny_inputs(**kw):
    wl = TINY.with_(**kw)
    return wl, synth.make_inputs(wl)


# ------------------------------------------------------------ golden files

def test_golden_worked_routing():
    g = golden("worked_routing.json")
    c = g["config"]
    cfg = oracle.make_cfg(1, c["H"], c["E"], c["k"], 1, 0, c["routed_scaling"], c["renormalize"])
    x = f32_to_bf16_bits([g["x"]])
    r = oracle.route(cfg, x, np.array(g["router_w"], np.float32), np.array(g["router_b"], np.float32))
    assert r["ids"][0].tolist() == g["expect"]["ids"]
    np.testing.assert_allclose(r["w"][0], g["expect"]["w"], atol=g["tol"], rtol=0)
    assert abs(r["gap"][0] - g["expect"]["gap"]) < g["tol"]


@pytest.mark.parametrize("with_shared", [False, True])
def test_golden_layout_example(with_shared):
    g = golden("layout_example.json")
    c = g["config"]
    Is = 1 if with_shared else 0
    cfg = oracle.make_cfg(1, c["H"], c["E"], c["k"], c["I"], Is, c["routed_scaling"], c["renormalize"])
    sh = {}
    if with_shared:
        sh = dict(ws_gate=f32_to_bf16_bits(g["ws_gate"]), ws_up=f32_to_bf16_bits(g["ws_up"]),
                  ws_down=f32_to_bf16_bits(g["ws_down"]))
    inp = inputs(f32_to_bf16_bits([g["x"]]), g["router_w"], g["router_b"],
                 f32_to_bf16_bits(g["w_gate"]), f32_to_bf16_bits(g["w_up"]),
                 f32_to_bf16_bits(g["w_down"]), **sh)
    out = oracle.forward(cfg, inp)
    assert out["ids"][0].tolist() == g["expect"]["ids"]
    np.testing.assert_allclose(out["w"][0], g["expect"]["w"], atol=g["tol"], rtol=0)
    key = "y_with_shared" if with_shared else "y_routed_only"
    np.testing.assert_allclose(out["y"][0], g["expect"][key], atol=g["tol"], rtol=0)


def test_golden_swiglu_scalar():
    g = golden("swiglu_scalar.json")
    for case in g["cases"]:
        rows = f32_to_bf16_bits([[1.0]])
        h, o = oracle.expert(rows, f32_to_bf16_bits([[case["gate"]]]), f32_to_bf16_bits([[case["up"]]]),
                             f32_to_bf16_bits([[1.0]]), limit=case["limit"])
        assert abs(o[0, 0] - case["o"]) <= g["tol"] * max(1.0, abs(case["o"])), case
        assert abs(h[0, 0] - case["o"]) <= g["tol"] * max(1.0, abs(case["o"])), case


# ------------------------------------------------------------- selection

def _dominates(key, a, b):
    """(key desc, index asc) order: does expert a rank before expert b?"""
    return key[a] > key[b] or (key[a] == key[b] and a < b)


@pytest.mark.parametrize("ties", [False, True])
def test_topk_brute_force(ties):
    """Exactly one k-subset beats every expert outside it, and it is ids."""
    wl = TINY.with_(T=24)
    inp = synth.make_inputs(wl)
    rw, rb = inp.router_w, inp.router_b
    if ties:  # coarse keys with many exact ties: only the bias decides
        rw = np.zeros_like(rw)
        rb = (np.arange(wl.E) % 5).astype(np.float32) * 0.25
    r = oracle.route(oracle.cfg_of(wl), inp.x, rw, rb, want_keys=True)
    for t in range(wl.T):
        key = r["keys"][t]
        winners = []
        for S in itertools.combinations(range(wl.E), wl.k):
            inside = set(S)
            if all(_dominates(key, a, b) for a in S for b in range(wl.E) if b not in inside):
                winners.append(S)
        assert len(winners) == 1
        assert sorted(r["ids"][t].tolist()) == list(winners[0])
        # ids come in rank order
        for j in range(wl.k - 1):
            assert _dominates(key, r["ids"][t][j], r["ids"][t][j + 1])
        srt = sorted(range(wl.E), key=lambda e: (-key[e], e))
        assert r["gap"][t] == key[srt[wl.k - 1]] - key[srt[wl.k]]


def test_all_tied():
    wl, inp = tiny_inputs(T=8)
    r = oracle.route(oracle.cfg_of(wl), inp.x, np.zeros_like(inp.router_w), np.zeros(wl.E, np.float32))
    for t in range(wl.T):
        assert r["ids"][t].tolist() == list(range(wl.k))
        assert np.all(r["w"][t] == 3.0 / wl.k)
        assert r["gap"][t] == 0.0
    # full shape: 3/8 = 0.375 exactly
    cfg = oracle.make_cfg(2, 64, 288, 8, 64, 0)
    x = synth.normal_bf16(0, 1, 2 * 64, 1.0).reshape(2, 64)
    r = oracle.route(cfg, x, np.zeros((288, 64), np.float32), None)
    assert np.all(r["w"] == 0.375) and r["ids"].tolist() == [list(range(8))] * 2


def test_bias_alone_selects():
    wl, inp = tiny_inputs(T=8)
    b = inp.router_b
    assert len(set(b.tolist())) == wl.E
    r = oracle.route(oracle.cfg_of(wl), inp.x, np.zeros_like(inp.router_w), b)
    expect = np.argsort(-b.astype(np.float64), kind="stable")[: wl.k]
    for t in range(wl.T):
        assert r["ids"][t].tolist() == expect.tolist()
        assert np.all(r["w"][t] == 3.0 / wl.k)


def test_bias_never_changes_weights():
    """The bias moves the selection but never the gating weights."""
    wl = TINY.with_(T=1)
    for seed in range(6):
        inp = synth.make_inputs(wl.with_(seed=seed))
        cfg = oracle.cfg_of(wl)
        base = oracle.route(cfg, inp.x, inp.router_w, inp.router_b, want_keys=True)
        S = base["ids"][0]
        # (a) perturbation that keeps the selected set: same weights, bit for bit
        b2 = inp.router_b.copy()
        mask = np.zeros(wl.E, bool)
        mask[S] = True
        b2[mask] += np.float32(0.5)
        b2[~mask] -= np.float32(0.5)
        r2 = oracle.route(cfg, inp.x, inp.router_w, b2)
        assert r2["ids"][0].tolist() == S.tolist()
        assert np.array_equal(r2["w"][0], base["w"][0])
        # (b) two different biases that select the same other set: same weights
        rng = np.random.default_rng(seed)
        S2 = rng.choice(wl.E, wl.k, replace=False)
        b3 = np.zeros(wl.E, np.float32)
        b3[S2] = 10.0
        b4 = rng.normal(0, 0.01, wl.E).astype(np.float32)
        b4[S2] = 5.0
        r3 = oracle.route(cfg, inp.x, inp.router_w, b3, want_keys=True)
        r4 = oracle.route(cfg, inp.x, inp.router_w, b4)
        assert sorted(r3["ids"][0].tolist()) == sorted(S2.tolist())
        assert r3["ids"][0].tolist() == r4["ids"][0].tolist()
        assert np.array_equal(r3["w"][0], r4["w"][0])
        # weights are proportional to the bias-free scores of the chosen set
        s = r3["scores"][0]
        ids = r3["ids"][0]
        np.testing.assert_allclose(r3["w"][0] / r3["w"][0][0], s[ids] / s[ids[0]], rtol=1e-14)
        # the scores do not depend on the bias at all
        np.testing.assert_array_equal(r3["scores"][0], base["scores"][0])


@pytest.mark.parametrize("name", ["tiny"])
def test_weights_sum_to_scaling(name):
    wl = synth.WORKLOADS[name].with_(T=64)
    inp = synth.make_inputs(wl)
    r = oracle.route(oracle.cfg_of(wl), inp.x, inp.router_w, inp.router_b)
    assert np.all(np.abs(r["w"].sum(1) - 3.0) < 1e-13)
    assert np.all(r["w"] > 0)
    # without renormalisation the weights are 3 * s, which do not sum to 3
    r2 = oracle.route(oracle.cfg_of(wl.with_(renormalize=False)), inp.x, inp.router_w,
                      inp.router_b, want_keys=True)
    s = np.take_along_axis(r2["scores"], r2["ids"].astype(np.int64), 1)
    np.testing.assert_allclose(r2["w"], 3.0 * s, rtol=1e-15)
    assert np.max(np.abs(r2["w"].sum(1) - 3.0)) > 1e-3


def test_weights_sum_full_shape():
    """Sigma w = 3 on the full router shape (288 experts, top-8, H = 4096)."""
    wl = synth.WORKLOADS["decode"].with_(T=16)
    x = synth.gen_x(wl)
    wg, b, _ = synth.gen_router(wl)
    r = oracle.route(oracle.cfg_of(wl), x, wg, b)
    assert np.all(np.abs(r["w"].sum(1) - 3.0) < 1e-13)
    assert all(len(set(row)) == 8 for row in r["ids"].tolist())


# -------------------------------------------------------------- experts

def _np_swiglu_mlp(x_bits, gate_bits, up_bits, down_bits, limit=0.0):
    """Dense SwiGLU MLP by library matmuls in float64 (a textbook MLP)."""
    X = bf16_bits_to_f32(x_bits).astype(np.float64)
    G = X @ bf16_bits_to_f32(gate_bits).astype(np.float64).T
    U = X @ bf16_bits_to_f32(up_bits).astype(np.float64).T
    if limit > 0:
        G = np.minimum(G, limit)
        U = np.clip(U, -limit, limit)
    A = G / (1.0 + np.exp(-G)) * U
    return A, A @ bf16_bits_to_f32(down_bits).astype(np.float64).T


@pytest.mark.parametrize("limit", [0.0, 0.05])
def test_expert_matches_library_mlp(limit):
    wl, inp = tiny_inputs(T=32)
    h, o = oracle.expert(inp.x, inp.w_gate[3], inp.w_up[3], inp.w_down[3], limit=limit)
    A, O = _np_swiglu_mlp(inp.x, inp.w_gate[3], inp.w_up[3], inp.w_down[3], limit)
    np.testing.assert_allclose(h, A, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o, O, rtol=1e-12, atol=1e-13)
    if limit:
        _, O0 = _np_swiglu_mlp(inp.x, inp.w_gate[3], inp.w_up[3], inp.w_down[3], 0.0)
        assert np.max(np.abs(O - O0)) > 1e-3  # the clamp is active on these inputs


def test_zero_routed_scaling_is_dense_mlp():
    """routed_scaling = 0 leaves the shared expert alone: a dense SwiGLU MLP."""
    wl, inp = tiny_inputs(T=16, routed_scaling=0.0)
    y = oracle.forward(oracle.cfg_of(wl), inp)["y"]
    _, O = _np_swiglu_mlp(inp.x, inp.ws_gate, inp.ws_up, inp.ws_down)
    np.testing.assert_allclose(y, O, rtol=1e-12, atol=1e-13)


def test_single_expert_is_scaled_mlp():
    """E = k = 1 and no shared expert: y = 3 * f(x) for the one expert."""
    wl, inp = tiny_inputs(T=16, E=1, k=1, Is=0)
    inp.ws_gate = np.zeros((0, wl.H), np.uint16)
    inp.ws_up = np.zeros((0, wl.H), np.uint16)
    inp.ws_down = np.zeros((wl.H, 0), np.uint16)
    out = oracle.forward(oracle.cfg_of(wl), inp)
    _, O = _np_swiglu_mlp(inp.x, inp.w_gate[0], inp.w_up[0], inp.w_down[0])
    np.testing.assert_allclose(out["y"], 3.0 * O, rtol=1e-12, atol=1e-13)
    assert np.all(out["w"] == 3.0)


def test_identical_experts_closed_form():
    """All routed experts identical: routed part = 3.0 * f(x); y = shared + 3 f."""
    wl, inp = tiny_inputs(T=16)
    for name in ("w_gate", "w_up", "w_down"):
        arr = getattr(inp, name)
        setattr(inp, name, np.ascontiguousarray(np.broadcast_to(arr[5], arr.shape)))
    y = oracle.forward(oracle.cfg_of(wl), inp)["y"]
    _, O = _np_swiglu_mlp(inp.x, inp.w_gate[0], inp.w_up[0], inp.w_down[0])
    _, Os = _np_swiglu_mlp(inp.x, inp.ws_gate, inp.ws_up, inp.ws_down)
    np.testing.assert_allclose(y, Os + 3.0 * O, rtol=1e-11, atol=1e-12)


def test_clamp_limits_applied_separately():
    """The routed and the shared limits act on their own experts only."""
    wl, inp = tiny_inputs(T=16)
    big = 0.02
    base = oracle.forward(oracle.cfg_of(wl), inp)["y"]
    r_only = oracle.forward(oracle.cfg_of(wl.with_(limit=big)), inp)["y"]
    s_only = oracle.forward(oracle.cfg_of(wl.with_(limit_shared=big)), inp)["y"]
    _, Os = _np_swiglu_mlp(inp.x, inp.ws_gate, inp.ws_up, inp.ws_down)
    _, Os_c = _np_swiglu_mlp(inp.x, inp.ws_gate, inp.ws_up, inp.ws_down, big)
    np.testing.assert_allclose(s_only - base, Os_c - Os, rtol=1e-9, atol=1e-12)
    assert np.max(np.abs(r_only - base)) > 1e-4


# --------------------------------------------------------- layer invariants

def test_token_independence_and_subsets():
    wl, inp = tiny_inputs(T=32)
    cfg = oracle.cfg_of(wl)
    full = oracle.forward(cfg, inp)
    sub = np.array([31, 0, 7, 7, 19])
    part = oracle.forward(cfg, inp, tokens=sub)
    assert np.array_equal(part["y"], full["y"][sub])
    assert np.array_equal(part["ids"], full["ids"][sub])


def test_expert_relabelling_equivariance():
    wl, inp = tiny_inputs(T=32)
    cfg = oracle.cfg_of(wl)
    full = oracle.forward(cfg, inp)
    perm = np.random.default_rng(1).permutation(wl.E)  # new expert i is old expert perm[i]
    inv = np.argsort(perm)
    relab = inputs(inp.x, inp.router_w[perm], inp.router_b[perm], inp.w_gate[perm], inp.w_up[perm],
                   inp.w_down[perm], inp.ws_gate, inp.ws_up, inp.ws_down)
    out = oracle.forward(cfg, relab)
    assert np.array_equal(perm[out["ids"]], full["ids"])  # no exact key ties on these inputs
    np.testing.assert_array_equal(out["w"], full["w"])
    np.testing.assert_array_equal(out["y"], full["y"])
    assert inv.size == wl.E


def test_forced_ids_recompute_weights():
    wl, inp = tiny_inputs(T=4)
    cfg = oracle.cfg_of(wl)
    r = oracle.route(cfg, inp.x, inp.router_w, inp.router_b, want_keys=True)
    forced = np.tile(np.arange(wl.k, dtype=np.int32), (wl.T, 1))
    out = oracle.forward(cfg, inp, forced_ids=forced)
    s = r["scores"][:, : wl.k]
    np.testing.assert_allclose(out["w"], 3.0 * s / s.sum(1, keepdims=True), rtol=1e-15)
    assert np.array_equal(out["ids"], forced)


# --------------------------------------------------------------- permute

@pytest.mark.parametrize("T,E,k", [(16, 16, 4), (300, 288, 8), (1, 5, 5), (0, 7, 2)])
def test_permute_matches_stable_argsort(T, E, k):
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32) \
        if T else np.zeros((0, k), np.int32)
    off, srt, pos = oracle.permute(ids, E)
    flat = ids.ravel()
    expect = np.argsort(flat, kind="stable")
    assert np.array_equal(srt, expect)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(pos[srt], np.arange(T * k))
    assert off[-1] == T * k


# ------------------------------------------------------ shape cross-check

def test_parameter_count_matches_pages():
    """Three H x I matrices per routed and shared expert reproduce the pages'
    ~196B total / ~11B active (sglang-jax issue, Model configuration; the
    inference-research record's 196.81B vendor / 195.8B config arithmetic)."""
    H, V, L = 4096, 128896, 45
    moe_layers = len(range(3, 45))                       # moe_layers_enum 3..44
    E, k, I, Is, dense_I = 288, 8, 1280, 1280, 11264
    head_dim, kv = 128, 8
    full_layers, sliding_layers = 12, 33                 # 3:1 pattern over 45 layers
    q_full, q_sliding = 64, 96

    def attn(nq):
        return H * nq * head_dim * 2 + 2 * H * kv * head_dim + H * nq  # q,o + k,v + head gate

    attention = full_layers * attn(q_full) + sliding_layers * attn(q_sliding)
    dense = (L - moe_layers) * 3 * H * dense_I
    expert = 3 * H * I
    per_moe = E * expert + 3 * H * Is + E * H + E
    total = 2 * V * H + attention + dense + moe_layers * per_moe
    active = 2 * V * H + attention + dense + moe_layers * (k * expert + 3 * H * Is + E * H)
    assert abs(total / 196e9 - 1) < 0.015
    assert abs(active / 11e9 - 1) < 0.10
    # two matrices per expert instead of three would miss by a third
    assert abs((total - moe_layers * E * H * I) / 196e9 - 1) > 0.25


# ------------------------------------------------------ FP8 (e4m3) weights

def test_e4m3_decode_matches_library_and_named_values():
    """OCP FP8 E4M3 (e4m3fn): every code against torch's float8_e4m3fn, and
    the format's named values."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), codes[~same]
    named = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x3C: 1.5, 0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in named.items():
        assert got[c] == v, hex(c)
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.signbit(got[0x80]) and got[0x80] == 0.0
    assert np.nanmax(np.abs(got)) == 448.0


def test_synth_e4m3_encoder_matches_library():
    """The input generator's encoder (round to nearest even) against torch's
    conversion, over the normal and subnormal ranges."""
    import torch
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 0.01, 20000),
                        rng.uniform(-2 ** -6, 2 ** -6, 20000), [0.0, -0.0, 448.0, -448.0]])
    v = v.astype(np.float32).astype(np.float64)  # values torch sees exactly
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(synth.e4m3_encode(v), ref)


def _fp8_exact_case(seed):
    """Experts whose e4m3-times-scale weights are exactly bf16 weights: random
    codes of magnitude < 2^4 (no subnormals) and power-of-two scales per row."""
    wl = TINY.with_(T=12)
    inp = synth.make_inputs(wl)
    rng = np.random.default_rng(seed)
    E, I, H = wl.E, wl.I, wl.H

    def codes(shape):
        ex = rng.integers(1, 11, size=shape)           # exponent field 1..10: 2^-6 .. 2^3
        man = rng.integers(0, 8, size=shape)
        sign = rng.integers(0, 2, size=shape)
        return ((sign << 7) | (ex << 3) | man).astype(np.uint8)

    def scales(shape):
        return np.ldexp(1.0, rng.integers(-12, -2, size=shape)).astype(np.float32)

    fp8 = synth.Fp8Experts(codes((E, I, H)), scales((E, I)), codes((E, I, H)), scales((E, I)),
                           codes((E, H, I)), scales((E, H)))

    def as_bf16(c, s):
        vals = oracle.e4m3_decode(c) * s[..., None].astype(np.float64)
        return f32_to_bf16_bits(vals.astype(np.float32))

    bf = dict(w_gate=as_bf16(fp8.w8_gate, fp8.s_gate), w_up=as_bf16(fp8.w8_up, fp8.s_up),
              w_down=as_bf16(fp8.w8_down, fp8.s_down))
    # bf16 holds these values exactly (8 significant bits >= e4m3's 4)
    for name, c, s in (("w_gate", fp8.w8_gate, fp8.s_gate), ("w_down", fp8.w8_down, fp8.s_down)):
        assert np.array_equal(bf16_bits_to_f32(bf[name]).astype(np.float64),
                              oracle.e4m3_decode(c) * s[..., None])
    return wl, inp, fp8, bf


def test_fp8_forward_equals_bf16_forward_on_same_weights():
    wl, inp, fp8, bf = _fp8_exact_case(11)
    cfg = oracle.cfg_of(wl)
    ref = oracle.forward(cfg, inp.__class__(**{**inp.__dict__, **bf}))
    got = oracle.forward_fp8(cfg, inp, fp8)
    assert np.array_equal(got["ids"], ref["ids"])
    assert np.array_equal(got["y"], ref["y"])


def test_fp8_row_scale_scales_one_output_unit():
    """Doubling the scale of down row d of every expert doubles the routed
    part of y[:, d] and leaves the other units alone (a scale per output row,
    not per input column)."""
    wl, inp, fp8, _ = _fp8_exact_case(12)
    wl = wl.with_(Is=0)
    inp = inp.__class__(**{**inp.__dict__, "ws_gate": None, "ws_up": None, "ws_down": None})
    cfg = oracle.cfg_of(wl)
    base = oracle.forward_fp8(cfg, inp, fp8)["y"]
    d = 5
    s2 = fp8.s_down.copy()
    s2[:, d] *= 2
    fp8b = synth.Fp8Experts(fp8.w8_gate, fp8.s_gate, fp8.w8_up, fp8.s_up, fp8.w8_down, s2)
    got = oracle.forward_fp8(cfg, inp, fp8b)["y"]
    assert np.array_equal(got[:, d], 2 * base[:, d])
    others = np.arange(wl.H) != d
    assert np.array_equal(got[:, others], base[:, others])
