"""The seeded input generator: determinism, independence of slices and streams,
and the distributions the workload recipes ask for."""
import math

import numpy as np
from scipy import stats

import synth


def test_deterministic_and_sliceable():
    a = synth.normal_f32(0, 4, 200_000, 1.0)
    b = synth.normal_f32(0, 4, 200_000, 1.0)
    assert np.array_equal(a, b)
    # element i depends only on (seed, tensor, i): a shorter draw is a prefix
    c = synth.normal_f32(0, 4, 1000, 1.0)
    assert np.array_equal(a[:1000], c)
    # threads do not change the bytes (large draw is split over workers)
    w = synth.words(0, 4, 10)
    assert len(set(w.tolist())) == 10


def test_streams_and_seeds_differ():
    a = synth.normal_f32(0, 1, 1000, 1.0)
    b = synth.normal_f32(0, 2, 1000, 1.0)
    c = synth.normal_f32(1, 1, 1000, 1.0)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.1


def test_splitmix64_is_a_counter_stream():
    # word(i) of a stream equals the (i+1)-th SplitMix64 step from the stream base:
    # consecutive outputs of the stepping generator must match the counter form.
    seq = synth.splitmix64_sequence(12345, 5)
    assert len(set(seq)) == 5 and all(0 <= v < 2**64 for v in seq)
    seq2 = synth.splitmix64_sequence(12345, 6)
    assert seq2[:5] == seq


def test_normal_distribution():
    v = synth.normal_f32(0, 9, 400_000, 0.25).astype(np.float64)
    assert abs(v.mean()) < 0.003
    assert abs(v.std() - 0.25) < 0.002
    assert stats.kstest(v / 0.25, "norm").pvalue > 1e-3


def test_bf16_rounding_is_nearest_even():
    bits = synth.normal_bf16(0, 5, 100_000, 1.0)
    f = synth.normal_f32(0, 5, 100_000, 1.0)
    back = synth.bf16_to_f32(bits)
    err = np.abs(back.astype(np.float64) - f.astype(np.float64))
    ulp = np.abs(f).astype(np.float64) * 2.0 ** -8
    assert np.all(err <= ulp * 1.0001)
    # same bits as numpy's own round-to-nearest-even on the upper half
    u = f.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(bits, rne)


def test_uniform_and_choose():
    u = synth.uniform_f32(0, 11, 100_000, 0.5, 2.0)
    assert u.min() >= 0.5 and u.max() <= 2.0
    assert abs(u.mean() - 1.25) < 0.01
    hot = synth.choose(0, 10, 288, 16)
    assert len(set(hot.tolist())) == 16 and hot.min() >= 0 and hot.max() < 288
    assert np.array_equal(hot, synth.choose(0, 10, 288, 16))


def test_workload_recipes():
    wl = synth.WORKLOADS["tiny"]
    inp = synth.make_inputs(wl)
    assert inp.x.shape == (16, 256) and inp.x.dtype == np.uint16
    assert inp.router_w.shape == (16, 256) and inp.router_w.dtype == np.float32
    assert inp.w_gate.shape == (16, 64, 256) and inp.w_down.shape == (16, 256, 64)
    assert inp.ws_gate.shape == (64, 256) and inp.ws_down.shape == (256, 64)
    # N(0, v) is read as variance v: router weight std = 1/sqrt(H)
    assert abs(inp.router_w.std() - 1 / math.sqrt(256)) < 0.002
    wd = synth.bf16_to_f32(inp.w_down).astype(np.float64)
    assert abs(wd.std() - 1 / math.sqrt(64)) < 0.003

    sk = synth.WORKLOADS["skewed"].with_(T=4, H=256, I=64, Is=64)
    wg, b, hot = synth.gen_router(sk)
    assert hot.size == 16 and np.all(b[hot] == 2.0)
    assert np.all(np.abs(np.delete(b, hot)) < 2.0)

    lg = synth.WORKLOADS["long"].with_(T=64, H=512)
    x = synth.bf16_to_f32(synth.gen_x(lg)).astype(np.float64)
    rs = x.std(1)
    assert rs.min() > 0.35 and rs.max() < 2.4
