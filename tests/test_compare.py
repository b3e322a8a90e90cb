"""The parity protocol's routing comparison (tests/gpu_util.compare_route)
on hand-made oracle results: every rule it enforces rejects the mistake it
exists for, and accepts what the protocol allows.  CPU only."""
import numpy as np
import pytest

from tests import gpu_util as gu


def _ref(keys, scores, k):
    """What oracle.route returns, computed here from the keys by the rule the
    pages fix (key descending, equal keys -> lower index first)."""
    keys = np.asarray(keys, np.float64)
    scores = np.asarray(scores, np.float64)
    T, E = keys.shape
    ids = np.empty((T, k), np.int32)
    gap = np.empty(T)
    w = np.empty((T, k))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-keys[t, e], e))
        ids[t] = order[:k]
        gap[t] = keys[t, order[k - 1]] - keys[t, order[k]] if k < E else np.inf
        s = scores[t, ids[t]]
        w[t] = 3.0 * s / s.sum()
    return dict(ids=ids, w=w, gap=gap, keys=keys, scores=scores)


WL = None  # compare_route does not read the workload


def _case(keys, k=2):
    scores = np.full_like(np.asarray(keys, np.float64), 0.5)
    return _ref(keys, scores, k)


def test_identical_passes():
    ref = _case([[0.9, 0.1, 0.5, 0.3]])
    rep = gu.compare_route(WL, ref["ids"].copy(), ref["w"].astype(np.float32), ref)
    assert rep.mismatched == [] and rep.order_swaps == 0


def test_exact_tie_order_must_match():
    # experts 1 and 2 tie exactly: the lower index ranks first
    ref = _case([[0.1, 0.7, 0.7, 0.2]])
    assert ref["ids"].tolist() == [[1, 2]]
    w = ref["w"].astype(np.float32)
    gu.compare_route(WL, np.array([[1, 2]], np.int32), w, ref)
    with pytest.raises(AssertionError):
        gu.compare_route(WL, np.array([[2, 1]], np.int32), w, ref)


def test_exact_tie_at_the_cut_is_not_exempt():
    # experts 1 and 3 tie exactly for the last slot: 1 must be chosen
    ref = _case([[0.9, 0.4, 0.1, 0.4]])
    assert ref["gap"][0] == 0.0 and ref["ids"].tolist() == [[0, 1]]
    w = ref["w"].astype(np.float32)
    with pytest.raises(AssertionError):
        gu.compare_route(WL, np.array([[0, 3]], np.int32), w, ref)


def test_near_tie_swap_in_rank_order_allowed():
    ref = _case([[0.5, 0.5 + 3e-6, 0.1, 0.2]])
    rep = gu.compare_route(WL, np.array([[0, 1]], np.int32), ref["w"].astype(np.float32), ref)
    assert rep.order_swaps == 1


def test_near_tie_at_the_cut_allowed_and_counted():
    ref = _case([[0.9, 0.4, 0.1, 0.4 - 2e-6]])
    rep = gu.compare_route(WL, np.array([[0, 3]], np.int32), np.full((1, 2), 1.5, np.float32), ref)
    assert rep.mismatched == [0] and rep.near_tie == [0]


def test_wrong_expert_rejected():
    ref = _case([[0.9, 0.4, 0.1, 0.3]])
    with pytest.raises(AssertionError):
        gu.compare_route(WL, np.array([[0, 3]], np.int32), ref["w"].astype(np.float32), ref)


def test_far_swap_rejected():
    ref = _case([[0.9, 0.4, 0.1, 0.3]])
    with pytest.raises(AssertionError):
        gu.compare_route(WL, np.array([[1, 0]], np.int32), ref["w"][:, ::-1].astype(np.float32),
                         ref)


def test_weight_error_rejected():
    ref = _case([[0.9, 0.4, 0.1, 0.3]])
    w = ref["w"].astype(np.float32)
    w[0, 0] += 2e-5
    with pytest.raises(AssertionError):
        gu.compare_route(WL, ref["ids"].copy(), w, ref)


def test_repeated_expert_rejected():
    ref = _case([[0.9, 0.4, 0.1, 0.4 - 2e-6]], k=2)
    with pytest.raises(AssertionError):
        gu.compare_route(WL, np.array([[1, 1]], np.int32), ref["w"].astype(np.float32), ref)


def test_per_token_rel_err():
    ref = np.array([[1.0, -2.0], [0.01, 0.0]])
    got = np.array([[1.0, -2.02], [0.0101, 0.0]], np.float32)
    assert abs(gu.per_token_rel_err(got, ref) - 0.01) < 1e-6


def test_exact_ties_counted_once_per_token():
    # equal keys inside the set and at the cut: one token
    ref = _case([[0.7, 0.7, 0.7, 0.1]])
    rep = gu.compare_route(WL, ref["ids"].copy(), ref["w"].astype(np.float32), ref)
    assert rep.exact_ties == 1


def test_exact_tie_at_the_cut_with_a_near_neighbour_is_exempt():
    # experts 2 and 3 tie exactly at the cut (top 2: 0 and 2); expert 1 is
    # 1e-8 above them, so fp32 may rank 1 below the tied pair: {0, 2} and
    # {0, 1} are both valid sets
    ref = _case([[0.9, 0.4 + 1e-8, 0.4, 0.4]], k=3)
    assert ref["ids"].tolist() == [[0, 1, 2]] and ref["gap"][0] == 0.0
    rep = gu.compare_route(WL, np.array([[0, 2, 3]], np.int32), np.full((1, 3), 1.0, np.float32),
                           ref)
    assert rep.mismatched == [0] and rep.near_tie == [0]
    # the tied pair itself must still come lower index first
    with pytest.raises(AssertionError):
        gu.compare_route(WL, np.array([[0, 3, 2]], np.int32), np.full((1, 3), 1.0, np.float32),
                         ref)
