"""The near-tie check of the GPU parity helpers, on the CPU: a GPU selection
that differs from the oracle's on an exempt token passes only when it is a
valid resolution of the near-tie under the oracle's float64 scores.  The
"GPU" results here are built by hand from the oracle's own."""
import numpy as np
import pytest

import oracle
from parity import check_near_tie, compare_gate


@pytest.fixture(scope="module")
def o():
    return oracle.load()


def _weights(s, ids, scale):
    ss = s[ids]
    return (scale * ss / ss.sum()).astype(np.float32)


def _one_group_case(o, gap):
    """E=16, one group, top-4: the 4th and 5th choice scores differ by gap."""
    rng = np.random.default_rng(1)
    L = rng.standard_normal(16)
    b = np.zeros(16, np.float32)
    order = np.argsort(-L)
    L[order[4]] = L[order[3]] - gap          # 4th and 5th logits a gap apart
    r = o.select(L[None, :], b, 1, 1, 4, 2.5, with_scores=True)
    return r, order


def test_single_group_swap_at_the_boundary_is_valid(o):
    r, order = _one_group_case(o, 1e-9)
    assert r.margins[0, 0] < 1e-6
    ids = np.sort(np.r_[order[:3], order[4]]).astype(np.int32)      # 5th instead of 4th
    sc = r.scores
    w = _weights(sc.affinity[0], ids, 2.5)
    check_near_tie(ids, w, sc.affinity[0], sc.choice[0], None, 1, 2.5)
    st = compare_gate(w[None, :], ids[None, :], r, 2.5)
    assert st["exempt"] == 1 and st["exempt_differ_valid"] == 1


def test_single_group_far_loser_is_rejected(o):
    r, order = _one_group_case(o, 1e-9)
    ids = np.sort(np.r_[order[:3], order[6]]).astype(np.int32)      # 7th: far below
    sc = r.scores
    w = _weights(sc.affinity[0], ids, 2.5)
    with pytest.raises(AssertionError, match="not a valid resolution"):
        check_near_tie(ids, w, sc.affinity[0], sc.choice[0], None, 1, 2.5)
    with pytest.raises(AssertionError):
        compare_gate(w[None, :], ids[None, :], r, 2.5)


def test_wrong_weights_on_a_valid_set_are_rejected(o):
    r, order = _one_group_case(o, 1e-9)
    ids = np.sort(np.r_[order[:3], order[4]]).astype(np.int32)
    sc = r.scores
    w = _weights(sc.affinity[0], ids, 2.5)
    w[0] *= 1.001
    with pytest.raises(AssertionError, match="weights off"):
        check_near_tie(ids, w, sc.affinity[0], sc.choice[0], None, 1, 2.5)


def test_exempt_difference_without_scores_fails(o):
    r, order = _one_group_case(o, 1e-9)
    ids = np.sort(np.r_[order[:3], order[4]]).astype(np.int32)
    w = _weights(r.scores.affinity[0], ids, 2.5)
    bare = oracle.GateResult(r.weights, r.indices, r.margins)
    with pytest.raises(AssertionError, match="needs the oracle's scores"):
        compare_gate(w[None, :], ids[None, :], bare, 2.5)


def _group_case(o, group_gap):
    """E=32 in 4 groups of 8, keep 2, top-4: groups 1 and 2 tie within
    group_gap at the keep boundary; group 0 is clearly kept, group 3 clearly
    dropped."""
    E, G, S = 32, 4, 8
    v = np.full(E, 0.1)
    v[0:2] = [0.9, 0.85]                              # group 0: best (two high)
    v[8:16] = np.linspace(0.5, 0.45, 8)               # group 1
    v[16:24] = np.linspace(0.5, 0.45, 8)              # group 2: equal to group 1...
    v[16] -= group_gap                                # ...but for the gap
    v[24:32] = np.linspace(0.2, 0.1, 8)               # group 3: clearly dropped
    L = np.log(v / (1.0 - v))                         # sigmoid(L) = v, no bias
    b = np.zeros(E, np.float32)
    return o.select(L[None, :], b, G, 2, 4, 1.0, with_scores=True)


def test_group_boundary_swap_is_valid(o):
    r = _group_case(o, 1e-9)
    assert r.margins[0, 1] < 1e-6
    assert set(r.indices[0] // 8) == {0, 1}
    sc = r.scores
    # the other resolution keeps group 2: its two best with group 0's two best
    ids = np.array([0, 1, 16, 17], np.int32)
    w = _weights(sc.affinity[0], ids, 1.0)
    check_near_tie(ids, w, sc.affinity[0], sc.choice[0], sc.group[0], 2, 1.0)
    st = compare_gate(w[None, :], ids[None, :], r, 1.0, topk_group=2)
    assert st["exempt_differ_valid"] == 1


def test_group_boundary_with_a_clear_gap_is_rejected(o):
    r = _group_case(o, 1e-3)
    sc = r.scores
    ids = np.array([0, 1, 16, 17], np.int32)          # keeps the worse group
    w = _weights(sc.affinity[0], ids, 1.0)
    with pytest.raises(AssertionError, match="not a valid resolution"):
        check_near_tie(ids, w, sc.affinity[0], sc.choice[0], sc.group[0], 2, 1.0)


def test_winner_from_a_dropped_group_is_rejected(o):
    r = _group_case(o, 1e-9)
    sc = r.scores
    ids = np.array([0, 1, 8, 24], np.int32)           # group 3 was clearly dropped
    w = _weights(sc.affinity[0], ids, 1.0)
    with pytest.raises(AssertionError, match="not a valid resolution"):
        check_near_tie(ids, w, sc.affinity[0], sc.choice[0], sc.group[0], 2, 1.0)
