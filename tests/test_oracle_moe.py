"""Pins of the routing / combine oracle (oracle.moe) against definitions
computed another way: brute-force ranking, scipy's softmax, one-hot and
linearity properties, constructed ties."""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

from oracle import moe
from synthetic import router_logits


def _brute_topk(row, k):
    # rank expert i before j when l_i > l_j, or l_i == l_j and i < j (pairwise definition)
    e = len(row)
    score = [sum(1 for j in range(e) if row[j] > row[i] or (row[j] == row[i] and j < i)) for i in range(e)]
    return [i for _, i in sorted(zip(score, range(e)))][:k]


def test_topk_matches_pairwise_ranking():
    logits = router_logits(3, 40, 12)
    r = moe.route(logits, 4)
    for t in range(40):
        assert r.topk[t].tolist() == _brute_topk(logits[t].tolist(), 4)


def test_ties_go_to_the_lower_expert_id():
    logits = np.array([[1.0, 2.0, 2.0, 0.5, 2.0],
                       [0.0, 0.0, 0.0, 0.0, 0.0],
                       [3.0, -1.0, 3.0, 3.0, -1.0]], dtype=np.float32)
    r = moe.route(logits, 3)
    assert r.topk.tolist() == [[1, 2, 4], [0, 1, 2], [0, 2, 3]]
    np.testing.assert_allclose(r.weights, 1.0 / 3.0, rtol=0, atol=1e-15)


def test_weights_are_the_softmax_over_the_chosen_experts():
    logits = router_logits(4, 30, 9)
    r = moe.route(logits, 3)
    chosen = np.take_along_axis(logits, r.topk, 1).astype(np.float64)
    np.testing.assert_allclose(r.weights, softmax(chosen, axis=1), rtol=1e-13)
    np.testing.assert_allclose(r.weights.sum(1), 1.0, rtol=1e-14)
    assert np.all(np.diff(r.weights, axis=1) <= 0)        # decreasing with the logit order
    # k = E: the full softmax of the row, in logit order
    full = moe.route(logits, 9)
    np.testing.assert_allclose(full.weights, np.take_along_axis(softmax(logits.astype(np.float64), 1), full.topk, 1),
                               rtol=1e-13)


@pytest.mark.parametrize("t,e,k", [(64, 8, 2), (257, 64, 8), (5, 3, 1), (7, 4, 4)])
def test_slot_layout_invariants(t, e, k):
    logits = router_logits(t + e, t, e)
    r = moe.route(logits, k)
    assert r.group_offsets[0] == 0 and r.group_offsets[-1] == t * k
    assert np.all(np.diff(r.group_offsets) >= 0)
    assert np.array_equal(np.bincount(r.a_rows, minlength=t), np.full(t, k))
    assert sorted(r.slot_of.reshape(-1).tolist()) == list(range(t * k))
    for ex in range(e):
        rows = r.a_rows[r.group_offsets[ex]:r.group_offsets[ex + 1]]
        assert np.all(np.diff(rows) > 0)                    # tokens ascending, no repeats
        assert all(ex in r.topk[tok] for tok in rows)
        assert len(rows) == int(np.sum(r.topk == ex))
    for tok, j in itertools.product(range(t), range(k)):
        s = r.slot_of[tok, j]
        assert r.a_rows[s] == tok
        assert r.group_offsets[r.topk[tok, j]] <= s < r.group_offsets[r.topk[tok, j] + 1]


def test_combine_one_hot_and_linearity():
    rng = np.random.default_rng(8)
    logits = router_logits(9, 20, 6)
    r = moe.route(logits, 3)
    y_slots = rng.standard_normal((60, 5))
    # one-hot weights pick the slot row
    for j in range(3):
        w = np.zeros((20, 3))
        w[:, j] = 1.0
        np.testing.assert_array_equal(moe.combine(y_slots, r.slot_of, w), y_slots[r.slot_of[:, j]])
    # linear in the slot outputs and in the weights
    y2 = rng.standard_normal((60, 5))
    np.testing.assert_allclose(moe.combine(2 * y_slots - y2, r.slot_of, r.weights),
                               2 * moe.combine(y_slots, r.slot_of, r.weights) - moe.combine(y2, r.slot_of, r.weights),
                               rtol=1e-12, atol=1e-12)
    # constant slot outputs combine to the constant (weights sum to one)
    np.testing.assert_allclose(moe.combine(np.full((60, 5), 7.0), r.slot_of, r.weights), 7.0, rtol=1e-14)


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        moe.route(np.zeros((3, 4), np.float32), 5)
    with pytest.raises(ValueError):
        moe.route(np.array([[np.nan, 1.0]], np.float32), 1)
