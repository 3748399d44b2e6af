"""Pins for the oracle's indexer score and exhaustive top-k.

* The worked example of the paper-daily.com explainer ("代表向量为什么要学？"
  widget), stored in tests/golden/worked_example.json with its citation.
* Brute force with plain Python floats (math.fsum) on tiny inputs, which
  catches a transposed operand or a wrong reduction axis in the vectorised
  code.
* Special cases that reduce to a library routine: one head with weight 1 and
  no clipping is numpy's inner product; with no clipping the score is linear
  in the key, so a mean key scores the mean of its members (the identity the
  page contrasts the ReLU score with).
"""
import json
import math
import os

import numpy as np

from oracle.index import exhaustive_topk, topk_sorted
from oracle.score import indexer_scores, score_error_scale

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _worked():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        return json.load(f)


def test_worked_example_scalar():
    g = _worked()
    q = np.array([[[g["query"]]]])                      # T=1, H=1, d=1
    w = np.array([[g["head_weight"]]])
    members = np.array(g["members"])[:, None]
    mean = members.mean(axis=0, keepdims=True)
    assert mean[0, 0] == g["rep_is_mean"]
    assert indexer_scores(q, w, mean)[0, 0] == g["rep_score"]
    s = indexer_scores(q, w, members)[0]
    assert s.tolist() == g["member_scores"]
    assert s.mean() == g["mean_of_member_scores"]
    assert members[np.argmax(s), 0] == g["member_that_should_be_selected"]


def test_worked_example_embedded_in_dsa_shape():
    """Same numbers with H=4 heads, d=32, weights (1, 0, 0, 0); the other heads
    carry arbitrary vectors but zero weight."""
    g = _worked()
    rng = np.random.default_rng(3)
    d, H = 32, 4
    q = rng.standard_normal((1, H, d))
    q[0, 0] = 0.0
    q[0, 0, 5] = g["query"]
    w = np.array([[g["head_weight"], 0.0, 0.0, 0.0]])
    members = np.zeros((2, d))
    members[:, 5] = g["members"]
    members[:, 9] = rng.standard_normal(2)              # orthogonal to head 0's query
    mean = members.mean(axis=0, keepdims=True)
    s_rep = indexer_scores(q, w, np.where(np.arange(d) == 5, mean, 0.0))[0, 0]
    assert s_rep == g["rep_score"]
    s = indexer_scores(q, w, members)[0]
    assert s.tolist() == g["member_scores"]


def test_scores_match_python_brute_force():
    rng = np.random.default_rng(4)
    T, H, d, N = 3, 5, 7, 11
    q = rng.standard_normal((T, H, d))
    w = rng.standard_normal((T, H))
    k = rng.standard_normal((N, d))
    s = indexer_scores(q, w, k)
    for t in range(T):
        for j in range(N):
            terms = []
            for h in range(H):
                dot = math.fsum(float(q[t, h, i]) * float(k[j, i]) for i in range(d))
                terms.append(float(w[t, h]) * max(0.0, dot))
            assert abs(s[t, j] - math.fsum(terms)) <= 1e-12 * (1 + abs(s[t, j]))


def test_single_head_without_clipping_is_inner_product():
    rng = np.random.default_rng(5)
    q = np.abs(rng.standard_normal((1, 1, 16)))
    k = np.abs(rng.standard_normal((9, 16)))
    s = indexer_scores(q, np.ones((1, 1)), k)[0]
    assert np.allclose(s, k @ q[0, 0], rtol=1e-14, atol=0)


def test_mean_key_scores_mean_when_nothing_clips():
    rng = np.random.default_rng(6)
    H, d = 8, 32
    q = np.abs(rng.standard_normal((1, H, d)))
    w = rng.standard_normal((1, H))
    members = np.abs(rng.standard_normal((10, d)))      # all q_h . k >= 0
    s_mean = indexer_scores(q, w, members.mean(0, keepdims=True))[0, 0]
    assert np.isclose(s_mean, indexer_scores(q, w, members)[0].mean(), rtol=1e-12, atol=1e-12)


def test_error_scale_bounds_score():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((4, 6, 16))
    w = rng.standard_normal((4, 6))
    k = rng.standard_normal((20, 16))
    assert np.all(score_error_scale(q, w, k) >= np.abs(indexer_scores(q, w, k)) - 1e-12)


def _brute_topk(scores, n, k):
    order = sorted(range(n), key=lambda j: (-scores[j], j))[:k]
    return order + [-1] * (k - len(order))


def test_exhaustive_topk_matches_brute_force_with_ties_and_padding():
    rng = np.random.default_rng(8)
    T, H, d, N, k = 12, 3, 4, 40, 7
    # small integers make exact score ties common
    q = rng.integers(-2, 3, (T, H, d)).astype(np.float64)
    w = rng.integers(-1, 3, (T, H)).astype(np.float64)
    kv = rng.integers(-2, 3, (N, d)).astype(np.float64)
    q_pos0 = 0                                           # first queries have n < k
    idx, sc = exhaustive_topk(kv, q, w, q_pos0, k)
    full = indexer_scores(q, w, kv)
    for t in range(T):
        n = q_pos0 + t + 1
        ref = _brute_topk(full[t].tolist(), n, k)
        assert idx[t].tolist() == ref
        for j, s in zip(ref, sc[t]):
            assert (s == -np.inf) if j < 0 else (s == full[t, j])


def test_topk_sorted_order():
    cand = np.array([9, 3, 5, 1, 7])
    s = np.array([1.0, 2.0, 2.0, -1.0, 2.0])
    idx, sc = topk_sorted(cand, s, 4)
    assert idx.tolist() == [3, 5, 7, 9]
    assert sc.tolist() == [2.0, 2.0, 2.0, 1.0]
    idx, sc = topk_sorted(cand, s, 7)
    assert idx.tolist() == [3, 5, 7, 9, 1, -1, -1]
    assert sc[-1] == -np.inf
