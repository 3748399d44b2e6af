"""Exact-order fp32 clustering arithmetic for seal and refit, CPU oracle side.

Test infrastructure.  The pages say keys are grouped by distance (paper-daily
explainer, "代表向量为什么要学？": the method keeps grouping by distance and only
corrects the representative) with size-capped k-means at seal (kurate.org,
"Core Contribution", item 1) and one round of assignment plus update at refit
(paper-daily, "索引怎么边算边建？", item 3).  They give no arithmetic order.  We
fix one so that two implementations can agree bit for bit:

* squared distance D(x, c) = sum over i = 0..d-1 in ascending order of
  (x_i - c_i)^2: t = x_i - c_i rounded to fp32, then acc = t*t + acc rounded
  once to fp32 (a fused multiply-add, round-to-nearest-even), from acc = +0.0;
* mean of a cluster = fp32 running sum of its members in ascending key
  position starting from +0.0, then one IEEE fp32 division by the count.

Seal (our reading of "size-capped"): Lloyd iterations from evenly spaced
keys; the assignment step is the global greedy one that walks all
(distance, key, cluster) triples in ascending order and gives a key to a
cluster when the key is still free and the cluster holds fewer than `cap`
keys.  Empty clusters keep their centroid during the iterations.
"""
from __future__ import annotations

import numpy as np


def fma32(a, b, c) -> np.ndarray:
    """a*b + c for fp32 arrays, rounded once to fp32 (nearest, ties to even), for
    finite results.

    The product of two fp32 values is exact in fp64 (48 significant bits).  Its
    fp64 sum with c is rounded once; the two-sum formulas give that rounding's
    exact error e, so a*b + c = s + e exactly.  Rounding s to fp32 is then the
    correct rounding of a*b + c unless s landed exactly on the midpoint of two
    fp32 neighbours while e != 0 (the fp64 rounding moved a value off one side of
    the midpoint onto it); in that case the side is the sign of e.
    """
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    c = np.asarray(c, dtype=np.float32)
    p = a.astype(np.float64) * b.astype(np.float64)    # exact
    c64 = c.astype(np.float64)
    s = p + c64
    bv = s - p                                         # two-sum: p + c64 = s + e
    e = (p - (s - bv)) + (c64 - bv)
    r = s.astype(np.float32)                           # nearest fp32, ties to even
    r64 = r.astype(np.float64)
    toward = np.where(s > r64, np.float32(np.inf), np.float32(-np.inf))
    other = np.nextafter(r, toward)                    # the fp32 neighbour on s's side
    at_mid = (s != r64) & (s == (r64 + other.astype(np.float64)) * 0.5)
    out = np.where(at_mid & (e > 0), np.maximum(r, other), r)
    out = np.where(at_mid & (e < 0), np.minimum(r, other), out)
    return out.astype(np.float32)


def sqdist_exact(X: np.ndarray, C: np.ndarray) -> np.ndarray:
    """X [n, d] fp32, C [m, d] fp32 -> D [n, m] fp32 in the fixed order above."""
    X = np.asarray(X, dtype=np.float32)
    C = np.asarray(C, dtype=np.float32)
    acc = np.zeros((X.shape[0], C.shape[0]), dtype=np.float32)
    for i in range(X.shape[1]):
        diff = X[:, i:i + 1] - C[None, :, i]      # fp32 subtraction
        acc = fma32(diff, diff, acc)              # diff^2 + acc, one rounding; dimension i after i-1
    return acc


def mean_exact(rows: np.ndarray) -> np.ndarray:
    """Mean of rows [n, d] (already in ascending key position), fp32, fixed order."""
    rows = np.asarray(rows, dtype=np.float32)
    s = np.zeros(rows.shape[1], dtype=np.float32)
    for r in rows:
        s = s + r
    return s / np.float32(rows.shape[0])


def nearest(D: np.ndarray) -> np.ndarray:
    """Index of the smallest entry per row; the lowest index wins a tie."""
    return np.argmin(D, axis=1)


def capped_greedy_assign(D: np.ndarray, cap: int) -> np.ndarray:
    """Assign each key (row) to one cluster (column), at most `cap` per cluster.

    Walk the triples (D[j, c], j, c) in ascending order; key j goes to cluster c
    if j is still unassigned and c holds fewer than cap keys.  Requires
    cap * n_clusters >= n_keys, which guarantees every key is placed.
    """
    n, m = D.shape
    if cap * m < n:
        raise ValueError("cap too small to place every key")
    flat = D.reshape(-1)
    key_of = np.repeat(np.arange(n), m)
    cl_of = np.tile(np.arange(m), n)
    order = np.lexsort((cl_of, key_of, flat))      # by D, then key, then cluster
    assign = np.full(n, -1, dtype=np.int64)
    count = np.zeros(m, dtype=np.int64)
    placed = 0
    for t in order:
        j = key_of[t]
        c = cl_of[t]
        if assign[j] < 0 and count[c] < cap:
            assign[j] = c
            count[c] += 1
            placed += 1
            if placed == n:
                break
    return assign


def seal_blocks(X: np.ndarray, n_clusters: int):
    """Positional clusters of one window (the block-routing baseline): cluster i is
    the contiguous block of keys [i*b, (i+1)*b), b = W / n_clusters, and its
    centroid is the exact-order mean of the block.

    This is the position-block grouping of the comparison method the pages call
    HiSA (paper-daily explainer, "它到底在解决什么问题？": keys cut into contiguous
    blocks by position, each block represented by its mean, blocks ranked by the
    representative's score); AttentionIndex replaces the blocks by content clusters.
    Returns (assign [W] int64, centroids [n_clusters, d] fp32, alive [n_clusters] bool).
    """
    X = np.asarray(X, dtype=np.float32)
    W = X.shape[0]
    if W % n_clusters:
        raise ValueError("window must split into equal blocks")
    b = W // n_clusters
    assign = np.arange(W) // b
    C = np.stack([mean_exact(X[i * b:(i + 1) * b]) for i in range(n_clusters)])
    return assign, C, np.ones(n_clusters, dtype=bool)


def seal_window(X: np.ndarray, n_clusters: int, cap: int, iters: int):
    """Size-capped k-means on one window of keys X [W, d] (ascending position).

    Initial centroids are the keys at offsets floor((2i+1) W / (2 n_clusters)).
    Each of `iters` iterations computes D, the capped greedy assignment, and
    the exact-order mean of every non-empty cluster.
    Returns (assign [W] int64, centroids [n_clusters, d] fp32, alive [n_clusters] bool).
    The returned centroids are the means of the returned assignment.
    """
    if iters < 1:
        raise ValueError("seal needs at least one iteration")
    X = np.asarray(X, dtype=np.float32)
    W = X.shape[0]
    init = [((2 * i + 1) * W) // (2 * n_clusters) for i in range(n_clusters)]
    C = X[init].copy()
    for _ in range(iters):
        D = sqdist_exact(X, C)
        assign = capped_greedy_assign(D, cap)
        for c in range(n_clusters):
            idx = np.nonzero(assign == c)[0]
            if idx.size:
                C[c] = mean_exact(X[idx])
    alive = np.array([np.any(assign == c) for c in range(n_clusters)])
    return assign, C, alive
