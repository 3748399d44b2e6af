"""Pins for the refit's starting centroids and for the cluster count, independent of
OracleIndex.warm_start.

What fixes each check (paper-daily.com explainer of AttentionIndex):
* "索引怎么边算边建？" item 3: a refit does not start from scratch; it starts from
  the previous refit's cluster centres and adds a few new centres taken from the
  most recent keys, then runs one assignment round and one update round.  Our
  reading: the new centres are the centroids of the windows sealed since the
  previous refit (keys [B_{r-1}, B_r), B_r = S + r*R), i.e. each is the mean of
  one seal cluster whose members all lie in that range.
* "查询时怎么挑候选？": with about 128 keys per cluster, the number of clusters is
  about one over a hundred and some of the prefix length.

The start set is assembled here from those rules alone (window ranges from the
boundary formula, centres as float64 means of the seal members), the assignment
is recomputed by float64 brute force, and the updated centres by float64 means.
An oracle that dropped the seal centres of later refits, took the windows of
the wrong range, or carried dead clusters would fail here.
"""
import numpy as np
import pytest
from scipy.spatial.distance import cdist

import datagen
from datagen.workloads import WORKLOADS
from oracle import OracleConfig, OracleIndex


def _index(name, refit_every=None, n_keys=None):
    wl = dict(WORKLOADS[name])
    if refit_every is not None:
        wl["refit_every"] = refit_every
    N = wl["N"] if n_keys is None else n_keys
    inp = datagen.workload_inputs(wl["seed"], wl["N"], wl["T"], wl["q_pos0"], wl["H"], wl["d"], wl["M"],
                                  wl["dtype"])
    cfg = OracleConfig(heads=wl["H"], dim=wl["d"], dtype=wl["dtype"], n_sink=wl["n_sink"], window=wl["window"],
                       cluster_size=wl["cluster_size"], seal_cap=wl["seal_cap"], seal_iters=wl["seal_iters"],
                       refit_every=wl["refit_every"])
    ix = OracleIndex(cfg)
    ix.append(inp["keys"][:N], None if inp["k_scale"] is None else inp["k_scale"][:N])
    while ix.refit_due():
        ix.refit()
        ix.publish()
    return ix


def _start_set(ix, r):
    """(slots, float64 centres) refit r starts from, built from the rules in the
    module docstring without the oracle's warm_start."""
    cfg = ix.cfg
    S, W, R, Cs = cfg.n_sink, cfg.window, cfg.refit_every, cfg.n_clusters
    b_prev, b_r = S + (r - 1) * R, S + r * R
    slots, cents = [], []
    if r >= 2:
        for c in ix.epochs[r - 1]:                       # previous centres, live ones only
            if c.members.size:
                slots.append(c.slot)
                cents.append(c.centroid.astype(np.float64))
    # windows whose keys are exactly the keys added since the previous refit
    w_lo, w_hi = (b_prev - S) // W, (b_r - S) // W
    assert S + w_lo * W == b_prev and S + w_hi * W == b_r
    for w in range(w_lo, w_hi):
        for i, c in enumerate(ix.seals[w]):
            if not c.members.size:
                continue
            assert c.slot == w * Cs + i
            assert c.members.min() >= b_prev and c.members.max() < b_r, "a new centre from outside the new keys"
            mean64 = ix.X[c.members].astype(np.float64).mean(axis=0)
            assert np.allclose(c.centroid, mean64, rtol=0, atol=1e-5), "a new centre is not its members' mean"
            slots.append(c.slot)
            cents.append(mean64)
    return np.array(slots), np.stack(cents)


@pytest.fixture(scope="module", params=[("c1r", None), ("c1r", 1024), ("c1", 1024)])
def refitted(request):
    name, R = request.param
    return _index(name, refit_every=R)


def test_refit_starts_from_previous_centres_plus_new_seal_centres(refitted):
    ix = refitted
    cfg = ix.cfg
    S = cfg.n_sink
    assert ix.computed >= 2, "the case must cover a refit after the first"
    for r in range(1, ix.computed + 1):
        slots, C = _start_set(ix, r)
        b_r = S + r * cfg.refit_every
        X = ix.X[S:b_r].astype(np.float64)
        D = cdist(X, C, "sqeuclidean")
        part = np.partition(D, 1, axis=1) if C.shape[0] > 1 else np.concatenate([D, D + 1], axis=1)
        clear = part[:, 1] - part[:, 0] > 1e-5 * (part[:, 1] + 1e-12)
        want = slots[np.argmin(D, axis=1)]
        owner = np.full(b_r, -1)
        for c in ix.epochs[r]:
            owner[c.members] = c.slot
        got = owner[S:]
        assert np.all(got >= 0), f"refit {r}: a covered key has no cluster"
        assert clear.mean() > 0.99
        assert np.array_equal(got[clear], want[clear]), f"refit {r}: assignment is not the nearest start centre"
        # update: every live cluster's centre is the mean of its members
        for c in ix.epochs[r]:
            if c.members.size:
                m64 = ix.X[c.members].astype(np.float64).mean(axis=0)
                assert np.allclose(c.centroid, m64, rtol=0, atol=1e-5), f"refit {r}: slot {c.slot} centre"
        # the epoch's slots are exactly the start slots; no other slot is live
        live = sorted(c.slot for c in ix.epochs[r] if c.members.size)
        assert set(live) <= set(slots.tolist())
        assert len(ix.epochs[r]) == r * cfg.slots_per_refit


def test_cluster_count_is_about_prefix_over_cluster_size(refitted):
    """About 128 keys per cluster: the live clusters of each epoch number between
    1/200 and 1/100 of the covered prefix (a hundred and some keys each)."""
    ix = refitted
    cfg = ix.cfg
    for r in range(1, ix.computed + 1):
        covered = r * cfg.refit_every
        n_live = sum(1 for c in ix.epochs[r] if c.members.size)
        per = covered / n_live
        assert 100 <= per <= 200, f"refit {r}: {n_live} live clusters for {covered} keys ({per:.1f} per cluster)"
        assert n_live >= 0.9 * covered / cfg.cluster_size


def test_planted_mistakes_fail_the_start_pin():
    """The pin above rejects the two plausible slips named in its docstring: a
    warm start without the newest seal centres, and one from the wrong windows."""
    ix = _index("c1r", refit_every=1024)
    r = ix.computed
    slots, C = _start_set(ix, r)
    cfg = ix.cfg
    S, W, Cs = cfg.n_sink, cfg.window, cfg.n_clusters
    b_r = S + r * cfg.refit_every
    X = ix.X[S:b_r].astype(np.float64)
    good = slots[np.argmin(cdist(X, C, "sqeuclidean"), axis=1)]
    # slip 1: drop the seal centres of the new windows
    keep = slots < (r - 1) * cfg.slots_per_refit
    bad1 = slots[keep][np.argmin(cdist(X, C[keep], "sqeuclidean"), axis=1)]
    assert np.mean(bad1 != good) > 0.05
    # slip 2: new centres from the window one before the right one
    w_wrong = (S + (r - 1) * cfg.refit_every - S) // W - 1
    wrong = np.stack([c.centroid.astype(np.float64) for c in ix.seals[w_wrong] if c.members.size])
    C2 = np.concatenate([C[keep], wrong])
    s2 = np.concatenate([slots[keep], np.arange(wrong.shape[0]) + 10 ** 6])
    bad2 = s2[np.argmin(cdist(X, C2, "sqeuclidean"), axis=1)]
    assert np.mean(bad2 != good) > 0.05
    # and the oracle's own epoch agrees with the right start
    owner = np.full(b_r, -1)
    for c in ix.epochs[r]:
        owner[c.members] = c.slot
    assert np.mean(owner[S:] == good) > 0.99
