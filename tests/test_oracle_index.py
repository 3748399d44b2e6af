"""Pins for the oracle's index: budget fill, versions, refit, routing invariants.

What fixes each check (paper-daily.com explainer of AttentionIndex unless noted):
* "核心想法" + "查询时怎么挑候选？": the fine stage scores candidates exactly, so
  every error comes from the coarse stage; a budget that holds the whole
  prefix reproduces the exhaustive top-k exactly (recall 1.0).
* "索引怎么边算边建？" item 2: before the first seal queries score exhaustively.
* same section, last paragraph: a query uses a version only when its prefix
  holds every key of that version (causality audit).
* "查询时怎么挑候选？": each query scores about (#clusters + budget) keys; the
  candidate count is min(prefix, max(budget, sinks + open window)).
* The refit assignment is the nearest centroid: checked against scipy's
  float64 distances wherever the two nearest differ by more than the fp32
  error bound.
* The worked example (tests/golden/worked_example.json) run through a real
  index: a cluster whose mean scores 0 hides a member that scores 2.
"""
import json
import os

import numpy as np
import pytest
from scipy.spatial.distance import cdist

import datagen
from datagen.workloads import WORKLOADS
from oracle import OracleConfig, OracleIndex, fill_budget
from oracle.index import Cluster, make_cluster
from oracle.kmeans import mean_exact
from oracle.recall import recall_per_query

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _build(name, n_keys=None, publish=True, **over):
    wl = dict(WORKLOADS[name], **over)
    N = wl["N"] if n_keys is None else n_keys
    inp = datagen.workload_inputs(wl["seed"], wl["N"], wl["T"], wl["q_pos0"], wl["H"], wl["d"], wl["M"],
                                  wl["dtype"])
    cfg = OracleConfig(heads=wl["H"], dim=wl["d"], dtype=wl["dtype"], n_sink=wl["n_sink"], window=wl["window"],
                       cluster_size=wl["cluster_size"], seal_cap=wl["seal_cap"], seal_iters=wl["seal_iters"],
                       refit_every=wl["refit_every"])
    ix = OracleIndex(cfg)
    ix.append(inp["keys"][:N], None if inp["k_scale"] is None else inp["k_scale"][:N])
    while publish and ix.refit_due():
        ix.refit()
        ix.publish()
    return wl, inp, ix


@pytest.fixture(scope="module")
def c1r():
    return _build("c1r")


def test_structural_constants_from_the_pages():
    with open(os.path.join(GOLDEN, "structural_constants.json")) as f:
        g = json.load(f)
    cfg = OracleConfig(heads=64, dim=128, dtype="bf16", window=g["window"], cluster_size=g["cluster_size"],
                       refit_every=g["refit_every"])
    assert cfg.n_clusters == g["clusters_per_seal"]
    assert cfg.windows_per_refit == g["refit_every"] // g["window"]
    assert WORKLOADS["c4"]["k"] == g["k"] and WORKLOADS["c2"]["window"] == g["window"]


def test_fill_budget_order_and_truncation():
    mk = lambda slot, mem: Cluster(slot, np.array(mem), None, None, 1.0, None)
    base = np.array([0, 1, 20, 21])
    ranked = [mk(5, [7, 9, 11]), mk(2, [3, 4]), mk(9, [12, 13, 14, 15])]
    cand, used = fill_budget(base, ranked, 10)
    assert cand.tolist() == [0, 1, 20, 21, 7, 9, 11, 3, 4, 12]
    assert used == [(5, 3), (2, 2), (9, 1)]
    cand, used = fill_budget(base, ranked, 3)           # sinks + open exceed the budget
    assert cand.tolist() == [0, 1, 20, 21] and used == []
    cand, used = fill_budget(base, ranked, 100)         # everything fits
    assert len(cand) == 4 + 9 and used[-1] == (9, 4)


def test_budget_covering_prefix_reproduces_exhaustive(c1r):
    wl, inp, ix = c1r
    idx, sc = ix.route(inp["q"], inp["q_scale"], inp["w"], wl["q_pos0"], wl["k"], budget=wl["N"])
    eidx, esc = ix.exhaustive(inp["q"], inp["q_scale"], inp["w"], wl["q_pos0"], wl["k"])
    assert np.array_equal(idx, eidx) and np.array_equal(sc, esc)
    assert np.all(recall_per_query(idx, eidx) == 1.0)


def test_before_first_seal_routing_is_exhaustive():
    wl, inp, ix = _build("c1", n_keys=1000)                # S + W = 1028 > 1000: nothing sealed
    assert len(ix.seals) == 0
    q = inp["q"][:200]
    idx, sc = ix.route(q, inp["q_scale"], inp["w"][:200], 800, wl["k"], budget=64)
    eidx, esc = ix.exhaustive(q, inp["q_scale"], inp["w"][:200], 800, wl["k"])
    assert np.array_equal(idx, eidx) and np.array_equal(sc, esc)


def test_counts_and_causality_of_every_query(c1r):
    wl, inp, ix = c1r
    cfg = ix.cfg
    _, _, dbg = ix.route(inp["q"], inp["q_scale"], inp["w"], wl["q_pos0"], wl["k"], wl["budget"], debug=True)
    for t, d in enumerate(dbg):
        n = wl["q_pos0"] + t + 1
        assert d["n"] == n
        r, m = d["epoch"], d["windows"]
        open_len = n - cfg.n_sink - m * cfg.window
        assert 0 <= open_len < cfg.window
        assert ix.boundary(r) <= cfg.n_sink + m * cfg.window <= n     # version inside the prefix
        assert d["cand"].size == min(n, max(wl["budget"], cfg.n_sink + open_len))
        assert np.all(d["cand"] < n) and np.unique(d["cand"]).size == d["cand"].size
        for c in ix.visible(n):
            assert c.members.max() < n
        # scored count ~ clusters + budget
        assert len(d["slots"]) + d["cand"].size <= len(ix.visible(n)) + max(wl["budget"], n)


def test_unpublished_epoch_is_not_used():
    wl, inp, ix = _build("c1r", publish=False)
    ix.refit()                                            # computed, not published
    assert ix.computed == 1 and ix.published == 0
    n = wl["N"]
    r, m = ix.version_of(n)
    assert r == 0 and m == len(ix.seals)
    ix.publish()
    assert ix.version_of(n)[0] == 1
    # a query whose prefix stops before the epoch boundary keeps seal clusters
    assert ix.version_of(ix.boundary(1) - 1)[0] == 0


def test_refit_assignment_is_nearest_centroid(c1r):
    _, _, ix = c1r
    cfg = ix.cfg
    for r in range(1, ix.computed + 1):
        warm = [c for c in ix.warm_start(r) if c.alive]
        lo, hi = cfg.n_sink, ix.boundary(r)
        X = ix.X[lo:hi].astype(np.float64)
        C = np.stack([c.centroid for c in warm]).astype(np.float64)
        D = cdist(X, C, "sqeuclidean")
        part = np.partition(D, 1, axis=1)
        clear = part[:, 1] - part[:, 0] > 1e-5 * part[:, 1]
        ref = np.array([warm[i].slot for i in np.argmin(D, axis=1)])
        owner = np.full(hi, -1)
        for c in ix.epochs[r]:
            owner[c.members] = c.slot
        assert np.all(owner[lo:] >= 0)                     # every sealed key placed once
        assert np.array_equal(owner[lo:][clear], ref[clear])
        for c in ix.epochs[r]:
            if c.alive:
                assert np.array_equal(c.centroid, mean_exact(ix.X[c.members]))
                assert np.all(np.diff(c.members) > 0)
        dead_warm = {c.slot for c in ix.warm_start(r) if not c.alive}
        assert all(not c.alive for c in ix.epochs[r] if c.slot in dead_warm)


def test_seal_clusters_partition_each_window(c1r):
    _, _, ix = c1r
    cfg = ix.cfg
    for w, clusters in enumerate(ix.seals):
        lo = cfg.n_sink + w * cfg.window
        allm = np.sort(np.concatenate([c.members for c in clusters]))
        assert np.array_equal(allm, np.arange(lo, lo + cfg.window))
        assert max(c.members.size for c in clusters) <= cfg.seal_cap
        assert [c.slot for c in clusters] == list(range(w * cfg.n_clusters, (w + 1) * cfg.n_clusters))


def test_worked_example_through_the_index():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    d = 32
    cfg = OracleConfig(heads=1, dim=d, dtype="f32", n_sink=0, window=2, cluster_size=2, seal_cap=2,
                       seal_iters=1, refit_every=0)
    ix = OracleIndex(cfg)
    keys = np.zeros((4, d), np.float32)
    keys[0:2, 5] = g["members"]                          # cluster A: mean 0
    keys[2:4, 5] = 0.5                                   # cluster B: mean 0.5
    ix.append(keys)
    assert ix.seals[0][0].centroid[5] == g["rep_is_mean"]
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 5] = g["query"]
    w = np.full((1, 1), g["head_weight"], np.float32)
    idx, sc, dbg = ix.route(q, None, w, 3, 1, budget=2, debug=True)
    assert dbg[0]["srep"].tolist() == [g["rep_score"], 0.5]
    assert dbg[0]["used"] == [(1, 2)]                    # the mean hides the key scoring 2
    eidx, esc = ix.exhaustive(q, None, w, 3, 1)
    assert esc[0, 0] == max(g["member_scores"]) and keys[eidx[0, 0], 5] == g["member_that_should_be_selected"]
    assert recall_per_query(idx, eidx)[0] == 0.0
    idx, sc = ix.route(q, None, w, 3, 1, budget=4)
    assert np.array_equal(idx, eidx)


def test_rep_quantisation_is_stored_with_cluster():
    c = make_cluster(3, np.array([1, 2]), np.float32([1.0, -2.0, 0.5]), "e4m3")
    assert c.rep_scale == np.float32(np.float32(2.0) / np.float32(448.0))
    assert np.allclose(c.rep_value, [1.0, -2.0, 0.5], rtol=2 ** -4)


def test_positional_index_routes_whole_blocks():
    """Block routing: clusters are the windows' contiguous 128-key blocks; with a budget of
    sinks + open window + two blocks, the candidates are exactly the two blocks whose mean
    representative scores highest, in rank order."""
    from oracle import OracleConfig, OracleIndex
    from oracle.index import query_values
    from oracle.score import indexer_scores
    import datagen
    inp = datagen.workload_inputs(7, 4096, 1, 4095, 2, 32, 16, "f32")
    cfg = OracleConfig(heads=2, dim=32, dtype="f32", n_sink=4, window=1024, cluster_size=128, refit_every=0,
                       positional=True)
    ix = OracleIndex(cfg)
    ix.append(inp["keys"], None)
    assert len(ix.seals) == 3
    for w, clusters in enumerate(ix.seals):
        for i, c in enumerate(clusters):
            lo = 4 + w * 1024 + i * 128
            assert np.array_equal(c.members, np.arange(lo, lo + 128))
    n = 4096
    open_len = n - (4 + 3 * 1024)
    budget = 4 + open_len + 256
    idx, sc, dbg = ix.route(inp["q"], None, inp["w"], 4095, 64, budget, debug=True)
    d = dbg[0]
    qv = query_values(inp["q"], None, "f32")
    reps = np.stack([c.rep_value for w in ix.seals for c in w])
    s = indexer_scores(qv, inp["w"].astype(np.float64), reps)[0]
    top2 = np.argsort(-s, kind="stable")[:2]
    assert [u for u, _ in d["used"]] == top2.tolist()
    blocks = np.concatenate([np.arange(4 + 128 * b, 4 + 128 * (b + 1)) for b in top2])
    assert np.array_equal(d["cand"][4 + open_len:], blocks)
    with pytest.raises(ValueError):
        OracleConfig(heads=2, dim=32, dtype="f32", refit_every=16384, positional=True)


def test_route_at_positions_matches_single_query_routes():
    """A decode batch at scattered positions routes each query exactly as a one-query
    call at that position (the version, candidates and top-k depend only on it)."""
    from oracle import OracleConfig, OracleIndex
    import datagen
    inp = datagen.workload_inputs(11, 6000, 6000, 0, 2, 32, 16, "f32")
    cfg = OracleConfig(heads=2, dim=32, dtype="f32", n_sink=4, window=1024, cluster_size=128, refit_every=2048)
    ix = OracleIndex(cfg)
    ix.append(inp["keys"], None)
    while ix.refit_due():
        ix.refit()
        ix.publish()
    pos = np.array([5999, 3, 1027, 4100, 2051, 5000])
    q, w = inp["q"][pos], inp["w"][pos]
    idx, sc = ix.route_at(q, None, w, pos, 32, 1500)
    for t, p in enumerate(pos):
        i1, s1 = ix.route(q[t:t + 1], None, w[t:t + 1], int(p), 32, 1500)
        assert np.array_equal(idx[t], i1[0]) and np.array_equal(sc[t], s1[0])
        assert np.all(idx[t][idx[t] >= 0] <= p)
    with pytest.raises(Exception):
        ix.route_at(q[:1], None, w[:1], np.array([6000]), 32, 1500)


def test_hand_computed_index():
    """The oracle's routing over a hand-built epoch reproduces every value worked out
    by hand in tests/golden/hand_index.json (representative scores, version, cluster
    order and takes, candidate list, top-k, exhaustive top-k)."""
    import hand_fixture as hf
    from oracle.index import make_cluster
    from oracle.index import CausalityError
    g = hf.load()
    c = g["config"]
    cfg = OracleConfig(heads=hf.H, dim=hf.D, dtype="f32", **c)
    ix = OracleIndex(cfg)
    ix.append(hf.keys(g))
    assert ix.refit_due()
    sizes, flat, cents, reps = hf.epoch_arrays(g)
    offs = np.concatenate([[0], np.cumsum(sizes)])
    clusters = [make_cluster(s, flat[offs[s]:offs[s + 1]], cents[s], "f32", reps[s]) for s in range(len(sizes))]
    bad = [make_cluster(s, cl.members, cl.centroid, "f32") for s, cl in enumerate(clusters)]
    bad[2] = make_cluster(2, np.array([3, 8]), cents[2], "f32")            # key 8 is beyond the epoch
    with pytest.raises(CausalityError):
        ix.install_epoch(bad)
    assert ix.install_epoch(clusters) == 1
    ix.publish()
    q, w = hf.query(g)
    for case in g["queries"]:
        p = case["position"]
        idx, sc, dbg = ix.route(q, None, w, p, case["k"], case["budget"], debug=True)
        d = dbg[0]
        if "rep_scores" in case:
            assert d["slots"].tolist() == list(range(len(case["rep_scores"])))
            assert d["srep"].tolist() == case["rep_scores"]
        if "version" in case:
            r, m = d["epoch"], d["windows"]
            assert [r, m, m * cfg.n_clusters, cfg.n_sink + m * cfg.window] == case["version"]
        assert [u for u, _ in d["used"]] == case["order"]
        assert [t for _, t in d["used"]] == case["take"]
        assert d["cand"].tolist() == case["candidates"]
        assert idx[0].tolist() == case["topk"] and sc[0].tolist() == case["topk_scores"]
        if "exhaustive_topk" in case:
            eidx, _ = ix.exhaustive(q, None, w, p, case["k"])
            assert eidx[0].tolist() == case["exhaustive_topk"]
            if "recall" in case:
                assert recall_per_query(idx, eidx)[0] == case["recall"]
