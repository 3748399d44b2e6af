"""GPU tests of hand-built versions, version read-back and the refit failure paths.

* The pages' worked example (paper-daily explainer, "代表向量为什么要学？": one
  cluster with members -2 and 2 has mean 0, so a query 1 scores its representative
  0 and skips it although one member scores 2) run through the library's kernels,
  embedded at d = 32 with four heads and head weights (1, 0, 0, 0): once as two
  sealed windows, once as an imported epoch.
* The hand-computed index of tests/golden/hand_index.json, imported with
  idx_import_version and routed; every value is compared with the fixture and with
  the oracle's routing over the same epoch.
* A refit after an imported epoch starts from its centres (bit-exact against the
  oracle), and idx_export_version returns what the oracle's version rule makes
  visible.
* Failure paths of the side-stream refit: a refit that is launched and never
  published is never used, and an abandoned one is recomputed identically; routes
  keep to the published epoch and equal the oracle under the same schedule.
"""
import json
import os

import numpy as np
import pytest

import hand_fixture as hf
from gpu_common import (RTOL, check_routed_query, compare_epoch, compare_seal_store, ensure_built, gpu_index,
                        oracle_cfg, say, to_dev, workload)
from oracle import OracleConfig, OracleIndex
from oracle.index import make_cluster, query_values
from oracle.kmeans import mean_exact

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _route_dbg(ivf, ix, q, w, pos0, k, budget, n_slots, cand_cap):
    import torch
    T = q.shape[0]
    dbg = ivf.make_route_debug(T, cand_cap, max(n_slots, 1), max(n_slots, 1))
    idx, sc = ivf.idx_route_topk(ix, q, None, w, pos0, k, budget, debug=dbg)
    torch.cuda.synchronize()
    d = {kk: v.cpu().numpy() for kk, v in dbg.items() if hasattr(v, "cpu")}
    d["topk_idx"], d["topk_score"] = idx.cpu().numpy(), sc.cpu().numpy()
    return d


def _worked_keys(g, d=32):
    keys = np.zeros((4, d), np.float32)
    keys[0:2, 5] = g["members"]          # cluster A: members -2 and 2, mean 0
    keys[2:4, 5] = 0.5                   # cluster B: mean 0.5
    q = np.zeros((1, 4, d), np.float32)
    q[0, 0, 5] = g["query"]
    q[0, 1:, 7] = [1.0, -3.0, 2.0]       # other heads carry weight 0
    w = np.array([[g["head_weight"], 0.0, 0.0, 0.0]], np.float32)
    return keys, q, w


def _check_worked(ivf, ix, g, keys, q, w):
    import torch
    qd, wd = to_dev(q), to_dev(w)
    d = _route_dbg(ivf, ix, qd, wd, 3, 1, 2, 2, 64)
    assert d["rep_scores"][0, :2].tolist() == [g["rep_score"], 0.5]
    assert d["order"][0, :1].tolist() == [1] and d["order_take"][0, :1].tolist() == [2]
    assert d["cand"][0, :int(d["cand_len"][0])].tolist() == [2, 3]
    assert d["topk_idx"][0].tolist() == [2]          # ties at 0.5 go to the lower position
    eidx, esc = ivf.idx_exhaustive_topk(to_dev(keys), None, "f32", 4, qd, None, wd, 3, 1)
    torch.cuda.synchronize()
    assert eidx.cpu().tolist() == [[1]] and esc.cpu().tolist() == [[max(g["member_scores"])]]
    assert keys[1, 5] == g["member_that_should_be_selected"]
    # the whole prefix as budget finds it
    idx, _ = ivf.idx_route_topk(ix, qd, None, wd, 3, 1, 4)
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == [[1]]


def test_worked_example_sealed():
    import ivf_top_key_amd as ivf
    ensure_built()
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    keys, q, w = _worked_keys(g)
    say("worked example, two sealed windows of two keys")
    ix = ivf.idx_create(heads=4, dim=32, dtype="f32", max_keys=4, n_sink=0, window=2, cluster_size=2, seal_cap=2,
                        seal_iters=1, refit_every=0, max_queries=1, max_budget=4, max_k=1)
    try:
        ivf.idx_build_seal(ix, to_dev(keys))
        seal = ivf.idx_export(ix, -1)
        assert seal["centroids"][0, 5] == g["rep_is_mean"] and seal["sizes"].tolist() == [2, 2]
        _check_worked(ivf, ix, g, keys, q, w)
    finally:
        ivf.idx_destroy(ix)


def test_worked_example_imported():
    import ivf_top_key_amd as ivf
    ensure_built()
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    keys, q, w = _worked_keys(g)
    say("worked example, an imported epoch of two clusters")
    ix = ivf.idx_create(heads=4, dim=32, dtype="f32", max_keys=4, n_sink=0, window=2, cluster_size=2, seal_cap=2,
                        seal_iters=1, refit_every=4, max_queries=1, max_budget=4, max_k=1)
    try:
        ivf.idx_build_seal(ix, to_dev(keys))
        cents = np.stack([keys[0:2].mean(0), keys[2:4].mean(0)]).astype(np.float32)
        ivf.idx_import_version(ix, 4, [2, 2], [0, 1, 2, 3], cents, cents)
        assert ivf.idx_publish(ix) == 1
        v = ivf.idx_export_version(ix, 4)
        assert v["epoch"] == 1 and v["windows"] == 2 and v["centroids"][0, 5] == 0.0
        _check_worked(ivf, ix, g, keys, q, w)
    finally:
        ivf.idx_destroy(ix)


def _hand_index(ivf):
    g = hf.load()
    c = g["config"]
    keys = hf.keys(g)
    ix = ivf.idx_create(heads=hf.H, dim=hf.D, dtype="f32", max_keys=keys.shape[0], max_queries=4, max_budget=64,
                        max_k=8, **c)
    ivf.idx_build_seal(ix, to_dev(keys))
    return g, keys, ix


def test_hand_computed_index_through_the_library():
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    g, keys, ix = _hand_index(ivf)
    say("hand-computed index (tests/golden/hand_index.json)")
    try:
        sizes, flat, cents, reps = hf.epoch_arrays(g)
        ivf.idx_import_version(ix, g["epoch1"]["prefix_len"], sizes, flat, cents, reps)
        assert ivf.idx_get_info(ix)["computed_epoch"] == 1
        assert ivf.idx_publish(ix) == 1
        exp = ivf.idx_export(ix, 1)
        assert exp["sizes"].tolist() == sizes.tolist() and exp["members"].tolist() == flat.tolist()
        assert np.array_equal(exp["reps"], reps) and np.array_equal(exp["centroids"], cents)
        assert exp["n_screened"] == -1                    # an imported epoch has no refit statistics
        # the oracle over the same epoch
        cfg = OracleConfig(heads=hf.H, dim=hf.D, dtype="f32", **g["config"])
        oix = OracleIndex(cfg)
        oix.append(keys)
        offs = np.concatenate([[0], np.cumsum(sizes)])
        oix.install_epoch([make_cluster(s, flat[offs[s]:offs[s + 1]], cents[s], "f32", reps[s])
                           for s in range(len(sizes))])
        oix.publish()
        q, w = hf.query(g)
        qd, wd = to_dev(q), to_dev(w)
        for case in g["queries"]:
            p, k, B = case["position"], case["k"], case["budget"]
            d = _route_dbg(ivf, ix, qd, wd, p, k, B, 4, 64)
            n_ord = int(d["n_order"][0])
            assert d["order"][0, :n_ord].tolist() == case["order"]
            assert d["order_take"][0, :n_ord].tolist() == case["take"]
            assert d["cand"][0, :int(d["cand_len"][0])].tolist() == case["candidates"]
            assert d["topk_idx"][0].tolist() == case["topk"]
            assert d["topk_score"][0].tolist() == case["topk_scores"]
            if "rep_scores" in case:
                assert d["rep_scores"][0, :4].tolist() == case["rep_scores"]
            if "version" in case:
                assert d["version"][0].tolist() == case["version"]
            if "exhaustive_topk" in case:
                eidx, _ = ivf.idx_exhaustive_topk(to_dev(keys), None, "f32", hf.H, qd, None, wd, p, k)
                torch.cuda.synchronize()
                assert eidx.cpu().numpy()[0].tolist() == case["exhaustive_topk"]
            _, _, od = oix.route(q, None, w, p, k, B, debug=True)
            stats = dict(order_swaps=0, topk_exempt=0, max_err=0.0)
            check_routed_query(0, d, od[0], oix, query_values(q, None, "f32"), w.astype(np.float64), k, B, "f32",
                               stats)
            assert stats["order_swaps"] == 0 and stats["topk_exempt"] == 0
        # the version read back for a prefix of 10 keys is the oracle's visible set
        v = ivf.idx_export_version(ix, 10)
        assert (v["epoch"], v["windows"]) == oix.version_of(10)
        assert v["sizes"].tolist() == [c.members.size for c in oix.visible(10)]
    finally:
        ivf.idx_destroy(ix)


def test_import_errors():
    import ivf_top_key_amd as ivf
    ensure_built()
    g, keys, ix = _hand_index(ivf)
    say("import argument and state errors")
    try:
        sizes, flat, cents, reps = hf.epoch_arrays(g)

        def expect(code, *a, **kw):
            with pytest.raises(ivf.IdxError) as ei:
                ivf.idx_import_version(ix, *a, **kw)
            assert ei.value.code == code, str(ei.value)

        beyond = flat.copy()
        beyond[0] = 8                                            # key 8 lies beyond the epoch's 8 keys
        expect(ivf.IDX_ECAUSAL, 8, sizes, beyond, cents, reps)
        expect(ivf.IDX_EINVAL, 16, sizes, flat, cents, reps)     # not the next epoch's boundary
        dup = flat.copy()
        dup[1] = dup[0]
        expect(ivf.IDX_EINVAL, 8, sizes, dup, cents, reps)       # a key twice
        unsorted = flat.copy()
        unsorted[2], unsorted[3] = unsorted[3], unsorted[2]
        expect(ivf.IDX_EINVAL, 8, sizes, unsorted, cents, reps)  # not ascending within a slot
        expect(ivf.IDX_EINVAL, 8, sizes[:3], flat[:6], cents[:3], reps[:3])      # wrong slot count
        short = sizes.copy()
        short[3] = 1
        expect(ivf.IDX_EINVAL, 8, short, flat[:7], cents, reps)  # a key left out
        bad = reps.copy()
        bad[1, 0] = np.inf
        expect(ivf.IDX_EINVAL, 8, sizes, flat, cents, bad)
        # the index is unchanged and still accepts the valid set; then a second import
        # while the first is unpublished is refused
        assert ivf.idx_get_info(ix)["computed_epoch"] == 0
        ivf.idx_import_version(ix, 8, sizes, flat, cents, reps)
        expect(ivf.IDX_ESTATE, 8, sizes, flat, cents, reps)
    finally:
        ivf.idx_destroy(ix)
    ix = ivf.idx_create(heads=4, dim=32, dtype="f32", max_keys=64, n_sink=0, window=4, cluster_size=2, seal_cap=4,
                        seal_iters=1, refit_every=8, max_queries=1, max_budget=64, max_k=8)
    try:
        ivf.idx_build_seal(ix, to_dev(keys[:6]))                # keys below 8 not all inserted
        sizes, flat, cents, reps = hf.epoch_arrays(g)
        with pytest.raises(ivf.IdxError) as ei:
            ivf.idx_import_version(ix, 8, sizes, flat, cents, reps)
        assert ei.value.code == ivf.IDX_ECAUSAL
    finally:
        ivf.idx_destroy(ix)


def _partition_epoch(oix, r, dtype):
    """A cluster set for epoch r that no refit would produce: key x of [S, B_r) goes to
    slot (7x) mod (r*Q); centroids are exact-order means (slots left empty are dead)."""
    cfg = oix.cfg
    S, B = cfg.n_sink, oix.boundary(r)
    ns = r * cfg.slots_per_refit
    pos = np.arange(S, B)
    slot = (7 * pos) % ns
    out = []
    for s in range(ns):
        mem = pos[slot == s]
        cent = mean_exact(oix.X[mem]) if mem.size else np.zeros(cfg.dim, np.float32)
        out.append(make_cluster(s, mem, cent, dtype))
    return out


def _import_clusters(ivf, ix, prefix_len, clusters):
    sizes = np.array([c.members.size for c in clusters], np.int32)
    flat = np.concatenate([c.members for c in clusters]).astype(np.int32)
    ivf.idx_import_version(ix, prefix_len, sizes, flat, np.stack([c.centroid for c in clusters]),
                           np.stack([c.rep_raw for c in clusters]),
                           np.array([c.rep_scale for c in clusters], np.float32))


def _check_routes(ivf, gix, oix, wl, inp, q_pos0, T, label):
    cfg = oix.cfg
    k, budget, dt = wl["k"], wl["budget"], wl["dtype"]
    q = to_dev(inp["q"][:T])
    qs = to_dev(inp["q_scale"][:T]) if inp["q_scale"] is not None else None
    w = to_dev(inp["w"][:T])
    n_slots = ((q_pos0 + T - cfg.n_sink) // cfg.window) * cfg.n_clusters
    import torch
    dbg = ivf.make_route_debug(T, max(budget, cfg.n_sink + cfg.window) + 32, max(n_slots, 1), max(n_slots, 1))
    idx, sc = ivf.idx_route_topk(gix, q, qs, w, q_pos0, k, budget, debug=dbg)
    torch.cuda.synchronize()
    d = {kk: v.cpu().numpy() for kk, v in dbg.items() if hasattr(v, "cpu")}
    d["topk_idx"], d["topk_score"] = idx.cpu().numpy(), sc.cpu().numpy()
    qraw = inp["q"][:T]
    qsc = None if inp["q_scale"] is None else inp["q_scale"][:T]
    _, _, od = oix.route(qraw, qsc, inp["w"][:T], q_pos0, k, budget, debug=True)
    stats = dict(order_swaps=0, topk_exempt=0, max_err=0.0)
    qv = query_values(qraw, qsc, dt)
    for t in range(T):
        check_routed_query(t, d, od[t], oix, qv, inp["w"][:T].astype(np.float64), k, budget, dt, stats)
    say(f"  {label}: {T} queries at {q_pos0}.. match the oracle {stats}")
    return d


@pytest.mark.parametrize("name", ["c1r", "e4m3_small"])
def test_refit_after_imported_epoch(name):
    """Import a partition no refit would make as epoch 1, route over it, then let
    refit 2 start from it: epoch 2 is bit-exact to the oracle's refit from the same
    set, and the version read-back matches the oracle's visible clusters."""
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload(name)
    R, S, W = wl["refit_every"], wl["n_sink"], wl["window"]
    n1 = S + 2 * R + W                      # refit 1 due, refit 2 not yet
    n2 = S + 2 * R + 2 * W                  # refit 2 due
    say(f"import {name}: epoch 1 imported at {n1} keys, refit 2 at {n2}")
    gix = ivf.idx_create(heads=wl["H"], dim=wl["d"], dtype=wl["dtype"], max_keys=wl["N"], max_queries=256,
                         max_budget=wl["budget"], max_k=wl["k"], n_sink=S, window=W,
                         cluster_size=wl["cluster_size"], seal_cap=wl["seal_cap"], seal_iters=wl["seal_iters"],
                         refit_every=R)
    try:
        keys = to_dev(inp["keys"])
        ks = to_dev(inp["k_scale"]) if inp["k_scale"] is not None else None
        ivf.idx_build_seal(gix, keys[:n1], None if ks is None else ks[:n1])
        oix = OracleIndex(oracle_cfg(wl))
        oix.append(inp["keys"][:n1], None if inp["k_scale"] is None else inp["k_scale"][:n1])
        clusters = _partition_epoch(oix, 1, wl["dtype"])
        _import_clusters(ivf, gix, S + R, clusters)
        oix.install_epoch(clusters)
        ivf.idx_publish(gix)
        oix.publish()
        compare_epoch(ivf, gix, oix, 1, "imported")
        _check_routes(ivf, gix, oix, wl, inp, n1 - 200, 200, "over the imported epoch")
        for n in (S + R, S + R + W - 1, n1):
            v = ivf.idx_export_version(gix, n)
            assert (v["epoch"], v["windows"]) == oix.version_of(n), n
            vis = {c.slot: c for c in oix.visible(n)}
            for s, sz in enumerate(v["sizes"]):
                if sz == 0:
                    assert s not in vis
                    continue
                mem = v["members"][v["offsets"][s]:v["offsets"][s] + sz]
                assert np.array_equal(mem, vis[s].members) and np.array_equal(v["reps"][s], vis[s].rep_raw)
        # refit 2 starts from the imported centres (every key screened: no bounds carried)
        ivf.idx_build_seal(gix, keys[n1:n2], None if ks is None else ks[n1:n2])
        oix.append(inp["keys"][n1:n2], None if inp["k_scale"] is None else inp["k_scale"][n1:n2])
        assert ivf.idx_refit(gix)
        assert ivf.idx_publish(gix) == 2
        oix.refit()
        oix.publish()
        ex = compare_epoch(ivf, gix, oix, 2, "refit after import")
        assert ex["n_screened"] == 2 * R           # the imported keys carried no bounds
        compare_seal_store(ivf, gix, oix, "after import")
        _check_routes(ivf, gix, oix, wl, inp, n2 - 200, 200, "after refit 2")
    finally:
        ivf.idx_destroy(gix)


def test_unpublished_and_abandoned_refits():
    """A refit that is launched but never published is never used; an abandoned
    one is recomputed to the same epoch; a store that a later refit reused is not
    routed even after that refit is abandoned."""
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload("c1r", refit_every=1024)
    S, W = wl["n_sink"], wl["window"]
    N = wl["N"]
    gix = ivf.idx_create(heads=wl["H"], dim=wl["d"], dtype=wl["dtype"], max_keys=N, max_queries=256,
                         max_budget=wl["budget"], max_k=wl["k"], n_sink=S, window=W,
                         cluster_size=wl["cluster_size"], seal_cap=wl["seal_cap"], seal_iters=wl["seal_iters"],
                         refit_every=1024)
    import torch
    side = torch.cuda.Stream()
    try:
        keys = to_dev(inp["keys"])
        oix = OracleIndex(oracle_cfg(wl))
        n = S + 2 * W
        ivf.idx_build_seal(gix, keys[:n])
        oix.append(inp["keys"][:n])
        # refit 1 launched on the side stream and never published
        assert ivf.idx_refit(gix, side_stream=side)
        ivf.idx_build_seal(gix, keys[n:n + W])                  # a third window sealed meanwhile
        oix.append(inp["keys"][n:n + W])
        n += W
        assert not ivf.idx_refit(gix, side_stream=side)         # the unpublished one blocks the next
        info = ivf.idx_get_info(gix)
        assert info["computed_epoch"] == 1 and info["published_epoch"] == 0
        _check_routes(ivf, gix, oix, wl, inp, n - 128, 128, "refit launched, not published")
        # abandon it: routes unchanged; the next launch recomputes epoch 1 identically
        assert ivf.idx_abandon_refit(gix) == 1
        assert ivf.idx_abandon_refit(gix) == 0
        _check_routes(ivf, gix, oix, wl, inp, n - 128, 128, "refit abandoned")
        assert ivf.idx_refit(gix, side_stream=side)
        assert ivf.idx_publish(gix) == 1
        oix.refit()
        oix.publish()
        compare_epoch(ivf, gix, oix, 1, "relaunched")
        _check_routes(ivf, gix, oix, wl, inp, n - 128, 128, "epoch 1 published")
        while ivf.idx_refit(gix, side_stream=side):
            ivf.idx_publish(gix)
            oix.refit()
            oix.publish()
        # epochs 1..3 computed and published; refit 4 reuses epoch 1's store
        ivf.idx_build_seal(gix, keys[n:S + 4 * W])
        oix.append(inp["keys"][n:S + 4 * W])
        n = S + 4 * W
        assert ivf.idx_get_info(gix)["published_epoch"] == 3
        assert ivf.idx_refit(gix, side_stream=side)
        assert ivf.idx_abandon_refit(gix) == 4
        q = to_dev(inp["q"][:1])
        w = to_dev(inp["w"][:1])
        with pytest.raises(ivf.IdxError) as ei:                 # position 1500 routes over epoch 1
            ivf.idx_route_topk_pos(gix, q, None, w, [1500], wl["k"], wl["budget"])
        assert ei.value.code == ivf.IDX_ESTATE
        with pytest.raises(ivf.IdxError) as ei:
            ivf.idx_export(gix, 1)
        assert ei.value.code == ivf.IDX_ESTATE
        _check_routes(ivf, gix, oix, wl, inp, n - 128, 128, "epoch 3 after refit 4 was abandoned")
        assert ivf.idx_refit(gix, side_stream=side)
        ivf.idx_publish(gix)
        oix.refit()
        oix.publish()
        compare_epoch(ivf, gix, oix, 4, "refit 4 relaunched")
        _check_routes(ivf, gix, oix, wl, inp, n - 128, 128, "epoch 4 published")
        torch.cuda.synchronize()
    finally:
        ivf.idx_destroy(gix)
