"""GPU parity at the full benchmark sizes.

32K bf16 (4096 queries, k = 2048, budget 8192): the oracle builds the whole index
itself, so every sealed window and the refit epoch are compared bit for bit, and
every one of the 4096 queries is routed by the oracle over its own index and
compared with the library (versions, representative scores, cluster order and
takes, candidate lists, top-k); 64 seeded queries are also checked on the
exhaustive path.

1M-token prefix, E4M3 (the benchmark's workload: the index streamed 16384 keys at
a time with every refit published, 4096 tail queries routed in one call, k = 2048,
budget 8192).  An oracle rebuild of a 1M-key index takes hours, so the checks are
the ones the oracle can make one output at a time:
* 64 seeded queries on the exhaustive path against float64 scores of every key of
  their prefix;
* 32 seeded sealed windows recomputed by the oracle, bit for bit;
* every cluster of the newest epoch: centroid = exact-order mean of its members,
  members ascending, representative = the oracle's quantisation;
* every key's assignment at the newest refit = its nearest warm-start centroid
  (epoch r-1's centroids and the newer seal centroids): a float64 distance screen,
  then the fixed-order fp32 distances for each key whose two nearest lie within
  the fp32 evaluation's error bound of each other;
* 1024 seeded routed queries = the oracle's routing over the published clusters.
"""
import numpy as np
import pytest

from gpu_common import (RTOL, check_refit_bounds, check_routed_query, compare_epoch, compare_seal_store,
                        ensure_built, oracle_index, say, to_dev, workload)
from oracle import OracleConfig, OracleIndex
from oracle import codec
from oracle.index import key_values, make_cluster, query_values
from oracle.kmeans import mean_exact, nearest, seal_window, sqdist_exact
from oracle.score import indexer_scores, score_error_scale

pytestmark = pytest.mark.gpu


def _build(wl, inp, ivf, chunk):
    import torch
    N = wl["N"]
    ix = ivf.idx_create(heads=wl["H"], dim=wl["d"], dtype=wl["dtype"], max_keys=N, n_sink=wl["n_sink"],
                        window=wl["window"], cluster_size=wl["cluster_size"], seal_cap=wl["seal_cap"],
                        seal_iters=wl["seal_iters"], refit_every=wl["refit_every"], max_queries=wl["T"],
                        max_budget=16384, max_k=wl["k"])
    keys = to_dev(inp["keys"])
    ks = to_dev(inp["k_scale"]) if inp["k_scale"] is not None else None
    for a in range(0, N, chunk):
        ivf.idx_build_seal(ix, keys[a:a + chunk], None if ks is None else ks[a:a + chunk])
        while ivf.idx_refit(ix):
            ivf.idx_publish(ix)
    torch.cuda.synchronize()
    return ix, keys, ks


def _route_all(ivf, ix, wl, inp):
    import torch
    T, q_pos0, k = wl["T"], wl["q_pos0"], wl["k"]
    q = to_dev(inp["q"])
    qs = to_dev(inp["q_scale"]) if inp["q_scale"] is not None else None
    w = to_dev(inp["w"])
    Cs = wl["window"] // wl["cluster_size"]
    vis_slots = ((q_pos0 + T - wl["n_sink"]) // wl["window"]) * Cs
    dbg = ivf.make_route_debug(T, wl["budget"] + 32, vis_slots, vis_slots)
    idx, sc = ivf.idx_route_topk(ix, q, qs, w, q_pos0, k, wl["budget"], debug=dbg)
    ws = torch.empty(ivf.idx_exhaustive_workspace_bytes(wl["N"], 256) // 4, dtype=torch.float32, device="cuda")
    return q, qs, w, dbg, idx, sc, ws


def _exhaustive_check(eidx, esc, picks, kv, qv, wv, q_pos0, k, dt, chunk=65536):
    """Float64 scores of the picked queries against every key of their prefix (the
    oracle's score applied to key chunks), then per query: the GPU's top-k equals the
    float64 top-k except positions scoring within the tolerance of the k-th score,
    and every returned score is within the tolerance of its float64 value."""
    pos = q_pos0 + picks
    n = int(pos.max()) + 1
    S = np.empty((picks.size, n))
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        S[:, a:b] = indexer_scores(qv[picks], wv[picks], kv[a:b], block=picks.size)
    exempt = 0
    for i, t in enumerate(picks):
        nt = int(pos[i]) + 1
        row = S[i, :nt]
        kk = min(k, nt)
        kth_val = np.partition(row, nt - kk)[nt - kk]
        cand = np.nonzero(row >= kth_val)[0]
        order = np.lexsort((cand, -row[cand]))[:kk]
        ref = cand[order]
        g = eidx[t][eidx[t] >= 0]
        assert g.size == kk, f"exhaustive query {t}: {g.size} entries"
        sig_g = score_error_scale(qv[t:t + 1], wv[t:t + 1], kv[g])[0]
        err = np.abs(esc[t][:kk].astype(np.float64) - row[g])
        assert np.all(err <= RTOL[dt] * sig_g + 1e-30), f"exhaustive query {t}: score error"
        diff = np.array(sorted(set(g.tolist()) ^ set(ref.tolist())), dtype=np.int64)
        if diff.size:
            sig_d = score_error_scale(qv[t:t + 1], wv[t:t + 1], kv[np.append(diff, ref[-1])])[0]
            tol = 2 * RTOL[dt] * np.maximum(sig_d[:-1], sig_d[-1])
            assert np.all(np.abs(row[diff] - row[ref[-1]]) <= tol), f"exhaustive query {t}: not a top-k"
            exempt += diff.size
    return exempt


def _assignment_check(X, owner, warm_c, warm_alive, S, B, chunk=8192):
    """Every key of [S, B) belongs to its nearest live warm centroid under the
    fixed-order fp32 distance (ties to the lower slot).  A float64 screen gives each
    key's two nearest; where they are further apart than twice the fp32 evaluation's
    relative error bound (d + 2) * 2^-24, the float64 winner is the fp32 winner;
    the other keys are evaluated in the fixed order.  Returns the number of those."""
    ids = np.nonzero(warm_alive)[0]
    C = warm_c[ids].astype(np.float64)
    CT = np.ascontiguousarray(C.T)
    cn = (C * C).sum(1)
    d = X.shape[1]
    gamma = 1.01 * (d + 2) * 2.0 ** -24
    rows = np.arange(chunk)
    n_exact = 0
    for a in range(S, B, chunk):
        b = min(B, a + chunk)
        x = X[a:b].astype(np.float64)
        D = x @ CT
        D *= -2.0
        D += cn[None, :]
        best = D.argmin(1)
        r = rows[:b - a]
        d1 = D[r, best].copy()
        D[r, best] = np.inf
        d2 = D.min(1)
        xn = (x * x).sum(1)
        d1 += xn
        d2 += xn
        want = ids[best]
        amb = np.nonzero(d2 - d1 <= 4 * gamma * np.abs(d2) + 1e-12)[0]
        if amb.size:
            want[amb] = ids[nearest(sqdist_exact(X[a + amb], warm_c[ids]))]
            n_exact += amb.size
        got = owner[a:b]
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"key {a + bad[0]}: slot {got[bad[0]]}, nearest warm centroid {want[bad[0]]}"
    return n_exact


def _clusters(exp, dtype):
    out = []
    for s in range(exp["sizes"].shape[0]):
        sz, off = int(exp["sizes"][s]), int(exp["offsets"][s])
        out.append(make_cluster(s, exp["members"][off:off + sz].astype(np.int64), exp["centroids"][s], dtype))
    return out


def _debug_rows(dbg, picks):
    import torch
    rows = torch.from_numpy(picks).cuda()
    d = {}
    for kk, v in dbg.items():
        if hasattr(v, "cpu"):
            full = np.zeros(tuple(v.shape), dtype=v[:1].cpu().numpy().dtype)   # only picked rows filled
            full[picks] = v.index_select(0, rows).cpu().numpy()
            d[kk] = full
    return d


def test_scale_1m_e4m3():
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload("c4")
    dt, T, k, q_pos0, N = wl["dtype"], wl["T"], wl["k"], wl["q_pos0"], wl["N"]
    S, W, R = wl["n_sink"], wl["window"], wl["refit_every"]
    Cs = W // wl["cluster_size"]
    say(f"scale c4: N={N} dtype={dt} T={T}")
    ix, keys, ks = _build(wl, inp, ivf, R)
    rng = np.random.default_rng(1)
    try:
        q, qs, w, dbg, idx, sc, ws = _route_all(ivf, ix, wl, inp)
        eidx, esc = ivf.idx_exhaustive_topk(keys, ks, dt, wl["H"], q, qs, w, q_pos0, k, workspace=ws)
        torch.cuda.synchronize()
        idx, sc, eidx, esc = idx.cpu().numpy(), sc.cpu().numpy(), eidx.cpu().numpy(), esc.cpu().numpy()
        info = ivf.idx_get_info(ix)
        P = info["published_epoch"]
        kv = key_values(inp["keys"], inp["k_scale"], dt)
        X = codec.dequantize(inp["keys"], inp["k_scale"], dt)
        qv = query_values(inp["q"], inp["q_scale"], dt)
        wv = inp["w"].astype(np.float64)

        picks = np.sort(rng.choice(T, 64, replace=False))
        ex = _exhaustive_check(eidx, esc, picks, kv, qv, wv, q_pos0, k, dt)
        say(f"  exhaustive: 64 seeded queries match float64 ({ex} near-tie exemptions)")

        seal = ivf.idx_export(ix, -1)
        for wi in rng.choice(info["sealed_windows"], 32, replace=False):
            lo = S + wi * W
            a, C, alive = seal_window(X[lo:lo + W], Cs, wl["seal_cap"], wl["seal_iters"])
            for c in range(Cs):
                s = wi * Cs + c
                mem = lo + np.nonzero(a == c)[0]
                off, sz = int(seal["offsets"][s]), int(seal["sizes"][s])
                assert sz == mem.size and np.array_equal(seal["members"][off:off + sz], mem), f"window {wi}"
                assert np.array_equal(seal["centroids"][s].view(np.uint32), C[c].view(np.uint32)), f"window {wi}"
        say("  seal: 32 seeded windows bit-exact")

        assert P >= 2
        ep = ivf.idx_export(ix, P)
        n_live = 0
        for s in range(ep["sizes"].shape[0]):
            off, sz = int(ep["offsets"][s]), int(ep["sizes"][s])
            if not sz:
                continue
            n_live += 1
            mem = ep["members"][off:off + sz].astype(np.int64)
            assert np.all(np.diff(mem) > 0)
            assert np.array_equal(ep["centroids"][s].view(np.uint32), mean_exact(X[mem]).view(np.uint32)), s
            raw, rs = codec.quantize_rep(ep["centroids"][s], dt)
            assert np.array_equal(ep["reps"][s], raw) and np.float32(ep["rep_scale"][s]) == rs, s
        Q = ep["sizes"].shape[0] // P
        prev = ivf.idx_export(ix, P - 1)
        warm_c = np.concatenate([prev["centroids"], seal["centroids"][(P - 1) * Q:P * Q]])
        warm_alive = np.concatenate([prev["sizes"] > 0, seal["sizes"][(P - 1) * Q:P * Q] > 0])
        owner = np.full(N, -1)
        for s in range(ep["sizes"].shape[0]):
            off, sz = int(ep["offsets"][s]), int(ep["sizes"][s])
            owner[ep["members"][off:off + sz]] = s
        B = S + P * R
        assert np.all(owner[S:B] >= 0) and np.all(owner[B:] == -1)
        n_exact = _assignment_check(X, owner, warm_c, warm_alive, S, B)
        say(f"  epoch {P}: all {n_live} live clusters exact means; all {B - S} keys nearest "
            f"({n_exact} decided by the fixed-order distances)")
        nchk, frac = check_refit_bounds(ivf, ix, wl, kv, sample=2000, seed=1)
        say(f"  bounds of {nchk} sampled keys hold; the last refit screened {frac:.3f} of its prefix")

        cfg = OracleConfig(heads=wl["H"], dim=wl["d"], dtype=dt, n_sink=S, window=W,
                           cluster_size=wl["cluster_size"], seal_cap=wl["seal_cap"],
                           seal_iters=wl["seal_iters"], refit_every=R)
        oix = OracleIndex(cfg)
        oix.kv = kv
        oix.X = X
        sc_all = _clusters(seal, dt)
        oix.seals = [sc_all[i:i + Cs] for i in range(0, len(sc_all), Cs)]
        oix.epochs[P] = _clusters(ep, dt)
        oix.computed = oix.published = P
        picks = np.sort(rng.choice(T, 1024, replace=False))
        d = _debug_rows(dbg, picks)
        d["topk_idx"], d["topk_score"] = idx, sc
        stats = dict(order_swaps=0, topk_exempt=0, max_err=0.0)
        for t in picks:
            _, _, od = oix.route(inp["q"][t:t + 1], inp["q_scale"][t:t + 1], inp["w"][t:t + 1], q_pos0 + int(t), k,
                                 wl["budget"], debug=True)
            check_routed_query(int(t), d, od[0], oix, qv, wv, k, wl["budget"], dt, stats)
        say(f"  routed: 1024 seeded queries match the oracle's routing over the published clusters {stats}")
        rec = np.mean([np.intersect1d(a[a >= 0], b[b >= 0]).size / k for a, b in zip(idx, eidx)])
        say(f"  recall vs exhaustive {rec:.4f}")
    finally:
        ivf.idx_destroy(ix)


def test_scale_32k_bf16():
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload("c2")
    dt, T, k, q_pos0 = wl["dtype"], wl["T"], wl["k"], wl["q_pos0"]
    say(f"scale c2: N={wl['N']} dtype={dt} T={T}: the oracle builds the index and routes every query")
    ix, keys, ks = _build(wl, inp, ivf, wl["refit_every"])
    try:
        q, qs, w, dbg, idx, sc, ws = _route_all(ivf, ix, wl, inp)
        eidx, esc = ivf.idx_exhaustive_topk(keys, ks, dt, wl["H"], q, qs, w, q_pos0, k, workspace=ws)
        torch.cuda.synchronize()
        d = {kk: v.cpu().numpy() for kk, v in dbg.items() if hasattr(v, "cpu")}
        d["topk_idx"], d["topk_score"] = idx.cpu().numpy(), sc.cpu().numpy()
        eidx, esc = eidx.cpu().numpy(), esc.cpu().numpy()
        oix = oracle_index(wl, inp)
        assert ivf.idx_get_info(ix)["published_epoch"] == oix.published == 1
        compare_seal_store(ivf, ix, oix, "c2")
        compare_epoch(ivf, ix, oix, 1, "c2")
        say(f"  index: all {len(oix.seals)} windows and epoch 1 bit-exact")
        qv = query_values(inp["q"], None, dt)
        wv = inp["w"].astype(np.float64)
        stats = dict(order_swaps=0, topk_exempt=0, max_err=0.0)
        for t0 in range(0, T, 256):
            _, _, od = oix.route(inp["q"][t0:t0 + 256], None, inp["w"][t0:t0 + 256], q_pos0 + t0, k, wl["budget"],
                                 debug=True)
            for i, o in enumerate(od):
                check_routed_query(t0 + i, d, o, oix, qv, wv, k, wl["budget"], dt, stats)
            if t0 % 1024 == 0:
                say(f"  routed {t0 + 256} of {T} queries: {stats}")
        say(f"  routed: all {T} queries match the oracle {stats}")
        picks = np.sort(np.random.default_rng(2).choice(T, 64, replace=False))
        ex = _exhaustive_check(eidx, esc, picks, oix.kv, qv, wv, q_pos0, k, dt)
        say(f"  exhaustive: 64 seeded queries match float64 ({ex} near-tie exemptions)")
    finally:
        ivf.idx_destroy(ix)
