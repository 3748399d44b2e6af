"""Shared helpers of the GPU parity tests: inputs, building both sides, comparisons.

Tolerances.  Scores are compared against the oracle's float64 scores relative to
sigma(t, j) = sum_h |w| * sum_i |q_i k_i| (the error scale of any fp32
evaluation).  The fp32 MFMA accumulation over d terms plus the fp32 sum over H
heads is off by at most about (d + H) * 2^-24 * sigma = 1.2e-5 sigma for d=128,
H=64, and 2.1e-6 sigma for d=32, H=4.  Tests assert 1e-5 sigma for fp32 (the
stated bar) and 1e-4 sigma for bf16/E4M3 (tighter than the stated 2e-2), and
treat two candidates whose oracle scores are within that tolerance of each
other as a near tie, where either order is correct.
"""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import datagen  # noqa: E402
from datagen.workloads import WORKLOADS  # noqa: E402
from oracle import OracleConfig, OracleIndex, fill_budget  # noqa: E402
from oracle.index import query_values, topk_sorted  # noqa: E402
from oracle.score import indexer_scores, score_error_scale  # noqa: E402

RTOL = {"f32": 1e-5, "bf16": 1e-4, "e4m3": 1e-4}
CFG_KEYS = ("n_sink", "window", "cluster_size", "seal_cap", "seal_iters", "refit_every")


def ensure_built():
    from ivf_top_key_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from ivf_top_key_amd.build import build
        build()


def say(msg):
    print(msg, flush=True)


def workload(name, **over):
    wl = dict(WORKLOADS[name], **over)
    inp = datagen.workload_inputs(wl["seed"], wl["N"], wl["T"], wl["q_pos0"], wl["H"], wl["d"], wl["M"],
                                  wl["dtype"])
    return wl, inp


def oracle_cfg(wl):
    return OracleConfig(heads=wl["H"], dim=wl["d"], dtype=wl["dtype"], positional=wl.get("positional", False),
                        **{k: wl[k] for k in CFG_KEYS})


def oracle_index(wl, inp, n_keys=None):
    n = wl["N"] if n_keys is None else n_keys
    ix = OracleIndex(oracle_cfg(wl))
    ix.append(inp["keys"][:n], None if inp["k_scale"] is None else inp["k_scale"][:n])
    while ix.refit_due():
        ix.refit()
        ix.publish()
    return ix


def to_dev(a, device="cuda"):
    import torch
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def gpu_index(wl, inp, n_keys=None, chunk=None, max_queries=None, max_budget=None, max_k=None, rescore="auto"):
    """Insert keys (in chunks) and run every due refit, published at once."""
    import ivf_top_key_amd as ivf
    n = wl["N"] if n_keys is None else n_keys
    ix = ivf.idx_create(heads=wl["H"], dim=wl["d"], dtype=wl["dtype"], max_keys=wl["N"],
                        max_queries=max_queries or wl["T"], max_budget=max_budget or max(wl["budget"], wl["N"]),
                        max_k=max_k or wl["k"], rescore=rescore,
                        clusters="positional" if wl.get("positional") else "content",
                        **{k: wl[k] for k in CFG_KEYS})
    keys = to_dev(inp["keys"][:n])
    ks = to_dev(inp["k_scale"][:n]) if inp["k_scale"] is not None else None
    chunk = chunk or n
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        ivf.idx_build_seal(ix, keys[a:b], None if ks is None else ks[a:b])
        while ivf.idx_refit(ix):
            ivf.idx_publish(ix)
    return ix


def compare_cluster_set(got, clusters, n_members_base, dtype, label):
    """Bit-exact comparison of an exported cluster set with oracle clusters (slot order)."""
    assert got["sizes"].shape[0] == len(clusters), label
    for c in clusters:
        s = c.slot
        size = int(got["sizes"][s])
        assert size == c.members.size, f"{label}: slot {s} size {size} vs oracle {c.members.size}"
        if size:
            off = int(got["offsets"][s])
            mem = got["members"][off:off + size]
            assert np.array_equal(mem, c.members), f"{label}: slot {s} members differ"
            assert np.array_equal(got["centroids"][s].view(np.uint32), c.centroid.view(np.uint32)), \
                f"{label}: slot {s} centroid bits differ (max abs diff " \
                f"{np.abs(got['centroids'][s] - c.centroid).max():.3g})"
            assert np.array_equal(got["reps"][s], c.rep_raw), f"{label}: slot {s} representative differs"
            assert np.float32(got["rep_scale"][s]) == np.float32(c.rep_scale), f"{label}: slot {s} rep scale"


def compare_seal_store(ivf, gix, oix, label):
    got = ivf.idx_export(gix, -1)
    clusters = [c for w in oix.seals for c in w]
    compare_cluster_set(got, clusters, 0, oix.cfg.dtype, label + " seal")
    return got


def compare_epoch(ivf, gix, oix, r, label):
    got = ivf.idx_export(gix, r)
    compare_cluster_set(got, oix.epochs[r], 0, oix.cfg.dtype, f"{label} epoch {r}")
    return got


def check_scores(idx, sc, qv, w, kv, t, dtype, label):
    """GPU scores of the returned positions against float64 within rtol * sigma."""
    ok = idx >= 0
    j = idx[ok]
    ref = indexer_scores(qv[t:t + 1], w[t:t + 1], kv[j])[0]
    sig = score_error_scale(qv[t:t + 1], w[t:t + 1], kv[j])[0]
    err = np.abs(sc[ok].astype(np.float64) - ref)
    bound = RTOL[dtype] * sig + 1e-30
    assert np.all(err <= bound), f"{label}: score error {np.max(err / bound):.3g} x tolerance"
    return float(np.max(err / np.maximum(sig, 1e-30))) if err.size else 0.0


def topk_matches(got_idx, cand, qv, w, kv, t, k, dtype):
    """True if got_idx is a correct top-k of `cand` up to near ties (oracle float64 scores).

    Returns (ok, n_exempt): every position in the symmetric difference with the
    oracle's top-k must score within the tolerance of the oracle's k-th score."""
    cand = np.asarray(cand, dtype=np.int64)
    s = indexer_scores(qv[t:t + 1], w[t:t + 1], kv[cand])[0]
    sig = score_error_scale(qv[t:t + 1], w[t:t + 1], kv[cand])[0]
    ref_idx, ref_sc = topk_sorted(cand, s, k)
    g = set(int(x) for x in got_idx if x >= 0)
    r = set(int(x) for x in ref_idx if x >= 0)
    if len(g) != len(r):
        return False, 0
    diff = g ^ r
    if not diff:
        return True, 0
    kth = ref_sc[min(k, len(r)) - 1]
    pos = {int(c): i for i, c in enumerate(cand)}
    tol_k = RTOL[dtype] * sig[pos[int(ref_idx[min(k, len(r)) - 1])]]
    for x in diff:
        i = pos.get(x)
        if i is None:
            return False, 0
        if abs(s[i] - kth) > 2 * max(RTOL[dtype] * sig[i], tol_k):
            return False, 0
    return True, len(diff)


def check_routed_query(t, d, od, oix, qv, wv, k, budget, dt, stats):
    """One routed query of the GPU (debug outputs d, row t) against the oracle's
    routing of the same query (od) over the index oix.  See test_gpu_route."""
    cfg = oix.cfg
    idx = d["topk_idx"]
    sc = d["topk_score"]
    r, m = od["epoch"], od["windows"]
    assert d["version"][t].tolist() == [r, m, m * cfg.n_clusters, cfg.n_sink + m * cfg.window], \
        f"query {t}: version {d['version'][t].tolist()} vs ({r}, {m})"
    vis = {c.slot: c for c in oix.visible(od["n"])}
    srep, ssig = {}, {}
    if vis:
        slots = np.array(sorted(vis))
        reps = np.stack([vis[s].rep_value for s in slots])
        ref = indexer_scores(qv[t:t + 1], wv[t:t + 1], reps)[0]
        sig = score_error_scale(qv[t:t + 1], wv[t:t + 1], reps)[0]
        err = np.abs(d["rep_scores"][t, slots].astype(np.float64) - ref)
        assert np.all(err <= RTOL[dt] * sig + 1e-30), f"query {t}: representative score error"
        srep = dict(zip(slots.tolist(), ref.tolist()))
        ssig = dict(zip(slots.tolist(), sig.tolist()))
    n_ord = int(d["n_order"][t])
    g_order = d["order"][t, :n_ord].tolist()
    g_take = d["order_take"][t, :n_ord].tolist()
    o_used = od["used"]
    L = int(d["cand_len"][t])
    g_cand = d["cand"][t, :L]
    if [s for s, _ in o_used] == g_order:
        assert [tk for _, tk in o_used] == g_take, f"query {t}: takes differ"
        assert np.array_equal(g_cand, od["cand"]), f"query {t}: candidate list differs"
    else:
        # near ties only: a valid ranking under the tolerance, and the oracle's fill
        # with this order reproduces the GPU's list exactly
        stats["order_swaps"] += 1
        tol = lambda a, b: 2 * RTOL[dt] * max(ssig[a], ssig[b])
        for a, b in zip(g_order, g_order[1:]):
            assert srep[a] >= srep[b] - tol(a, b), f"query {t}: clusters {a},{b} out of order"
        chosen = set(g_order)
        last = g_order[-1]
        for u in vis:
            if u not in chosen:
                assert srep[u] <= srep[last] + tol(u, last), f"query {t}: skipped cluster {u}"
        cand, used = fill_budget(oix.base_candidates(od["n"]), [vis[s] for s in g_order], budget)
        assert [s for s, _ in used] == g_order and [x for _, x in used] == g_take
        assert np.array_equal(g_cand, cand), f"query {t}: fill with the GPU order differs"
    # the selection itself, exactly: top k of the GPU's own candidate scores
    gs = d["cand_scores"][t, :L]
    order = np.lexsort((g_cand, -gs.astype(np.float64)))[:k]
    assert np.array_equal(idx[t][:min(k, L)], g_cand[order]), f"query {t}: selection differs from " \
        f"the exact top-k of the GPU's own scores"
    ok, ex = topk_matches(idx[t], g_cand, qv, wv, oix.kv, t, k, dt)
    assert ok, f"query {t}: top-k is not a top-k of the candidates"
    stats["topk_exempt"] += ex
    valid = idx[t] >= 0
    assert valid.sum() == min(k, L)
    gj = idx[t][valid]
    ref = indexer_scores(qv[t:t + 1], wv[t:t + 1], oix.kv[gj])[0]
    sig = score_error_scale(qv[t:t + 1], wv[t:t + 1], oix.kv[gj])[0]
    err = np.abs(sc[t][valid].astype(np.float64) - ref)
    assert np.all(err <= RTOL[dt] * sig + 1e-30), f"query {t}: candidate score error"
    if err.size:
        stats["max_err"] = max(stats["max_err"], float(np.max(err / np.maximum(sig, 1e-300))))


def check_refit_bounds(ivf, gix, wl, keys_f64, sample=None, seed=0):
    """Bound state of the newest refit epoch e against distances computed here in
    float64: every key's upper bound covers the distance to its assigned warm
    centroid, which is the nearest one (up to fp32 near ties), and its lower bound
    stays below the distance to every other live warm centroid.  The warm set of
    refit e is epoch e-1's centroids for slots below (e-1)*Q and the seal centroids
    above.  Returns (keys checked, fraction of the prefix the refit screened)."""
    info = ivf.idx_get_info(gix)
    e = info["computed_epoch"]
    assert e >= 1
    Q = info["slots_per_epoch"]
    cur = ivf.idx_export(gix, e)
    seal = ivf.idx_export(gix, -1)
    if e >= 2:
        prev = ivf.idx_export(gix, e - 1)
        warm = np.concatenate([prev["centroids"][:(e - 1) * Q], seal["centroids"][(e - 1) * Q:e * Q]])
        alive = np.concatenate([prev["sizes"][:(e - 1) * Q] > 0, seal["sizes"][(e - 1) * Q:e * Q] > 0])
    else:
        warm, alive = seal["centroids"][:Q], seal["sizes"][:Q] > 0
    warm = warm.astype(np.float64)
    S, nb = wl["n_sink"], cur["n_bound_keys"]
    assert nb == e * wl["refit_every"]
    idx = np.arange(nb)
    if sample is not None and sample < nb:
        idx = np.sort(np.random.default_rng(seed).choice(nb, sample, replace=False))
    X = keys_f64[S + idx]
    D2 = (X * X).sum(1)[:, None] + (warm * warm).sum(1)[None, :] - 2.0 * (X @ warm.T)
    D = np.sqrt(np.maximum(D2, 0.0))
    D[:, ~alive] = np.inf
    a = cur["assign"][idx]
    assert np.all((a >= 0) & (a < e * Q)) and np.all(alive[a]), "assigned to a dead or missing slot"
    rows = np.arange(idx.size)
    own = D[rows, a]
    assert np.all(own <= D.min(1) * (1 + 1e-6) + 1e-12), "assignment is not the nearest warm centroid"
    assert np.all(cur["ub"][idx] >= own * (1 - 1e-6)), "upper bound below the distance to the own centroid"
    D[rows, a] = np.inf
    other = D.min(1)
    lb = cur["lb"][idx].astype(np.float64)
    assert np.all(lb <= other * (1 + 1e-6) + 1e-12), "lower bound above the distance to another centroid"
    return idx.size, cur["n_screened"] / nb


def route_parity(name, budget=None, k=None, T=None, q_pos0=None, list_cap=0, **over):
    """Route the workload's queries on the GPU (with debug outputs) and check every
    query against the oracle's routing over the same index (check_routed_query)."""
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    if T is not None:
        over["T"] = T
    if q_pos0 is not None:
        over["q_pos0"] = q_pos0
    wl, inp = workload(name, **over)
    budget = wl["budget"] if budget is None else budget
    k = wl["k"] if k is None else k
    T, q_pos0 = wl["T"], wl["q_pos0"]
    dt = wl["dtype"]
    say(f"route {name} dtype={dt} T={T} q_pos0={q_pos0} k={k} budget={budget}")
    gix = gpu_index(wl, inp, max_budget=max(budget, wl["budget"]), max_queries=T, max_k=max(k, wl["k"]))
    try:
        oix = oracle_index(wl, inp)
        q = to_dev(inp["q"][:T])
        qs = to_dev(inp["q_scale"][:T]) if inp["q_scale"] is not None else None
        w = to_dev(inp["w"][:T])
        cfg = oix.cfg
        cand_cap = max(budget, cfg.n_sink + cfg.window) + 32
        n_slots = ((q_pos0 + T - cfg.n_sink) // cfg.window) * cfg.n_clusters
        dbg = ivf.make_route_debug(T, cand_cap, max(n_slots, 1), max(n_slots, 1))
        dbg["list_cap"] = list_cap
        idx, sc = ivf.idx_route_topk(gix, q, qs, w, q_pos0, k, budget, debug=dbg)
        torch.cuda.synchronize()
        idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
        d = {kk: v.cpu().numpy() for kk, v in dbg.items() if hasattr(v, "cpu")}
        d["topk_idx"], d["topk_score"] = idx, sc
        qraw = inp["q"][:T]
        qsc = None if inp["q_scale"] is None else inp["q_scale"][:T]
        ridx, rsc, odbg = oix.route(qraw, qsc, inp["w"][:T], q_pos0, k, budget, debug=True)
        qv = query_values(qraw, qsc, dt)
        wv = inp["w"][:T].astype(np.float64)
        stats = dict(order_swaps=0, topk_exempt=0, max_err=0.0)
        for t in range(T):
            check_routed_query(t, d, odbg[t], oix, qv, wv, k, budget, dt, stats)
        say(f"  ok {stats}")
        return stats
    finally:
        ivf.idx_destroy(gix)
