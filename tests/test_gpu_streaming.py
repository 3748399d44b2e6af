"""Streaming prefill: the index grows chunk by chunk while the chunk's own queries
are routed (AttentionIndex, paper-daily.com explainer, "索引怎么边算边建？": new keys
are candidates at once, windows seal as they fill, refits run on a side stream,
and a query only uses versions whose keys all lie in its prefix).

Protocol per chunk: insert the chunk's keys (sealing full windows), publish the
refit launched after the previous chunk (publication lag of one chunk), route the
chunk's queries, launch the next refit if one is due (side stream).

* reduced bf16 run: sampled queries of every chunk against the oracle following
  the same protocol;
* the 128K bf16 workload (16 chunks of 8192): every query's candidates lie in
  its prefix, its version is the one the protocol publishes, and the candidate
  count is min(prefix, max(budget, sinks + open window)); and 16 seeded queries of
  every chunk equal the oracle's routing over the clusters the library published
  (read back with idx_export: the sealed windows and the epochs the chunk uses).
"""
import numpy as np
import pytest

from gpu_common import check_routed_query, ensure_built, oracle_cfg, say, to_dev, workload
from oracle import OracleIndex, codec
from oracle.index import key_values, make_cluster, query_values

pytestmark = pytest.mark.gpu


def _exported_clusters(exp, dtype):
    out = []
    for s in range(exp["sizes"].shape[0]):
        sz, off = int(exp["sizes"][s]), int(exp["offsets"][s])
        out.append(make_cluster(s, exp["members"][off:off + sz].astype(np.int64), exp["centroids"][s], dtype))
    return out


def _stream(name, check_every=None, exported_every=None, seed=0, **over):
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload(name, **over)
    N, T, chunk, k, budget, dt = wl["N"], wl["N"], wl["chunk"], wl["k"], wl["budget"], wl["dtype"]
    S, W, R = wl["n_sink"], wl["window"], wl["refit_every"]
    wpr = R // W
    Cs = W // wl["cluster_size"]
    say(f"stream {name}: N={N} chunk={chunk} R={R} dtype={dt}")
    ix = ivf.idx_create(heads=wl["H"], dim=wl["d"], dtype=dt, max_keys=N, n_sink=S, window=W,
                        cluster_size=wl["cluster_size"], seal_cap=wl["seal_cap"], seal_iters=wl["seal_iters"],
                        refit_every=R, max_queries=chunk, max_budget=budget, max_k=k)
    side = torch.cuda.Stream()
    keys = to_dev(inp["keys"])
    ks = to_dev(inp["k_scale"]) if inp["k_scale"] is not None else None
    oix = OracleIndex(oracle_cfg(wl)) if check_every else None
    rng = np.random.default_rng(seed)
    stats = dict(order_swaps=0, topk_exempt=0, max_err=0.0)
    if exported_every:
        kv_all = key_values(inp["keys"], inp["k_scale"], dt)
        X_all = codec.dequantize(inp["keys"], inp["k_scale"], dt)
        n_exported = 0
    try:
        for c0 in range(0, N, chunk):
            c1 = min(N, c0 + chunk)
            n_q = c1 - c0
            ivf.idx_build_seal(ix, keys[c0:c1], None if ks is None else ks[c0:c1])
            P = ivf.idx_publish(ix)
            qd = to_dev(_queries(inp, c0, c1, wl))
            qsd = to_dev(_qscale(inp, c0, c1, wl))
            wd = to_dev(_weights(inp, c0, c1, wl))
            n_slots = max(1, ((c1 - S) // W) * Cs)
            dbg = ivf.make_route_debug(n_q, budget + W + 64, n_slots, n_slots)
            idx, sc = ivf.idx_route_topk(ix, qd, qsd, wd, c0, k, budget, debug=dbg)
            launched = ivf.idx_refit(ix, side_stream=side)
            torch.cuda.synchronize()
            d = {kk: v.cpu().numpy() for kk, v in dbg.items() if hasattr(v, "cpu")}
            d["topk_idx"], d["topk_score"] = idx.cpu().numpy(), sc.cpu().numpy()
            # properties of every query of the chunk
            n_t = c0 + 1 + np.arange(n_q)
            m_t = np.where(n_t >= S, (n_t - S) // W, 0)
            r_t = np.minimum(P, m_t // wpr)
            assert np.array_equal(d["version"][:, 0], r_t), f"chunk at {c0}: epoch per query"
            assert np.array_equal(d["version"][:, 1], m_t), f"chunk at {c0}: windows per query"
            open_t = np.maximum(0, n_t - (S + m_t * W))
            base = np.minimum(S, n_t) + open_t
            assert np.array_equal(d["cand_len"], np.minimum(n_t, np.maximum(budget, base)))
            cand = d["cand"][:, :budget + W + 64]
            valid = np.arange(cand.shape[1])[None, :] < d["cand_len"][:, None]
            assert np.all(np.where(valid, cand, 0) >= 0)
            assert np.all(np.where(valid, cand, -1).max(axis=1) < n_t), f"chunk at {c0}: a query sees a future key"
            rows = rng.choice(n_q, min(512, n_q), replace=False)
            srt = np.sort(np.where(valid[rows], cand[rows], -1), axis=1)
            dup = (srt[:, 1:] == srt[:, :-1]) & (srt[:, 1:] >= 0)
            assert not dup.any(), f"chunk at {c0}: repeated candidate"
            got = d["topk_idx"]
            assert np.all(np.where(got >= 0, got, -1).max(axis=1) < n_t)
            if oix is not None:
                oix.append(inp["keys"][c0:c1], None if inp["k_scale"] is None else inp["k_scale"][c0:c1])
                oix.publish()
                assert oix.published == P
                qv = query_values(_queries(inp, c0, c1, wl), _qscale(inp, c0, c1, wl), dt)
                wv = _weights(inp, c0, c1, wl).astype(np.float64)
                for t in np.sort(rng.choice(n_q, min(check_every, n_q), replace=False)):
                    _, _, od = oix.route(_queries(inp, c0 + t, c0 + t + 1, wl, base=c0),
                                         _qscale(inp, c0 + t, c0 + t + 1, wl, base=c0),
                                         _weights(inp, c0 + t, c0 + t + 1, wl, base=c0), c0 + int(t), k, budget,
                                         debug=True)
                    check_routed_query(int(t), d, od[0], oix, qv, wv, k, budget, dt, stats)
                if oix.refit_due() and oix.computed == oix.published:
                    oix.refit()
                assert launched == (oix.computed > oix.published)
            if exported_every:
                # the oracle routes over the clusters the library published: every sealed
                # window, and the epochs this chunk's queries use (synchronized above, so a
                # refit launched after the route has finished and wrote a newer epoch slot)
                eix = OracleIndex(oracle_cfg(wl))
                eix.kv, eix.X = kv_all, X_all
                seal = _exported_clusters(ivf.idx_export(ix, -1), dt)
                eix.seals = [seal[i:i + Cs] for i in range(0, len(seal), Cs)]
                for r in sorted(set(r_t.tolist())):
                    if r >= 1:
                        eix.epochs[r] = _exported_clusters(ivf.idx_export(ix, r), dt)
                eix.computed = eix.published = P
                qv = query_values(_queries(inp, c0, c1, wl), _qscale(inp, c0, c1, wl), dt)
                wv = _weights(inp, c0, c1, wl).astype(np.float64)
                for t in np.sort(rng.choice(n_q, min(exported_every, n_q), replace=False)):
                    _, _, od = eix.route(_queries(inp, c0 + t, c0 + t + 1, wl), _qscale(inp, c0 + t, c0 + t + 1, wl),
                                         _weights(inp, c0 + t, c0 + t + 1, wl), c0 + int(t), k, budget, debug=True)
                    check_routed_query(int(t), d, od[0], eix, qv, wv, k, budget, dt, stats)
                    n_exported += 1
        say(f"  ok, {N} queries; oracle comparisons {stats}"
            + (f"; {n_exported} of them over the exported clusters" if exported_every else ""))
    finally:
        ivf.idx_destroy(ix)


def _queries(inp, a, b, wl, base=None):
    # queries of positions [a, b) are rows [a, b) of the query array
    return inp["q"][a:b]


def _qscale(inp, a, b, wl, base=None):
    return None if inp["q_scale"] is None else inp["q_scale"][a:b]


def _weights(inp, a, b, wl, base=None):
    return inp["w"][a:b]


def test_streaming_parity_bf16_reduced():
    _stream("c3", check_every=96, N=20480, T=20480, chunk=2048, refit_every=4096, k=256, budget=2048, M=512)


def test_streaming_causality_128k_bf16():
    _stream("c3", check_every=None, exported_every=16, T=131072)
