"""Learned representatives (idx_set_encoder) against the CPU oracle.

paper-daily explainer, "代表向量为什么要学？": the encoder only replaces the
representative.  Checked on seal clusters and refit epochs: members and centroids
bit-exact as without an encoder; the fp32 representative within 1e-4 of the
oracle's float64 encoder output (the network sums a few hundred fp32 products and
applies tanh); the key-format representative is exactly the quantization of the
library's own fp32 representative; routing over the library's learned
representatives matches the oracle's routing over the same clusters."""
import numpy as np
import pytest

import datagen
from gpu_common import check_routed_query, ensure_built, oracle_cfg, say, to_dev, workload
from oracle import OracleIndex, codec
from oracle.encoder import encode
from oracle.index import Cluster, query_values

pytestmark = pytest.mark.gpu

ATOL = 1e-4


def _compare(got, clusters, X, weights, dt, label):
    worst = 0.0
    for c in clusters:
        s = c.slot
        sz = int(got["sizes"][s])
        assert sz == c.members.size, f"{label}: slot {s} size"
        if not sz:
            continue
        off = int(got["offsets"][s])
        assert np.array_equal(got["members"][off:off + sz], c.members), f"{label}: slot {s} members"
        assert np.array_equal(got["centroids"][s].view(np.uint32), c.centroid.view(np.uint32)), f"{label}: slot {s}"
        ref = encode(X[c.members], c.centroid, weights)
        err = np.abs(got["rep_f32"][s].astype(np.float64) - ref).max()
        worst = max(worst, err)
        assert err <= ATOL, f"{label}: slot {s} learned representative off by {err:.3g}"
        raw, sc = codec.quantize_rep(got["rep_f32"][s], dt)
        assert np.array_equal(got["reps"][s], raw) and np.float32(got["rep_scale"][s]) == sc, \
            f"{label}: slot {s} key-format representative"
    return worst


def _clusters_from(exp, dt):
    out = []
    for s in range(exp["sizes"].shape[0]):
        sz, off = int(exp["sizes"][s]), int(exp["offsets"][s])
        raw, sc = exp["reps"][s], np.float32(exp["rep_scale"][s])
        value = codec.decode_codes(raw, dt).astype(np.float64) * np.float64(sc)
        out.append(Cluster(s, exp["members"][off:off + sz].astype(np.int64), exp["centroids"][s].copy(), raw.copy(),
                           sc, value))
    return out


@pytest.mark.parametrize("name", ["c1r", "bf16_small", "e4m3_small"])
def test_learned_representatives(name):
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload(name)
    dt, d = wl["dtype"], wl["d"]
    weights = datagen.encoder_weights(17, d, alpha=0.25)
    say(f"encoder {name}: N={wl['N']} dtype={dt} R={wl['refit_every']}")
    ix = ivf.idx_create(heads=wl["H"], dim=d, dtype=dt, max_keys=wl["N"], n_sink=wl["n_sink"],
                        window=wl["window"], cluster_size=wl["cluster_size"], seal_cap=wl["seal_cap"],
                        seal_iters=wl["seal_iters"], refit_every=wl["refit_every"], max_queries=wl["T"],
                        max_budget=wl["budget"], max_k=wl["k"])
    try:
        ivf.idx_set_encoder(ix, to_dev(weights))
        keys = to_dev(inp["keys"])
        ks = to_dev(inp["k_scale"]) if inp["k_scale"] is not None else None
        for a in range(0, wl["N"], 3000):
            b = min(wl["N"], a + 3000)
            ivf.idx_build_seal(ix, keys[a:b], None if ks is None else ks[a:b])
            while ivf.idx_refit(ix):
                ivf.idx_publish(ix)
        cfg = oracle_cfg(wl)
        cfg.encoder = weights
        oix = OracleIndex(cfg)
        oix.append(inp["keys"], inp["k_scale"])
        while oix.refit_due():
            oix.refit()
            oix.publish()
        seal = ivf.idx_export(ix, -1)
        worst = _compare(seal, [c for w in oix.seals for c in w], oix.X, weights, dt, f"{name} seal")
        P = oix.published
        if P >= 1:
            ep = ivf.idx_export(ix, P)
            worst = max(worst, _compare(ep, oix.epochs[P], oix.X, weights, dt, f"{name} epoch {P}"))
        # routing over the library's learned representatives
        gix_seals = _clusters_from(seal, dt)
        Cs = cfg.n_clusters
        oix.seals = [gix_seals[i:i + Cs] for i in range(0, len(gix_seals), Cs)]
        if P >= 1:
            oix.epochs[P] = _clusters_from(ep, dt)
        T, k, budget, q_pos0 = wl["T"], wl["k"], wl["budget"], wl["q_pos0"]
        q = to_dev(inp["q"])
        qs = to_dev(inp["q_scale"]) if inp["q_scale"] is not None else None
        w = to_dev(inp["w"])
        n_slots = ((q_pos0 + T - cfg.n_sink) // cfg.window) * Cs
        dbg = ivf.make_route_debug(T, max(budget, cfg.n_sink + cfg.window) + 32, n_slots, n_slots)
        idx, sc = ivf.idx_route_topk(ix, q, qs, w, q_pos0, k, budget, debug=dbg)
        torch.cuda.synchronize()
        dd = {kk: v.cpu().numpy() for kk, v in dbg.items() if hasattr(v, "cpu")}
        dd["topk_idx"], dd["topk_score"] = idx.cpu().numpy(), sc.cpu().numpy()
        _, _, odbg = oix.route(inp["q"], inp["q_scale"], inp["w"], q_pos0, k, budget, debug=True)
        qv = query_values(inp["q"], inp["q_scale"], dt)
        wv = inp["w"].astype(np.float64)
        stats = dict(order_swaps=0, topk_exempt=0, max_err=0.0)
        for t in range(T):
            check_routed_query(t, dd, odbg[t], oix, qv, wv, k, budget, dt, stats)
        say(f"  ok: representative error <= {worst:.2e}; routing {stats}")
    finally:
        ivf.idx_destroy(ix)
