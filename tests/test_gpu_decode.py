"""Decode-shaped routing (idx_route_topk_pos) against the CPU oracle.

After a prefill, keys arrive one per step (idx_build_seal with n = 1; windows seal
and refits run and are published as they fall due) and each step routes a batch
of queries at mixed positions: the newest token, its predecessor and tokens of
earlier positions, as a serving batch of several requests over one prefix would.
Every query is checked like the prefill routing (version, representative scores,
cluster order and takes, candidate list, exact top-k of the GPU's scores, top-k
of the oracle up to near ties)."""
import numpy as np
import pytest

from gpu_common import check_routed_query, ensure_built, oracle_cfg, say, to_dev, workload
from oracle import OracleIndex
from oracle.index import query_values

pytestmark = pytest.mark.gpu


def _decode(name, n_prefill, steps, k, budget, seed, **over):
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload(name, **over)
    N, dt = wl["N"], wl["dtype"]
    assert wl["q_pos0"] == 0 and wl["T"] == N   # a query for every position
    say(f"decode {name}: prefill {n_prefill}, {steps} steps, k={k} budget={budget}")
    ix = ivf.idx_create(heads=wl["H"], dim=wl["d"], dtype=dt, max_keys=N, n_sink=wl["n_sink"], window=wl["window"],
                        cluster_size=wl["cluster_size"], seal_cap=wl["seal_cap"], seal_iters=wl["seal_iters"],
                        refit_every=wl["refit_every"], max_queries=16, max_budget=budget, max_k=k)
    oix = OracleIndex(oracle_cfg(wl))
    keys = to_dev(inp["keys"])
    ks = to_dev(inp["k_scale"]) if inp["k_scale"] is not None else None
    q_all = to_dev(inp["q"])
    qs_all = to_dev(inp["q_scale"]) if inp["q_scale"] is not None else None
    w_all = to_dev(inp["w"])
    rng = np.random.default_rng(seed)
    stats = dict(order_swaps=0, topk_exempt=0, max_err=0.0)

    def insert(a, b):
        ivf.idx_build_seal(ix, keys[a:b], None if ks is None else ks[a:b])
        oix.append(inp["keys"][a:b], None if inp["k_scale"] is None else inp["k_scale"][a:b])
        while ivf.idx_refit(ix):
            ivf.idx_publish(ix)
        while oix.refit_due():
            oix.refit()
            oix.publish()

    try:
        insert(0, n_prefill)
        n = n_prefill
        for step in range(steps):
            insert(n, n + 1)
            n += 1
            earlier = rng.integers(0, n, size=5)
            pos = np.array([n - 1, n - 2, *earlier, 3])
            pt = torch.from_numpy(pos).to("cuda")
            q = q_all.index_select(0, pt)
            qs = qs_all.index_select(0, pt) if qs_all is not None else None
            w = w_all.index_select(0, pt)
            T = pos.size
            cfg = oix.cfg
            n_slots = ((n - cfg.n_sink) // cfg.window) * cfg.n_clusters
            dbg = ivf.make_route_debug(T, max(budget, cfg.n_sink + cfg.window) + 32, max(n_slots, 1), max(n_slots, 1))
            idx, sc = ivf.idx_route_topk_pos(ix, q, qs, w, pos, k, budget, debug=dbg)
            torch.cuda.synchronize()
            d = {kk: v.cpu().numpy() for kk, v in dbg.items() if hasattr(v, "cpu")}
            d["topk_idx"], d["topk_score"] = idx.cpu().numpy(), sc.cpu().numpy()
            qraw = inp["q"][pos]
            qsc = None if inp["q_scale"] is None else inp["q_scale"][pos]
            _, _, odbg = oix.route_at(qraw, qsc, inp["w"][pos], pos, k, budget, debug=True)
            qv = query_values(qraw, qsc, dt)
            wv = inp["w"][pos].astype(np.float64)
            for t in range(T):
                check_routed_query(t, d, odbg[t], oix, qv, wv, k, budget, dt, stats)
            assert np.all(d["topk_idx"].max(axis=1) <= pos), "a decode query saw a future key"
        say(f"  ok: {steps} steps to n={n}, epoch {oix.published}; {stats}")
    finally:
        ivf.idx_destroy(ix)


def test_decode_fp32_across_seals_and_refits():
    # 2040 prefill keys + 70 steps cross the seal of window 2 (keys up to 2052) and the
    # refit boundary S + 2048
    _decode("c1r", 2000, 70, 32, 512, seed=3, N=2200, T=2200, q_pos0=0)


def test_decode_bf16():
    # crosses the seal of window 8 (keys up to 9220)
    _decode("bf16_small", 9200, 40, 128, 2048, seed=4, N=9300, T=9300, q_pos0=0, refit_every=4096)


def test_decode_single_query_matches_prefill_route():
    """T = 1 at the newest position equals the same query routed by idx_route_topk."""
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload("c1r")
    from gpu_common import gpu_index
    gix = gpu_index(wl, inp)
    try:
        t = wl["T"] - 1
        p = wl["q_pos0"] + t
        q = to_dev(inp["q"][t:t + 1])
        w = to_dev(inp["w"][t:t + 1])
        a, sa = ivf.idx_route_topk(gix, q, None, w, p, wl["k"], wl["budget"])
        b, sb = ivf.idx_route_topk_pos(gix, q, None, w, [p], wl["k"], wl["budget"])
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(sa, sb)
    finally:
        ivf.idx_destroy(gix)
