"""GPU parity: routed top-k (idx_route_topk) against the CPU oracle.

Per query: the version (epoch, sealed windows, open window) must match exactly;
representative scores within the score tolerance; the ranked clusters and the
candidate list must equal the oracle's, except that clusters whose oracle
representative scores are within the tolerance of each other may swap (then the
oracle's fill, fed the GPU's cluster order, must reproduce the GPU's candidate
list exactly and the GPU's order must be a valid ranking); the top-k must be a
correct top-k of the candidates up to near ties, with scores within tolerance.
Also: a budget covering the prefix makes the routed output bit-identical to the
GPU's exhaustive output (same scores through the same score tile)."""
import numpy as np
import pytest

from gpu_common import (RTOL, check_routed_query, ensure_built, gpu_index, oracle_index, route_parity, say,
                        to_dev, topk_matches, workload)
from oracle import fill_budget
from oracle.index import query_values
from oracle.score import indexer_scores, score_error_scale

pytestmark = pytest.mark.gpu


def test_route_fp32_tiny():
    route_parity("c1")


def test_route_fp32_with_refits():
    route_parity("c1r")


def test_route_bf16():
    route_parity("bf16_small")


def test_route_e4m3():
    route_parity("e4m3_small")


def test_route_queries_straddling_windows_and_epochs():
    """Queries from before the first seal to past the second refit boundary in one
    call: several versions inside one chunk (epochs 0, 1 and 2, windows 0..7)."""
    route_parity("c1r", q_pos0=900, T=3300, budget=1200)


def test_route_full_cut_kernel():
    """A tiny list capacity sends most queries to the full (radix-select) cut kernel."""
    route_parity("c1r", list_cap=3)
    route_parity("e4m3_small", list_cap=5)


def test_route_sinks_and_open_window_exceed_budget():
    route_parity("c1r", budget=96, k=64, q_pos0=5000, T=200)


def test_route_budget_covering_prefix_is_exhaustive_bit_exact():
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload("bf16_small")
    T, q_pos0, k = 64, wl["N"] - 64, wl["k"]
    budget = 16384
    gix = gpu_index(wl, inp, max_budget=budget)
    try:
        q = to_dev(inp["q"][:T])
        w = to_dev(inp["w"][:T])
        idx, sc = ivf.idx_route_topk(gix, q, None, w, q_pos0, k, budget)
        eidx, esc = ivf.idx_exhaustive_topk(to_dev(inp["keys"]), None, "bf16", wl["H"], q, None, w, q_pos0, k)
        torch.cuda.synchronize()
        assert torch.equal(idx, eidx)
        assert torch.equal(sc.view(torch.int32), esc.view(torch.int32))
    finally:
        ivf.idx_destroy(gix)


@pytest.mark.parametrize("batch", [200, 64])
@pytest.mark.parametrize("zero_queries", [False, True])
def test_route_exact_ties(zero_queries, batch):
    """Integer-valued fp32 keys and queries give exactly equal scores (all zero when
    the queries are zero): GPU and oracle must then agree exactly, ties going to the
    lower position (the crowded-cut-bin and all-equal paths of the top-k).  Batches of
    64 run the small-batch kernels (split scoring, 1024-thread cut and selection)."""
    import torch
    import ivf_top_key_amd as ivf
    from oracle import OracleConfig, OracleIndex
    ensure_built()
    rng = np.random.default_rng(11)
    N, T, H, d, k, budget = 6000, 200, 4, 32, 300, 1500
    keys = rng.integers(-1, 2, (N, d)).astype(np.float32)
    q = np.zeros((T, H, d), np.float32) if zero_queries else rng.integers(0, 2, (T, H, d)).astype(np.float32)
    w = np.ones((T, H), np.float32)
    cfg = dict(heads=H, dim=d, dtype="f32", n_sink=4, window=1024, cluster_size=128, seal_cap=256,
               seal_iters=3, refit_every=2048)
    gix = ivf.idx_create(max_keys=N, max_queries=T, max_budget=budget, max_k=k, **cfg)
    try:
        kd = to_dev(keys)
        ivf.idx_build_seal(gix, kd)
        while ivf.idx_refit(gix):
            ivf.idx_publish(gix)
        q_pos0 = N - T
        qd, wd = to_dev(q), to_dev(w)
        parts = []
        for a in range(0, T, batch):
            b = min(T, a + batch)
            parts.append(ivf.idx_route_topk(gix, qd[a:b], None, wd[a:b], q_pos0 + a, k, budget))
        torch.cuda.synchronize()
        idx = torch.cat([pp[0] for pp in parts])
        sc = torch.cat([pp[1] for pp in parts])
        oix = OracleIndex(OracleConfig(**cfg))
        oix.append(keys)
        while oix.refit_due():
            oix.refit()
            oix.publish()
        ridx, rsc = oix.route(q, None, w, q_pos0, k, budget)
        assert np.array_equal(idx.cpu().numpy(), ridx)
        assert np.array_equal(sc.cpu().numpy().astype(np.float64), rsc)
    finally:
        ivf.idx_destroy(gix)


@pytest.mark.parametrize("name", ["bf16_small", "e4m3_small"])
def test_route_positional_blocks(name):
    """The same routing over position blocks (the block-routing baseline)."""
    route_parity(name, positional=True, refit_every=0)


@pytest.mark.parametrize("name,over", [
    ("c1", {}),
    ("bf16_small", {}),
    ("e4m3_small", dict(T=300, q_pos0=11000)),
])
def test_route_rescore_modes_bit_identical(name, over):
    """The fused cut + rescoring kernel (auto), query-major rescoring from a candidate
    list in memory and cluster-major rescoring give the same candidates, scores and
    top-k bits."""
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload(name, **over)
    T, k, budget = wl["T"], wl["k"], wl["budget"]
    q = to_dev(inp["q"])
    qs = to_dev(inp["q_scale"]) if inp["q_scale"] is not None else None
    w = to_dev(inp["w"])
    out = {}
    for mode in ("auto", "query", "cluster"):
        ix = gpu_index(wl, inp, rescore=mode)
        try:
            dbg = ivf.make_route_debug(T, budget + wl["window"] + 64, 8, 8)
            idx, sc = ivf.idx_route_topk(ix, q, qs, w, wl["q_pos0"], k, budget, debug=dbg)
            torch.cuda.synchronize()
            out[mode] = (idx.cpu().numpy(), sc.cpu().numpy(), dbg["cand"].cpu().numpy(),
                         dbg["cand_scores"].cpu().numpy(), dbg["cand_len"].cpu().numpy())
        finally:
            ivf.idx_destroy(ix)
    a = out["query"]
    for other in ("auto", "cluster"):
        b = out[other]
        assert np.array_equal(a[4], b[4]), f"{other}: candidate counts differ"
        for t in range(T):
            L = int(a[4][t])
            assert np.array_equal(a[2][t, :L], b[2][t, :L]), f"{other}, query {t}: candidate lists differ"
            assert np.array_equal(a[3][t, :L].view(np.uint32), b[3][t, :L].view(np.uint32)), \
                f"{other}, query {t}: scores differ"
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32)), \
            f"{other}: top-k differs"
    say(f"  {name}: {T} queries, fused, query-major and cluster-major bit-identical")


@pytest.mark.parametrize("name", ["c1r", "e4m3_small"])
def test_route_small_batches_bit_identical(name):
    """Batches of at most 64 queries score their candidates with blocks that split
    each list; the outputs must equal those of one large batch bit for bit."""
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload(name)
    T, k, budget, q_pos0 = 160, wl["k"], wl["budget"], wl["q_pos0"]
    q = to_dev(inp["q"][:T])
    qs = to_dev(inp["q_scale"][:T]) if inp["q_scale"] is not None else None
    w = to_dev(inp["w"][:T])
    ix = gpu_index(wl, inp, max_queries=max(T, wl["T"]))
    try:
        cap = budget + wl["window"] + 64
        dbg = ivf.make_route_debug(T, cap, 8, 8)
        idx, sc = ivf.idx_route_topk(ix, q, qs, w, q_pos0, k, budget, debug=dbg)
        torch.cuda.synchronize()
        big = (idx.cpu().numpy(), sc.cpu().numpy(), dbg["cand_scores"].cpu().numpy(), dbg["cand_len"].cpu().numpy())
        parts = []
        for a, b in ((0, 64), (64, 65), (65, 100), (100, 160)):
            d2 = ivf.make_route_debug(b - a, cap, 8, 8)
            i2, s2 = ivf.idx_route_topk(ix, q[a:b], None if qs is None else qs[a:b], w[a:b], q_pos0 + a, k, budget,
                                        debug=d2)
            torch.cuda.synchronize()
            parts.append((i2.cpu().numpy(), s2.cpu().numpy(), d2["cand_scores"].cpu().numpy(),
                          d2["cand_len"].cpu().numpy()))
        small = [np.concatenate([pp[i] for pp in parts]) for i in range(4)]
        assert np.array_equal(big[3], small[3])
        for t in range(T):
            L = int(big[3][t])
            assert np.array_equal(big[2][t, :L].view(np.uint32), small[2][t, :L].view(np.uint32)), f"query {t}"
        assert np.array_equal(big[0], small[0]) and np.array_equal(big[1].view(np.uint32), small[1].view(np.uint32))
        say(f"  {name}: {T} queries as one batch and as batches of 64, 1, 35 and 60: bit-identical")
    finally:
        ivf.idx_destroy(ix)


def test_route_overflow_list_across_calls():
    """The fused kernel hands queries whose short cluster list overflows to the
    overflow kernel through a device list that each call leaves empty.  Calls in a
    row that alternate between many overflowing queries (a cluster-list capacity of
    3) and none, over queries from before the first seal to past two refits, give
    the bits of the list-based path every time."""
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload("c1r", q_pos0=900, T=3300)
    T, k, budget, q_pos0 = wl["T"], wl["k"], 1200, wl["q_pos0"]
    q = to_dev(inp["q"][:T])
    w = to_dev(inp["w"][:T])
    ref = {}
    ix = gpu_index(wl, inp, rescore="query", max_queries=T, max_budget=budget)
    try:
        for cap in (0, 3):
            idx, sc = ivf.idx_route_topk(ix, q, None, w, q_pos0, k, budget, debug={"list_cap": cap})
            torch.cuda.synchronize()
            ref[cap] = (idx.cpu().numpy(), sc.cpu().numpy())
    finally:
        ivf.idx_destroy(ix)
    assert np.array_equal(ref[0][0], ref[3][0]) and np.array_equal(ref[0][1].view(np.uint32), ref[3][1].view(np.uint32))
    ix = gpu_index(wl, inp, rescore="auto", max_queries=T, max_budget=budget)
    try:
        for call, cap in enumerate((3, 0, 3, 3, 0)):
            idx, sc = ivf.idx_route_topk(ix, q, None, w, q_pos0, k, budget, debug={"list_cap": cap})
            torch.cuda.synchronize()
            assert np.array_equal(idx.cpu().numpy(), ref[cap][0]), f"call {call} (list capacity {cap}): top-k differs"
            assert np.array_equal(sc.cpu().numpy().view(np.uint32), ref[cap][1].view(np.uint32)), \
                f"call {call} (list capacity {cap}): scores differ"
    finally:
        ivf.idx_destroy(ix)
    say(f"  {T} queries, five calls alternating overflow and none: fused = list-based, bit for bit")


def test_route_debug_events_null_entries_skipped():
    """Timing events in the debug struct: all eight marks, or only some (NULL entries
    are not recorded), leave the outputs bit-identical to a call without events, and
    the recorded marks give ordered, non-negative spans."""
    import ctypes
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload("e4m3_small")
    T, k, budget, q_pos0 = wl["T"], wl["k"], wl["budget"], wl["q_pos0"]
    q = to_dev(inp["q"])
    qs = to_dev(inp["q_scale"])
    w = to_dev(inp["w"])
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]

    def event():
        ev = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def elapsed(a, b):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    ix = gpu_index(wl, inp)
    try:
        runs = {}
        all8 = [event() for _ in range(8)]
        some = [event(), None, event(), event(), None, None, None, None]
        for name, dbg in (("none", None), ("all", {"events": all8}), ("some", {"events": some})):
            idx, sc = ivf.idx_route_topk(ix, q, qs, w, q_pos0, k, budget, debug=dbg)
            torch.cuda.synchronize()
            runs[name] = (idx.cpu().numpy(), sc.cpu().numpy())
        for name in ("all", "some"):
            assert np.array_equal(runs["none"][0], runs[name][0]), name
            assert np.array_equal(runs["none"][1].view(np.uint32), runs[name][1].view(np.uint32)), name
        spans = [elapsed(all8[i], all8[i + 1]) for i in range(7)]
        assert all(x >= 0.0 for x in spans), spans
        assert elapsed(some[0], some[2]) >= 0.0 and elapsed(some[2], some[3]) > 0.0
        say(f"  {T} queries: outputs unchanged by events; spans (ms) {[round(x, 4) for x in spans]}")
        for e in all8 + [e for e in some if e]:
            hip.hipEventDestroy(ctypes.c_void_p(e))
    finally:
        ivf.idx_destroy(ix)
