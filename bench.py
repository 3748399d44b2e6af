"""Benchmark: routed indexer top-k at a 1M-token prefix on one MI355X.

Workload (synthetic, seeded; the pages' models and datasets are not available):
1,048,576 E4M3 keys with per-token fp32 scales, H=64 heads, d=128, 4096 queries at
the tail of the prefix (positions 1,044,480 .. 1,048,575), k=2048, budget 8192.
The index is built first (untimed; its seal and refit costs are reported apart),
then one step = one idx_route_topk call over the 4096 queries: version select,
representative scores, cluster cut + fill, candidate rescoring + top-k.

Reported next to the routed throughput: the exhaustive top-k time on the same
queries (our own baseline), recall of routed vs exhaustive, a budget sweep
(4096 / 8192 / 16384), per-kernel times from HIP events recorded around each
kernel during the timed steps, the roofline of the dominant kernel, and the CPU
oracle timed on a bounded sample of the same queries.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routed top-k queries/s at 1M-token prefix, k=2048, 8K budget; recall vs exhaustive"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3


PMC_SUMMARY = os.path.join(ROOT, "profiles", "route_rescore_c4_e4m3_pmc.md")
PMC_KERNEL = "route_rescore"
PMC_SOURCES = ("rescore.h", "cut.h", "routing.h", "dev.h", "params.h")
PMC_FETCH_SCALE = 2.0    # FETCH_SIZE read 524,316 KiB for a copy that reads 1,048,576 KiB
PMC_WRITE_SCALE = 1.0    # WRITE_SIZE read the 1,048,576 KiB the copy writes


def kernel_source_hash():
    """First 16 hex digits of the sha256 over the sources the rescoring kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for f in PMC_SOURCES:
        with open(os.path.join(ROOT, "ivf_top_key_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, budget):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a 1 GiB copy), or None when the summary
    is for another kernel or workload or the kernel's sources changed since."""
    if kernel != PMC_KERNEL or workload != "c4" or budget != 8192 or not os.path.exists(PMC_SUMMARY):
        return None
    vals = {}
    with open(PMC_SUMMARY) as fh:
        for line in fh:
            if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "source_sha256_16"):
                key, v = line.split(":", 1)
                vals[key] = v.strip()
    if vals.get("source_sha256_16") != kernel_source_hash():
        return None
    return float(vals["traffic_bytes_per_launch"])


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Hip:
    """hipEvent helpers through the HIP runtime that torch already loaded."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def elapsed(self, a, b):
        ms = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    def sync(self, ev):
        self.h.hipEventSynchronize(ctypes.c_void_p(ev))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c4")
    ap.add_argument("--budget", type=int, default=8192)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--ablation", action="store_true",
                    help="also measure recall vs prefix length for seal-only, refit intervals and position blocks")
    ap.add_argument("--no-exhaustive", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rescore", default="auto", choices=["auto", "query", "cluster"],
                    help="candidate rescoring: query-major gathers (auto) or cluster-major")
    ap.add_argument("--cpu-sample", type=int, default=1024)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB elementwise copy (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by query with no exchange; see the design notes)", flush=True)
        sys.exit(2)

    import torch
    import datagen
    from datagen.workloads import WORKLOADS
    import ivf_top_key_amd as ivf
    from ivf_top_key_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from ivf_top_key_amd.build import build
        build()

    wl = dict(WORKLOADS[args.workload])
    N, T, H, d, k, dt = wl["N"], wl["T"], wl["H"], wl["d"], wl["k"], wl["dtype"]
    q_pos0, R, W = wl["q_pos0"], wl["refit_every"], wl["window"]
    budget = args.budget
    dev = torch.device("cuda:0")
    hip = Hip()

    t0 = time.time()
    inp = datagen.workload_inputs(wl["seed"], N, T, q_pos0, H, d, wl["M"], dt)
    log(f"inputs generated in {time.time() - t0:.1f}s")
    keys = torch.from_numpy(inp["keys"]).to(dev)
    ks = torch.from_numpy(inp["k_scale"]).to(dev) if inp["k_scale"] is not None else None
    q = torch.from_numpy(np.ascontiguousarray(inp["q"])).to(dev)
    qs = torch.from_numpy(inp["q_scale"]).to(dev) if inp["q_scale"] is not None else None
    w = torch.from_numpy(inp["w"]).to(dev)

    # ---- build the index by streaming the prefix, R keys at a time ----
    ix = ivf.idx_create(heads=H, dim=d, dtype=dt, max_keys=N, n_sink=wl["n_sink"], window=W,
                        cluster_size=wl["cluster_size"], seal_cap=wl["seal_cap"], seal_iters=wl["seal_iters"],
                        refit_every=R, max_queries=T, max_budget=16384, max_k=k, rescore=args.rescore)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    t0 = time.time()
    seal_ms, refit_ms = [], []
    for a in range(0, N, R):
        b = min(N, a + R)
        e0, e1 = hip.event(), hip.event()
        hip.h.hipEventRecord(ctypes.c_void_p(e0), ctypes.c_void_p(stream.cuda_stream))
        ivf.idx_build_seal(ix, keys[a:b], None if ks is None else ks[a:b])
        hip.h.hipEventRecord(ctypes.c_void_p(e1), ctypes.c_void_p(stream.cuda_stream))
        r0, r1 = hip.event(), hip.event()
        hip.h.hipEventRecord(ctypes.c_void_p(r0), ctypes.c_void_p(stream.cuda_stream))
        launched = ivf.idx_refit(ix, stream=stream, side_stream=side)
        hip.h.hipEventRecord(ctypes.c_void_p(r1), ctypes.c_void_p(side.cuda_stream))
        ivf.idx_publish(ix, stream=stream)
        hip.sync(e1)
        hip.sync(r1)
        seal_ms.append((hip.elapsed(e0, e1), (b - a) // W))
        if launched:
            refit_ms.append(hip.elapsed(r0, r1))
    torch.cuda.synchronize()
    build_s = time.time() - t0
    info = ivf.idx_get_info(ix)
    log(f"index built in {build_s:.2f}s: {info}")
    screened = None
    if info["computed_epoch"] >= 1:
        ex = ivf.idx_export(ix, info["computed_epoch"])
        screened = dict(keys=ex["n_bound_keys"], screened=ex["n_screened"], brute=ex["n_brute"])
        del ex

    if args.copy_calibration:
        # a plain copy of known size: 1 GiB read + 1 GiB written
        xa = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        ya = torch.empty_like(xa)
        torch.mul(xa, 1.0, out=ya)
        torch.cuda.synchronize()
        del xa, ya

    # ---- routed steps ----
    out_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    out_sc = torch.empty((T, k), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        ivf.idx_route_topk(ix, q, qs, w, q_pos0, k, budget, out_idx, out_sc)
    torch.cuda.synchronize()
    # timed region: K steps, with HIP events recorded by the library around each kernel
    # on its launch stream (per-kernel times and the roofline's launch duration come
    # from the same steps as the throughput).  The library records events in pairs
    # around its four stages; with the default mode and more than 64 queries the cut,
    # rescoring and top-k run as one kernel, so only three marks are recorded (every
    # record costs stream time): the start, the start of the fused kernel (the
    # representative scores' span includes the launch gap) and its end.  The overflow
    # launch that follows (queries whose short cluster list overflowed: none here) is
    # inside the step but not timed on its own.
    fused = args.rescore == "auto" and T > 64 and max(budget, wl["n_sink"] + W) <= 8192
    if fused:
        evs = [[hip.event(), None, hip.event(), hip.event(), None, None, None, None] for _ in range(args.steps)]
    else:
        evs = [[hip.event() for _ in range(8)] for _ in range(args.steps)]
    start, stop = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.h.hipEventRecord(ctypes.c_void_p(start), ctypes.c_void_p(stream.cuda_stream))
    for s in range(args.steps):
        ivf.idx_route_topk(ix, q, qs, w, q_pos0, k, budget, out_idx, out_sc, debug={"events": evs[s]})
    hip.h.hipEventRecord(ctypes.c_void_p(stop), ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    ms_per_step = hip.elapsed(start, stop) / args.steps
    if fused:
        names = ["rep_score", "route_rescore"]
        kern = {"rep_score": float(np.mean([hip.elapsed(e[0], e[2]) for e in evs])),
                "route_rescore": float(np.mean([hip.elapsed(e[2], e[3]) for e in evs]))}
    else:
        names = ["rep_score", "route_select", "cluster_score", "rescore_topk"]
        kern = {n: float(np.mean([hip.elapsed(e[2 * i], e[2 * i + 1]) for e in evs])) for i, n in enumerate(names)}
    value = T / (ms_per_step / 1e3)
    log(f"routed: {ms_per_step:.3f} ms/step, {value:.0f} q/s; kernels {kern}")

    # ---- algorithmic work of one step ----
    Cs = W // wl["cluster_size"]
    S = wl["n_sink"]
    n_t = q_pos0 + 1 + np.arange(T, dtype=np.int64)
    m_t = (n_t - S) // W
    c_vis = m_t * Cs
    open_t = n_t - S - m_t * W
    base_t = np.minimum(n_t, S) + open_t                      # sinks + open window
    cand_t = np.minimum(n_t, np.maximum(budget, base_t))
    clus_t = cand_t - base_t                                  # candidates from selected clusters
    rb = d * {"f32": 4, "bf16": 2, "e4m3": 1}[dt]
    scale_b = 4 if dt == "e4m3" else 0
    peak_mfma = {"e4m3": FP8_PEAK_TFLOPS, "bf16": BF16_PEAK_TFLOPS, "f32": FP32_PEAK_TFLOPS}[dt]
    work = {
        # contractions: flops against the MFMA peak of the format
        "rep_score": ("mfma", float(2 * H * d * c_vis.sum())),
        "cluster_score": ("mfma", float(2 * H * d * clus_t.sum())),
        # cut + fill: read each query's representative scores and the visible clusters'
        # sizes (one array shared by every query, counted once), write its list (the
        # gather row of every candidate)
        "route_select": ("hbm", float((c_vis * 4).sum() + c_vis.max() * 4 + cand_t.sum() * 4)),
    }
    if fused:
        # the cut's reads (each query's representative scores; the visible clusters'
        # sizes, one array shared by every query, counted once) and the method's
        # rescoring bytes: every candidate's key row and scale, the query (row, head
        # weight and scale per head), the top-k written (position and score); the
        # member positions this design also reads are not counted
        work["route_rescore"] = ("hbm", float((c_vis * 4).sum() + c_vis.max() * 4 + cand_t.sum() * (rb + scale_b)
                                              + T * H * (rb + 8) + T * k * 8))
        work["split_score"] = ("mfma", 0.0)
        work["overflow_path"] = ("hbm", 0.0)
    elif args.rescore == "cluster":
        # sink / open-window rows gathered and scored, cluster scores and positions read, top-k written
        work["rescore_topk"] = ("hbm", float(base_t.sum() * (rb + scale_b + 8) + clus_t.sum() * 8
                                             + T * H * (rb + 8) + T * k * 8))
    else:
        # the method's bytes: every candidate's key row and scale, the query (row, head
        # weight and scale per head), the top-k written (position and score); the gather
        # rows and member positions this design also reads are not counted
        work["rescore_topk"] = ("hbm", float(cand_t.sum() * (rb + scale_b) + T * H * (rb + 8) + T * k * 8))
        work["cluster_score"] = ("mfma", 0.0)
    rescore_flops = float(2 * H * d * cand_t.sum())
    keys_scored = float((c_vis + cand_t).sum())

    def roof_of(name):
        bound, amount = work[name]
        sec = kern[name] * 1e-3
        if bound == "mfma":
            ach = amount / sec / 1e12
            return dict(kernel=name, bound="mfma", achieved=round(ach, 2), peak=peak_mfma, unit="TFLOP/s",
                        frac=round(ach / peak_mfma, 4), traffic=None, algorithmic_flops=amount,
                        avg_launch_ms=round(kern[name], 4))
        ach = amount / sec / 1e9
        traffic = measured_traffic(name, args.workload, budget)
        out = dict(kernel=name, bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                   frac=round(ach / HBM_PEAK_GBS, 4), traffic=traffic, algorithmic_bytes=amount,
                   avg_launch_ms=round(kern[name], 4))
        if traffic is not None:
            out["traffic_calibration"] = {"FETCH_SIZE": PMC_FETCH_SCALE, "WRITE_SIZE": PMC_WRITE_SCALE,
                                          "from": "one 1 GiB elementwise copy in the profiled process"}
        return out

    dominant = max(kern, key=kern.get)
    roof = roof_of(dominant)
    if fused and dominant == "route_rescore":
        # the candidates' contraction against the MFMA peak of the format, next to the
        # bytes that bound the kernel
        roof["algorithmic_flops"] = rescore_flops
        roof["mfma_frac"] = round(rescore_flops / (kern[dominant] * 1e-3) / 1e12 / peak_mfma, 4)
    kernel_roofs = {n: {kk: v for kk, v in roof_of(n).items() if kk in ("bound", "achieved", "unit", "frac")}
                    for n in names if work[n][1] > 0}

    # ---- exhaustive baseline + recall ----
    extra = {}
    if not args.no_exhaustive:
        # one pass: the streamed selection needs about 200 KB per query, not a score row
        ws = torch.empty(ivf.idx_exhaustive_workspace_bytes(q_pos0 + T, T) // 4, dtype=torch.float32, device=dev)
        e_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        e_sc = torch.empty((T, k), dtype=torch.float32, device=dev)
        ivf.idx_exhaustive_topk(keys, ks, dt, H, q, qs, w, q_pos0, k, e_idx, e_sc, workspace=ws)
        torch.cuda.synchronize()
        reps = 2
        a0, a1 = hip.event(), hip.event()
        hip.h.hipEventRecord(ctypes.c_void_p(a0), ctypes.c_void_p(stream.cuda_stream))
        for _ in range(reps):
            ivf.idx_exhaustive_topk(keys, ks, dt, H, q, qs, w, q_pos0, k, e_idx, e_sc, workspace=ws)
        hip.h.hipEventRecord(ctypes.c_void_p(a1), ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        exh_ms = hip.elapsed(a0, a1) / reps
        exh_flops = float(2 * H * d * n_t.sum())
        r_np, e_np = out_idx.cpu().numpy(), e_idx.cpu().numpy()
        rec = summarize(recall_per_query(r_np, e_np))
        extra.update(exhaustive_ms=round(exh_ms, 3), exhaustive_qps=round(T / (exh_ms * 1e-3), 1),
                     exhaustive_tflops=round(exh_flops / (exh_ms * 1e-3) / 1e12, 1),
                     routed_speedup_vs_exhaustive=round(exh_ms / ms_per_step, 2), recall=rec)
        log(f"exhaustive {exh_ms:.2f} ms, speedup {exh_ms / ms_per_step:.2f}x, recall {rec}")
        if not args.no_sweep:
            sweep = {}
            for B in (4096, 8192, 16384):
                for _ in range(5):
                    ivf.idx_route_topk(ix, q, qs, w, q_pos0, k, B, out_idx, out_sc)
                b0, b1 = hip.event(), hip.event()
                hip.h.hipEventRecord(ctypes.c_void_p(b0), ctypes.c_void_p(stream.cuda_stream))
                for _ in range(10):
                    ivf.idx_route_topk(ix, q, qs, w, q_pos0, k, B, out_idx, out_sc)
                hip.h.hipEventRecord(ctypes.c_void_p(b1), ctypes.c_void_p(stream.cuda_stream))
                torch.cuda.synchronize()
                bms = hip.elapsed(b0, b1) / 10
                rb_ = summarize(recall_per_query(out_idx.cpu().numpy(), e_np))
                sweep[str(B)] = dict(ms=round(bms, 3), qps=round(T / (bms * 1e-3), 1), recall=rb_,
                                     speedup_vs_exhaustive=round(exh_ms / bms, 2))
                log(f"budget {B}: {bms:.3f} ms, recall {rb_}")
            extra["budget_sweep"] = sweep
        del ws

    # ---- decode-shaped routing: batches of queries at scattered positions ----
    rng = np.random.default_rng(5)
    dec = {}
    for B in (1, 64):
        pos = (N - 1 - rng.integers(0, 32768, size=B)).astype(np.int64)   # the two newest epochs
        sel = torch.from_numpy(rng.integers(0, T, size=B)).to(dev)
        qb = q.index_select(0, sel)
        qsb = qs.index_select(0, sel) if qs is not None else None
        wb = w.index_select(0, sel)
        for _ in range(3):
            ivf.idx_route_topk_pos(ix, qb, qsb, wb, pos, k, budget)
        d0, d1 = hip.event(), hip.event()
        hip.h.hipEventRecord(ctypes.c_void_p(d0), ctypes.c_void_p(stream.cuda_stream))
        for _ in range(20):
            ivf.idx_route_topk_pos(ix, qb, qsb, wb, pos, k, budget)
        hip.h.hipEventRecord(ctypes.c_void_p(d1), ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        dms = hip.elapsed(d0, d1) / 20
        devs = [[hip.event() for _ in range(8)] for _ in range(10)]
        for e in devs:
            ivf.idx_route_topk_pos(ix, qb, qsb, wb, pos, k, budget, debug={"events": e})
        torch.cuda.synchronize()
        dnames = ["rep_score", "route_select", "split_score", "rescore_topk"]
        dk = {n: round(float(np.mean([hip.elapsed(e[2 * i], e[2 * i + 1]) for e in devs])), 4)
              for i, n in enumerate(dnames)}
        dec[str(B)] = dict(ms_per_call=round(dms, 4), queries_per_s=round(B / (dms * 1e-3), 1), kernels_ms=dk)
    extra["decode_batches"] = dec
    log(f"decode batches {dec}")

    if args.ablation:
        extra["ablation"] = ablation(ivf, torch, wl, inp, keys, ks, q, qs, w, dev, budget, k)

    # ---- CPU oracle on a bounded sample of the same queries ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(ix, inp, wl, budget, args.cpu_sample)
        log(f"cpu baseline {cpu}")

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": f"{'1M' if N == 1 << 20 else str(N // 1024) + 'K'}-token prefix ({N} keys), {dt} "
                               f"keys+queries{' with fp32 scales' if dt == 'e4m3' else ''}, H={H}, d={d}, "
                               f"{T} tail queries, k={k}, budget {budget}",
                   "global_batch": T, "seq_len": N, "parallelism": "single GPU",
                   "rescore": "query-major" if args.rescore != "cluster" else "cluster-major"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "keys_scored_per_s": round(keys_scored / (ms_per_step * 1e-3), 1),
        "kernels_ms": {kk: round(v, 4) for kk, v in kern.items()},
        "kernel_rooflines": kernel_roofs,
        "candidate_scoring_tflops": round(rescore_flops / (sum(kern[n] for n in names[1:]) * 1e-3) / 1e12, 1),
        "maintenance": {
            "build_s": round(build_s, 3),
            "seal_ms_per_window_last_chunk": round(seal_ms[-1][0] / max(1, seal_ms[-1][1]), 4),
            "refits": len(refit_ms),
            "refit_ms_last": round(refit_ms[-1], 3) if refit_ms else None,
            "refit_ms_mean": round(float(np.mean(refit_ms)), 3) if refit_ms else None,
            "last_refit_keys": screened,
        },
        **extra,
    }
    ivf.idx_destroy(ix)
    print(json.dumps(res), flush=True)


def recall_per_query(routed, reference):
    """|routed_t & reference_t| / |reference_t| per query (padding -1 ignored)."""
    out = np.empty(routed.shape[0])
    for t in range(routed.shape[0]):
        ref = reference[t][reference[t] >= 0]
        out[t] = 1.0 if ref.size == 0 else np.intersect1d(ref, routed[t][routed[t] >= 0]).size / ref.size
    return out


def summarize(r):
    return dict(mean=round(float(np.mean(r)), 5), p5=round(float(np.percentile(r, 5)), 5),
                min=round(float(np.min(r)), 5))


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count()


def ablation(ivf, torch, wl, inp, keys, ks, q, qs, w, dev, budget, k, n_q=512,
             lengths=(16384, 65536, 262144, 1048576)):
    """Recall of routed vs exhaustive top-k (the same n_q queries placed at the end of
    each prefix length) for: seal-only clustering, refits every 8K / 16K / 32K tokens,
    and position blocks (the block-routing baseline).  The index is streamed once per
    configuration; each length is measured when the stream reaches it."""
    N, H, dt = wl["N"], wl["H"], wl["dtype"]
    lengths = [L for L in lengths if L <= N]
    qa, wa = q[:n_q], w[:n_q]
    qsa = qs[:n_q] if qs is not None else None
    ws = torch.empty(ivf.idx_exhaustive_workspace_bytes(max(lengths), n_q) // 4, dtype=torch.float32, device=dev)
    exh = {}
    for L in lengths:
        e_idx, _ = ivf.idx_exhaustive_topk(keys, ks, dt, H, qa, qsa, wa, L - n_q, k, workspace=ws, n_keys=L)
        exh[L] = e_idx.cpu().numpy()
    out = {}
    configs = [("seal-only", "content", 0), ("refit every 8K", "content", 8192),
               ("refit every 16K", "content", 16384), ("refit every 32K", "content", 32768),
               ("position blocks", "positional", 0)]
    for name, clusters, R in configs:
        ix = ivf.idx_create(heads=H, dim=wl["d"], dtype=dt, max_keys=N, n_sink=wl["n_sink"], window=wl["window"],
                            cluster_size=wl["cluster_size"], seal_cap=wl["seal_cap"], seal_iters=wl["seal_iters"],
                            refit_every=R, max_queries=n_q, max_budget=budget, max_k=k, clusters=clusters)
        res = {}
        done = 0
        chunk = 16384
        for L in lengths:
            while done < L:
                b = min(L, done + chunk)
                ivf.idx_build_seal(ix, keys[done:b], None if ks is None else ks[done:b])
                while ivf.idx_refit(ix):
                    ivf.idx_publish(ix)
                done = b
            r_idx, _ = ivf.idx_route_topk(ix, qa, qsa, wa, L - n_q, k, budget)
            res[str(L)] = summarize(recall_per_query(r_idx.cpu().numpy(), exh[L]))["mean"]
        ivf.idx_destroy(ix)
        out[name] = res
        log(f"ablation {name}: {res}")
    return dict(budget=budget, k=k, queries=n_q, recall_by_prefix=out,
                learned_representatives=learned_ablation(ivf, torch, wl, dev, budget, k, n_q))


def learned_ablation(ivf, torch, wl, dev, budget, k, n_q, N=524288, lengths=(65536, 131072, 262144, 524288)):
    """Mean vs learned representatives (seeded stand-in encoder weights) on the mixture
    whose components hide members of opposite sign along u_m, with queries along u_m;
    recall vs exhaustive and index build time (seals + refits with publication)."""
    import datagen
    H, d, dt, M = wl["H"], wl["d"], wl["dtype"], 4096
    kf = datagen.make_adversarial_keys(wl["seed"], N, d, M, a=1.0)
    keys_np, ks_np = datagen.cast_rows(kf, dt)
    qf = datagen.make_adversarial_queries(wl["seed"], n_q, H, d, M)
    if dt == "e4m3":
        qc, qsv = datagen.cast_rows(qf.reshape(n_q, H * d), dt)
        q_np, qs_np = qc.reshape(n_q, H, d), np.repeat(qsv[:, None], H, axis=1).astype(np.float32)
    else:
        q_np, qs_np = datagen.cast_rows(qf, dt)[0], None
    w_np = datagen.make_weights(wl["seed"], n_q, H)
    keys = torch.from_numpy(keys_np).to(dev)
    ks = torch.from_numpy(ks_np).to(dev) if ks_np is not None else None
    q = torch.from_numpy(np.ascontiguousarray(q_np)).to(dev)
    qs = torch.from_numpy(qs_np).to(dev) if qs_np is not None else None
    w = torch.from_numpy(w_np).to(dev)
    ws = torch.empty(ivf.idx_exhaustive_workspace_bytes(N, n_q) // 4, dtype=torch.float32, device=dev)
    exh = {}
    for L in lengths:
        e_idx, _ = ivf.idx_exhaustive_topk(keys, ks, dt, H, q, qs, w, L - n_q, k, workspace=ws, n_keys=L)
        exh[L] = e_idx.cpu().numpy()
    enc = torch.from_numpy(datagen.encoder_weights(wl["seed"], d, alpha=0.25)).to(dev)
    out = {}
    for name, use_enc in (("mean representatives", False), ("learned representatives (seeded weights)", True)):
        ix = ivf.idx_create(heads=H, dim=d, dtype=dt, max_keys=N, n_sink=wl["n_sink"], window=wl["window"],
                            cluster_size=wl["cluster_size"], seal_cap=wl["seal_cap"], seal_iters=wl["seal_iters"],
                            refit_every=wl["refit_every"], max_queries=n_q, max_budget=budget, max_k=k)
        if use_enc:
            ivf.idx_set_encoder(ix, enc)
        res, done, build_s = {}, 0, 0.0
        for L in lengths:
            torch.cuda.synchronize()
            t0 = time.time()
            while done < L:
                b = min(L, done + 16384)
                ivf.idx_build_seal(ix, keys[done:b], None if ks is None else ks[done:b])
                while ivf.idx_refit(ix):
                    ivf.idx_publish(ix)
                done = b
            torch.cuda.synchronize()
            build_s += time.time() - t0
            r_idx, _ = ivf.idx_route_topk(ix, q, qs, w, L - n_q, k, budget)
            res[str(L)] = summarize(recall_per_query(r_idx.cpu().numpy(), exh[L]))["mean"]
        ivf.idx_destroy(ix)
        out[name] = dict(recall_by_prefix=res, build_s=round(build_s, 3))
        log(f"learned-rep ablation {name}: {out[name]}")
    return out


def cpu_baseline(ix, inp, wl, budget, sample):
    """Time the CPU oracle's routing (representative scores, ranking, budget fill,
    fp64 rescoring, top-k) for `sample` of the tail queries over the same index.
    The oracle cannot rebuild a 1M-key index in a benchmark's time (each refit is a
    brute-force pass over every key), so its cluster tables are loaded from the
    library's export; only the routing is timed."""
    import ivf_top_key_amd as ivf
    from oracle import OracleConfig, OracleIndex
    from oracle.index import key_values, make_cluster

    cfg = OracleConfig(heads=wl["H"], dim=wl["d"], dtype=wl["dtype"], n_sink=wl["n_sink"], window=wl["window"],
                       cluster_size=wl["cluster_size"], seal_cap=wl["seal_cap"], seal_iters=wl["seal_iters"],
                       refit_every=wl["refit_every"])
    oix = OracleIndex(cfg)
    oix.kv = key_values(inp["keys"], inp["k_scale"], wl["dtype"])
    oix.X = np.zeros((oix.kv.shape[0], 0), np.float32)          # routing never reads fp32 keys
    info = ivf.idx_get_info(ix)
    P = info["published_epoch"]

    def clusters(exp, lo_slot=0):
        out = []
        for s in range(exp["sizes"].shape[0]):
            sz, off = int(exp["sizes"][s]), int(exp["offsets"][s])
            out.append(make_cluster(s, exp["members"][off:off + sz].astype(np.int64), exp["centroids"][s],
                                    wl["dtype"]))
        return out

    seal = clusters(ivf.idx_export(ix, -1))
    Cs = cfg.n_clusters
    oix.seals = [seal[i:i + Cs] for i in range(0, len(seal), Cs)]
    if P >= 1:
        oix.epochs[P] = clusters(ivf.idx_export(ix, P))
    oix.computed = oix.published = P
    rng = np.random.default_rng(0)
    T = wl["T"]
    pick = np.sort(rng.choice(T, size=min(sample, T), replace=False))

    def run(rows):
        t0 = time.perf_counter()
        for t in rows:
            oix.route(inp["q"][t:t + 1], None if inp["q_scale"] is None else inp["q_scale"][t:t + 1],
                      inp["w"][t:t + 1], wl["q_pos0"] + int(t), wl["k"], budget)
        return time.perf_counter() - t0

    threads = blas_threads()
    dt_s = run(pick)
    # the same oracle on one thread, over the first quarter of the sample
    one = pick[:max(1, len(pick) // 4)]
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            dt_1 = run(one)
        single = {"value": round(len(one) / dt_1, 3), "cores": 1, "sample": f"{len(one)} of the same queries; "
                  f"{dt_1:.1f} s"}
    except ImportError:
        single = None
    return {"value": round(len(pick) / dt_s, 3), "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(pick)} of the {T} tail queries (seeded), routed by the numpy oracle over the same "
                      f"1M-key index (cluster tables loaded from the library's export; fp64 scores; "
                      f"{threads} BLAS threads); {dt_s:.1f} s",
            "single_thread": single, "host": host_description()}


def host_description():
    """CPU model and logical CPU count of the machine running the oracle."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "usable_cpus": usable}


if __name__ == "__main__":
    main()
