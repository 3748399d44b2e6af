"""Named workload presets (plain numbers only).

Each preset gives the input shape (heads H, dimension d, storage format,
prefix length N, query chunk) and the selection parameters that the pages fix
for GLM-5.3: k = 2048 keys kept per query, windows of W = 1024 keys sealed into
8 clusters of about 128, a whole-prefix refit every R = 16384 tokens, a few
sink keys (4 here).  "c1r" and the "*_small" presets are reduced sizes that a
CPU oracle finishes in seconds while still covering several windows, refits,
tiles and a ragged tail.
"""

COMMON = dict(n_sink=4, window=1024, cluster_size=128, seal_cap=256, seal_iters=10)

WORKLOADS = {
    # tiny fp32 case: H=4, d=32, 4096 keys, the last 256 positions as queries
    "c1": dict(COMMON, H=4, d=32, dtype="f32", N=4096, T=256, q_pos0=3840, k=64, budget=1024,
               refit_every=16384, M=64, seed=1),
    # the same with a short refit period so that refits fire on a small prefix
    "c1r": dict(COMMON, H=4, d=32, dtype="f32", N=8192, T=512, q_pos0=7680, k=64, budget=1024,
                refit_every=2048, M=64, seed=11),
    # DSA-like shape at 32K, bf16
    "c2": dict(COMMON, H=64, d=128, dtype="bf16", N=32768, T=4096, q_pos0=28672, k=2048,
               budget=8192, refit_every=16384, M=4096, seed=2),
    # streaming prefill to 128K in chunks of 8192 queries, bf16
    "c3": dict(COMMON, H=64, d=128, dtype="bf16", N=131072, T=8192, q_pos0=0, k=2048,
               budget=8192, refit_every=16384, M=4096, seed=3, chunk=8192),
    # 1M-token prefix, E4M3 with per-token fp32 scales, 4096 queries at the tail
    "c4": dict(COMMON, H=64, d=128, dtype="e4m3", N=1048576, T=4096, q_pos0=1044480, k=2048,
               budget=8192, refit_every=16384, M=4096, seed=4),
    # reduced DSA-shaped cases with refits, small enough for full oracle parity
    "bf16_small": dict(COMMON, H=64, d=128, dtype="bf16", N=12288, T=640, q_pos0=11648, k=256,
                       budget=2048, refit_every=4096, M=256, seed=21),
    "e4m3_small": dict(COMMON, H=64, d=128, dtype="e4m3", N=12288, T=640, q_pos0=11648, k=256,
                       budget=2048, refit_every=4096, M=256, seed=22),
}
