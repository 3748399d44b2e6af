"""GPU parity across the supported shapes: every storage format with each head-tile
count (H <= 32, H <= 64, H <= 128, a ragged last head tile, a single head), d = 32 /
64 / 128, 1 / 2 / 4 / 8 clusters per window, window sizes 256 .. 1024, and the
largest k.  For each: seal stores and refit epochs bit for bit, routed queries
against the oracle (including queries before the first seal) and exhaustive top-k."""
import numpy as np
import pytest

from gpu_common import (compare_epoch, compare_seal_store, ensure_built, gpu_index, oracle_index, route_parity,
                        say, workload)
from test_gpu_exhaustive import _run as exhaustive_parity

pytestmark = pytest.mark.gpu

# (name, overrides of the tiny fp32 preset)
SHAPES = [
    ("f32_d64_h8_cs4", dict(dtype="f32", d=64, H=8, window=512, cluster_size=128, seal_cap=256, refit_every=1024,
                            N=4000, T=150, q_pos0=3850, k=100, budget=700, M=48, seed=31)),
    ("f32_d128_h128", dict(dtype="f32", d=128, H=128, refit_every=2048, N=5000, T=96, q_pos0=4904, k=128,
                           budget=1500, M=64, seed=32)),
    ("bf16_d64_h32_w256", dict(dtype="bf16", d=64, H=32, window=256, cluster_size=64, seal_cap=128,
                               refit_every=1024, N=4000, T=120, q_pos0=3880, k=64, budget=600, M=48, seed=33)),
    ("e4m3_d64_h100_cs4", dict(dtype="e4m3", d=64, H=100, cluster_size=256, seal_cap=512, refit_every=2048,
                               N=6000, T=128, q_pos0=5872, k=256, budget=2048, M=64, seed=34)),
    ("e4m3_d128_h1", dict(dtype="e4m3", d=128, H=1, refit_every=2048, N=5000, T=100, q_pos0=4900, k=64,
                          budget=1024, M=64, seed=35)),
    ("f32_d32_cs1", dict(dtype="f32", d=32, H=4, window=512, cluster_size=512, seal_cap=512, refit_every=1024,
                         N=4000, T=100, q_pos0=3900, k=64, budget=1200, M=32, seed=36)),
    ("bf16_d128_h64_cs2", dict(dtype="bf16", d=128, H=64, cluster_size=512, seal_cap=1024, refit_every=2048,
                               N=5000, T=96, q_pos0=4904, k=200, budget=1600, M=64, seed=37)),
]


@pytest.mark.parametrize("name,over", SHAPES, ids=[n for n, _ in SHAPES])
def test_shape_index_route_exhaustive(name, over):
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload("c1", **over)
    say(f"shape {name}: {wl['dtype']} d={wl['d']} H={wl['H']} W={wl['window']} Cs={wl['window'] // wl['cluster_size']}")
    gix = gpu_index(wl, inp)
    try:
        oix = oracle_index(wl, inp)
        compare_seal_store(ivf, gix, oix, name)
        for r in range(max(1, oix.published - 2), oix.published + 1):
            compare_epoch(ivf, gix, oix, r, name)
    finally:
        ivf.idx_destroy(gix)
    stats = route_parity("c1", **over)
    say(f"  routed tail ok {stats}")
    # queries from position 0: before the first seal, then across the first windows
    route_parity("c1", **dict(over, q_pos0=0, T=min(over["N"], over.get("window", 1024) + 300)))
    exhaustive_parity("c1", **over)


def test_largest_k():
    """k = 4096 (the largest) with an 8192-candidate budget: the selection's widest case,
    in a small batch (split scoring) and in a batch of more than 64 queries (the fused
    cut + rescoring kernel)."""
    route_parity("bf16_small", k=4096, budget=8192, T=48, q_pos0=12240)
    route_parity("e4m3_small", k=4096, budget=8192, T=100, q_pos0=12188)
    from test_gpu_exhaustive import _run
    _run("bf16_small", q_pos0=12240, T=48, k=4096)
