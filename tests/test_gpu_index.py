"""GPU parity: seal and refit clusters (idx_build_seal, idx_refit, idx_publish,
idx_export) against the CPU oracle, bit for bit: sizes, member lists, fp32
centroid bits, representative bits and scales."""
import numpy as np
import pytest

from gpu_common import (compare_epoch, compare_seal_store, ensure_built, gpu_index, oracle_index, say,
                        workload)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["c1", "c1r", "bf16_small", "e4m3_small"])
def test_index_bit_exact(name):
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload(name)
    say(f"index {name}: N={wl['N']} dtype={wl['dtype']} R={wl['refit_every']}")
    gix = gpu_index(wl, inp)
    try:
        oix = oracle_index(wl, inp)
        info = ivf.idx_get_info(gix)
        assert info["sealed_windows"] == len(oix.seals)
        assert info["published_epoch"] == oix.published
        compare_seal_store(ivf, gix, oix, name)
        for r in range(max(1, oix.published - 2), oix.published + 1):
            if r >= 1:
                compare_epoch(ivf, gix, oix, r, name)
        say(f"  ok: {len(oix.seals)} windows, epochs up to {oix.published}")
    finally:
        ivf.idx_destroy(gix)


@pytest.mark.parametrize("name", ["c1", "e4m3_small"])
def test_positional_blocks_bit_exact(name):
    """Block-routing baseline: every window's clusters are its contiguous blocks with
    exact-order means, bit for bit."""
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload(name, positional=True, refit_every=0)
    gix = gpu_index(wl, inp, chunk=1500)
    try:
        oix = oracle_index(wl, inp)
        got = compare_seal_store(ivf, gix, oix, name + " positional")
        b = wl["cluster_size"]
        assert np.all(got["sizes"] == b)
        say(f"  ok: {len(oix.seals)} windows of position blocks")
    finally:
        ivf.idx_destroy(gix)


def test_index_streamed_in_chunks_matches_one_shot():
    """Keys inserted 700 at a time (windows sealed across calls, refits launched as
    soon as due) give the same index as the oracle."""
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload("c1r")
    gix = gpu_index(wl, inp, chunk=700)
    try:
        oix = oracle_index(wl, inp)
        compare_seal_store(ivf, gix, oix, "chunked")
        compare_epoch(ivf, gix, oix, oix.published, "chunked")
    finally:
        ivf.idx_destroy(gix)


def test_seal_with_binding_cap():
    """Few mixture components per window make nearest assignment exceed the cap,
    so the greedy walk decides the clusters."""
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload("c1", M=3, seal_cap=140, N=3100, T=64, q_pos0=3000, refit_every=0)
    from oracle.kmeans import nearest, sqdist_exact
    gix = gpu_index(wl, inp)
    try:
        oix = oracle_index(wl, inp)
        compare_seal_store(ivf, gix, oix, "cap")
        # the cap really binds in at least one window
        sizes = [c.members.size for w in oix.seals for c in w]
        assert max(sizes) == 140
    finally:
        ivf.idx_destroy(gix)


@pytest.mark.parametrize("name", ["c1r", "bf16_small", "e4m3_small"])
def test_refit_bound_state_is_valid(name):
    """After the last refit every key's Hamerly bounds hold against its warm
    centroids (the state the next refit prunes with)."""
    import ivf_top_key_amd as ivf
    from gpu_common import check_refit_bounds
    from oracle.index import key_values
    ensure_built()
    wl, inp = workload(name)
    gix = gpu_index(wl, inp)
    try:
        kv = key_values(inp["keys"], inp["k_scale"], wl["dtype"])
        n, frac = check_refit_bounds(ivf, gix, wl, kv)
        say(f"  ok: {n} keys, last refit screened {frac:.3f} of its prefix")
    finally:
        ivf.idx_destroy(gix)
