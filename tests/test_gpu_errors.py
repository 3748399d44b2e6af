"""Error behaviour of a live index: every call validates on the host and returns the
documented status without touching the device state (the index stays usable)."""
import numpy as np
import pytest

from gpu_common import ensure_built, gpu_index, say, to_dev, workload

pytestmark = pytest.mark.gpu


def _codes(ivf):
    return dict(EINVAL=-1, ECAUSAL=-4, ESTATE=-5, ECAPACITY=-6)


def _expect(ivf, code, fn, *a, **kw):
    with pytest.raises(ivf.IdxError) as ei:
        fn(*a, **kw)
    assert ei.value.code == code, str(ei.value)


def test_route_argument_errors_leave_the_index_usable():
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload("c1r")
    T, k, budget = 64, wl["k"], wl["budget"]
    ix = gpu_index(wl, inp, max_queries=T, max_budget=budget)
    try:
        c = _codes(ivf)
        q, w = to_dev(inp["q"][:T]), to_dev(inp["w"][:T])
        N = wl["N"]
        _expect(ivf, c["ECAPACITY"], ivf.idx_route_topk, ix, to_dev(inp["q"][:T + 1]), None,
                to_dev(inp["w"][:T + 1]), N - T - 1, k, budget)                       # T > max_queries
        _expect(ivf, c["ECAPACITY"], ivf.idx_route_topk, ix, q, None, w, N - T, k + 1, budget)    # k > max_k
        _expect(ivf, c["EINVAL"], ivf.idx_route_topk, ix, q, None, w, N - T, k, k - 1)            # budget < k
        _expect(ivf, c["ECAPACITY"], ivf.idx_route_topk, ix, q, None, w, N - T, k, budget + 32)   # > max_budget
        _expect(ivf, c["ECAUSAL"], ivf.idx_route_topk, ix, q, None, w, N - T + 1, k, budget)      # key not inserted
        _expect(ivf, c["EINVAL"], ivf.idx_route_topk, ix, q, None, w, -1, k, budget)
        pos = np.full(T, N - 1, np.int64)
        pos[5] = N
        _expect(ivf, c["ECAUSAL"], ivf.idx_route_topk_pos, ix, q, None, w, pos, k, budget)
        pos[5] = -3
        _expect(ivf, c["EINVAL"], ivf.idx_route_topk_pos, ix, q, None, w, pos, k, budget)
        # a valid call still works and matches a second identical call
        a = ivf.idx_route_topk(ix, q, None, w, N - T, k, budget)
        b = ivf.idx_route_topk(ix, q, None, w, N - T, k, budget)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and (a[0][:, 0] >= 0).all()
    finally:
        ivf.idx_destroy(ix)


def test_capacity_retired_epoch_and_publication_state():
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload("c1r", N=12288, T=512, q_pos0=11776)   # five refit epochs
    N = wl["N"]
    ix = gpu_index(wl, inp)
    try:
        c = _codes(ivf)
        info = ivf.idx_get_info(ix)
        e = info["computed_epoch"]
        assert e >= 4 and info["published_epoch"] == e
        # no more room: the index was created for exactly N keys
        _expect(ivf, c["ECAPACITY"], ivf.idx_build_seal, ix, to_dev(inp["keys"][:1]))
        # epochs below computed - 2 are retired: exporting or routing with one is refused
        _expect(ivf, c["ESTATE"], ivf.idx_export, ix, e - 3)
        R, S, W = wl["refit_every"], wl["n_sink"], wl["window"]
        early = S + R + W    # a query there uses epoch 1
        assert e - 3 >= 1
        q, w = to_dev(inp["q"][:4]), to_dev(inp["w"][:4])
        _expect(ivf, c["ESTATE"], ivf.idx_route_topk, ix, q, None, w, early, wl["k"], wl["budget"])
        # nothing due: refit launches nothing, publish keeps the epoch
        assert ivf.idx_refit(ix) is False
        assert ivf.idx_publish(ix) == e
        say(f"  epochs 1..{e}: epoch {e - 3} retired, routing at {early} refused")
    finally:
        ivf.idx_destroy(ix)


def test_e4m3_needs_scales_and_encoder_size_is_checked():
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    wl, inp = workload("e4m3_small")
    ix = ivf.idx_create(heads=wl["H"], dim=wl["d"], dtype="e4m3", max_keys=4096, max_queries=8, max_budget=2048,
                        max_k=256)
    try:
        c = _codes(ivf)
        _expect(ivf, c["EINVAL"], ivf.idx_build_seal, ix, to_dev(inp["keys"][:2048]), None)
        ivf.idx_build_seal(ix, to_dev(inp["keys"][:2048]), to_dev(inp["k_scale"][:2048]))
        q, w = to_dev(inp["q"][:8]), to_dev(inp["w"][:8])
        _expect(ivf, c["EINVAL"], ivf.idx_route_topk, ix, q, None, w, 2000, 64, 1024)   # q_scale missing
        with pytest.raises(ValueError):
            ivf.idx_set_encoder(ix, torch.zeros(10, dtype=torch.float32, device="cuda"))
        i, s = ivf.idx_route_topk(ix, q, to_dev(inp["q_scale"][:8]), w, 2000, 64, 1024)
        torch.cuda.synchronize()
        assert (i[:, :64] >= 0).all()
    finally:
        ivf.idx_destroy(ix)
