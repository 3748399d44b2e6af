"""The no-allocation exhaustive entry point against the workspace one.

idx_exhaustive_topk_noalloc runs the same kernels as idx_exhaustive_topk with its
workspace (sample scores, survivor lists, the fallback's score rows) in the
library's per-GPU scratch array instead of a caller workspace, so its outputs must
equal the workspace entry point's bit for bit.  Two calls in a row (the second
smaller, on a different format) check that the array's contents from the previous
call do not leak into the next; 1500 queries over a 600K-key prefix are more than
the array holds at once, so two passes run; a prefix whose pass exceeds the array
is refused before any device work.
"""
import numpy as np
import pytest

from gpu_common import ensure_built, say

pytestmark = pytest.mark.gpu


def _case(ivf, torch, dtype, n, T, k, H=64, d=128, seed=0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    if dtype == "e4m3":
        keys = torch.randint(0, 126, (n, d), dtype=torch.uint8, device="cuda", generator=g)
        keys |= (torch.randint(0, 2, (n, d), dtype=torch.uint8, device="cuda", generator=g) << 7)
        ks = torch.rand(n, device="cuda", generator=g) * 0.01 + 1e-3
        q = torch.randint(0, 126, (T, H, d), dtype=torch.uint8, device="cuda", generator=g)
        qs = torch.rand(T, H, device="cuda", generator=g) * 0.01 + 1e-3
    else:
        keys = torch.randn(n, d, device="cuda", generator=g).to(torch.bfloat16)
        q = torch.randn(T, H, d, device="cuda", generator=g).to(torch.bfloat16)
        ks = qs = None
    w = torch.randn(T, H, device="cuda", generator=g) / H ** 0.5
    return keys, ks, q, qs, w


def _both(ivf, torch, dtype, n, T, k, seed):
    keys, ks, q, qs, w = _case(ivf, torch, dtype, n, T, k, seed=seed)
    q_pos0 = n - T
    ref_i, ref_s = ivf.idx_exhaustive_topk(keys, ks, dtype, 64, q, qs, w, q_pos0, k)
    got_i = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    got_s = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    ivf.idx_exhaustive_topk_noalloc(keys, ks, dtype, 64, q, qs, w, q_pos0, k, got_i, got_s)
    torch.cuda.synchronize()
    assert torch.equal(ref_i, got_i), f"{dtype} n={n} T={T}: indices differ"
    assert torch.equal(ref_s.view(torch.int32), got_s.view(torch.int32)), f"{dtype} n={n} T={T}: scores differ"
    assert (got_i[:, 0] >= 0).all()
    say(f"  {dtype} n={n} T={T} k={k}: identical")


def test_noalloc_matches_workspace_entry_point():
    import torch
    import ivf_top_key_amd as ivf
    ensure_built()
    say("no-alloc exhaustive: two calls, the second smaller; then a multi-pass prefix")
    _both(ivf, torch, "bf16", 20000, 300, 512, seed=1)
    _both(ivf, torch, "e4m3", 5000, 100, 256, seed=2)
    # 600K bf16 keys, k = 2048: about 100 KB per query (a 9375-key sample row and 8192
    # survivors), so the 128 MiB array holds about 1300 of the 1500 queries per pass
    _both(ivf, torch, "bf16", 600000, 1500, 2048, seed=3)


def test_noalloc_rejects_rows_beyond_the_array():
    import ctypes
    import ivf_top_key_amd as ivf
    ensure_built()
    lib = ivf.lib()
    p = ctypes.c_void_p(16)              # never dereferenced: the size check fails first
    n = (128 << 20) // 4 + 64            # the fallback's score row alone is longer than the array
    rc = lib.idx_exhaustive_topk_noalloc(p, None, n, 1, 64, 128, p, None, p, n - 1, 1, 8, p, None, None)
    assert rc == ivf.IDX_ECAPACITY
    assert "scratch" in ivf.idx_last_error()
