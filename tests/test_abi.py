"""The C ABI on the CPU: the library loads without a GPU, exports every function
include/ivftk.h declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ivftk.h")


@pytest.fixture(scope="module")
def lib():
    from ivf_top_key_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from ivf_top_key_amd.build import build
        build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(idx_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("idx_build_seal", "idx_refit", "idx_route_topk", "idx_exhaustive_topk", "idx_create",
                     "idx_destroy", "idx_last_error", "idx_publish", "idx_export", "idx_get_info",
                     "idx_exhaustive_workspace_bytes", "idx_export_version", "idx_import_version",
                     "idx_abandon_refit"):
        assert required in names


def test_every_declared_function_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    from ivf_top_key_amd._lib import SIGNATURES
    assert sorted(n for n, _, _ in SIGNATURES) == declared_functions()


def _cfg(**over):
    from ivf_top_key_amd._lib import idx_config
    base = dict(heads=64, dim=128, dtype=2, n_sink=4, window=1024, cluster_size=128, seal_cap=256, seal_iters=10,
                refit_every=16384, max_queries=4096, max_budget=8192, max_k=2048, rescore_mode=0, cluster_mode=0,
                max_keys=1 << 20)
    base.update(over)
    return idx_config(*[base[f] for f, _ in idx_config._fields_])


@pytest.mark.parametrize("over,code", [
    (dict(dtype=7), -1), (dict(heads=0), -1), (dict(heads=200), -1), (dict(dim=96), -7),
    (dict(dtype=1, dim=32), -7), (dict(window=1000), -1), (dict(cluster_size=64), -7),
    (dict(seal_cap=100), -1), (dict(seal_iters=0), -1), (dict(refit_every=1000), -1),
    (dict(max_k=5000), -1), (dict(max_budget=100), -1), (dict(max_keys=0), -1),
    (dict(max_keys=1 << 21), -6), (dict(max_budget=32768, max_k=4096), -6), (dict(rescore_mode=3), -1),
    (dict(cluster_mode=2), -1), (dict(cluster_mode=1), -1),
])
def test_create_rejects_bad_config(lib, over, code):
    h = ctypes.c_void_p()
    rc = lib.idx_create(ctypes.byref(_cfg(**over)), None, ctypes.byref(h))
    assert rc == code, lib.idx_last_error()
    assert h.value is None
    assert lib.idx_last_error()


def test_create_valid_config_on_any_host(lib):
    """A valid configuration either creates an index (a GPU is present) or fails
    with ENOMEM / EDEVICE and releases what it allocated (no GPU)."""
    h = ctypes.c_void_p()
    rc = lib.idx_create(ctypes.byref(_cfg(max_keys=1 << 16, max_queries=64)), None, ctypes.byref(h))
    assert rc in (0, -2, -3), lib.idx_last_error()
    if rc == 0:
        assert lib.idx_destroy(h) == 0
    else:
        assert h.value is None and lib.idx_last_error()


def test_calls_on_null_handle(lib):
    assert lib.idx_build_seal(None, None, None, 0, None) == -1
    assert lib.idx_refit(None, None, None, None) == -1
    assert lib.idx_publish(None, None, None) == -1
    assert lib.idx_route_topk(None, None, None, None, 0, 1, 1, 1, None, None, None, None) == -1
    assert lib.idx_route_topk_pos(None, None, None, None, None, 1, 1, 1, None, None, None, None) == -1
    assert lib.idx_export(None, -1, None) == -1
    assert lib.idx_export_version(None, 1, None, None, None) == -1
    assert lib.idx_import_version(None, 1, None, None) == -1
    assert lib.idx_abandon_refit(None, None, None) == -1
    assert lib.idx_get_info(None, None) == -1
    assert lib.idx_destroy(None) == 0


def test_exhaustive_rejects_bad_arguments(lib):
    p = ctypes.c_void_p(16)   # never dereferenced: every case fails validation first
    call = lambda **kw: lib.idx_exhaustive_topk(
        kw.get("keys", p), kw.get("ks", p), kw.get("n", 100), kw.get("dt", 1), kw.get("H", 64), kw.get("d", 128),
        p, kw.get("qs", p), p, kw.get("q0", 10), kw.get("T", 4), kw.get("k", 8), p, p, p, kw.get("ws", 1 << 20),
        None)
    assert call(dt=9) == -1
    assert call(H=0) == -1
    assert call(d=96) == -7
    assert call(keys=None) == -1
    assert call(dt=2, ks=None) == -1
    assert call(T=0) == -1
    assert call(k=0) == -1 and call(k=5000) == -1
    assert call(q0=-1) == -1
    assert call(q0=97, T=4) == -4        # query position 100 has no key
    assert call(ws=16) == -1             # workspace below one query row
    assert "workspace" in lib.idx_last_error().decode()


def test_create_rejects_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.idx_create(None, None, ctypes.byref(h)) == -1
    assert lib.idx_create(ctypes.byref(_cfg()), None, None) == -1


def test_workspace_size(lib):
    """The streamed exhaustive selection keeps, per query, one row of sample scores
    (every 64th key) and a survivor list, not a full score row; the workspace still
    holds at least one full row for the fallback."""
    n = 1 << 20
    one = lib.idx_exhaustive_workspace_bytes(n, 1)
    many = lib.idx_exhaustive_workspace_bytes(n, 1024)
    assert one >= n * 4
    assert many > one
    assert many < 1024 * n * 4 // 10
    per_query = (many - one) / 1023
    assert (n // 64) * 4 <= per_query <= (n // 64) * 4 + 16384 * 8 + 1024
    assert lib.idx_exhaustive_workspace_bytes(0, 3) == 0


def test_encoder_size_matches_the_packed_layout(lib):
    from oracle.encoder import encoder_floats
    for d in (32, 64, 128):
        assert lib.idx_encoder_floats(d) == encoder_floats(d)
    assert lib.idx_encoder_floats(96) == -1
    assert lib.idx_set_encoder(None, None, None) == -1
