"""Causal IVF-routed indexer top-k on AMD MI355X (gfx950): Python binding.

Each function here has the name of a C entry point in include/ivftk.h and only
marshals arguments: torch tensors on the GPU become device pointers, the
current torch stream becomes the HIP stream, and outputs are allocated with
torch when the caller passes none.  All computation runs in libivftk.so; when
the library is missing the calls raise instead of falling back to anything.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib

RESCORE = {"auto": 0, "query": 1, "cluster": 2}
CLUSTERS = {"content": 0, "positional": 1}
DTYPES = {"f32": 0, "bf16": 1, "e4m3": 2}
ELEM_BYTES = {"f32": 4, "bf16": 2, "e4m3": 1}
_HOST_DTYPE = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}
IDX_OK, IDX_EINVAL, IDX_ENOMEM, IDX_EDEVICE, IDX_ECAUSAL, IDX_ESTATE, IDX_ECAPACITY, IDX_ENOTIMPL = \
    0, -1, -2, -3, -4, -5, -6, -7


class IdxError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def lib():
    return _lib.load()


def idx_last_error() -> str:
    return (lib().idx_last_error() or b"").decode()


def _check(rc: int):
    if rc != IDX_OK:
        raise IdxError(rc, idx_last_error())


def _ptr(t, elem_bytes=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if elem_bytes is not None and t.element_size() != elem_bytes:
        raise ValueError(f"{name} must have {elem_bytes}-byte elements (got {t.element_size()})")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


class Index:
    """Handle of one index (C: idx_index*).  Holds its configuration for the binding."""

    def __init__(self, handle, cfg: dict):
        self.handle = handle
        self.cfg = cfg

    @property
    def dtype(self) -> str:
        return self.cfg["dtype"]


def idx_create(heads: int, dim: int, dtype: str, max_keys: int, n_sink: int = 4, window: int = 1024,
               cluster_size: int = 128, seal_cap: int = 256, seal_iters: int = 10, refit_every: int = 16384,
               max_queries: int = 4096, max_budget: int = 8192, max_k: int = 2048,
               rescore: str = "auto", clusters: str = "content", stream=None) -> Index:
    cfg = dict(heads=heads, dim=dim, dtype=dtype, n_sink=n_sink, window=window, cluster_size=cluster_size,
               seal_cap=seal_cap, seal_iters=seal_iters, refit_every=refit_every, max_queries=max_queries,
               max_budget=max_budget, max_k=max_k, rescore=rescore, clusters=clusters, max_keys=max_keys)
    c = _lib.idx_config(heads, dim, DTYPES[dtype], n_sink, window, cluster_size, seal_cap, seal_iters,
                        refit_every, max_queries, max_budget, max_k, RESCORE[rescore], CLUSTERS[clusters],
                        max_keys)
    h = ctypes.c_void_p()
    _check(lib().idx_create(ctypes.byref(c), _stream(stream), ctypes.byref(h)))
    return Index(h, cfg)


def idx_destroy(ix: Index):
    if ix.handle:
        _check(lib().idx_destroy(ix.handle))
        ix.handle = None


def idx_get_info(ix: Index) -> dict:
    info = _lib.idx_info()
    _check(lib().idx_get_info(ix.handle, ctypes.byref(info)))
    return {k: getattr(info, k) for k, _ in _lib.idx_info._fields_}


def idx_build_seal(ix: Index, keys: torch.Tensor, k_scale: torch.Tensor | None = None, stream=None):
    eb = ELEM_BYTES[ix.dtype]
    n = keys.shape[0]
    _check(lib().idx_build_seal(ix.handle, _ptr(keys, eb, "keys"), _ptr(k_scale, 4, "k_scale"), n,
                                _stream(stream)))


def idx_refit(ix: Index, stream=None, side_stream=None) -> bool:
    launched = ctypes.c_int32(0)
    side = side_stream if side_stream is not None else stream
    _check(lib().idx_refit(ix.handle, _stream(stream), _stream(side), ctypes.byref(launched)))
    return bool(launched.value)


def idx_publish(ix: Index, stream=None) -> int:
    pub = ctypes.c_int32(0)
    _check(lib().idx_publish(ix.handle, _stream(stream), ctypes.byref(pub)))
    return pub.value


def idx_abandon_refit(ix: Index, stream=None) -> int:
    """Give up the launched, unpublished refit; returns its epoch (0 if none)."""
    ab = ctypes.c_int32(0)
    _check(lib().idx_abandon_refit(ix.handle, _stream(stream), ctypes.byref(ab)))
    return ab.value


def make_route_debug(T: int, cand_cap: int, order_cap: int, rep_cap: int, device="cuda") -> dict:
    """Device buffers for the optional debug outputs of idx_route_topk."""
    i32 = dict(dtype=torch.int32, device=device)
    return dict(cand=torch.full((T, cand_cap), -1, **i32), cand_len=torch.zeros(T, **i32),
                order=torch.full((T, order_cap), -1, **i32), order_take=torch.zeros((T, order_cap), **i32),
                n_order=torch.zeros(T, **i32),
                rep_scores=torch.zeros((T, rep_cap), dtype=torch.float32, device=device),
                version=torch.zeros((T, 4), **i32),
                cand_scores=torch.full((T, cand_cap), float("nan"), dtype=torch.float32, device=device))


def _route_debug(debug: dict | None):
    if debug is None:
        return None
    ev = debug.get("events")
    if ev is not None:
        ev = ctypes.cast((ctypes.c_void_p * len(ev))(*ev), ctypes.POINTER(ctypes.c_void_p))
    return _lib.idx_route_debug(
        _ptr(debug.get("cand")), debug["cand"].shape[1] if debug.get("cand") is not None else 0,
        _ptr(debug.get("cand_len")), _ptr(debug.get("order")), _ptr(debug.get("order_take")),
        debug["order"].shape[1] if debug.get("order") is not None else 0, _ptr(debug.get("n_order")),
        _ptr(debug.get("rep_scores")),
        debug["rep_scores"].shape[1] if debug.get("rep_scores") is not None else 0,
        _ptr(debug.get("version")), ev, int(debug.get("list_cap", 0)), _ptr(debug.get("cand_scores")))


def idx_route_topk_pos(ix: Index, q: torch.Tensor, q_scale, w: torch.Tensor, positions, k: int, budget: int,
                       topk_idx=None, topk_score=None, debug: dict | None = None, stream=None):
    """Decode batch: query t at positions[t] (host integers)."""
    T = q.shape[0]
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64).reshape(-1))
    if pos.shape[0] != T:
        raise ValueError("one position per query")
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=q.device)
    if topk_score is None:
        topk_score = torch.empty((T, k), dtype=torch.float32, device=q.device)
    dbg = _route_debug(debug)
    _check(lib().idx_route_topk_pos(ix.handle, _ptr(q, ELEM_BYTES[ix.dtype], "q"), _ptr(q_scale, 4, "q_scale"),
                                    _ptr(w, 4, "w"), pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), T, k,
                                    budget, _ptr(topk_idx, 4, "topk_idx"), _ptr(topk_score, 4, "topk_score"),
                                    ctypes.byref(dbg) if dbg is not None else None, _stream(stream)))
    return topk_idx, topk_score


def idx_route_topk(ix: Index, q: torch.Tensor, q_scale, w: torch.Tensor, q_pos0: int, k: int, budget: int,
                   topk_idx=None, topk_score=None, debug: dict | None = None, stream=None):
    T = q.shape[0]
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=q.device)
    if topk_score is None:
        topk_score = torch.empty((T, k), dtype=torch.float32, device=q.device)
    dbg = _route_debug(debug)
    _check(lib().idx_route_topk(ix.handle, _ptr(q, ELEM_BYTES[ix.dtype], "q"), _ptr(q_scale, 4, "q_scale"),
                                _ptr(w, 4, "w"), q_pos0, T, k, budget, _ptr(topk_idx, 4, "topk_idx"),
                                _ptr(topk_score, 4, "topk_score"), ctypes.byref(dbg) if dbg is not None else None,
                                _stream(stream)))
    return topk_idx, topk_score


def idx_exhaustive_workspace_bytes(n_keys: int, T: int) -> int:
    return int(lib().idx_exhaustive_workspace_bytes(n_keys, T))


def idx_exhaustive_topk(keys: torch.Tensor, k_scale, dtype: str, heads: int, q: torch.Tensor, q_scale,
                        w: torch.Tensor, q_pos0: int, k: int, topk_idx=None, topk_score=None, workspace=None,
                        n_keys: int | None = None, stream=None):
    T = q.shape[0]
    d = keys.shape[-1]
    n_keys = keys.shape[0] if n_keys is None else n_keys
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=q.device)
    if topk_score is None:
        topk_score = torch.empty((T, k), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = idx_exhaustive_workspace_bytes(q_pos0 + T, T)
        workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=q.device)
    eb = ELEM_BYTES[dtype]
    _check(lib().idx_exhaustive_topk(_ptr(keys, eb, "keys"), _ptr(k_scale, 4, "k_scale"), n_keys, DTYPES[dtype],
                                     heads, d, _ptr(q, eb, "q"), _ptr(q_scale, 4, "q_scale"), _ptr(w, 4, "w"),
                                     q_pos0, T, k, _ptr(topk_idx, 4, "topk_idx"), _ptr(topk_score, 4, "topk_score"),
                                     _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))
    return topk_idx, topk_score


def idx_exhaustive_topk_noalloc(keys: torch.Tensor, k_scale, dtype: str, heads: int, q: torch.Tensor, q_scale,
                                w: torch.Tensor, q_pos0: int, k: int, topk_idx: torch.Tensor,
                                topk_score: torch.Tensor | None = None, n_keys: int | None = None, stream=None):
    """idx_exhaustive_topk without a workspace (the library's own scratch array):
    the caller passes the outputs, nothing is allocated."""
    d = keys.shape[-1]
    n_keys = keys.shape[0] if n_keys is None else n_keys
    eb = ELEM_BYTES[dtype]
    _check(lib().idx_exhaustive_topk_noalloc(_ptr(keys, eb, "keys"), _ptr(k_scale, 4, "k_scale"), n_keys,
                                             DTYPES[dtype], heads, d, _ptr(q, eb, "q"), _ptr(q_scale, 4, "q_scale"),
                                             _ptr(w, 4, "w"), q_pos0, q.shape[0], k, _ptr(topk_idx, 4, "topk_idx"),
                                             _ptr(topk_score, 4, "topk_score"), _stream(stream)))
    return topk_idx, topk_score


def idx_export(ix: Index, which: int) -> dict:
    """Host copy of one cluster set: which=-1 sealed windows, which=e epoch e.  For the
    newest computed epoch it also holds the refit's counts (n_screened, n_brute) and
    the per-key bound state (assign, ub, lb for positions S .. S + e*R - 1)."""
    buf = _lib.idx_export_buf()
    _check(lib().idx_export(ix.handle, which, ctypes.byref(buf)))
    ns, nm, d, nb = buf.n_slots, buf.n_members, ix.cfg["dim"], buf.n_bound_keys
    out = dict(sizes=np.zeros(ns, np.int32), offsets=np.zeros(ns, np.int32), members=np.zeros(nm, np.int32),
               centroids=np.zeros((ns, d), np.float32),
               reps=np.zeros((ns, d), _HOST_DTYPE[ix.dtype]),
               rep_scale=np.zeros(ns, np.float32), rep_f32=np.zeros((ns, d), np.float32),
               assign=np.zeros(nb, np.int32), ub=np.zeros(nb, np.float32), lb=np.zeros(nb, np.float32))
    for k in out:
        setattr(buf, k, out[k].ctypes.data if out[k].size else None)
    _check(lib().idx_export(ix.handle, which, ctypes.byref(buf)))
    out["n_screened"], out["n_brute"], out["n_bound_keys"] = int(buf.n_screened), int(buf.n_brute), int(nb)
    if nb == 0:
        for k in ("assign", "ub", "lb"):
            del out[k]
    return out


def idx_export_version(ix: Index, prefix_len: int) -> dict:
    """Host copy of the clusters a query with `prefix_len` keys in its prefix routes
    over: slots [0, m*C), the epoch's below e*Q and seal clusters above; also 'epoch'
    and 'windows' (e and m)."""
    buf = _lib.idx_export_buf()
    ep, win = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().idx_export_version(ix.handle, prefix_len, ctypes.byref(ep), ctypes.byref(win), ctypes.byref(buf)))
    ns, nm, d = buf.n_slots, buf.n_members, ix.cfg["dim"]
    out = dict(sizes=np.zeros(ns, np.int32), offsets=np.zeros(ns, np.int32), members=np.zeros(nm, np.int32),
               centroids=np.zeros((ns, d), np.float32), reps=np.zeros((ns, d), _HOST_DTYPE[ix.dtype]),
               rep_scale=np.zeros(ns, np.float32), rep_f32=np.zeros((ns, d), np.float32))
    for k in out:
        setattr(buf, k, out[k].ctypes.data if out[k].size else None)
    _check(lib().idx_export_version(ix.handle, prefix_len, ctypes.byref(ep), ctypes.byref(win), ctypes.byref(buf)))
    out["epoch"], out["windows"] = ep.value, win.value
    return out


def idx_import_version(ix: Index, prefix_len: int, sizes, members, centroids, reps, rep_scale=None, rep_f32=None,
                       stream=None):
    """Install a host-built cluster set as the next refit epoch (see the C header).
    sizes [n_slots], members (slot by slot, ascending within a slot), centroids
    [n_slots, d] fp32, reps [n_slots, d] in the key format (uint16 bf16 bits, uint8
    E4M3 codes), rep_scale [n_slots] for E4M3, rep_f32 optional."""
    d = ix.cfg["dim"]
    arrs = dict(sizes=np.ascontiguousarray(sizes, dtype=np.int32),
                members=np.ascontiguousarray(members, dtype=np.int32),
                centroids=np.ascontiguousarray(centroids, dtype=np.float32).reshape(-1, d),
                reps=np.ascontiguousarray(reps, dtype=_HOST_DTYPE[ix.dtype]).reshape(-1, d),
                rep_scale=None if rep_scale is None else np.ascontiguousarray(rep_scale, dtype=np.float32),
                rep_f32=None if rep_f32 is None else np.ascontiguousarray(rep_f32, dtype=np.float32).reshape(-1, d))
    ns = arrs["sizes"].shape[0]
    if arrs["centroids"].shape[0] != ns or arrs["reps"].shape[0] != ns:
        raise ValueError("centroids and reps need one row per slot")
    buf = _lib.idx_import_buf(ns, *[arrs[k].ctypes.data if arrs[k] is not None and arrs[k].size else None
                                    for k in ("sizes", "members", "centroids", "reps", "rep_scale", "rep_f32")])
    _check(lib().idx_import_version(ix.handle, prefix_len, ctypes.byref(buf), _stream(stream)))


def idx_encoder_floats(dim: int) -> int:
    return int(lib().idx_encoder_floats(dim))


def idx_set_encoder(ix: Index, weights: torch.Tensor | None, stream=None):
    """Learned representatives from now on (weights: float32 device tensor in the packed
    layout, idx_encoder_floats(dim) values), or None for mean representatives."""
    if weights is not None:
        if weights.dtype != torch.float32 or weights.numel() != idx_encoder_floats(ix.cfg["dim"]):
            raise ValueError("encoder weights must be float32 with idx_encoder_floats(dim) values")
        weights = weights.contiguous()
    _check(lib().idx_set_encoder(ix.handle, _ptr(weights, 4, "weights"), _stream(stream)))


__all__ = ["IdxError", "Index", "idx_create", "idx_destroy", "idx_last_error", "idx_get_info", "idx_build_seal",
           "idx_refit", "idx_publish", "idx_abandon_refit", "idx_route_topk", "idx_route_topk_pos",
           "idx_exhaustive_workspace_bytes", "idx_exhaustive_topk", "idx_exhaustive_topk_noalloc", "idx_export", "idx_export_version",
           "idx_import_version", "idx_encoder_floats", "idx_set_encoder", "make_route_debug", "DTYPES"]
