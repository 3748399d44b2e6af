"""ctypes declarations of the C ABI in include/ivftk.h and the library loader."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libivftk.so")

c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64
c_vp = ctypes.c_void_p


class idx_config(ctypes.Structure):
    _fields_ = [("heads", c_i32), ("dim", c_i32), ("dtype", c_i32), ("n_sink", c_i32), ("window", c_i32),
                ("cluster_size", c_i32), ("seal_cap", c_i32), ("seal_iters", c_i32), ("refit_every", c_i32),
                ("max_queries", c_i32), ("max_budget", c_i32), ("max_k", c_i32), ("rescore_mode", c_i32), ("cluster_mode", c_i32),
                ("max_keys", c_i64)]


class idx_info(ctypes.Structure):
    _fields_ = [("n_keys", c_i64), ("sealed_windows", c_i32), ("computed_epoch", c_i32),
                ("published_epoch", c_i32), ("clusters_per_window", c_i32), ("slots_per_epoch", c_i32),
                ("device_bytes", c_i64)]


class idx_route_debug(ctypes.Structure):
    _fields_ = [("cand", c_vp), ("cand_cap", c_i32), ("cand_len", c_vp), ("order", c_vp), ("order_take", c_vp),
                ("order_cap", c_i32), ("n_order", c_vp), ("rep_scores", c_vp), ("rep_cap", c_i32),
                ("version", c_vp), ("events", ctypes.POINTER(c_vp)), ("list_cap", c_i32),
                ("cand_scores", c_vp)]


class idx_export_buf(ctypes.Structure):
    _fields_ = [("n_slots", c_i32), ("n_members", c_i32), ("sizes", c_vp), ("offsets", c_vp), ("members", c_vp),
                ("centroids", c_vp), ("reps", c_vp), ("rep_scale", c_vp), ("rep_f32", c_vp),
                ("n_screened", c_i64), ("n_brute", c_i64), ("n_bound_keys", c_i64), ("assign", c_vp), ("ub", c_vp),
                ("lb", c_vp)]


class idx_import_buf(ctypes.Structure):
    _fields_ = [("n_slots", c_i32), ("sizes", c_vp), ("members", c_vp), ("centroids", c_vp), ("reps", c_vp),
                ("rep_scale", c_vp), ("rep_f32", c_vp)]


# (name, restype, argtypes) of every exported function
SIGNATURES = [
    ("idx_create", c_i32, [ctypes.POINTER(idx_config), c_vp, ctypes.POINTER(c_vp)]),
    ("idx_destroy", c_i32, [c_vp]),
    ("idx_last_error", ctypes.c_char_p, []),
    ("idx_get_info", c_i32, [c_vp, ctypes.POINTER(idx_info)]),
    ("idx_build_seal", c_i32, [c_vp, c_vp, c_vp, c_i64, c_vp]),
    ("idx_refit", c_i32, [c_vp, c_vp, c_vp, ctypes.POINTER(c_i32)]),
    ("idx_publish", c_i32, [c_vp, c_vp, ctypes.POINTER(c_i32)]),
    ("idx_abandon_refit", c_i32, [c_vp, c_vp, ctypes.POINTER(c_i32)]),
    ("idx_route_topk", c_i32, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_vp,
                               ctypes.POINTER(idx_route_debug), c_vp]),
    ("idx_route_topk_pos", c_i32, [c_vp, c_vp, c_vp, c_vp, ctypes.POINTER(c_i64), c_i32, c_i32, c_i32, c_vp, c_vp,
                                   ctypes.POINTER(idx_route_debug), c_vp]),
    ("idx_exhaustive_workspace_bytes", c_i64, [c_i64, c_i32]),
    ("idx_exhaustive_topk", c_i32, [c_vp, c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_i64, c_i32, c_i32,
                                    c_vp, c_vp, c_vp, c_i64, c_vp]),
    ("idx_exhaustive_topk_noalloc", c_i32, [c_vp, c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_i64, c_i32,
                                            c_i32, c_vp, c_vp, c_vp]),
    ("idx_export", c_i32, [c_vp, c_i32, ctypes.POINTER(idx_export_buf)]),
    ("idx_export_version", c_i32, [c_vp, c_i64, ctypes.POINTER(c_i32), ctypes.POINTER(c_i32),
                                   ctypes.POINTER(idx_export_buf)]),
    ("idx_import_version", c_i32, [c_vp, c_i64, ctypes.POINTER(idx_import_buf), c_vp]),
    ("idx_encoder_floats", c_i64, [c_i32]),
    ("idx_set_encoder", c_i32, [c_vp, c_vp, c_vp]),
]

_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libivftk.so (or the build named by IVFTK_LIBRARY, e.g. the host
    AddressSanitizer build); raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("IVFTK_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m ivf_top_key_amd.build` "
                          "(hipcc, gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
