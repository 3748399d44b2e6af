"""Recall of a routed top-k against the exhaustive top-k (test infrastructure).

paper-daily.com explainer, end of "它到底在解决什么问题？": recall is an
evaluation metric only.  The indexer scores every key offline, its top k is
the reference answer, and recall is the share of that answer that the coarse
plus fine selection also returns.  The system does not know it at inference.
"""
from __future__ import annotations

import numpy as np


def recall_per_query(routed: np.ndarray, reference: np.ndarray) -> np.ndarray:
    """|R_t intersect E_t| / |E_t| per query (padding entries -1 ignored)."""
    out = np.empty(routed.shape[0], dtype=np.float64)
    for t in range(routed.shape[0]):
        ref = reference[t][reference[t] >= 0]
        got = routed[t][routed[t] >= 0]
        out[t] = 1.0 if ref.size == 0 else np.intersect1d(ref, got).size / ref.size
    return out


def summarize(r: np.ndarray) -> dict:
    return dict(mean=float(np.mean(r)), p5=float(np.percentile(r, 5)), min=float(np.min(r)))
