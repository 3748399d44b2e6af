"""DSA indexer score in float64, CPU oracle side (test infrastructure).

paper-daily.com explainer, sections "它到底在解决什么问题？" and
"代表向量为什么要学？": the indexer gives query t a score for each earlier key j
by taking, per head h, the inner product of the head's query vector with the
key, passing it through ReLU, and adding the results with per-head weights:

    s(t, j) = sum_h w[t, h] * ReLU(q[t, h] . k[j])

Stored vectors are dequantised first: an E4M3 query row is its codes times its
fp32 scale, an E4M3 key is its codes times its per-token fp32 scale.  All of
these are exact in float64, and the inner products here are float64, so the
values below are the true scores up to ~1e-16 relative.
"""
from __future__ import annotations

import numpy as np


def indexer_scores(qv: np.ndarray, w: np.ndarray, kv: np.ndarray, block: int = 8) -> np.ndarray:
    """qv [T, H, d], w [T, H], kv [N, d] (all real values) -> scores [T, N] float64."""
    qv = np.asarray(qv, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    T, H, d = qv.shape
    out = np.empty((T, kv.shape[0]), dtype=np.float64)
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        dots = qv[t0:t1].reshape(-1, d) @ kv.T                # [(t, h), j]
        dots = np.maximum(dots, 0.0).reshape(t1 - t0, H, -1)  # ReLU per head
        out[t0:t1] = np.einsum("th,thj->tj", w[t0:t1], dots)
    return out


def score_error_scale(qv: np.ndarray, w: np.ndarray, kv: np.ndarray, block: int = 8) -> np.ndarray:
    """sigma(t, j) = sum_h |w[t,h]| * sum_i |q[t,h,i] * k[j,i]|.

    The scale of the rounding error of any evaluation of s(t, j) in a lower
    precision; sigma >= |s(t, j)|.  Tolerances are stated relative to it.
    """
    return indexer_scores(np.abs(np.asarray(qv, np.float64)), np.abs(np.asarray(w, np.float64)),
                          np.abs(np.asarray(kv, np.float64)), block=block)
