"""Learned cluster representatives, CPU oracle side (test infrastructure).

paper-daily.com explainer, "代表向量为什么要学？": a cluster's mean scores badly
under the indexer score (per-head ReLU before the weighted sum), so the method
keeps grouping by distance and only corrects the representative.  One small
network per layer reads the cluster's summaries: the mean of the member keys, the
log of the cluster size, and the mean and the maximum over members of a learned
per-member transform; it outputs a bounded correction that is added to the mean
(zero correction = plain mean).  It runs when a seal or a refit creates clusters;
queries then score the representatives as before.

Readings (the pages give the structure, not the sizes):
* per-member transform: phi(x) = W2 ReLU(W1 x + b1) + b2, hidden width h;
* head: o = Wb ReLU(Wa z + ba) + bb with z = [mean, log n, mean_m phi, max_m phi];
* correction: alpha * tanh(o), so every coordinate moves by less than alpha;
* weights are inputs (trained ones are not available here: tests use seeded
  random ones).  Packed order, all float32: W1 [h, d], b1 [h], W2 [h, h], b2 [h],
  Wa [h, d + 1 + 2h], ba [h], Wb [d, h], bb [d], alpha.
Arithmetic in float64.
"""
from __future__ import annotations

import numpy as np


def encoder_floats(d: int, h: int = 128) -> int:
    return h * d + h + h * h + h + h * (d + 1 + 2 * h) + h + d * h + d + 1


def unpack(weights: np.ndarray, d: int, h: int = 128) -> dict:
    w = np.asarray(weights, dtype=np.float64).reshape(-1)
    if w.size != encoder_floats(d, h):
        raise ValueError("encoder weights have the wrong size")
    out, o = {}, 0
    for name, shape in (("W1", (h, d)), ("b1", (h,)), ("W2", (h, h)), ("b2", (h,)), ("Wa", (h, d + 1 + 2 * h)),
                        ("ba", (h,)), ("Wb", (d, h)), ("bb", (d,)), ("alpha", ())):
        size = int(np.prod(shape)) if shape else 1
        out[name] = w[o:o + size].reshape(shape) if shape else w[o]
        o += size
    return out


def encode(members_x: np.ndarray, mean: np.ndarray, weights: np.ndarray, h: int = 128) -> np.ndarray:
    """Representative of one cluster: members_x [n, d] (key values), mean [d] (the
    cluster's fp32 centroid).  Returns float64 [d]."""
    X = np.asarray(members_x, dtype=np.float64)
    ybar = np.asarray(mean, dtype=np.float64)
    d = ybar.shape[0]
    P = unpack(weights, d, h)
    n = X.shape[0]
    if n == 0:
        return ybar.copy()
    phi = np.maximum(X @ P["W1"].T + P["b1"], 0.0) @ P["W2"].T + P["b2"]      # [n, h]
    z = np.concatenate([ybar, [np.log(n)], phi.mean(axis=0), phi.max(axis=0)])
    o = P["Wb"] @ np.maximum(P["Wa"] @ z + P["ba"], 0.0) + P["bb"]
    return ybar + P["alpha"] * np.tanh(o)
