"""The hand-computed tiny index of tests/golden/hand_index.json, as arrays.

Shared by the oracle pin (CPU) and the library test (GPU): both build the same
keys, queries and imported epoch from the fixture's numbers, then compare with
the expected values the fixture states.
"""
import json
import os

import numpy as np

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_index.json")
D, H = 32, 4


def load():
    with open(PATH) as f:
        return json.load(f)


def keys(g):
    v = np.asarray(g["v"], np.float32)
    k = np.zeros((v.size, D), np.float32)
    k[:, 0] = v
    k[:, 1] = 0.25 * (np.arange(v.size) + 1)
    return k


def query(g):
    q = np.zeros((1, H, D), np.float32)
    q[0, 0, 0] = 1.0
    for h, row in enumerate(g["other_heads"], start=1):
        q[0, h, :3] = row
    w = np.array([[1.0, 0.0, 0.0, 0.0]], np.float32)
    return q, w


def epoch_arrays(g):
    """sizes, flat members, centroids (float32 means of the members) and
    representatives (fp32, coordinate 0 from the fixture) of the imported epoch."""
    mem = g["epoch1"]["members"]
    k = keys(g)
    sizes = np.array([len(m) for m in mem], np.int32)
    flat = np.concatenate([np.asarray(m, np.int32) for m in mem])
    cents = np.stack([k[m].astype(np.float64).mean(0).astype(np.float32) for m in mem])
    reps = np.zeros((len(mem), D), np.float32)
    reps[:, 0] = g["epoch1"]["rep0"]
    return sizes, flat, cents, reps
