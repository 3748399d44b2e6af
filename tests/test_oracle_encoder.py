"""Oracle pins for the learned-representative encoder (paper-daily explainer,
"代表向量为什么要学？"): zero output layer = plain mean, permutation invariance over
members, the bound alpha, and the pages' two-member example worked by hand."""
import numpy as np
import pytest

import datagen
from oracle.encoder import encode, encoder_floats, unpack


def _pack(d, h, W1, b1, W2, b2, Wa, ba, Wb, bb, alpha):
    parts = [np.asarray(a, dtype=np.float64).reshape(-1) for a in (W1, b1, W2, b2, Wa, ba, Wb, bb)]
    return np.concatenate(parts + [np.array([alpha])])


def test_sizes_and_unpack_roundtrip():
    d, h = 5, 3
    w = np.arange(encoder_floats(d, h), dtype=np.float64)
    P = unpack(w, d, h)
    assert P["W1"].shape == (3, 5) and P["Wa"].shape == (3, 5 + 1 + 6) and P["Wb"].shape == (5, 3)
    assert P["alpha"] == w[-1] and P["W1"][0, 0] == 0 and P["b1"][0] == 15
    w2 = datagen.encoder_weights(0, 32)
    assert w2.size == encoder_floats(32) and w2.dtype == np.float32


def test_zero_output_layer_gives_the_mean():
    """With Wb = 0 and bb = 0 the correction vanishes: the plain-IVF mean (the pages:
    the correction starts at zero, so the index starts as plain IVF)."""
    rng = np.random.default_rng(1)
    d = 16
    w = datagen.encoder_weights(1, d, h=8).astype(np.float64)
    P = unpack(w, d, 8)
    off = encoder_floats(d, 8) - 1 - d - d * 8
    w[off:-1] = 0.0
    X = rng.standard_normal((7, d)).astype(np.float32)
    m = X.mean(axis=0).astype(np.float32)
    assert np.array_equal(encode(X, m, w, h=8), m.astype(np.float64))
    assert P["Wb"].shape == (d, 8)


def test_permutation_invariance_and_bound():
    rng = np.random.default_rng(2)
    d = 32
    w = datagen.encoder_weights(2, d, alpha=0.3)
    X = rng.standard_normal((40, d)).astype(np.float32)
    m = X.mean(axis=0).astype(np.float32)
    r1 = encode(X, m, w)
    r2 = encode(X[rng.permutation(40)], m, w)
    assert np.allclose(r1, r2, rtol=0, atol=1e-12)
    assert np.all(np.abs(r1 - m) < 0.3)
    assert np.any(np.abs(r1 - m) > 1e-3)          # random weights do move the representative


def test_two_member_example_by_hand():
    """The pages' example: members -2 and 2 (one head, weight 1, query 1).  The mean 0
    scores ReLU(1 * 0) = 0.  With h = 1, W1 = W2 = 1, Wa = [0, 0, 1, 1], Wb = 1, all
    biases 0, alpha = 0.5: phi = [0, 2], mean 1, max 2, z = [0, log 2, 1, 2], u = 3,
    o = 3, representative 0.5 * tanh(3); the query now scores it above zero."""
    w = _pack(1, 1, [[1.0]], [0.0], [[1.0]], [0.0], [[0.0, 0.0, 1.0, 1.0]], [0.0], [[1.0]], [0.0], 0.5)
    X = np.array([[-2.0], [2.0]], dtype=np.float32)
    r = encode(X, np.zeros(1, np.float32), w, h=1)
    assert r.shape == (1,) and r[0] == pytest.approx(0.5 * np.tanh(3.0), rel=1e-15)
    assert max(1.0 * r[0], 0.0) > 0.0


def test_index_with_encoder_keeps_clusters_and_moves_reps():
    """An encoder changes only the representatives: members and centroids are those of
    the plain index, and each representative is the encoder's output for its cluster."""
    from oracle import OracleConfig, OracleIndex
    from oracle.encoder import encode
    from oracle import codec
    inp = datagen.workload_inputs(5, 4200, 1, 4199, 2, 32, 8, "f32")
    w = datagen.encoder_weights(5, 32)
    base = dict(heads=2, dim=32, dtype="f32", n_sink=4, window=1024, cluster_size=128, refit_every=2048)
    a, b = OracleIndex(OracleConfig(**base)), OracleIndex(OracleConfig(**base, encoder=w))
    for ix in (a, b):
        ix.append(inp["keys"], None)
        while ix.refit_due():
            ix.refit()
            ix.publish()
    for ca, cb in zip([c for s in a.seals for c in s] + a.epochs[a.published],
                      [c for s in b.seals for c in s] + b.epochs[b.published]):
        assert np.array_equal(ca.members, cb.members) and np.array_equal(ca.centroid, cb.centroid)
        if cb.members.size:
            ref = encode(b.X[cb.members], cb.centroid, w).astype(np.float32)
            raw, _ = codec.quantize_rep(ref, "f32")
            assert np.array_equal(cb.rep_raw, raw)
            assert not np.array_equal(cb.rep_raw, ca.rep_raw)
