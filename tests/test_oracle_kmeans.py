"""Pins for the oracle's exact-order clustering arithmetic.

* Distances and means against float64 (scipy / numpy) within the fp32 error
  bound of a sequential sum, which fails on a dropped term, a transposed
  operand or a wrong axis.
* The fused multiply-add (one rounding of a*b + c) against rational
  arithmetic rounded to fp32 from the format's definition, including values a
  hair off a midpoint of two fp32 neighbours, and the distance chain replayed
  term by term in rational arithmetic (which a two-rounding chain fails).
* The capped greedy assignment against an independent certificate: an
  assignment equals the greedy walk over (distance, key, cluster) in ascending
  order if and only if, for every key, each cluster it prefers to its own is
  full of keys whose triples come earlier (a short exchange argument shows
  that only one assignment satisfies this).
* A non-binding cap reduces seal to textbook Lloyd from the same initial
  centres: scikit-learn's KMeans (algorithm="lloyd") is the library reference.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy.spatial.distance import cdist
from sklearn.cluster import KMeans

from oracle.kmeans import capped_greedy_assign, fma32, mean_exact, nearest, seal_window, sqdist_exact

U = 2.0 ** -24


def _round_f32(x: Fraction) -> float:
    """The fp32 value nearest to the rational x, ties to the even significand
    (written from the format's definition: 24-bit significands, subnormals below
    2^-126 with quantum 2^-149, no overflow handling)."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    q = x / quantum
    n = q.numerator // q.denominator
    rest = q - n
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n * quantum)


def _fma_ref(a, b, c) -> float:
    return _round_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def test_fma32_is_the_single_rounding_of_a_times_b_plus_c():
    rng = np.random.default_rng(13)
    n = 3000
    a = (rng.standard_normal(n) * 2.0 ** rng.integers(-30, 30, n)).astype(np.float32)
    b = (rng.standard_normal(n) * 2.0 ** rng.integers(-30, 30, n)).astype(np.float32)
    c = (rng.standard_normal(n) * 2.0 ** rng.integers(-60, 60, n)).astype(np.float32)
    got = fma32(a, b, c)
    want = np.array([_fma_ref(x, y, z) for x, y, z in zip(a, b, c)], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # a plain product-then-sum rounds twice and differs somewhere
    assert not np.array_equal((a * b + c).view(np.uint32), want.view(np.uint32))


def test_fma32_when_the_wide_sum_lands_on_a_midpoint():
    """a*b + c a hair off the midpoint of two fp32 neighbours, closer than fp64 can
    tell apart: a rounding of the fp64 sum would take the even neighbour, the single
    rounding must take the side the exact value is on."""
    u = 2.0 ** -24
    c = np.float32(1 + 2 * u)                       # odd last bit
    a = np.float32(1 + 2.0 ** -15)
    b = np.float32((1 - 2.0 ** -15) * u)            # a*b = u (1 - 2^-30)
    assert float(fma32(a, b, c)) == float(c)        # just below c + u: stays at c
    assert float(fma32(-a, b, c)) == float(c)       # just above c - u: rounds up to c
    assert _fma_ref(a, b, c) == float(c) and _fma_ref(-a, b, c) == float(c)
    # an exact tie goes to the even neighbour
    h = np.float32(2.0 ** -12)
    assert float(fma32(h, h, c)) == 1 + 4 * u == _fma_ref(h, h, c)


def test_sqdist_is_the_fused_chain_in_ascending_dimension():
    """Each term: t = x_i - c_i rounded to fp32, then acc = t*t + acc rounded once,
    i ascending from acc = +0; replayed here in rational arithmetic."""
    rng = np.random.default_rng(14)
    X = rng.standard_normal((6, 24)).astype(np.float32)
    C = rng.standard_normal((4, 24)).astype(np.float32)
    D = sqdist_exact(X, C)
    for j in range(6):
        for c in range(4):
            acc = 0.0
            for i in range(24):
                t = _round_f32(Fraction(float(X[j, i])) - Fraction(float(C[c, i])))
                acc = _round_f32(Fraction(t) * Fraction(t) + Fraction(acc))
            assert float(D[j, c]) == acc
    # the plain two-rounding chain gives other bits on these rows
    two = np.zeros((6, 4), np.float32)
    for i in range(24):
        t = X[:, i:i + 1] - C[None, :, i]
        two = two + t * t
    assert not np.array_equal(two.view(np.uint32), D.view(np.uint32))


def test_sqdist_within_sequential_sum_bound():
    rng = np.random.default_rng(10)
    X = rng.standard_normal((200, 128)).astype(np.float32)
    C = (rng.standard_normal((17, 128)) * 0.5).astype(np.float32)
    D = sqdist_exact(X, C).astype(np.float64)
    ref = cdist(X.astype(np.float64), C.astype(np.float64), "sqeuclidean")
    gamma = (128 + 2) * U
    assert np.all(np.abs(D - ref) <= gamma * ref * 1.01)
    assert np.array_equal(nearest(D), np.argmin(D, axis=1))


def test_sqdist_is_exact_on_small_integers():
    rng = np.random.default_rng(11)
    X = rng.integers(-50, 50, (30, 32)).astype(np.float32)
    C = rng.integers(-50, 50, (5, 32)).astype(np.float32)
    ref = ((X[:, None, :].astype(np.int64) - C[None].astype(np.int64)) ** 2).sum(-1)
    assert np.array_equal(sqdist_exact(X, C), ref.astype(np.float32))


def test_mean_within_bound_and_exact_on_integers():
    rng = np.random.default_rng(12)
    rows = rng.standard_normal((300, 64)).astype(np.float32)
    m = mean_exact(rows).astype(np.float64)
    ref = rows.astype(np.float64).mean(0)
    bound = (300 + 1) * U * np.abs(rows.astype(np.float64)).mean(0) * 1.01 + 1e-30
    assert np.all(np.abs(m - ref) <= bound)
    ints = rng.integers(-1000, 1000, (64, 8)).astype(np.float32)
    assert np.array_equal(mean_exact(ints), (ints.astype(np.float64).sum(0) / 64).astype(np.float32))


def _certificate_holds(D, assign, cap):
    n, m = D.shape
    key = lambda j, c: (D[j, c], j, c)      # the global order of triples
    members = {c: np.nonzero(assign == c)[0] for c in range(m)}
    if any(len(v) > cap for v in members.values()) or np.any(assign < 0):
        return False
    for j in range(n):
        mine = key(j, assign[j])
        for c in range(m):
            if c == assign[j] or key(j, c) > mine:
                continue
            full_early = len(members[c]) == cap and all(key(jj, c) < key(j, c) for jj in members[c])
            if not full_early:
                return False
    return True


@pytest.mark.parametrize("seed", range(6))
def test_capped_greedy_matches_certificate(seed):
    rng = np.random.default_rng(20 + seed)
    n, m = 48, 4
    cap = 12 + seed % 3
    # clustered data so that the cap binds
    X = np.concatenate([rng.standard_normal((36, 3)) * 0.2, rng.standard_normal((12, 3)) + 3]).astype(np.float32)
    C = X[rng.choice(n, m, replace=False)]
    D = sqdist_exact(X, C)
    if seed % 2:                      # exact distance ties
        D = np.round(D * 2) / 2
    a = capped_greedy_assign(D, cap)
    assert _certificate_holds(D, a, cap)
    # a plausible wrong walk (by key first) usually breaks the certificate
    order = np.lexsort((np.tile(np.arange(m), n), D.reshape(-1), np.repeat(np.arange(n), m)))
    wrong = np.full(n, -1)
    cnt = np.zeros(m, int)
    for t in order:
        j, c = divmod(t, m)
        if wrong[j] < 0 and cnt[c] < cap:
            wrong[j] = c
            cnt[c] += 1
    if not np.array_equal(wrong, a):
        assert not _certificate_holds(D, wrong, cap)


def test_capped_greedy_equals_nearest_when_cap_does_not_bind():
    rng = np.random.default_rng(30)
    X = rng.standard_normal((100, 8)).astype(np.float32)
    C = X[:5].copy()
    D = sqdist_exact(X, C)
    near = nearest(D)
    cap = int(np.bincount(near, minlength=5).max())
    assert np.array_equal(capped_greedy_assign(D, cap), near)
    assert np.array_equal(capped_greedy_assign(D, 100), near)


def test_seal_without_binding_cap_is_textbook_lloyd():
    rng = np.random.default_rng(31)
    centres = rng.standard_normal((8, 16)) * 4
    X = (centres[rng.integers(0, 8, 1024)] + rng.standard_normal((1024, 16)) * 0.3).astype(np.float32)
    a, C, alive = seal_window(X, 8, cap=1024, iters=10)
    init = np.array([((2 * i + 1) * 1024) // 16 for i in range(8)])
    km = KMeans(n_clusters=8, init=X[init], n_init=1, max_iter=10, tol=0.0, algorithm="lloyd").fit(X)
    assert np.array_equal(a, km.labels_)
    assert np.allclose(C[alive], km.cluster_centers_[alive], rtol=0, atol=1e-5)


def test_seal_capped_result_is_a_greedy_fixed_point():
    rng = np.random.default_rng(32)
    X = (rng.standard_normal((256, 8)) * np.r_[np.ones(4) * 3, np.ones(4) * 0.1]).astype(np.float32)
    X[:200] *= 0.05                                      # one dense blob: the cap must bind
    a, C, alive = seal_window(X, 4, cap=80, iters=6)
    assert np.bincount(a, minlength=4).max() <= 80
    for c in range(4):
        if alive[c]:
            assert np.array_equal(C[c], mean_exact(X[a == c]))


def test_seal_blocks_are_contiguous_means():
    """Positional blocks: block i is keys [i*b, (i+1)*b) and its centroid is their mean
    (the plain mean in float64 agrees to fp32 rounding)."""
    from oracle.kmeans import seal_blocks
    rng = np.random.default_rng(3)
    X = rng.standard_normal((1024, 32)).astype(np.float32)
    a, C, alive = seal_blocks(X, 8)
    assert alive.all()
    assert np.array_equal(a, np.repeat(np.arange(8), 128))
    for i in range(8):
        ref = X[i * 128:(i + 1) * 128].astype(np.float64).mean(axis=0)
        assert np.allclose(C[i], ref, rtol=0, atol=1e-5)
    with pytest.raises(ValueError):
        seal_blocks(X[:1001], 8)
