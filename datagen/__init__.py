"""Seeded synthetic inputs for the indexer top-k workloads.

This module is shared by the CPU oracle, the tests and the benchmark.  It only
draws random numbers and casts them to the stored formats (fp32, bf16 bit
patterns, OCP E4M3 codes with a per-token fp32 scale).  It holds none of the
selection method's arithmetic: no scores, no clustering, no routing.

Recipe (the pages evaluate on LongBench-v2, RULER and InfiniteBench with real
models; none of that is available, so a Gaussian mixture of the DSA indexer's
shape stands in for it):

* M unit-norm centres mu_m = g / |g|, g ~ N(0, I_d).
* Key j belongs to a component that drifts slowly with position
  (phi(j) = floor(j*M/N)): with probability 0.8 it is phi(j)+U{-2..2} mod M,
  otherwise a uniform component (content that recurs across the sequence).
  k_j = mu_z + (0.3/sqrt(d)) * eps, eps ~ N(0, I_d).
* Query (t, h) picks a uniform component and adds the same noise.
* Head weights w[t, h] ~ N(0, 1/H) (may be negative).
* bf16 is round-to-nearest-even from fp32; E4M3 uses a per-token scale
  amax/448 and a round-to-nearest-even, saturating encode.

Every stream comes from numpy's PCG64 seeded with SeedSequence([seed, stream]).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "make_keys",
    "make_queries",
    "make_weights",
    "cast_rows",
    "bf16_bits_from_f32",
    "e4m3_codes_from_f32",
    "STREAM_CENTRES",
]

STREAM_CENTRES = 0
STREAM_KEY_COMPONENT = 1
STREAM_KEY_NOISE = 2
STREAM_QUERY = 3
STREAM_WEIGHT = 4
STREAM_ADVERSARIAL = 5
STREAM_ENCODER = 6


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(stream)]))


def centres(seed: int, M: int, d: int) -> np.ndarray:
    g = _rng(seed, STREAM_CENTRES).standard_normal((M, d))
    return g / np.linalg.norm(g, axis=1, keepdims=True)


def make_keys(seed: int, N: int, d: int, M: int, noise: float = 0.3,
              p_drift: float = 0.8, start: int = 0, count: int | None = None) -> np.ndarray:
    """fp32 keys for positions [start, start+count) of an N-key sequence.

    Generating a sub-range gives exactly the rows of the full draw, so a
    benchmark can stream a long prefix chunk by chunk.
    """
    if count is None:
        count = N - start
    mu = centres(seed, M, d)
    out = np.empty((count, d), dtype=np.float32)
    comp_rng = _rng(seed, STREAM_KEY_COMPONENT)
    noise_rng = _rng(seed, STREAM_KEY_NOISE)
    block = 1 << 16
    # draw in fixed blocks of the full sequence so that sub-ranges agree
    b0 = start // block
    b1 = (start + count + block - 1) // block
    for b in range(b1):
        lo, hi = b * block, min(N, (b + 1) * block)
        if hi <= lo:
            break
        u = comp_rng.random(hi - lo)
        off = comp_rng.integers(-2, 3, size=hi - lo)
        uni = comp_rng.integers(0, M, size=hi - lo)
        eps = noise_rng.standard_normal((hi - lo, d))
        if b < b0:
            continue
        j = np.arange(lo, hi, dtype=np.int64)
        phi = (j * M) // N
        z = np.where(u < p_drift, (phi + off) % M, uni)
        rows = mu[z] + (noise / np.sqrt(d)) * eps
        s0, s1 = max(lo, start), min(hi, start + count)
        if s1 > s0:
            out[s0 - start:s1 - start] = rows[s0 - lo:s1 - lo].astype(np.float32)
    return out


def make_queries(seed: int, T: int, H: int, d: int, M: int, noise: float = 0.3) -> np.ndarray:
    rng = _rng(seed, STREAM_QUERY)
    mu = centres(seed, M, d)
    m = rng.integers(0, M, size=(T, H))
    eps = rng.standard_normal((T, H, d))
    return (mu[m] + (noise / np.sqrt(d)) * eps).astype(np.float32)


def make_weights(seed: int, T: int, H: int) -> np.ndarray:
    rng = _rng(seed, STREAM_WEIGHT)
    return (rng.standard_normal((T, H)) / np.sqrt(H)).astype(np.float32)


def adversarial_directions(seed: int, M: int, d: int) -> np.ndarray:
    """u_m: a unit direction orthogonal to each centre mu_m."""
    rng = _rng(seed, STREAM_ADVERSARIAL + 100)
    mu = centres(seed, M, d)
    g = rng.standard_normal((M, d))
    g -= (g * mu).sum(1, keepdims=True) * mu
    return g / np.linalg.norm(g, axis=1, keepdims=True)


def make_adversarial_queries(seed: int, T: int, H: int, d: int, M: int, noise: float = 0.3) -> np.ndarray:
    """Queries along the hidden directions: q_{t,h} = u_m + noise for a uniform m."""
    rng = _rng(seed, STREAM_QUERY + 100)
    u = adversarial_directions(seed, M, d)
    m = rng.integers(0, M, size=(T, H))
    eps = rng.standard_normal((T, H, d))
    return (u[m] + (noise / np.sqrt(d)) * eps).astype(np.float32)


def make_adversarial_keys(seed: int, N: int, d: int, M: int, a: float = 1.0,
                          noise: float = 0.3) -> np.ndarray:
    """Mixture whose components hold members of opposite sign along u_m.

    k = mu_m + s * a * u_m + noise with s = +-1 and u_m orthogonal to mu_m, so a
    component's mean hides its members that align with u_m.
    """
    rng = _rng(seed, STREAM_ADVERSARIAL)
    mu = centres(seed, M, d)
    u = adversarial_directions(seed, M, d)
    j = np.arange(N)
    z = np.where(rng.random(N) < 0.8, ((j * M) // N + rng.integers(-2, 3, N)) % M,
                 rng.integers(0, M, N))
    s = np.where(rng.random(N) < 0.5, -1.0, 1.0)
    eps = rng.standard_normal((N, d))
    return (mu[z] + (s * a)[:, None] * u[z] + (noise / np.sqrt(d)) * eps).astype(np.float32)


def encoder_weights(seed: int, d: int, alpha: float = 0.25, h: int = 128) -> np.ndarray:
    """Seeded stand-in weights for the learned-representative encoder (packed order:
    W1 [h, d], b1 [h], W2 [h, h], b2 [h], Wa [h, d + 1 + 2h], ba [h], Wb [d, h], bb [d],
    alpha), matrices N(0, 1/fan_in), biases zero."""
    rng = _rng(seed, STREAM_ENCODER)
    parts = []
    for rows, cols in ((h, d), (h, h), (h, d + 1 + 2 * h), (d, h)):
        parts.append((rng.standard_normal((rows, cols)) / np.sqrt(cols)).reshape(-1))
        parts.append(np.zeros(rows))
    parts.append(np.array([alpha]))
    return np.concatenate(parts).astype(np.float32)


# --------------------------------------------------------------------------
# casts to the stored formats
# --------------------------------------------------------------------------

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def e4m3_codes_from_f32(x: np.ndarray) -> np.ndarray:
    """OCP E4M3 (e4m3fn) codes: round to nearest even, saturate at +-448.

    Input values must be finite.  The sign bit of the input is kept (so a
    negative value that rounds to zero gives code 0x80).  Works on the fp32
    bit pattern: a normal E4M3 value keeps 3 of fp32's 23 mantissa bits, and
    the subnormal range (below 2**-6) is a multiple of 2**-9.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    sign = (bits >> 31).astype(np.uint8)
    mag = bits & np.uint32(0x7FFFFFFF)
    # round the fp32 pattern to 3 mantissa bits (ties to even); the result is
    # (exponent << 3 | mantissa) with fp32's exponent bias 127, E4M3's is 7
    r = (mag + np.uint32(0x7FFFF) + ((mag >> 20) & np.uint32(1))) >> 20
    code_normal = r.astype(np.int64) - (120 << 3)
    code_sub = np.rint(np.abs(x) * np.float32(512.0)).astype(np.int64)
    code = np.where(mag >= np.uint32(0x3C800000), code_normal, code_sub)
    code = np.minimum(code, 0x7E)
    return (code.astype(np.uint8) | (sign << 7)).astype(np.uint8)


def cast_rows(x: np.ndarray, dtype: str):
    """Cast fp32 rows [..., d] to the stored format.

    Returns (data, scale): data is float32 / uint16 (bf16 bits) / uint8 (E4M3
    codes); scale is None except for E4M3, where it is the fp32 per-row scale
    amax/448 (1.0 for an all-zero row).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy(), None
    if dtype == "bf16":
        return bf16_bits_from_f32(x), None
    if dtype == "e4m3":
        amax = np.abs(x).max(axis=-1).astype(np.float32)
        scale = (amax / np.float32(448.0)).astype(np.float32)
        scale = np.where(amax > 0, scale, np.float32(1.0)).astype(np.float32)
        codes = np.empty(x.shape, dtype=np.uint8)
        flat_x = x.reshape(-1, x.shape[-1])
        flat_c = codes.reshape(-1, x.shape[-1])
        flat_s = scale.reshape(-1)
        step = 16384
        for r0 in range(0, flat_x.shape[0], step):
            r1 = min(flat_x.shape[0], r0 + step)
            flat_c[r0:r1] = e4m3_codes_from_f32(flat_x[r0:r1] / flat_s[r0:r1, None])
        return codes, scale
    raise ValueError(f"unknown dtype {dtype!r}")


def workload_inputs(seed: int, N: int, T: int, q_pos0: int, H: int, d: int, M: int, dtype: str,
                    key_start: int = 0, key_count: int | None = None):
    """Keys (stored form + scale), queries (stored form + per (t, h) scale) and weights.

    Query scales for E4M3 are per token (one amax over all heads), repeated
    over heads so the [T, H] layout is the same for every format.
    """
    kf = make_keys(seed, N, d, M, start=key_start, count=key_count)
    keys, kscale = cast_rows(kf, dtype)
    qf = make_queries(seed, T, H, d, M)
    if dtype == "e4m3":
        flat = qf.reshape(T, H * d)
        qcodes, qs = cast_rows(flat, dtype)
        q = qcodes.reshape(T, H, d)
        qscale = np.repeat(qs[:, None], H, axis=1).astype(np.float32)
    else:
        q, _ = cast_rows(qf, dtype)
        qscale = None
    w = make_weights(seed, T, H)
    return dict(keys=keys, k_scale=kscale, q=q, q_scale=qscale, w=w,
                N=N, T=T, q_pos0=q_pos0, H=H, d=d, dtype=dtype)
