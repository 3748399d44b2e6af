// Device-side building blocks shared by every kernel of the library (gfx950, wave64).
//
// * Stored formats: fp32, bf16, OCP E4M3 (e4m3fn).  Decoding is exact (E4M3 through
//   the hardware conversion); encoding is round-to-nearest-even, saturating at +-448
//   for E4M3.
// * Composite sort keys: (order-preserving bits of an fp32 score) << 32 | ~position,
//   so that a larger key means a higher score and, among equal scores, a lower
//   position (the tie rule of the top-k and of cluster ranking).
// * LDS bitonic sort and a weighted radix select over such keys.
// * The indexer-score tile: for one query (H heads) against 32 keys, MFMA contracts
//   q[h] . k[j] over d with fp32 accumulation, then the epilogue reduces
//   sum_h w'[h] * max(acc[h][j], 0) over heads inside the wave.  The same tile serves
//   representative scoring, candidate rescoring and exhaustive scoring, so a (query,
//   key) pair gets bit-identical scores on every path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef IVFTK_SWZ8
#define IVFTK_SWZ8(r) ((r) >> 1)
#endif

namespace ivftk {

enum { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2 };

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT>
struct Elem;
template <>
struct Elem<DT_F32> { static constexpr int bytes = 4; };
template <>
struct Elem<DT_BF16> { static constexpr int bytes = 2; };
template <>
struct Elem<DT_E4M3> { static constexpr int bytes = 1; };

// ---------------------------------------------------------------------------
// stored formats
// ---------------------------------------------------------------------------

// E4M3 code (low byte of the word) -> fp32 (exact).  gfx950's conversion instructions
// decode the OCP E4M3 format (bias 7, exponent field 0 subnormal: m * 2^-9, no
// infinities) exactly for every finite code; the NaN codes are never stored.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) { return __builtin_amdgcn_cvt_f32_fp8((int)code, 0); }

// The four E4M3 codes of a word (byte b is element b) -> fp32, two per instruction.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t word, float& x0, float& x1, float& x2, float& x3) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
  x0 = lo[0], x1 = lo[1], x2 = hi[0], x3 = hi[1];
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// fp32 -> E4M3 code, round to nearest even, saturating at 448, sign bit kept.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t mag = b & 0x7FFFFFFFu;
  uint32_t code;
  if (mag >= 0x43E00000u) {                 // >= 448
    code = 0x7Eu;
  } else if (mag >= 0x3C800000u) {          // >= 2^-6: normal, keep 3 mantissa bits
    const uint32_t r = (mag + 0x7FFFFu + ((mag >> 20) & 1u)) >> 20;
    code = r - (120u << 3);
    if (code > 0x7Eu) code = 0x7Eu;
  } else {                                  // subnormal: multiple of 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(mag) * 512.0f);
  }
  return code | sign;
}

// Element i of a stored row as fp32 (no scale).
template <int DT>
__device__ __forceinline__ float load_elem(const uint8_t* row, int i) {
  if constexpr (DT == DT_F32) {
    return reinterpret_cast<const float*>(row)[i];
  } else if constexpr (DT == DT_BF16) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[i]);
  } else {
    return e4m3_to_f32(row[i]);
  }
}

// N consecutive elements of a stored row as fp32 times sk (sk = 1 for unscaled
// formats): 16-byte loads first, then the conversion, so all loads are in flight
// together.  row must be 16-byte aligned and N * element size a multiple of 16.
template <int DT, int N>
__device__ __forceinline__ void load_row_f32(float (&x)[N], const uint8_t* row, float sk) {
  constexpr int EB = DT == DT_F32 ? 4 : (DT == DT_BF16 ? 2 : 1);
  constexpr int NV = N * EB / 16;
  static_assert(N * EB % 16 == 0, "whole 16-byte chunks");
  uint32_t w[4 * NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const uint4 q = reinterpret_cast<const uint4*>(row)[v];
    w[4 * v] = q.x, w[4 * v + 1] = q.y, w[4 * v + 2] = q.z, w[4 * v + 3] = q.w;
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if constexpr (DT == DT_F32) {
      x[i] = __uint_as_float(w[i]);
    } else if constexpr (DT == DT_BF16) {
      x[i] = bf16_to_f32((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
    }
  }
  if constexpr (DT == DT_E4M3) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      e4m3x4_to_f32(w[i >> 2], x[i], x[i + 1], x[i + 2], x[i + 3]);
#pragma unroll
      for (int u = 0; u < 4; ++u) x[i + u] = x[i + u] * sk;
    }
  }
}

// The elements of one 16-byte chunk of a stored row as fp32 times sk (sk = 1 for the
// unscaled formats).
template <int DT>
__device__ __forceinline__ void chunk_to_f32(const uint32_t (&wds)[4], float (&x)[16 / Elem<DT>::bytes], float sk) {
#pragma unroll
  for (int e = 0; e < 16 / Elem<DT>::bytes; ++e) {
    if constexpr (DT == DT_F32) {
      x[e] = __uint_as_float(wds[e]);
    } else if constexpr (DT == DT_BF16) {
      x[e] = bf16_to_f32((wds[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    }
  }
  if constexpr (DT == DT_E4M3) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      e4m3x4_to_f32(wds[q], x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
#pragma unroll
      for (int u = 0; u < 4; ++u) x[4 * q + u] = x[4 * q + u] * sk;
    }
  }
}

// ---------------------------------------------------------------------------
// composite keys
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t order_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;              // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_order_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o ^ 0x80000000u) : ~o);
}

__device__ __forceinline__ uint64_t make_comp(float score, uint32_t id) {
  return ((uint64_t)order_bits(score) << 32) | (uint64_t)(~id);
}

__device__ __forceinline__ uint32_t comp_id(uint64_t c) { return ~(uint32_t)c; }
__device__ __forceinline__ float comp_score(uint64_t c) { return from_order_bits((uint32_t)(c >> 32)); }

// The first K of a descending composite list of `avail` entries; missing entries
// (zero composites or past avail) are -1 / -inf.
__device__ inline void write_topk(const uint64_t* buf, int avail, int K, int* oi, float* os) {
  for (int i = threadIdx.x; i < K; i += blockDim.x) {
    const uint64_t v = i < avail ? buf[i] : 0ull;
    oi[i] = v ? (int)comp_id(v) : -1;
    if (os) os[i] = v ? comp_score(v) : -__builtin_inff();
  }
}

__host__ __device__ __forceinline__ int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// ---------------------------------------------------------------------------
// block-wide helpers (all threads of the block must call them)
// ---------------------------------------------------------------------------

// Sort a[0..n) (n a power of two) into descending order.
__device__ inline void bitonic_sort_desc(uint64_t* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = a[i], y = a[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            a[i] = y;
            a[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Sort v (one entry per lane, 64 lanes) into descending order across the wave.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v) {
  const int lane = threadIdx.x & 63;
  for (int k = 2; k <= 64; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)v, j), hi = __shfl_xor((uint32_t)(v >> 32), j);
      const uint64_t o = ((uint64_t)hi << 32) | lo;
      // segments of k lanes alternate direction; the last pass (k = 64) is descending
      const bool desc = (lane & k) == 0;
      const bool low = (lane & j) == 0;
      v = (low == desc) ? (v > o ? v : o) : (v < o ? v : o);
    }
  }
  return v;
}

// Sort a[0..n) (n a power of two) into ascending order.
__device__ inline void bitonic_sort_asc(uint64_t* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = a[i], y = a[ixj];
          const bool asc = (i & k) == 0;
          if (asc ? (x > y) : (x < y)) {
            a[i] = y;
            a[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

struct SelectScratch {
  int hist[256];
  int cnt[256];
  uint64_t prefix;
  int need;
  int count;
  uint64_t result;
};

// Weighted radix select over unique nonzero keys a[0..n).  Returns the key T with
//   sum_{a > T} w < target <= sum_{a >= T} w,
// where w = wts[i] (or 1 when wts is null).  Requires 1 <= target <= sum of w.
// Keys equal to 0 are ignored (padding).
__device__ inline uint64_t radix_select_desc(const uint64_t* a, const int* wts, int n, int target,
                                             SelectScratch& sc) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    sc.prefix = 0;
    sc.need = target;
  }
  __syncthreads();
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += blockDim.x) {
      sc.hist[i] = 0;
      sc.cnt[i] = 0;
    }
    __syncthreads();
    const uint64_t prefix = sc.prefix;
    const uint64_t mask = (shift == 56) ? 0ull : (~0ull << (shift + 8));
    for (int i = tid; i < n; i += blockDim.x) {
      const uint64_t v = a[i];
      if (v != 0 && (v & mask) == prefix) {
        const int d = (int)((v >> shift) & 255u);
        atomicAdd(&sc.hist[d], wts ? wts[i] : 1);
        atomicAdd(&sc.cnt[d], 1);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // lane L owns digits 255-4L .. 252-4L (descending)
      const int lane = tid;
      int s = 0;
      for (int q = 0; q < 4; ++q) s += sc.hist[255 - 4 * lane - q];
      int incl = s;
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      const int excl = incl - s;
      const int need = sc.need;
      if (excl < need && need <= incl) {
        int acc = excl;
        for (int q = 0; q < 4; ++q) {
          const int d = 255 - 4 * lane - q;
          if (acc + sc.hist[d] >= need) {
            sc.need = need - acc;
            sc.prefix = prefix | ((uint64_t)d << shift);
            sc.count = sc.cnt[d];
            break;
          }
          acc += sc.hist[d];
        }
      }
    }
    __syncthreads();
    if (sc.count == 1 || shift == 0) {
      const uint64_t p = sc.prefix;
      const uint64_t m2 = ~0ull << shift;
      for (int i = tid; i < n; i += blockDim.x) {
        const uint64_t v = a[i];
        if (v != 0 && (v & m2) == p) sc.result = v;
      }
      __syncthreads();
      return sc.result;
    }
  }
  return 0;  // not reached
}

struct Select32Scratch {
  int hist[256];
  uint32_t prefix;
  int need;
  int above;
};

// Radix select over 32-bit keys a[0..n): returns T with
//   count(a > T) < target <= count(a >= T); sc.above receives count(a > T).
// Requires 1 <= target <= n.  All threads of the block must call it.
__device__ inline uint32_t radix_select32_desc(const uint32_t* a, int n, int target, Select32Scratch& sc) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    sc.prefix = 0;
    sc.need = target;
    sc.above = 0;
  }
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += blockDim.x) sc.hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = sc.prefix;
    const uint32_t mask = (shift == 24) ? 0u : (~0u << (shift + 8));
    for (int i = tid; i < n; i += blockDim.x) {
      const uint32_t v = a[i];
      if ((v & mask) == prefix) atomicAdd(&sc.hist[(v >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 64) {
      const int lane = tid;
      int s = 0;
      for (int q = 0; q < 4; ++q) s += sc.hist[255 - 4 * lane - q];
      int incl = s;
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      const int excl = incl - s;
      const int need = sc.need;
      if (excl < need && need <= incl) {
        int acc = excl;
        for (int q = 0; q < 4; ++q) {
          const int d = 255 - 4 * lane - q;
          if (acc + sc.hist[d] >= need) {
            sc.need = need - acc;
            sc.above += acc;
            sc.prefix = prefix | ((uint32_t)d << shift);
            break;
          }
          acc += sc.hist[d];
        }
      }
    }
    __syncthreads();
  }
  return sc.prefix;
}

// Block-wide min and max of 32-bit keys (threads pass their partial min/max).
// tmp must hold 2 * (blockDim.x / 64) uints.
__device__ inline void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t a = __shfl_xor(mn, off), b = __shfl_xor(mx, off);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  if (lane == 0) {
    tmp[2 * wave] = mn;
    tmp[2 * wave + 1] = mx;
  }
  __syncthreads();
  mn = 0xFFFFFFFFu;
  mx = 0u;
  for (int i = 0; i < nw; ++i) {
    mn = tmp[2 * i] < mn ? tmp[2 * i] : mn;
    mx = tmp[2 * i + 1] > mx ? tmp[2 * i + 1] : mx;
  }
  __syncthreads();
}

// Monotone binning of scores by value: the keys' scores in [lo, hi] (lo, hi = the
// scores of the smallest and largest key) map to bin = trunc((x - lo) * nbin / (hi -
// lo)), clamped to [0, nbin).  Subtraction of a constant, multiplication by a
// positive constant and truncation never reverse an order, so a higher score never
// lands in a lower bin and equal scores share a bin.  Binning by value spreads a
// block's scores over the bins (keys in order-key space are logarithmic in the
// magnitude, which crowds most scores into a few bins and serialises the histogram
// atomics).
struct ValBins {
  float lo;
  float scale;
  int top;
  __device__ __forceinline__ uint32_t operator()(uint32_t okey) const {
    const float x = from_order_bits(okey);
    const int b = (int)((x - lo) * scale);
    return (uint32_t)(b < 0 ? 0 : (b > top ? top : b));
  }
};

// mn_key < mx_key are order keys; returns bins over their scores.
__device__ __forceinline__ ValBins make_bins(uint32_t mn_key, uint32_t mx_key, int nbin) {
  ValBins b;
  b.lo = from_order_bits(mn_key);
  const float span = from_order_bits(mx_key) - b.lo;
  b.scale = (span > 0.0f && span < __builtin_inff()) ? (float)nbin / span : 0.0f;
  b.top = nbin - 1;
  return b;
}

// Exclusive scan of v over the block in thread order; *total receives the sum.
// tmp must hold one int per wave (blockDim.x / 64 <= 16).
__device__ inline int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  int incl = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int x = tmp[i];
    if (i < wave) base += x;
    tot += x;
  }
  __syncthreads();
  if (total) *total = tot;
  return base + incl - v;
}

// ---------------------------------------------------------------------------
// the indexer-score tile
// ---------------------------------------------------------------------------
//
// MFMA shapes (32x32 output, 16 accumulators per lane):
//   fp32: v_mfma_f32_32x32x2_f32, bf16: v_mfma_f32_32x32x16_bf16,
//   E4M3: v_mfma_f32_32x32x64_f8f6f4 (both operands OCP E4M3).
// Operand layout: lane l feeds row/column (l & 31) and holds a contiguous half of
// that row, bytes [g*RB/2, (g+1)*RB/2) with g = l >> 5, consumed in KS steps.  A
// and B use the same split of the d dimension, so the contraction is over all of
// d whatever order the unit walks the elements of one step in.
// Output: lane l holds column (l & 31), rows 8*(v>>2) + 4*g + (v&3), v = 0..15.

template <int DT, int D>
struct Geo {
  static constexpr int RB = D * Elem<DT>::bytes;   // bytes per row
  static constexpr int HW = RB / 8;                // dwords per lane (half a row)
  static constexpr int KD = (DT == DT_F32) ? 1 : (DT == DT_BF16 ? 4 : 8);  // dwords per MFMA step
  static constexpr int KS = HW / KD;               // MFMA steps per 32x32 tile
  static_assert(HW % 4 == 0, "half row must be a multiple of 16 bytes");
};

template <int DT>
__device__ __forceinline__ void mfma_step(v16f& acc, const uint32_t* a, const uint32_t* b) {
  if constexpr (DT == DT_F32) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[0]), __uint_as_float(b[0]), acc, 0, 0, 0);
  } else if constexpr (DT == DT_BF16) {
    v8bf av, bv;
    __builtin_memcpy(&av, a, 16);
    __builtin_memcpy(&bv, b, 16);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
  } else {
    v8i av, bv;
    __builtin_memcpy(&av, a, 32);
    __builtin_memcpy(&bv, b, 32);
    // format selectors 0/0 = E4M3 for A and B; zero scales select the unscaled op
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
  }
}

// Load this lane's half row (HW dwords) from `row` (the row's first byte).
template <int DT, int D>
__device__ __forceinline__ void load_half_row(uint32_t* r, const uint8_t* row) {
  const int g = (threadIdx.x >> 5) & 1;
  const uint4* p = reinterpret_cast<const uint4*>(row + g * (Geo<DT, D>::RB / 2));
#pragma unroll
  for (int i = 0; i < Geo<DT, D>::HW / 4; ++i) {
    const uint4 v = p[i];
    r[4 * i + 0] = v.x;
    r[4 * i + 1] = v.y;
    r[4 * i + 2] = v.z;
    r[4 * i + 3] = v.w;
  }
}

// One query's A operands: HT tiles of 32 heads (rows beyond H are zero), and the
// head weights of the accumulator rows this lane holds: w[ht][4j + e] is the
// weight of head ht*32 + 8j + 4g + e (g = lane >> 5).
template <int DT, int D, int HT>
struct QueryFrag {
  uint32_t a[HT][Geo<DT, D>::HW];
  float w[HT][16];
};

// q_t: the query's [H][RB] rows.
template <int DT, int D, int HT>
__device__ __forceinline__ void load_query(QueryFrag<DT, D, HT>& f, const uint8_t* q_t, int H) {
  const int r = threadIdx.x & 31;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int head = ht * 32 + r;
    if (head < H) {
      load_half_row<DT, D>(f.a[ht], q_t + (size_t)head * Geo<DT, D>::RB);
    } else {
#pragma unroll
      for (int i = 0; i < Geo<DT, D>::HW; ++i) f.a[ht][i] = 0;
    }
  }
}

// Head weights of one query into LDS: wq[h] = w[h] * q_scale[h] for h < H, 0 up to
// HT*32.  Called by the wave that uses them (lane-strided).
template <int HT>
__device__ __forceinline__ void load_query_weights(float* wq, const float* w_t, const float* qs_t, int H) {
  const int lane = threadIdx.x & 63;
  for (int h = lane; h < HT * 32; h += 64) wq[h] = (h < H) ? (qs_t ? w_t[h] * qs_t[h] : w_t[h]) : 0.0f;
}

// This lane's head weights from the query's LDS weights (after a barrier).
template <int DT, int D, int HT>
__device__ __forceinline__ void load_query_wregs(QueryFrag<DT, D, HT>& f, const float* wq) {
  const int g = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 w4 = *reinterpret_cast<const float4*>(wq + ht * 32 + 8 * j + 4 * g);
      f.w[ht][4 * j + 0] = w4.x;
      f.w[ht][4 * j + 1] = w4.y;
      f.w[ht][4 * j + 2] = w4.z;
      f.w[ht][4 * j + 3] = w4.w;
    }
  }
}

// ReLU as one integer max on the bit pattern: every negative float (and -0) has
// the sign bit set, so it is below 0 as an int32 and becomes +0; non-negative
// values pass unchanged.  Accumulators are never NaN here.  A float max would
// also quiet signalling NaNs first, which costs a second instruction.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// The contraction of one 32-key tile: acc[ht] = q (head tile ht) . k over d.
template <int DT, int D, int HT>
__device__ __forceinline__ void tile_mfma(const QueryFrag<DT, D, HT>& f, const uint32_t* b, v16f (&acc)[HT]) {
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[ht][v] = 0.0f;
#pragma unroll
    for (int s = 0; s < Geo<DT, D>::KS; ++s)
      mfma_step<DT>(acc[ht], &f.a[ht][s * Geo<DT, D>::KD], &b[s * Geo<DT, D>::KD]);
  }
}

// This lane's half of the score of its column (key): sum over the head rows the lane
// holds (rows 8j + 4g + e of each head tile, in the order ht, j, e) of
// w' * ReLU(q . k).  The other half is in lane l ^ 32.
template <int DT, int D, int HT>
__device__ __forceinline__ float tile_epilogue(const QueryFrag<DT, D, HT>& f, const v16f (&acc)[HT]) {
  float p = 0.0f;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
    for (int v = 0; v < 16; ++v) p = __builtin_fmaf(f.w[ht][v], relu(acc[ht][v]), p);
  }
  return p;
}

template <int DT, int D, int HT>
__device__ __forceinline__ float tile_partial(const QueryFrag<DT, D, HT>& f, const uint32_t* b) {
  v16f acc[HT];
  tile_mfma<DT, D, HT>(f, b, acc);
  return tile_epilogue<DT, D, HT>(f, acc);
}

// Score of this lane's column (key) against the query, before the key scale.
// Lanes l and l+32 return the same value: the lower half's partial plus the upper
// half's, after one cross-half swap.
template <int DT, int D, int HT>
__device__ __forceinline__ float score_tile(const QueryFrag<DT, D, HT>& f, const uint32_t* b) {
  const float p = tile_partial<DT, D, HT>(f, b);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Scores of two tiles of 32 keys at once: lane l < 32 returns the score of column l
// of tile A, lane l >= 32 that of column l - 32 of tile B.  One swap exchanges the
// upper half of A's partials with the lower half of B's, so each lane adds the
// lower-half partial and the upper-half partial of its column: the same two fp32
// values, added once, as score_tile, hence the same bits.
template <int DT, int D, int HT>
__device__ __forceinline__ float pair_epilogue(const QueryFrag<DT, D, HT>& f, const v16f (&accA)[HT],
                                               const v16f (&accB)[HT]) {
  const float pA = tile_epilogue<DT, D, HT>(f, accA);
  const float pB = tile_epilogue<DT, D, HT>(f, accB);
  // after the swap: r[0] = [pA lanes 0..31, pB lanes 0..31], r[1] = [pA lanes 32..63, pB lanes 32..63]
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(pA), __float_as_uint(pB), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DT, int D, int HT>
__device__ __forceinline__ float score_tile_pair(const QueryFrag<DT, D, HT>& f, const uint32_t* bA,
                                                 const uint32_t* bB) {
  v16f accA[HT], accB[HT];
  tile_mfma<DT, D, HT>(f, bA, accA);
  tile_mfma<DT, D, HT>(f, bB, accB);
  return pair_epilogue<DT, D, HT>(f, accA, accB);
}

// Score column blocks blk = first, first + step, ... < nblk of one query with a ring
// of DEPTH row buffers: the rows of block i + (DEPTH-1)*step are in flight while
// block i is contracted.  fetch(blk, buf, scale) issues this lane's loads for a
// block; sink(blk, score) consumes the score of this lane's column.
template <int DT, int D, int HT, int DEPTH, class Fetch, class Sink>
__device__ __forceinline__ void score_blocks(const QueryFrag<DT, D, HT>& f, int first, int step, int nblk, Fetch fetch,
                                             Sink sink) {
  uint32_t buf[DEPTH][Geo<DT, D>::HW];
  float sc[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    const int blk = first + d * step;
    if (blk < nblk) fetch(blk, buf[d], sc[d]);
  }
  for (int base = first; base < nblk; base += DEPTH * step) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int blk = base + d * step;
      if (blk < nblk) {
        const float x = score_tile<DT, D, HT>(f, buf[d]) * sc[d];
        sink(blk, x);
        const int nxt = blk + DEPTH * step;
        if (nxt < nblk) fetch(nxt, buf[d], sc[d]);
      }
    }
  }
}

// score_blocks for gathered rows: index(blk) loads this lane's row index for block
// blk, row(j, buf, scale) issues the loads of row j.  Loads retire in issue order,
// so a row load that needs an index issued just before it would also wait for
// every row load in flight; instead each index is loaded DEPTH blocks before its
// row (a second ring), and the row loads of DEPTH blocks stay in flight.  Every
// load is unconditional (block numbers past the end are clamped to the last
// block) so that the compiler can count the loads in flight exactly; tiles past
// the end are computed and dropped (sink is not called for them).
template <int DT, int D, int HT, int DEPTH, class Index, class Row, class Sink>
__device__ __forceinline__ void score_gather(const QueryFrag<DT, D, HT>& f, int first, int step, int nblk,
                                             Index index, Row row, Sink sink) {
  if (first >= nblk) return;
  const int last = nblk - 1;
  uint32_t buf[DEPTH][Geo<DT, D>::HW];
  float sc[DEPTH];
  int jx[DEPTH];   // row index of the block DEPTH blocks after the one in buf[d]
  int j0[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) j0[d] = index(min(first + d * step, last));
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) jx[d] = index(min(first + (DEPTH + d) * step, last));
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) row(j0[d], buf[d], sc[d]);
  for (int base = first; base < nblk; base += DEPTH * step) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int blk = base + d * step;
      const float x = score_tile<DT, D, HT>(f, buf[d]) * sc[d];
      if (blk < nblk) sink(blk, x);
      const int jn = jx[d];
      jx[d] = index(min(blk + 2 * DEPTH * step, last));
      row(jn, buf[d], sc[d]);
    }
  }
}

// ---------------------------------------------------------------------------
// block-cooperative scoring of a shared run of rows
// ---------------------------------------------------------------------------
//
// When every wave of a block scores the same rows (representatives, or a chunk of
// keys) against its own query, each row is read from memory once per block: a
// stage of SR rows is loaded with row-contiguous 16-byte chunks (a row is one or
// more whole cache lines per group of lanes), written to LDS with an XOR swizzle
// of the chunk index, and every wave reads its MFMA operand layout from there.
// Two LDS buffers alternate; the loads of stage s+1 are in flight while stage s is
// contracted, and one barrier per stage separates reuse of a buffer.

template <int DT, int D>
struct Stage {
  static constexpr int RB = Geo<DT, D>::RB;
  static constexpr int CPR = RB / 16;                          // 16-byte chunks per row
  static constexpr int SR = (16384 / RB) < 32 ? 32 : 16384 / RB;  // rows per stage (16 KB)
  static constexpr int CHUNKS = SR * CPR;                      // chunks per stage
};

// LDS slot of chunk ch of stage row r.  Rows of 128 bytes pair up in a 256-byte
// bank line, so their swizzle key steps every second row; longer rows use the row.
template <int CPR>
__device__ __forceinline__ int stage_slot(int r, int ch) {
  const int key = (CPR == 8) ? (IVFTK_SWZ8(r)) : r;
  return r * CPR + (ch ^ (key & (CPR - 1)));
}

// Buffer resource over `bytes` bytes at `base` (raw, no stride): loads at offsets
// past the end return zeros, which lets the staged loads run without clamping.
// base and bytes must be the same in every lane; they are read from the first
// active lane so that the resource lives in scalar registers.
constexpr int BUF_WORD3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* u = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, __builtin_amdgcn_readfirstlane(bytes), BUF_WORD3);
}

// LDS of one staged scorer: two stage buffers of rows and their scales.  The two
// buffers are separate arrays so that the compiler can tell a load into one from a
// read of the other (and need not wait for the next stage's loads before reading the
// current stage).
template <int DT, int D>
struct StageLds {
  u32x4 rows0[Stage<DT, D>::CHUNKS];
  u32x4 rows1[Stage<DT, D>::CHUNKS];
  float sc0[Stage<DT, D>::SR];
  float sc1[Stage<DT, D>::SR];
};

// Scores rows [0, nrows) of a dense run: row i at base + i * RB (16-byte aligned),
// its scale at scale[i] (scale null: 1).  nrows * RB must fit in 31 bits.  Every
// thread of the block calls, with uniform arguments; NW waves of 64 lanes.
// sink(i, x): score x of row i, called once per row by the lane that holds it (i may
// be >= nrows: rows past the end read as zeros and the callers drop them).  When a
// stage holds an even number of 32-row tiles and a half row fits in 16 registers,
// tiles are scored in pairs and lane l holds row r0 + l of the pair; otherwise lanes
// 0..31 hold the rows of one tile.
// Stages go from memory straight to LDS (buffer loads with an LDS destination): each
// lane loads the chunk whose swizzled LDS slot is its own, 64 consecutive slots per
// wave and load, so no registers hold a stage in flight.  Stage s + 1 loads while
// stage s is scored; even stages use buffer 0, odd stages buffer 1.
template <int DT, int D, int HT, int NW, class Sink>
__device__ __forceinline__ void score_staged(const QueryFrag<DT, D, HT>& f, const uint8_t* base, const float* scale,
                                             int nrows, StageLds<DT, D>& lds, Sink sink) {
  using S = Stage<DT, D>;
  using G = Geo<DT, D>;
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int NT = NW * 64;
  constexpr int CPT = S::CHUNKS / NT;
  constexpr int TPS = S::SR / 32;            // 32-row tiles per stage
  constexpr bool PAIR = TPS % 2 == 0 && G::HW <= 16;
  static_assert(S::CHUNKS % (NT) == 0, "stage chunks must split evenly over the block");
  static_assert(S::SR <= NT && (S::SR % 64 == 0 || S::SR == 32), "stage scales: one per lane of whole waves");
  // The swizzle key of row tt*32 + c equals that of row c (CPR <= 32, and for CPR = 8
  // the key is the row over two), so tile tt's slots are tile 0's plus tt*32*CPR.
  static_assert(S::CPR <= 32 && 32 % S::CPR == 0, "tile offsets independent of the swizzle");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = tid & 31, g = (tid >> 5) & 1;
  // nrows is the same in every lane (often read from LDS, which the compiler cannot
  // tell): the stage loop and the loads' scalar offsets stay in scalar registers
  const int nst = __builtin_amdgcn_readfirstlane((nrows + S::SR - 1) / S::SR);
  if (nst == 0) return;
  const __amdgpu_buffer_rsrc_t rrow = buffer_rsrc(base, nrows * S::RB);
  const __amdgpu_buffer_rsrc_t rscl = buffer_rsrc(scale, scale ? nrows * 4 : 0);
  // load k of this wave fills LDS slots (k * NW + wave) * 64 + lane of a stage buffer;
  // the slot's row r and swizzled chunk give the source chunk (the swizzle is an XOR,
  // its own inverse)
  int voff[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int slot = (k * NW + wave) * 64 + lane;
    const int r = slot / S::CPR;
    const int key = (S::CPR == 8) ? (IVFTK_SWZ8(r)) : r;
    voff[k] = r * S::RB + (((slot % S::CPR) ^ (key & (S::CPR - 1))) * 16);
  }
  // LDS slots of this lane's operand chunks in tile 0
  int rslot[G::HW / 4];
#pragma unroll
  for (int i = 0; i < G::HW / 4; ++i) rslot[i] = stage_slot<S::CPR>(col, g * (S::CPR / 2) + i);
  if (!scale) {
    for (int i = tid; i < S::SR; i += NT) {
      lds.sc0[i] = 1.0f;
      lds.sc1[i] = 1.0f;
    }
  }
  // st is the same in every lane: its offsets are read into scalar registers
  auto dma = [&](int st, u32x4* rows, float* sc) {
    const int soff = __builtin_amdgcn_readfirstlane(st * S::SR * S::RB);
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rrow, (lds_void*)(rows + (k * NW + wave) * 64), 16, voff[k],
                                               soff, 0, 0);
    if (scale && wave * 64 < S::SR)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rscl, (lds_void*)(sc + wave * 64), 4, (wave * 64 + lane) * 4,
                                               __builtin_amdgcn_readfirstlane(st * S::SR * 4), 0, 0);
  };
  auto operand = [&](uint32_t* bf, const u32x4* tb, int tt) {
#pragma unroll
    for (int i = 0; i < G::HW / 4; ++i) {
      const u32x4 v = tb[tt * 32 * S::CPR + rslot[i]];
      bf[4 * i + 0] = v.x;
      bf[4 * i + 1] = v.y;
      bf[4 * i + 2] = v.z;
      bf[4 * i + 3] = v.w;
    }
  };
  // Paired tiles hand their scores to the sink one stage late, right after the next
  // barrier: the sink's stores (or its ballot and branch) then neither split the
  // stage's contraction into separate blocks of code nor hold up the barrier's
  // wait for this wave's memory operations.
  constexpr int NPEND = PAIR ? TPS / 2 : 1;
  float pend[NPEND];
  int pend_st = -1;
  auto flush = [&]() {
    if (pend_st >= 0) {
#pragma unroll
      for (int i = 0; i < NPEND; ++i) sink(pend_st * S::SR + 2 * i * 32 + lane, pend[i]);
    }
  };
  auto compute = [&](int st, const u32x4* tb, const float* sb) {
    if constexpr (PAIR) {
      // rows past nrows are zeros (the loads return zeros past the end) and their sink
      // calls are dropped by the callers, so every pair of the stage is scored
      flush();
      float scl[NPEND];
#pragma unroll
      for (int tt = 0; tt < TPS; tt += 2) scl[tt / 2] = sb[tt * 32 + lane];
#pragma unroll
      for (int tt = 0; tt < TPS; tt += 2) {
        uint32_t bA[G::HW], bB[G::HW];
        operand(bA, tb, tt);
        operand(bB, tb, tt + 1);
        pend[tt / 2] = score_tile_pair<DT, D, HT>(f, bA, bB) * scl[tt / 2];
      }
      pend_st = st;
    } else {
#pragma unroll
      for (int tt = 0; tt < TPS; ++tt) {
        const int r0 = st * S::SR + tt * 32;
        if (r0 < nrows) {
          uint32_t bf[G::HW];
          operand(bf, tb, tt);
          const float x = score_tile<DT, D, HT>(f, bf) * sb[tt * 32 + col];
          if (lane < 32) sink(r0 + col, x);
        }
      }
    }
  };
  // vmcnt(0) before each barrier: this wave's loads into LDS have landed
  dma(0, lds.rows0, lds.sc0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    if (st + 1 < nst) dma(st + 1, lds.rows1, lds.sc1);
    compute(st, lds.rows0, lds.sc0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (st + 1 >= nst) break;
    if (st + 2 < nst) dma(st + 2, lds.rows0, lds.sc0);
    compute(st + 1, lds.rows1, lds.sc1);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  if constexpr (PAIR) flush();
}

}  // namespace ivftk
