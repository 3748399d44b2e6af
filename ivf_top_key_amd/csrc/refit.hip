// Refit: one round of assignment + update over the whole sealed prefix, warm-started.
//
// AttentionIndex, paper-daily.com explainer, "索引怎么边算边建？" item 3 and the
// paragraph after it: every R tokens the whole prefix is regrouped, starting from
// the previous centres plus new centres from recent keys; every key keeps an upper
// bound on the distance to its own centre and a lower bound on the distance to the
// others, and only new keys and keys whose bounds no longer certify their cluster
// are compared with every centre; one assignment and one update, no convergence;
// it runs on another stream.  kurate.org assessment, "Core Contribution" item 1:
// warm-started refits with Elkan/Hamerly-style bounds.
//
// Epoch r starts from slots [0, r*Q): epoch r-1's centroids for s < (r-1)*Q and the
// seal centroids of the R/W newest windows (the new centres) above.  The result is
// the exact nearest-centroid assignment (fp32 distances in the fixed order, each term
// t = x_i - c_i then one fused multiply-add, ties to the lower slot) of every key in
// [S, B_r) followed by exact-order means, i.e. the
// bounds only skip work.  Bound arithmetic keeps a relative slack far above the
// fp32 error of a 128-term distance (about 8e-6), so a certified key is never a
// near tie.
//
// Bound state per key (Hamerly): ub >= distance to its own warm centroid, lb <=
// distance to every other live warm centroid.  After the update, drift[s] bounds
// how far centroid s moved.  A single lower bound shrunk by the largest drift
// certifies almost nothing here (a few centroids move far in every update), so the
// next refit lists the most-moved quarter of the old slots together with the new
// ones: a key keeps its slot when its distance (ub widened by its own slot's drift,
// else exact) is below A - E for every listed slot (the matrix-core screen below) and
// below lb shrunk by the largest drift of an unlisted slot.  Every other key, and
// every new key, is screened against all slots.
#include "dispatch.h"
#include "launch.h"
#include "params.h"

namespace ivftk {

constexpr float EPS_B = 1e-5f;   // relative slack on distance bounds
constexpr float EPS_D = 1e-4f;   // relative slack on squared distances in the test
constexpr int REFIT_TILE_SLOTS = 64;

template <int DT, int D>
__device__ __forceinline__ void load_key_f32(float (&x)[D], const RefitParams& p, int64_t pos) {
  const uint8_t* row = p.keys + (size_t)pos * (D * Elem<DT>::bytes);
  load_row_f32<DT, D>(x, row, DT == DT_E4M3 ? p.kscale[pos] : 1.0f);
}

template <int D>
__device__ __forceinline__ float sqdist(const float (&x)[D], const float* c) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const float t = x[i] - c[i];
    acc = __builtin_fmaf(t, t, acc);
  }
  return acc;
}

// Four distances at once (four independent chains, each in the fixed order).
template <int D>
__device__ __forceinline__ void sqdist4(const float (&x)[D], const float* c, float& d0, float& d1, float& d2,
                                        float& d3) {
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const float t0 = x[i] - c[i];
    const float t1 = x[i] - c[D + i];
    const float t2 = x[i] - c[2 * D + i];
    const float t3 = x[i] - c[3 * D + i];
    a0 = __builtin_fmaf(t0, t0, a0);
    a1 = __builtin_fmaf(t1, t1, a1);
    a2 = __builtin_fmaf(t2, t2, a2);
    a3 = __builtin_fmaf(t3, t3, a3);
  }
  d0 = a0;
  d1 = a1;
  d2 = a2;
  d3 = a3;
}

// sqdist of key row `row` (scale sk) to c, streaming the row 16 bytes at a time
// (few registers; the row is in cache): the same values and the same fixed order as
// load_key_f32 followed by sqdist.
template <int DT, int D>
__device__ __forceinline__ float sqdist_row(const uint8_t* row, float sk, const float* c) {
  constexpr int EPC = 16 / Elem<DT>::bytes;   // elements per 16-byte chunk
  float acc = 0.0f;
#pragma unroll 1
  for (int i0 = 0; i0 < D; i0 += EPC) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(row + (size_t)i0 * Elem<DT>::bytes);
    const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
    float cv[EPC];
#pragma unroll
    for (int e = 0; e < EPC; e += 4) {
      const float4 c4 = *reinterpret_cast<const float4*>(c + i0 + e);
      cv[e] = c4.x;
      cv[e + 1] = c4.y;
      cv[e + 2] = c4.z;
      cv[e + 3] = c4.w;
    }
    float xv[EPC];
    chunk_to_f32<DT>(wds, xv, sk);
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const float t = xv[e] - cv[e];
      acc = __builtin_fmaf(t, t, acc);
    }
  }
  return acc;
}

// warm centroid and liveness of slot s
__device__ __forceinline__ const float* warm_cent(const RefitParams& p, int s, int D) {
  return (s < (p.r - 1) * p.Q) ? p.prev.cent + (size_t)s * D : p.seal.cent + (size_t)s * D;
}
__device__ __forceinline__ bool warm_alive(const RefitParams& p, int s) {
  return ((s < (p.r - 1) * p.Q) ? p.prev.size : p.seal.size)[s] > 0;
}

// tile[c * D + i] = row(c)[i] for c < nt (fp32 centroid rows): 16-byte loads, eight
// per thread issued before any store.  Every thread of the block calls.
template <int D, class Row>
__device__ __forceinline__ void load_cent_tile(float* tile, int nt, Row row) {
  constexpr int VPR = D / 4;   // 16-byte vectors per row
  const int nv = nt * VPR;
  for (int v0 = threadIdx.x; v0 < nv; v0 += 8 * blockDim.x) {
    float4 r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int v = min(v0 + u * (int)blockDim.x, nv - 1);
      r[u] = reinterpret_cast<const float4*>(row(v / VPR))[v % VPR];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int v = v0 + u * (int)blockDim.x;
      if (v < nv) reinterpret_cast<float4*>(tile)[v] = r[u];
    }
  }
}

__global__ void k_refit_begin(RefitParams p) {
  if (threadIdx.x == 0) {
    *p.work_count = 0;
    *p.ovf_count = 0;
    *p.drift_max = 0.0f;
  }
  if (threadIdx.x == 0) p.tile_cmax[0] = 0u;
}

// The slots listed for certifying the keys of epoch r-1: the m live old slots that
// moved most in the last update (m = a quarter of the old slots, rounded up to a
// whole tile, at least 32), then the Q new ones.  rest_drift bounds the drift of
// every live old slot left out.
__global__ __launch_bounds__(1024) void k_refit_hsel(RefitParams p) {
  __shared__ Select32Scratch sc;
  __shared__ int s_alive, s_n;
  const int tid = threadIdx.x;
  const int n_old = (p.r - 1) * p.Q;
  if (tid == 0) {
    s_alive = 0;
    s_n = 0;
  }
  __syncthreads();
  int alive = 0;
  for (int s = tid; s < n_old; s += blockDim.x) {
    const bool a = p.prev.size[s] > 0;
    // drifts are >= 0, so their bits order like their values; 0 marks a dead slot
    p.hkey[s] = a ? __float_as_uint(p.prev_drift[s]) + 1u : 0u;
    alive += a ? 1 : 0;
  }
  if (alive) atomicAdd(&s_alive, alive);
  __syncthreads();
  const int m = min(n_old, max(32, (n_old / 4 + 31) / 32 * 32));
  uint32_t T = 0u;   // listed: live slots with key > T
  if (s_alive > m) T = radix_select32_desc(p.hkey, n_old, m + 1, sc);
  __syncthreads();
  // hkey[s] becomes slot s's place in the list (0xFFFFFFFF: not listed), which the
  // certifying screen uses to find the one tile that holds a key's own slot
  for (int s = tid; s < n_old; s += blockDim.x) {
    uint32_t at = 0xFFFFFFFFu;
    if (p.hkey[s] > T) {
      at = (uint32_t)atomicAdd(&s_n, 1);
      p.hlist[at] = s;
    }
    p.hkey[s] = at;
  }
  __syncthreads();
  const int nh = s_n;
  for (int i = tid; i < p.Q; i += blockDim.x) p.hlist[nh + i] = n_old + i;
  if (tid == 0) {
    *p.nlist = nh + p.Q;
    *p.rest_drift = T > 0u ? __uint_as_float(T - 1u) : 0.0f;
  }
}

// new keys [B_prev, B_r) and the work list: nearest of every live warm centroid
template <int DT, int D>
__global__ __launch_bounds__(256) void k_refit_brute(RefitParams p) {
  __shared__ float tile[REFIT_TILE_SLOTS * D];
  __shared__ int alive[REFIT_TILE_SLOTS];
  // keys: new keys then the work list, or (brute_ovf) the screening's overflow list
  const int64_t n_new = p.brute_ovf ? 0 : p.B_r - p.B_prev;
  const int64_t total = p.brute_ovf ? (int64_t)*p.ovf_count : n_new + *p.work_count;
  const int* list = p.brute_ovf ? p.ovf : p.work;
  const int nslots = p.r * p.Q;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x; base < total; base += (int64_t)gridDim.x * blockDim.x) {
    const int64_t item = base + threadIdx.x;
    const bool active = item < total;
    int64_t x = 0;
    float xv[D];
    if (active) {
      x = item < n_new ? p.B_prev + item : (int64_t)list[item - n_new];
      x = min(max(x, (int64_t)p.S), p.B_r - 1);
      load_key_f32<DT, D>(xv, p, x);
    }
    float b1 = __builtin_inff(), b2 = __builtin_inff();
    int best = -1;
    for (int t0 = 0; t0 < nslots; t0 += REFIT_TILE_SLOTS) {
      const int nt = min(REFIT_TILE_SLOTS, nslots - t0);
      __syncthreads();
      load_cent_tile<D>(tile, nt, [&](int c) { return warm_cent(p, t0 + c, D); });
      for (int i = threadIdx.x; i < nt; i += blockDim.x) alive[i] = warm_alive(p, t0 + i);
      __syncthreads();
      if (active) {
        auto take = [&](float dd, int slot) {
          if (dd < b1) {
            b2 = b1;
            b1 = dd;
            best = slot;
          } else if (dd < b2) {
            b2 = dd;
          }
        };
        // ascending slot order keeps ties on the lower slot
        for (int c = 0; c < nt; ++c)
          if (alive[c]) take(sqdist<D>(xv, tile + c * D), t0 + c);
      }
    }
    if (active) {
      p.assign[x] = best;
      p.ub[x] = __builtin_sqrtf(b1) * (1.0f + EPS_B);
      p.lb[x] = (b2 < __builtin_inff()) ? __builtin_sqrtf(b2) * (1.0f - EPS_B) : __builtin_inff();
    }
  }
}

// ---------------------------------------------------------------------------
// screening: the nearest warm centroid of the new keys and the work list
// ---------------------------------------------------------------------------
// The exact answer is the fixed-order fp32 nearest centroid.  Matrix cores give an
// approximate squared distance A(x,c) = |x|^2 + |c|^2 - 2 <x, c>' where <x, c>' is
// accumulated in fp32 from split bf16 values, v = v_hi + v_lo + e with v_hi =
// bf16(v), v_lo = bf16(v - v_hi), |e| <= 2^-16 |v|, as hi.hi + hi.lo + lo.hi (the
// products are exact).  E4M3 codes and bf16 keys are exact in bf16, so for them the
// key is not split (x_lo = 0, and the E4M3 key scale multiplies the accumulated
// dot product inside the final fused multiply-add; the 2^-24 rounding of each
// scaled key value in the norm is far inside the bound below).  |A - D| for the fixed-order distance D is at most
//   E(x) = 2.5e-4 |x| cmax + 6e-5 (|x| + cmax)^2 + 1e-30   (cmax >= every |c|):
// the split drops lo.lo and e terms (< 3.1 * 2^-16 |x||c| per dot product), the
// fp32 sums of 3d products add < 384 * 2^-23 * 1.01 |x||c|, both doubled by the
// factor 2, and the norms, the final operations (one add, then one fused
// multiply-add that applies -2 and the key scale to the dot product) and the
// fixed-order evaluation's own error stay below 4e-5 (|x|+|c|)^2 for d <= 128.  The exact nearest c* has
// A(c*) - E <= D(c*) <= D(c_min) <= Amin + E, so only slots with A <= Amin + 2E can
// be it; those are evaluated in the fixed order, and the result equals the brute
// force.  The cut carries 1% slack on E against fp32 rounding of the comparison.  A
// key whose survivor list overflows goes to the brute-force kernel.

// split bf16 copies (hi rows [0, r*Q), lo rows [r*Q, 2*r*Q)) and squared norm of the
// warm centroids (+inf for empty slots), and the largest squared norm (tile_cmax[0])
template <int DT, int D>
__global__ __launch_bounds__(256) void k_refit_prep(RefitParams p) {
  const int nslots = p.r * p.Q;
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= nslots) return;
  const float* c = warm_cent(p, s, D);
  float nrm = 0.0f;
  for (int i = 0; i < D; ++i) {
    const float v = c[i];
    nrm = nrm + v * v;
    p.cbf[(size_t)s * D + i] = (uint16_t)f32_to_bf16(v);
  }
  for (int i = 0; i < D; ++i) {
    const float v = c[i];
    const float hi = __uint_as_float(f32_to_bf16(v) << 16);
    p.cbf[(size_t)(p.r * p.Q + s) * D + i] = (uint16_t)f32_to_bf16(v - hi);
  }
  const bool alive = warm_alive(p, s);
  p.cnrm[s] = alive ? nrm : __builtin_inff();
  if (alive) atomicMax(&p.tile_cmax[0], __float_as_uint(nrm));
}

constexpr int SCR_LIST = 8;   // candidate entries per lane (each half-wave sees half the slots)

// Per key (one column of a wave's 32), each lane keeps the smallest approximate
// distance Amin of its half of the slots, the slots with A <= Amin + 2E, and the
// smallest A of every slot that falls outside that cut (Aout); at the end the halves
// merge, the survivors are evaluated exactly, and the bounds for the next refit are
// ub = exact best, lb = min(second-best exact survivor, Aout - E) (every other slot
// has D >= A - E >= Aout - E).
template <int DT, int D, bool CERT>
__global__ __launch_bounds__(256) void k_refit_screen(RefitParams p) {
  using GB = Geo<DT_BF16, D>;
  constexpr int CPR = GB::RB / 16;
  constexpr int TCH = 2 * 32 * CPR;   // 16-byte chunks of one tile: hi rows, then lo rows
  constexpr int CPT = TCH / 256;      // chunks per thread
  static_assert(TCH % 256 == 0, "a tile must split evenly over the block");
  // two tile buffers: the loads of tile t+1 are in flight while tile t is contracted
  __shared__ u32x4 ctile[2][TCH];
  __shared__ float cn[2][32];
  __shared__ int csl[2][CERT ? 32 : 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31, g = (lane >> 5) & 1;
  const int64_t n_new = p.B_r - p.B_prev;
  const int64_t total = CERT ? p.B_prev - p.S : n_new + *p.work_count;
  const int nslots = p.r * p.Q;
  const int nL = CERT ? *p.nlist : nslots;   // slots screened: the list, or all
  const int ntl = (nL + 31) / 32;
  auto slot_of = [&](int li) { return CERT ? p.hlist[li] : li; };
  const float cmr = __builtin_sqrtf(__uint_as_float(p.tile_cmax[0])) * (1.0f + 1e-6f);
  auto gload = [&](int tl, u32x4 (&r)[CPT], float& cr, int& ci) {
    const int t0 = tl * 32;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int c = k * 256 + tid;
      const int h = c / (32 * CPR), cc = c % (32 * CPR);
      const int sl = slot_of(min(t0 + cc / CPR, nL - 1)) + h * nslots;
      r[k] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(p.cbf) + (size_t)sl * GB::RB +
                                             (cc % CPR) * 16);
    }
    ci = (tid < 32 && t0 + tid < nL) ? slot_of(t0 + tid) : -1;
    cr = ci >= 0 ? p.cnrm[ci] : __builtin_inff();
  };
  auto lstore = [&](int b, const u32x4 (&r)[CPT], float cr, int ci) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int c = k * 256 + tid;
      const int h = c / (32 * CPR), cc = c % (32 * CPR);
      ctile[b][h * 32 * CPR + stage_slot<CPR>(cc / CPR, cc % CPR)] = r[k];
    }
    if (tid < 32) {
      cn[b][tid] = cr;
      if constexpr (CERT) csl[b][tid] = ci;
    }
  };
  for (int64_t base = (int64_t)blockIdx.x * 128; base < total; base += (int64_t)gridDim.x * 128) {
    const int64_t item = base + wave * 32 + col;
    const bool active = item < total;
    int64_t x = p.S;
    if (CERT) x = p.S + item;
    else if (item < n_new) x = p.B_prev + item;
    else if (item < total) x = (int64_t)p.work[item - n_new];
    x = min(max(x, (int64_t)p.S), (CERT ? p.B_prev : p.B_r) - 1);
    const int own = CERT ? min(max(p.assign[x], 0), (p.r - 1) * p.Q - 1) : -1;
    // the tile of the list that holds the own slot (-1: the own slot is not listed);
    // only tiles that hold some lane's own slot compare slot ids
    const int own_tile = CERT ? (int)p.hkey[own] >> 5 : -1;
    // this lane's half of the key as bf16 (B operand), and the squared norm
    // B operand: this lane's half of the key in bf16.  E4M3 codes and bf16 keys are
    // exact in bf16 (the E4M3 scale multiplies the dot product afterwards), so one
    // copy suffices; fp32 keys are split hi + lo.
    constexpr bool SPLIT_KEY = DT == DT_F32;
    uint32_t bx[GB::HW], bl[SPLIT_KEY ? GB::HW : 1];
    float nh = 0.0f;
    const float ksc = (DT == DT_E4M3) ? p.kscale[x] : 1.0f;
    {
      const uint8_t* row = p.keys + (size_t)x * (D * Elem<DT>::bytes) + (size_t)g * (D / 2) * Elem<DT>::bytes;
      float xc[D / 2];   // the stored values (E4M3: codes, unscaled)
      load_row_f32<DT, D / 2>(xc, row, 1.0f);
#pragma unroll
      for (int i = 0; i < GB::HW; ++i) {
        const float ca = xc[2 * i], cb = xc[2 * i + 1];
        const uint32_t ah = f32_to_bf16(ca), bh = f32_to_bf16(cb);
        bx[i] = ah | (bh << 16);
        if constexpr (SPLIT_KEY)
          bl[i] = f32_to_bf16(ca - __uint_as_float(ah << 16)) | (f32_to_bf16(cb - __uint_as_float(bh << 16)) << 16);
        const float a = DT == DT_E4M3 ? ca * ksc : ca, b = DT == DT_E4M3 ? cb * ksc : cb;
        nh = nh + a * a;
        nh = nh + b * b;
      }
    }
    const float nx = nh + __shfl_xor(nh, 32);
    const float nxr = __builtin_sqrtf(nx) * (1.0f + 1e-6f);
    const float sum = nxr + cmr;
    const float E = (2.5e-4f * nxr * cmr + 6e-5f * sum * sum + 1e-30f) * (1.0f + 1e-5f);
    const float E2 = 2.02f * E;   // the cut Amin + 2E with 1% slack
    const float m2k = -2.0f * ksc;  // A = fma(-2 sk, <x, c>', |x|^2 + |c|^2): one rounding for the product term
    float amin = __builtin_inff();
    float aout = __builtin_inff();   // smallest A among slots that cannot survive the cut
    int ls[SCR_LIST];
    float la[SCR_LIST];
#pragma unroll
    for (int q = 0; q < SCR_LIST; ++q) {
      ls[q] = -1;
      la[q] = 0.0f;
    }
    bool ovf = false;
    u32x4 reg[CPT];
    float creg;
    int ireg;
    gload(0, reg, creg, ireg);
    lstore(0, reg, creg, ireg);
    __syncthreads();
    for (int tl = 0; tl < ntl; ++tl) {
      const int t0 = tl * 32, b = tl & 1;
      const bool more = tl + 1 < ntl;
      if (more) gload(tl + 1, reg, creg, ireg);
      v16f acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
      for (int i = 0; i < GB::HW / 4; ++i) {
        const u32x4 a4 = ctile[b][stage_slot<CPR>(col, g * (CPR / 2) + i)];
        const u32x4 l4 = ctile[b][32 * CPR + stage_slot<CPR>(col, g * (CPR / 2) + i)];
        const uint32_t a[4] = {a4.x, a4.y, a4.z, a4.w};
        const uint32_t al[4] = {l4.x, l4.y, l4.z, l4.w};
        mfma_step<DT_BF16>(acc, a, &bx[4 * i]);
        if constexpr (SPLIT_KEY) mfma_step<DT_BF16>(acc, a, &bl[4 * i]);
        mfma_step<DT_BF16>(acc, al, &bx[4 * i]);
      }
      float A[16];
      float tmin = __builtin_inff();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 c4 = *reinterpret_cast<const float4*>(&cn[b][8 * j + 4 * g]);
        const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) A[4 * j + e] = __builtin_fmaf(m2k, acc[4 * j + e], nx + cv[e]);
      }
      if (CERT && __ballot(own_tile == tl) != 0ull) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (csl[b][8 * (v >> 2) + 4 * g + (v & 3)] != own) tmin = __builtin_fminf(tmin, A[v]);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) tmin = __builtin_fminf(tmin, A[v]);
      }
      if constexpr (CERT) {
        amin = __builtin_fminf(amin, tmin);   // smallest A over the listed slots but the own one
      } else if (tmin <= amin + E2) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          if (A[v] <= amin + E2) {
            amin = __builtin_fminf(amin, A[v]);
            const float cut = amin + E2;
            bool placed = false;
#pragma unroll
            for (int q = 0; q < SCR_LIST; ++q) {
              if (ls[q] >= 0 && la[q] > cut) {
                aout = __builtin_fminf(aout, la[q]);
                ls[q] = -1;
              }
              if (!placed && ls[q] < 0) {
                ls[q] = t0 + 8 * (v >> 2) + 4 * g + (v & 3);
                la[q] = A[v];
                placed = true;
              }
            }
            ovf = ovf || !placed;
          } else {
            aout = __builtin_fminf(aout, A[v]);   // the cut only moves down
          }
        }
      } else {
        aout = __builtin_fminf(aout, tmin);
      }
      if (more) lstore(b ^ 1, reg, creg, ireg);
      __syncthreads();
    }
    if constexpr (CERT) {
      // the key keeps its slot if the slot is certainly nearest: its distance (upper
      // bound widened by the slot's drift, else the exact distance) is below the lower
      // bound of every listed slot (A - E) and of every unlisted one (the previous lower
      // bound shrunk by the largest drift among them)
      amin = __builtin_fminf(amin, __shfl_xor(amin, 32));
      const float m2 = amin - 1.01f * E;
      if (active && g == 0) {
        float u1 = (p.ub[x] + p.prev_drift[own]) * (1.0f + EPS_B);
        const float l1 = __builtin_fmaxf(p.lb[x] - *p.rest_drift, 0.0f) * (1.0f - EPS_B);
        const float ub2 = u1 * u1 * (1.0f + EPS_D);
        const float lb2 = l1 * l1 * (1.0f - EPS_D);
        bool keep = ub2 < lb2 && ub2 < m2;
        if (!keep) {
          const float da = sqdist_row<DT, D>(p.keys + (size_t)x * (D * Elem<DT>::bytes), ksc,
                                             p.prev.cent + (size_t)own * D);
          keep = da < lb2 && da < m2;
          if (keep) u1 = __builtin_sqrtf(da) * (1.0f + EPS_B);
        }
        if (keep) {
          p.ub[x] = u1;
          p.lb[x] = __builtin_fminf(l1, __builtin_sqrtf(__builtin_fmaxf(m2, 0.0f)) * (1.0f - EPS_B));
        } else {
          p.work[atomicAdd(p.work_count, 1)] = (int)x;
        }
      }
      continue;
    }
    // both halves of the wave hold the same key: final cut, then exact distances of
    // this lane's survivors
    amin = __builtin_fminf(amin, __shfl_xor(amin, 32));
    ovf = ovf || __shfl_xor((int)ovf, 32);
    const float cut = amin + E2;
#pragma unroll
    for (int q = 0; q < SCR_LIST; ++q)
      if (ls[q] >= 0 && la[q] > cut) aout = __builtin_fminf(aout, la[q]);
    aout = __builtin_fminf(aout, __shfl_xor(aout, 32));
    float e1 = __builtin_inff(), e2 = __builtin_inff();
    int s1 = 0x7fffffff;
    const uint8_t* krow = p.keys + (size_t)x * (D * Elem<DT>::bytes);
#pragma unroll
    for (int q = 0; q < SCR_LIST; ++q) {
      if (ls[q] < 0 || la[q] > cut) continue;
      const float de = sqdist_row<DT, D>(krow, ksc, warm_cent(p, ls[q], D));
      if (de < e1 || (de == e1 && ls[q] < s1)) {
        e2 = e1;
        e1 = de;
        s1 = ls[q];
      } else {
        e2 = __builtin_fminf(e2, de);
      }
    }
    const float pe1 = __shfl_xor(e1, 32), pe2 = __shfl_xor(e2, 32);
    const int ps1 = __shfl_xor(s1, 32);
    float b1, b2;
    int best;
    if (e1 < pe1 || (e1 == pe1 && s1 < ps1)) {
      b1 = e1;
      best = s1;
      b2 = __builtin_fminf(__builtin_fminf(e2, pe2), pe1);
    } else {
      b1 = pe1;
      best = ps1;
      b2 = __builtin_fminf(__builtin_fminf(e2, pe2), e1);
    }
    b2 = __builtin_fminf(b2, aout - 1.01f * E);   // every non-survivor has D >= A - E >= aout - E
    if (active && g == 0) {
      if (ovf || best == 0x7fffffff) {
        p.ovf[atomicAdd(p.ovf_count, 1)] = (int)x;
      } else {
        p.assign[x] = best;
        p.ub[x] = __builtin_sqrtf(b1) * (1.0f + EPS_B);
        p.lb[x] = (b2 < __builtin_inff()) ? __builtin_sqrtf(__builtin_fmaxf(b2, 0.0f)) * (1.0f - EPS_B)
                                          : __builtin_inff();
      }
    }
  }
}

// per tile of keys: count of keys per slot
__global__ __launch_bounds__(1024) void k_tile_hist(RefitParams p) {
  extern __shared__ int hist[];
  const int nslots = p.r * p.Q;
  for (int i = threadIdx.x; i < nslots; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const int64_t x0 = p.S + (int64_t)blockIdx.x * p.tile;
  for (int i = threadIdx.x; i < p.tile; i += blockDim.x) {
    const int64_t x = x0 + i;
    if (x < p.B_r) atomicAdd(&hist[min(max(p.assign[x], 0), nslots - 1)], 1);
  }
  __syncthreads();
  int* out = p.tile_cnt + (size_t)blockIdx.x * nslots;
  for (int i = threadIdx.x; i < nslots; i += blockDim.x) out[i] = hist[i];
}

// per slot: exclusive prefix over tiles, and the slot size (16 tiles' counts loaded
// together, then scanned: one memory round trip per 16 tiles)
__global__ void k_tile_colscan(RefitParams p) {
  const int nslots = p.r * p.Q;
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= nslots) return;
  int* col = p.tile_cnt + s;
  const int nt = p.n_tiles;
  int run = 0;
  for (int t0 = 0; t0 < nt; t0 += 16) {
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = col[(size_t)min(t0 + u, nt - 1) * nslots];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (t0 + u < nt) {
        col[(size_t)(t0 + u) * nslots] = run;
        run += v[u];
      }
    }
  }
  p.size[s] = run;
}

// exclusive scan of slot sizes -> offsets (one block)
__global__ __launch_bounds__(1024) void k_slot_scan(RefitParams p) {
  __shared__ int wtmp[16];
  const int nslots = p.r * p.Q;
  const int per = (nslots + blockDim.x - 1) / blockDim.x;
  const int lo = threadIdx.x * per;
  int s = 0;
  for (int i = lo; i < lo + per && i < nslots; ++i) s += p.size[i];
  int tot;
  int run = block_exclusive_scan(s, wtmp, &tot);
  for (int i = lo; i < lo + per && i < nslots; ++i) {
    p.off[i] = run;
    run += p.size[i];
  }
}

// per tile: stable placement of its keys (positions ascending within a slot)
__global__ __launch_bounds__(1024) void k_tile_scatter(RefitParams p) {
  __shared__ uint64_t kv[1024];
  const int nslots = p.r * p.Q;
  const int64_t x0 = p.S + (int64_t)blockIdx.x * p.tile;
  const int i = threadIdx.x;
  const int64_t x = x0 + i;
  kv[i] = (i < p.tile && x < p.B_r)
              ? (((uint64_t)(uint32_t)min(max(p.assign[x], 0), nslots - 1) << 32) | (uint32_t)x)
              : ~0ull;
  __syncthreads();
  bitonic_sort_asc(kv, 1024);
  const uint64_t v = kv[i];
  if (v != ~0ull) {
    const uint32_t s = (uint32_t)(v >> 32);
    int lo = 0, hi = i;   // first index with the same slot
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((uint32_t)(kv[mid] >> 32) < s) lo = mid + 1; else hi = mid;
    }
    const int dest = p.off[s] + p.tile_cnt[(size_t)blockIdx.x * nslots + s] + (i - lo);
    if (dest >= 0 && dest < p.B_r - p.S) p.members[dest] = (int)(uint32_t)v;
  }
}

// per (slot, dim): exact-order mean of the members (empty slots keep the warm centroid)
template <int DT, int D>
__global__ __launch_bounds__(256) void k_refit_mean(RefitParams p) {
  const int nslots = p.r * p.Q;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)nslots * D) return;
  const int s = (int)(gid / D), i = (int)(gid % D);
  const int nc = p.size[s];
  float out;
  if (nc > 0) {
    const int* mem = p.members + p.off[s];
    float acc = 0.0f;
    int r = 0;
    for (; r + 8 <= nc; r += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t pos = min(max((int64_t)mem[r + u], (int64_t)0), p.n_keys - 1);
        float e = load_elem<DT>(p.keys + (size_t)pos * (D * Elem<DT>::bytes), i);
        if constexpr (DT == DT_E4M3) e = e * p.kscale[pos];
        v[u] = e;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = acc + v[u];
    }
    for (; r < nc; ++r) {
      const int64_t pos = min(max((int64_t)mem[r], (int64_t)0), p.n_keys - 1);
      float e = load_elem<DT>(p.keys + (size_t)pos * (D * Elem<DT>::bytes), i);
      if constexpr (DT == DT_E4M3) e = e * p.kscale[pos];
      acc = acc + e;
    }
    out = acc / (float)nc;
  } else {
    out = warm_cent(p, s, D)[i];
  }
  p.cent[(size_t)s * D + i] = out;
  p.lrep[(size_t)s * D + i] = out;
}

// per slot: representative, drift of the centroid, largest drift
template <int DT, int D>
__global__ __launch_bounds__(128) void k_refit_finish(RefitParams p) {
  __shared__ uint32_t amax;
  const int s = blockIdx.x;
  const float* c = p.cent + (size_t)s * D;
  if (threadIdx.x == 0) amax = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < D; i += blockDim.x) {
    const float x = c[i];
    if constexpr (DT == DT_F32) {
      reinterpret_cast<float*>(p.rep)[(size_t)s * D + i] = x;
    } else if constexpr (DT == DT_BF16) {
      reinterpret_cast<uint16_t*>(p.rep)[(size_t)s * D + i] = (uint16_t)f32_to_bf16(x);
    } else {
      atomicMax(&amax, __float_as_uint(__builtin_fabsf(x)));
    }
  }
  __syncthreads();
  if constexpr (DT == DT_E4M3) {
    const float am = __uint_as_float(amax);
    const float sr = am / 448.0f;
    for (int i = threadIdx.x; i < D; i += blockDim.x)
      p.rep[(size_t)s * D + i] = (am == 0.0f) ? (uint8_t)0 : (uint8_t)f32_to_e4m3(c[i] / sr);
    if (threadIdx.x == 0) p.rsc[s] = (am == 0.0f) ? 1.0f : sr;
  } else {
    if (threadIdx.x == 0) p.rsc[s] = 1.0f;
  }
  if (threadIdx.x == 0) {
    float dr = 0.0f;
    if (p.size[s] > 0) {
      const float* wc = warm_cent(p, s, D);
      float acc = 0.0f;
      for (int i = 0; i < D; ++i) {
        const float t = c[i] - wc[i];
        acc = acc + t * t;
      }
      dr = __builtin_sqrtf(acc) * (1.0f + EPS_B);
      atomicMax(reinterpret_cast<unsigned int*>(p.drift_max), __float_as_uint(dr));
    }
    p.drift[s] = dr;
  }
}

template <int DT, int D>
static hipError_t launch_refit_t(const RefitParams& p, hipStream_t s) {
  const int nslots = p.r * p.Q;
  hipLaunchKernelGGL(k_refit_begin, dim3(1), dim3(64), 0, s, p);
  hipLaunchKernelGGL((k_refit_prep<DT, D>), dim3((nslots + 255) / 256), dim3(256), 0, s, p);
  const int64_t n_old = p.B_prev - p.S;
  if (n_old > 0) {
    hipLaunchKernelGGL(k_refit_hsel, dim3(1), dim3(1024), 0, s, p);
    hipLaunchKernelGGL((k_refit_screen<DT, D, true>), dim3(2048), dim3(256), 0, s, p);
  }
  hipLaunchKernelGGL((k_refit_screen<DT, D, false>), dim3(2048), dim3(256), 0, s, p);
  RefitParams po = p;
  po.brute_ovf = 1;
  hipLaunchKernelGGL((k_refit_brute<DT, D>), dim3(256), dim3(256), 0, s, po);
  const size_t hist_lds = (size_t)nslots * sizeof(int);
  hipError_t e = hipFuncSetAttribute((const void*)k_tile_hist, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)hist_lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_tile_hist, dim3(p.n_tiles), dim3(1024), hist_lds, s, p);
  hipLaunchKernelGGL(k_tile_colscan, dim3((nslots + 255) / 256), dim3(256), 0, s, p);
  hipLaunchKernelGGL(k_slot_scan, dim3(1), dim3(1024), 0, s, p);
  hipLaunchKernelGGL(k_tile_scatter, dim3(p.n_tiles), dim3(1024), 0, s, p);
  const int64_t nm = (int64_t)nslots * D;
  hipLaunchKernelGGL((k_refit_mean<DT, D>), dim3((unsigned)((nm + 255) / 256)), dim3(256), 0, s, p);
  hipLaunchKernelGGL((k_refit_finish<DT, D>), dim3(nslots), dim3(128), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_refit(const RefitParams& p, int dtype, int dim, hipStream_t s) {
  IVFTK_DISPATCH_D(launch_refit_t, dtype, dim, p, s);
}

}  // namespace ivftk
