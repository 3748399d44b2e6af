// Seal: size-capped k-means of one window of W keys into C = W/cluster_size clusters
// (one block per window, one thread per key; the window's keys staged in LDS).
//
// AttentionIndex, paper-daily.com explainer, "索引怎么边算边建？" item 2: each time
// the open window holds W keys it is clustered and the clusters are appended,
// older clusters untouched (GLM-5.3: W = 1024 into 8 clusters of about 128);
// kurate.org assessment, "Core Contribution" item 1: windows are sealed with
// size-capped k-means.
//
// Arithmetic (fixed so that the result is reproducible bit for bit):
//   D(x, c) = sum over i ascending of (x_i - c_i)^2: t = x_i - c_i rounded to fp32,
//   then acc = fma(t, t, acc), one rounding (the library is built with
//   floating-point contraction off, so no other operation fuses);
//   mean = fp32 running sum over members in ascending position, then one division.
// Initial centroids: keys at offsets floor((2c+1) W / (2C)).  Assignment: nearest
// centroid (ties to the lower cluster) when that respects the cap; otherwise the
// greedy walk over (D, key, cluster) triples in ascending order, which gives a key
// to a cluster while the key is free and the cluster holds fewer than `cap` keys.
// (When nearest assignment respects the cap the walk returns exactly it: every key
// meets its nearest cluster first and that cluster cannot be full yet.)
// The walk's result is computed here by deferred acceptance: each key proposes to its
// clusters in (D, cluster) order; a cluster with more than `cap` proposals keeps the
// `cap` first in (D, key) order and turns the rest away, and those move on to their
// next cluster, until no cluster is over its cap.  The two agree: the preferences of
// both sides come from the one strict order of the triples, and under such
// preferences exactly one assignment is stable (no key and cluster that would both
// rather have each other than what they hold).  The walk ends in a stable assignment
// (a key it passes over meets only clusters already full of earlier triples), and so
// does deferred acceptance; with cap * C >= W both place every key.
// The iterations stop early once an assignment repeats: from there on every iteration
// would reproduce the same members and centroids, so the result equals the one after
// the full iteration count.
#include "dispatch.h"
#include "launch.h"
#include "params.h"

namespace ivftk {

constexpr int SEAL_MAXW = 1024;

// The elements of one 32-bit word of a stored row as fp32 times sk (sk = 1 for the
// unscaled formats).
template <int DT>
__device__ __forceinline__ void word_to_f32(uint32_t w, float (&x)[4 / Elem<DT>::bytes], float sk) {
  if constexpr (DT == DT_F32) {
    x[0] = __uint_as_float(w);
  } else if constexpr (DT == DT_BF16) {
    x[0] = bf16_to_f32(w & 0xFFFFu);
    x[1] = bf16_to_f32(w >> 16);
  } else {
    e4m3x4_to_f32(w, x[0], x[1], x[2], x[3]);
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = x[u] * sk;
  }
}

template <int DT, int D, int CS>
__global__ __launch_bounds__(1024) void k_seal(SealParams p) {
  constexpr int RB = D * Elem<DT>::bytes;
  constexpr int EPC = 16 / Elem<DT>::bytes;   // elements per 16-byte chunk
  constexpr int CPR = RB / 16;                // chunks per row
  constexpr int DPW = 4 / Elem<DT>::bytes;    // elements per 32-bit word
  constexpr int QPR = D / DPW;                // words per row
  // The window's keys are staged in LDS, row after row, when they fit in 128 KB.  (The
  // distance pass reads whole rows, one per thread, and spends hundreds of VALU
  // operations per 16-byte chunk, so its bank conflicts cost little; the means read
  // words of one row across a wave, and address a row with one multiply-add.)
  constexpr bool STAGE = SEAL_MAXW * RB <= 131072;
  __shared__ uint4 kst[STAGE ? SEAL_MAXW * CPR : 1];
  __shared__ float ksc[(STAGE && DT == DT_E4M3) ? SEAL_MAXW : 1];
  __shared__ float cent[CS * D];
  __shared__ int cnt[CS], clo[CS], plo[CS], pfill[CS];
  __shared__ uint32_t amax[CS];
  __shared__ int wcnt[16 * CS];
  __shared__ int2 mem2[SEAL_MAXW];   // member list: key offset and the bits of its scale
  __shared__ __align__(16) uint64_t prop[SEAL_MAXW + 8 * CS];
  __shared__ int s_over;
  __shared__ uint32_t s_dirty;
  const int tid = threadIdx.x, bd = blockDim.x, lane = tid & 63, wv = tid >> 6, nwv = bd >> 6;
  const int W = p.W, cap = p.cap;
  const int w = p.w0 + blockIdx.x;
  const int64_t base = (int64_t)p.S + (int64_t)w * W;
  const uint8_t* const wrows = p.keys + (size_t)base * RB;

  // the window's rows into LDS: chunk c of the window (row c / CPR) by thread c mod bd,
  // all loads issued before the stores
  // (indices clamped into the window, stores masked, so the loads are unconditional)
  if constexpr (STAGE) {
    const int nch = W * CPR;
    for (int c0 = 0; c0 < nch; c0 += 4 * bd) {
      uint4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = reinterpret_cast<const uint4*>(wrows)[min(c0 + k * bd + tid, nch - 1)];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = c0 + k * bd + tid;
        const int m = c / CPR, ch = c % CPR;
        if (c < nch) kst[m * CPR + ch] = v[k];
      }
    }
    if constexpr (DT == DT_E4M3) {
      if (tid < W) ksc[tid] = p.kscale[base + tid];
    }
  }
  // chunk ch, word q, scale of window key m
  auto chunk = [&](int m, int ch) -> uint4 {
    if constexpr (STAGE) {
      return kst[m * CPR + ch];
    } else {
      return reinterpret_cast<const uint4*>(wrows + (size_t)m * RB)[ch];
    }
  };
  auto word = [&](int m, int q) -> uint32_t {
    if constexpr (STAGE) {
      return reinterpret_cast<const uint32_t*>(kst)[m * QPR + q];
    } else {
      return reinterpret_cast<const uint32_t*>(wrows + (size_t)m * RB)[q];
    }
  };
  auto key_scale = [&](int m) -> float {
    if constexpr (DT != DT_E4M3) return 1.0f;
    else if constexpr (STAGE) return ksc[m];
    else return p.kscale[base + m];
  };

  __syncthreads();
  for (int idx = tid; idx < CS * QPR; idx += bd) {
    const int c = idx / QPR, q = idx % QPR;
    const int m = ((2 * c + 1) * W) / (2 * CS);
    float x[DPW];
    word_to_f32<DT>(word(m, q), x, key_scale(m));
#pragma unroll
    for (int e = 0; e < DPW; ++e) cent[c * D + q * DPW + e] = x[e];
  }

  // A cluster whose members did not change keeps the same mean, bit for bit, so its
  // distances from the previous iteration still hold: distances and means are
  // recomputed only for the clusters in s_dirty (all of them at first).
  int prev_a = tid < W ? -2 : -1;   // this key's assignment in the previous iteration
  float acc[CS];                    // this key's distances, kept across iterations
#pragma unroll
  for (int c = 0; c < CS; ++c) acc[c] = 0.0f;
  if (tid == 0) s_dirty = (1u << CS) - 1u;
  __syncthreads();
  for (int it = 0; it < p.iters; ++it) {
    int a = -1;   // this key's cluster in this iteration
    if (p.positional) {
      // ---- position blocks: no distances, the means below are the centroids ----
      if (tid < W) a = tid / (W / CS);
    } else {
      // ---- distances to the changed centroids, nearest ----
      const uint32_t dirty = s_dirty;
      int tgt = 0;
      if (tid < W) {
        const float sk = key_scale(tid);
#pragma unroll
        for (int c = 0; c < CS; ++c)
          if ((dirty >> c) & 1u) acc[c] = 0.0f;
        for (int ch = 0; ch < CPR; ++ch) {
          const uint4 raw = chunk(tid, ch);
          const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
          float xv[EPC];
          chunk_to_f32<DT>(wds, xv, sk);
#pragma unroll
          for (int c = 0; c < CS; ++c) {
            if (!((dirty >> c) & 1u)) continue;
            float s = acc[c];
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
              const float t = xv[e] - cent[c * D + ch * EPC + e];
              s = __builtin_fmaf(t, t, s);
            }
            acc[c] = s;
          }
        }
        float bv = acc[0];
#pragma unroll
        for (int c = 1; c < CS; ++c)
          if (acc[c] < bv) bv = acc[c], tgt = c;
      }
      auto count_targets = [&]() {
        if (tid < CS) cnt[tid] = 0;
        if (tid == 0) s_over = 0;
        __syncthreads();
        if (tid < W) atomicAdd(&cnt[tgt], 1);
        __syncthreads();
        if (tid < CS && cnt[tid] > cap) s_over = 1;
        __syncthreads();
      };
      count_targets();

      // ---- deferred acceptance while a cluster is over its cap.  Every key always
      // targets one cluster; a key's proposal ranks in its cluster by (D, key). ----
      uint32_t refused = 0;   // clusters that turned this key away
      for (int round = 0; round < W * CS && s_over; ++round) {
        // each over-full cluster's proposals in a list of its own, padded to a multiple
        // of 8 with entries that rank behind every proposal
        if (tid == 0) {
          int run = 0;
          for (int c = 0; c < CS; ++c) {
            plo[c] = run;
            pfill[c] = 0;
            if (cnt[c] > cap) run += (cnt[c] + 7) & ~7;
          }
        }
        __syncthreads();
        const bool contested = tid < W && cnt[tgt] > cap;
        float dt = acc[0];
#pragma unroll
        for (int c = 1; c < CS; ++c)
          if (tgt == c) dt = acc[c];
        const uint64_t v = ((uint64_t)__float_as_uint(dt) << 32) | (uint32_t)tid;
        if (contested) prop[plo[tgt] + atomicAdd(&pfill[tgt], 1)] = v;
        if (tid < 8 * CS) {
          const int c = tid >> 3, n = cnt[c];
          if (n > cap && n + (tid & 7) < ((n + 7) & ~7)) prop[plo[c] + n + (tid & 7)] = ~0ull;
        }
        __syncthreads();
        if (contested) {
          // proposals ahead of this one in (D, key) order, 8 per step
          const uint4* L = reinterpret_cast<const uint4*>(prop + plo[tgt]);
          const int n8 = (cnt[tgt] + 7) >> 3;
          int ahead = 0;
          for (int r = 0; r < n8; ++r) {
            uint4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = L[4 * r + u];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              ahead += ((((uint64_t)x[u].y << 32) | x[u].x) < v) ? 1 : 0;
              ahead += ((((uint64_t)x[u].w << 32) | x[u].z) < v) ? 1 : 0;
            }
          }
          if (ahead >= cap) {
            // turned away: the next cluster in this key's (D, cluster) order
            refused |= 1u << tgt;
            int nb = -1;
            float nv = 0.0f;
#pragma unroll
            for (int c = 0; c < CS; ++c)
              if (!((refused >> c) & 1u) && (nb < 0 || acc[c] < nv)) nb = c, nv = acc[c];
            if (nb >= 0) tgt = nb;
          }
        }
        __syncthreads();
        count_targets();
      }
      if (tid < W) a = tgt;
    }

    // ---- stop at a fixed point: an unchanged assignment gives the same members and
    // means as the previous iteration, hence the same centroids and again the same
    // assignment, so the remaining iterations would change nothing ----
    if (tid == 0) s_dirty = 0u;
    if (!__syncthreads_or(a != prev_a)) break;
    // clusters that gained or lost a member get a new mean (and new distances)
    if (a != prev_a) atomicOr(&s_dirty, (a >= 0 ? 1u << a : 0u) | (prev_a >= 0 ? 1u << prev_a : 0u));
    prev_a = a;

    // ---- stable member lists: ascending position within each cluster ----
    int myrank = 0;
#pragma unroll
    for (int cc = 0; cc < CS; ++cc) {
      const uint64_t mask = __ballot(a == cc);
      if (lane == 0) wcnt[wv * CS + cc] = __popcll(mask);
      if (a == cc) myrank = __popcll(mask & ((1ull << lane) - 1ull));
    }
    __syncthreads();
    if (tid < CS) {
      int run = 0;
      for (int q = 0; q < nwv; ++q) {
        const int x = wcnt[q * CS + tid];
        wcnt[q * CS + tid] = run;
        run += x;
      }
      cnt[tid] = run;
    }
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int cc = 0; cc < CS; ++cc) {
        clo[cc] = run;
        run += cnt[cc];
      }
    }
    __syncthreads();
    if (tid < W) {
      const int r = clo[a] + wcnt[wv * CS + a] + myrank;
      mem2[r] = make_int2(tid, __float_as_int(key_scale(tid)));
    }
    __syncthreads();

    // ---- means of the changed clusters (empty clusters keep their centroid): one
    // thread per (cluster, 32-bit word of a row) ----
    const uint32_t dirty = s_dirty;
    for (int idx = tid; idx < CS * QPR; idx += bd) {
      const int c = idx / QPR, q = idx % QPR;
      const int nc = cnt[c];
      if (nc > 0 && ((dirty >> c) & 1u)) {
        const int2* mem = mem2 + clo[c];
        float s[DPW];
#pragma unroll
        for (int e = 0; e < DPW; ++e) s[e] = 0.0f;
        int r = 0;
        for (; r + 8 <= nc; r += 8) {
          uint32_t wd[8];
          float sk[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int2 me = mem[r + u];
            wd[u] = word(me.x, q);
            sk[u] = __int_as_float(me.y);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            float x[DPW];
            word_to_f32<DT>(wd[u], x, sk[u]);
#pragma unroll
            for (int e = 0; e < DPW; ++e) s[e] = s[e] + x[e];
          }
        }
        for (; r < nc; ++r) {
          float x[DPW];
          const int2 me = mem[r];
          word_to_f32<DT>(word(me.x, q), x, __int_as_float(me.y));
#pragma unroll
          for (int e = 0; e < DPW; ++e) s[e] = s[e] + x[e];
        }
#pragma unroll
        for (int e = 0; e < DPW; ++e) cent[c * D + q * DPW + e] = s[e] / (float)nc;
      }
    }
    __syncthreads();
  }

  // ---- publish the window's clusters ----
  const int slot0 = w * CS;
  if (tid < CS) {
    p.size[slot0 + tid] = cnt[tid];
    p.off[slot0 + tid] = w * W + clo[tid];
    amax[tid] = 0u;
    if constexpr (DT != DT_E4M3) p.rsc[slot0 + tid] = 1.0f;
  }
  for (int r = tid; r < W; r += bd) p.members[(size_t)w * W + r] = (int)(base + mem2[r].x);
  __syncthreads();
  for (int idx = tid; idx < CS * D; idx += bd) {
    const float x = cent[idx];
    p.cent[(size_t)slot0 * D + idx] = x;
    p.lrep[(size_t)slot0 * D + idx] = x;
    if constexpr (DT == DT_E4M3) atomicMax(&amax[idx / D], __float_as_uint(__builtin_fabsf(x)));
  }
  __syncthreads();
  for (int idx = tid; idx < CS * D; idx += bd) {
    const float x = cent[idx];
    const size_t o = (size_t)slot0 * D + idx;
    if constexpr (DT == DT_F32) {
      reinterpret_cast<float*>(p.rep)[o] = x;
    } else if constexpr (DT == DT_BF16) {
      reinterpret_cast<uint16_t*>(p.rep)[o] = (uint16_t)f32_to_bf16(x);
    } else {
      const float am = __uint_as_float(amax[idx / D]);
      const float sr = am / 448.0f;
      p.rep[o] = (am == 0.0f) ? (uint8_t)0 : (uint8_t)f32_to_e4m3(x / sr);
      if (idx % D == 0) p.rsc[slot0 + idx / D] = (am == 0.0f) ? 1.0f : sr;
    }
  }
}

template <int DT, int D, int CS>
static hipError_t launch_seal_cs(const SealParams& p, int n_windows, hipStream_t s) {
  const int threads = ((p.W + 63) / 64) * 64;
  hipLaunchKernelGGL((k_seal<DT, D, CS>), dim3(n_windows), dim3(threads), 0, s, p);
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_seal_t(const SealParams& p, int n_windows, hipStream_t s) {
  switch (p.Cs) {
    case 1: return launch_seal_cs<DT, D, 1>(p, n_windows, s);
    case 2: return launch_seal_cs<DT, D, 2>(p, n_windows, s);
    case 4: return launch_seal_cs<DT, D, 4>(p, n_windows, s);
    case 8: return launch_seal_cs<DT, D, 8>(p, n_windows, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_seal(const SealParams& p, int dtype, int dim, int n_windows, hipStream_t s) {
  IVFTK_DISPATCH_D(launch_seal_t, dtype, dim, p, n_windows, s);
}

// ---------------------------------------------------------------------------
// member-ordered key copies of a store
// ---------------------------------------------------------------------------
// ckeys[j] = keys[members[j]] and cscale[j] = kscale[members[j]] for j in [j0, j1):
// a cluster's keys then sit in one contiguous run (with their scales), which the
// rescoring gathers read instead of the position-ordered keys.  One thread per
// 16-byte chunk of a row.
__global__ __launch_bounds__(256) void k_copy_member_rows(const int* members, int64_t j0, int64_t j1,
                                                          const uint8_t* keys, const float* kscale, int64_t n_keys,
                                                          int rb, uint8_t* ckeys, float* cscale) {
  const int cpr = rb / 16;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t j = j0 + idx / cpr;
  if (j >= j1) return;
  const int c = (int)(idx % cpr);
  const int64_t pos = min(max((int64_t)members[j], (int64_t)0), n_keys - 1);
  reinterpret_cast<uint4*>(ckeys + (size_t)j * rb)[c] = reinterpret_cast<const uint4*>(keys + (size_t)pos * rb)[c];
  if (cscale && c == 0) cscale[j] = kscale[pos];
}

hipError_t launch_copy_member_rows(const int* members, int64_t j0, int64_t j1, const uint8_t* keys,
                                   const float* kscale, int64_t n_keys, int rb, uint8_t* ckeys, float* cscale,
                                   hipStream_t s) {
  if (j1 <= j0) return hipSuccess;
  const int64_t threads = (j1 - j0) * (rb / 16);
  hipLaunchKernelGGL(k_copy_member_rows, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, members, j0, j1,
                     keys, kscale, n_keys, rb, ckeys, cscale);
  return hipGetLastError();
}

}  // namespace ivftk
