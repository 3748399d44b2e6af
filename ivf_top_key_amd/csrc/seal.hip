// Seal: size-capped k-means of one window of W keys into C = W/cluster_size clusters
// (one block per window, one thread per key).
//
// AttentionIndex, paper-daily.com explainer, "索引怎么边算边建？" item 2: each time
// the open window holds W keys it is clustered and the clusters are appended,
// older clusters untouched (GLM-5.3: W = 1024 into 8 clusters of about 128);
// kurate.org assessment, "Core Contribution" item 1: windows are sealed with
// size-capped k-means.
//
// Arithmetic (fixed so that the result is reproducible bit for bit):
//   D(x, c) = sum over i ascending of (x_i - c_i)^2, each operation rounded to fp32
//   (the library is built with floating-point contraction off);
//   mean = fp32 running sum over members in ascending position, then one division.
// Initial centroids: keys at offsets floor((2c+1) W / (2C)).  Assignment: nearest
// centroid (ties to the lower cluster) when that respects the cap; otherwise the
// greedy walk over (D, key, cluster) triples in ascending order, which gives a key
// to a cluster while the key is free and the cluster holds fewer than `cap` keys.
// (When nearest assignment respects the cap the walk returns exactly it: every key
// meets its nearest cluster first and that cluster cannot be full yet.)  The
// iterations stop early once an assignment repeats: from there on every iteration
// would reproduce the same members and centroids, so the result equals the one
// after the full iteration count.
#include "dispatch.h"
#include "launch.h"
#include "params.h"

namespace ivftk {

constexpr int SEAL_MAXW = 1024;
constexpr int SEAL_SORT = 8192;

template <int DT, int D>
__device__ __forceinline__ float key_value(const SealParams& p, int64_t pos, int i) {
  const uint8_t* row = p.keys + (size_t)pos * (D * Elem<DT>::bytes);
  float v = load_elem<DT>(row, i);
  if constexpr (DT == DT_E4M3) v = v * p.kscale[pos];
  return v;
}

template <int DT, int D, int CS>
__global__ __launch_bounds__(1024) void k_seal(SealParams p) {
  constexpr int RB = D * Elem<DT>::bytes;
  constexpr int EPC = 16 / Elem<DT>::bytes;   // elements per 16-byte load
  __shared__ float cent[CS * D];
  __shared__ int cnt[CS], clo[CS];
  __shared__ uint32_t amax[CS];
  __shared__ int wcnt[16 * CS];
  __shared__ int member[SEAL_MAXW];
  __shared__ int asg[SEAL_MAXW];
  __shared__ int first_lane[SEAL_MAXW];
  __shared__ uint64_t sortbuf[SEAL_SORT];
  __shared__ int s_over;
  const int tid = threadIdx.x, bd = blockDim.x, lane = tid & 63, wv = tid >> 6, nwv = bd >> 6;
  const int W = p.W, cap = p.cap;
  const int w = p.w0 + blockIdx.x;
  const int64_t base = (int64_t)p.S + (int64_t)w * W;

  for (int idx = tid; idx < CS * D; idx += bd) {
    const int c = idx / D, i = idx % D;
    cent[idx] = key_value<DT, D>(p, base + ((2 * c + 1) * W) / (2 * CS), i);
  }
  __syncthreads();

  int prev_a = tid < W ? -2 : -1;   // this key's assignment in the previous iteration
  for (int it = 0; it < p.iters; ++it) {
    if (p.positional) {
      // ---- position blocks: no distances, the means below are the centroids ----
      if (tid < W) asg[tid] = tid / (W / CS);
      __syncthreads();
    } else {
      // ---- distances to every centroid, nearest ----
      float acc[CS];
#pragma unroll
      for (int c = 0; c < CS; ++c) acc[c] = 0.0f;
      int best = 0;
      if (tid < W) {
        const uint8_t* row = p.keys + (size_t)(base + tid) * RB;
        float sk = 1.0f;
        if constexpr (DT == DT_E4M3) sk = p.kscale[base + tid];
        for (int i0 = 0; i0 < D; i0 += EPC) {
          const uint4 raw = *reinterpret_cast<const uint4*>(row + i0 * Elem<DT>::bytes);
          const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            float xi;
            if constexpr (DT == DT_F32) {
              xi = __uint_as_float(wds[e]);
            } else if constexpr (DT == DT_BF16) {
              xi = bf16_to_f32((wds[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
            } else {
              xi = e4m3_to_f32((wds[e >> 2] >> (8 * (e & 3))) & 0xFFu) * sk;
            }
#pragma unroll
            for (int c = 0; c < CS; ++c) {
              const float t = xi - cent[c * D + i0 + e];
              acc[c] = acc[c] + t * t;
            }
          }
        }
#pragma unroll
        for (int c = 1; c < CS; ++c)
          if (acc[c] < acc[best]) best = c;
      }
      if (tid < CS) cnt[tid] = 0;
      if (tid == 0) s_over = 0;
      __syncthreads();
      if (tid < W) atomicAdd(&cnt[best], 1);
      __syncthreads();
      if (tid < CS && cnt[tid] > cap) s_over = 1;
      __syncthreads();

      if (!s_over) {
        if (tid < W) asg[tid] = best;
      } else {
        // ---- greedy walk over all (D, key, cluster) triples ----
        const int ntr = W * CS;
        const int P2 = next_pow2(ntr);
        if (tid < W) {
#pragma unroll
          for (int c = 0; c < CS; ++c)
            sortbuf[tid * CS + c] = ((uint64_t)__float_as_uint(acc[c]) << 32) | (uint32_t)(tid * CS + c);
        }
        for (int i = ntr + tid; i < P2; i += bd) sortbuf[i] = ~0ull;
        for (int j = tid; j < W; j += bd) {
          asg[j] = -1;
          first_lane[j] = 64;
        }
        if (tid < CS) cnt[tid] = 0;
        __syncthreads();
        bitonic_sort_asc(sortbuf, P2);
        if (tid < 64) {
          int placed = 0;
          for (int st = 0; st < ntr && placed < W; st += 64) {
            const int ti = st + lane;
            const bool valid = ti < ntr;
            const uint32_t id = valid ? (uint32_t)sortbuf[ti] : 0u;
            const int j = (int)(id / CS), c = (int)(id % CS);
            const bool elig = valid && asg[j] < 0 && cnt[c] < cap;
            bool conflict = false;
#pragma unroll
            for (int cc = 0; cc < CS; ++cc) {
              const int pend = __popcll(__ballot(elig && c == cc));
              const int have = cnt[cc];
              if (have < cap && have + pend > cap) conflict = true;
            }
            if (!conflict) {
              if (elig) atomicMin(&first_lane[j], lane);
              __builtin_amdgcn_wave_barrier();
              const bool win = elig && first_lane[j] == lane;
              __builtin_amdgcn_wave_barrier();
              if (elig) first_lane[j] = 64;
              if (win) asg[j] = c;
#pragma unroll
              for (int cc = 0; cc < CS; ++cc) {
                const int add = __popcll(__ballot(win && c == cc));
                if (lane == 0) cnt[cc] += add;
              }
              placed += __popcll(__ballot(win));
              __builtin_amdgcn_wave_barrier();
            } else {
              // a cluster fills inside this group: decide the 64 triples one by one in
              // order, with the state in registers (lane cc holds cluster cc's count)
              const bool free0 = valid && asg[j] < 0;
              int hv = lane < CS ? cnt[lane] : 0;
              bool taken = false, win = false;
              for (int q = 0; q < 64; ++q) {
                const int jq = __shfl(j, q), cq = __shfl(c, q);
                const bool fq = __shfl((int)(free0 && !taken), q) != 0;
                const bool ok = fq && __shfl(hv, cq) < cap;   // uniform across the wave
                if (ok) {
                  if (lane == q) win = true;
                  if (j == jq) taken = true;
                  if (lane == cq) hv += 1;
                }
              }
              if (win) asg[j] = c;
              if (lane < CS) cnt[lane] = hv;
              placed += __popcll(__ballot(win));
              __builtin_amdgcn_wave_barrier();
            }
          }
        }
        __syncthreads();
      }
    }

    // ---- stop at a fixed point: an unchanged assignment gives the same members and
    // means as the previous iteration, hence the same centroids and again the same
    // assignment, so the remaining iterations would change nothing ----
    const int a = tid < W ? asg[tid] : -1;
    if (!__syncthreads_or(a != prev_a)) break;
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
    if (tid < W) member[clo[a] + wcnt[wv * CS + a] + myrank] = tid;
    __syncthreads();

    // ---- means (empty clusters keep their centroid) ----
    for (int idx = tid; idx < CS * D; idx += bd) {
      const int c = idx / D, i = idx % D;
      const int nc = cnt[c];
      if (nc > 0) {
        const int* mem = member + clo[c];
        float s = 0.0f;
        int r = 0;
        for (; r + 8 <= nc; r += 8) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = key_value<DT, D>(p, base + mem[r + u], i);
#pragma unroll
          for (int u = 0; u < 8; ++u) s = s + v[u];
        }
        for (; r < nc; ++r) s = s + key_value<DT, D>(p, base + mem[r], i);
        cent[idx] = s / (float)nc;
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
  for (int r = tid; r < W; r += bd) p.members[(size_t)w * W + r] = (int)(base + member[r]);
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
