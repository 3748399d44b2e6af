// Indexer scoring kernels: exhaustive scores (streamed, and in rows for the
// fallback), representative scores, candidate rescoring with the top-k selection,
// and the top-k of exhaustive score rows.
//
// Score (AttentionIndex, paper-daily.com explainer, "它到底在解决什么问题？"):
//   s(t, j) = sum_h w[t,h] * ReLU(q[t,h] . k[j]); with E4M3, the per-(t,h) query
//   scale folds into the head weight and the per-key scale multiplies the sum.
// Every path evaluates s through score_tile (dev.h), so one (query, key) pair gets
// the same fp32 bits on the exhaustive and the routed path.
#include "dispatch.h"
#include "launch.h"
#include "params.h"
#include "routing.h"

namespace ivftk {

// ---------------------------------------------------------------------------
// exhaustive scores: block = 4 waves = 4 query rows, one chunk of keys
// ---------------------------------------------------------------------------
// Three waves per SIMD where a half row fits in 16 registers (E4M3 and bf16 at d = 64,
// fp32 at d = 32) and there are at most 64 heads; otherwise the compiler's choice.
template <int DT, int D, int HT>
constexpr int score_waves() { return (Geo<DT, D>::HW <= 16 && HT <= 2) ? 3 : 1; }

// Query of row r of a pass.
__device__ __forceinline__ int exh_query(const ExhParams& p, int r) { return p.t0 + (p.tlist ? p.tlist[r] : r); }

// Keys of the scored run that query t sees: its prefix, or (EXH_SAMPLE) the sample
// keys inside its prefix.
template <int MODE>
__device__ __forceinline__ int64_t exh_run_len(const ExhParams& p, int t) {
  const int64_t n = p.q_pos0 + t + 1;
  if constexpr (MODE == EXH_SAMPLE) return n > p.soff ? (n - p.soff + p.stride - 1) / p.stride : 0;
  else return n;
}

// EXH_ROWS: score rows into p.ws; EXH_SAMPLE: the sample's scores into p.srow;
// EXH_STREAM: no rows, only the scores at or above the row's threshold p.tau[tl]
// (with their positions) into p.surv, counted in p.cnt.
template <int DT, int D, int HT, int MODE>
__global__ __launch_bounds__(256, (score_waves<DT, D, HT>())) void k_exh_score(ExhParams p) {
  using G = Geo<DT, D>;
  __shared__ float wq_s[4][HT * 32];
  __shared__ StageLds<DT, D> stage;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tl = blockIdx.x * 4 + wave;
  const bool active = tl < p.Tb;
  const int tr = active ? tl : p.Tb - 1;   // idle waves still stage rows
  const int tc = exh_query(p, tr);
  load_query_weights<HT>(wq_s[wave], p.w + (size_t)tc * p.H, p.qscale ? p.qscale + (size_t)tc * p.H : nullptr, p.H);
  // the block's rows: keys [j0, j1) with j1 bounded by its longest prefix
  int64_t n_max = 0;
  for (int u = 0; u < 4; ++u) {
    const int64_t n = exh_run_len<MODE>(p, exh_query(p, min((int)blockIdx.x * 4 + u, p.Tb - 1)));
    n_max = n > n_max ? n : n_max;
  }
  const int64_t j0 = (int64_t)blockIdx.y * p.kchunk;
  const int64_t j1 = (j0 + p.kchunk < n_max) ? j0 + p.kchunk : n_max;
  __syncthreads();
  if (j0 >= j1) return;
  const int64_t n_own = exh_run_len<MODE>(p, tc);
  const int64_t j_end = active ? (j1 < n_own ? j1 : n_own) : j0;
  QueryFrag<DT, D, HT> f;
  load_query<DT, D, HT>(f, p.q + (size_t)tc * p.H * G::RB, p.H);
  load_query_wregs<DT, D, HT>(f, wq_s[wave]);
  const uint8_t* run = MODE == EXH_SAMPLE ? p.skeys : p.keys;
  const float* rsc = MODE == EXH_SAMPLE ? p.sscale : p.kscale;
  const uint8_t* base = run + (size_t)j0 * G::RB;
  const float* scl = DT == DT_E4M3 ? rsc + j0 : nullptr;
  if constexpr (MODE == EXH_STREAM) {
    const uint32_t tau = p.tau[tr];
    int* const cnt = p.cnt + tr;
    uint64_t* const sv = p.surv + (size_t)tr * p.caps;
    const int caps = p.caps;
    score_staged<DT, D, HT, 4>(f, base, scl, (int)(j1 - j0), stage, [&](int i, float x) {
      const int64_t j = j0 + i;
      const bool take = j < j_end && order_bits(x) >= tau;
      const uint64_t m = __ballot(take);
      if (m != 0ull) {   // rare: one atomic per wave for all of its lanes' survivors
        const int leader = __builtin_ctzll(m);
        int b = 0;
        if (lane == leader) b = atomicAdd(cnt, __popcll(m));
        b = __shfl(b, leader);
        const int at = b + __popcll(m & ((1ull << lane) - 1ull));
        if (take && at < caps) sv[at] = make_comp(x, (uint32_t)j);
      }
    });
  } else {
    float* out = MODE == EXH_SAMPLE ? p.srow + (size_t)tr * p.sld : p.ws + (size_t)tr * p.ld;
    score_staged<DT, D, HT, 4>(f, base, scl, (int)(j1 - j0), stage, [&](int i, float x) {
      const int64_t j = j0 + i;
      if (j < j_end) out[j] = x;
    });
  }
}

template <int DT, int D, int HT>
static hipError_t launch_exh_score_t(const ExhParams& p, int mode, int64_t n_max, hipStream_t s) {
  dim3 grid((p.Tb + 3) / 4, (unsigned)((n_max + p.kchunk - 1) / p.kchunk));
  if (mode == EXH_SAMPLE) hipLaunchKernelGGL((k_exh_score<DT, D, HT, EXH_SAMPLE>), grid, dim3(256), 0, s, p);
  else if (mode == EXH_STREAM) hipLaunchKernelGGL((k_exh_score<DT, D, HT, EXH_STREAM>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((k_exh_score<DT, D, HT, EXH_ROWS>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_exh_score(const ExhParams& p, int mode, int dtype, int dim, int ht, int64_t n_max, hipStream_t s) {
  IVFTK_DISPATCH(launch_exh_score_t, dtype, dim, ht, p, mode, n_max, s);
}

// ---------------------------------------------------------------------------
// streamed exhaustive selection
// ---------------------------------------------------------------------------
// The top k of a row are found without writing the row: (1) every stride-th key (the
// sample) is scored; (2) a threshold tau per row is read off the sample, at the rank
// where about `aim` (>= 2k) scores of the whole row are expected to reach it; (3) the
// full scoring pass keeps only the scores >= tau, with their positions, and counts
// them; (4) a row with at least min(k, prefix) and at most caps such scores holds its
// whole answer among them (every score above the k-th, and every tie with it, reaches
// tau), which is sorted; any other row goes to the fallback, which materializes the
// row and selects from it.  A prefix of at most caps keys takes tau = 0 (all keys).

// The sample's rows (and scales) in one dense run: sample s is key soff + s * stride.
__global__ __launch_bounds__(256) void k_exh_gather(ExhParams p, int rb, int64_t ns, uint8_t* srows, float* sscale) {
  const int cpr = rb / 16;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t smp = idx / cpr;
  if (smp >= ns) return;
  const int c = (int)(idx % cpr);
  const int64_t pos = p.soff + smp * p.stride;
  reinterpret_cast<uint4*>(srows + (size_t)smp * rb)[c] = reinterpret_cast<const uint4*>(p.keys + (size_t)pos * rb)[c];
  if (p.kscale && c == 0) sscale[smp] = p.kscale[pos];
}

hipError_t launch_exh_gather(const ExhParams& p, int rb, int64_t ns, hipStream_t s) {
  if (ns <= 0) return hipSuccess;
  const int64_t threads = ns * (rb / 16);
  hipLaunchKernelGGL(k_exh_gather, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p, rb, ns,
                     const_cast<uint8_t*>(p.skeys), const_cast<float*>(p.sscale));
  return hipGetLastError();
}

constexpr int EXH_SAMPLE_CAP = 16384;   // sample scores one threshold block holds

// tau of each row of the pass (one block per row); clears the row's count and, in
// block 0, the fallback list.
__global__ __launch_bounds__(1024) void k_exh_threshold(ExhParams p) {
  __shared__ uint32_t sk[EXH_SAMPLE_CAP];
  __shared__ Select32Scratch sc;
  const int tl = blockIdx.x, tid = threadIdx.x;
  const int t = exh_query(p, tl);
  const int64_t n = p.q_pos0 + t + 1;
  const int64_t ns = exh_run_len<EXH_SAMPLE>(p, t);
  if (tid == 0) {
    p.cnt[tl] = 0;
    if (tl == 0) p.failed[0] = 0;
  }
  uint32_t tau = 0u;
  if (n > p.caps && ns > 0 && ns <= EXH_SAMPLE_CAP) {
    // about aim of the n scores reach the sample's r-th largest
    const int64_t r = ((int64_t)p.aim * ns + n - 1) / n;
    if (r <= ns) {
      const float* row = p.srow + (size_t)tl * p.sld;
      for (int64_t i = tid; i < ns; i += blockDim.x) sk[i] = order_bits(row[i]);
      __syncthreads();
      tau = radix_select32_desc(sk, (int)ns, (int)r, sc);
    }
  }
  if (tid == 0) p.tau[tl] = tau;
}

hipError_t launch_exh_threshold(const ExhParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_exh_threshold, dim3(p.Tb), dim3(1024), 0, s, p);
  return hipGetLastError();
}

// Each row's top k from its survivors, or the row onto the fallback list: the k-th
// largest survivor (a radix select over the survivor list in memory) bounds the k
// survivors that are kept, which are then sorted.
__global__ __launch_bounds__(1024) void k_exh_finalize(ExhParams p) {
  __shared__ uint64_t sel[4096];
  __shared__ SelectScratch ss;
  __shared__ int s_n;
  const int tl = blockIdx.x, tid = threadIdx.x;
  const int t = exh_query(p, tl);
  const int64_t n = p.q_pos0 + t + 1;
  const int K = p.k;
  const int c = p.cnt[tl];
  const int need = n < K ? (int)n : K;
  if (c < need || c > p.caps) {
    if (tid == 0) p.failed[1 + atomicAdd(&p.failed[0], 1)] = tl;
    return;
  }
  const uint64_t* sv = p.surv + (size_t)tl * p.caps;
  const int m = c < K ? c : K;   // entries kept
  const int P2 = next_pow2(m);
  if (c <= K) {
    for (int i = tid; i < P2; i += blockDim.x) sel[i] = i < c ? sv[i] : 0ull;
  } else {
    const uint64_t kth = radix_select_desc(sv, nullptr, c, K, ss);   // composites are unique
    if (tid == 0) s_n = 0;
    __syncthreads();
    for (int i = tid; i < c; i += blockDim.x) {
      const uint64_t v = sv[i];
      if (v >= kth) sel[atomicAdd(&s_n, 1)] = v;
    }
    for (int i = K + tid; i < P2; i += blockDim.x) sel[i] = 0ull;
  }
  __syncthreads();
  bitonic_sort_desc(sel, P2);
  write_topk(sel, P2, K, p.topk_idx + (size_t)t * K, p.topk_score ? p.topk_score + (size_t)t * K : nullptr);
}

hipError_t launch_exh_finalize(const ExhParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_exh_finalize, dim3(p.Tb), dim3(1024), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// top-k of one exhaustive score row per block
// ---------------------------------------------------------------------------
constexpr int ROW_CAP = 8192;   // composites held in LDS

// Digit search over a histogram in descending digit order: finds d with
// count(> d) < need <= count(>= d).  All threads call; results in shared vars.
__device__ inline void block_find_digit(const int* hist, int nbins, int need, int* wtmp, int* o_digit,
                                        int* o_above, int* o_in) {
  const int tid = threadIdx.x, bd = blockDim.x;
  const int per = (nbins + bd - 1) / bd;
  int s = 0;
  for (int q = 0; q < per; ++q) {
    const int d = nbins - 1 - tid * per - q;
    if (d >= 0) s += hist[d];
  }
  int tot;
  const int excl = block_exclusive_scan(s, wtmp, &tot);
  if (excl < need && need <= excl + s) {
    int acc = excl;
    for (int q = 0; q < per; ++q) {
      const int d = nbins - 1 - tid * per - q;
      if (d < 0) break;
      if (acc + hist[d] >= need) {
        *o_digit = d;
        *o_above = acc;
        *o_in = hist[d];
        break;
      }
      acc += hist[d];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(1024) void k_topk_rows(ExhParams p) {
  __shared__ uint64_t buf[ROW_CAP];
  // the digit histograms share buf's memory: each is read to its last use (the
  // digit search) before buf collects anything, so two blocks fit on a CU
  static_assert(4096 * sizeof(int) <= ROW_CAP * sizeof(uint64_t), "histogram must fit in buf");
  int* const hist = reinterpret_cast<int*>(buf);
  __shared__ Select32Scratch sc32;
  __shared__ int wtmp[16];
  __shared__ int s_cnt, s_digit, s_above, s_in, s_taken;
  const int tid = threadIdx.x, bd = blockDim.x;
  const int tl = blockIdx.x, t = exh_query(p, tl);
  const int64_t n = p.q_pos0 + t + 1;
  const float* row = p.ws + (size_t)tl * p.ld;
  const int K = p.k;
  int* oi = p.topk_idx + (size_t)t * K;
  float* os = p.topk_score ? p.topk_score + (size_t)t * K : nullptr;

  if (n <= ROW_CAP) {
    const int P2 = next_pow2((int)n);
    for (int i = tid; i < P2; i += bd) buf[i] = i < n ? make_comp(row[i], (uint32_t)i) : 0ull;
    __syncthreads();
    bitonic_sort_desc(buf, P2);
    write_topk(buf, P2, K, oi, os);
    return;
  }
  // ---- sampled threshold: 8192 evenly spaced scores give a key tau that about
  // min(2k, (k + ROW_CAP) / 2) scores of the row reach; one vectorized pass gathers
  // every score >= tau.  If at least k and at most ROW_CAP do, their exact order gives
  // the answer (every score above the k-th, and every tie with it, is among them);
  // otherwise the digit passes below decide. ----
  if (K < ROW_CAP) {
    constexpr int NS = 8192;
    uint32_t* sk = reinterpret_cast<uint32_t*>(buf);   // [NS] sample keys
    {
      float v[NS / 1024];   // the kernel runs 1024 threads: eight samples each, loaded together
#pragma unroll
      for (int u = 0; u < NS / 1024; ++u) v[u] = row[((int64_t)(u * 1024 + tid) * n) / NS];
#pragma unroll
      for (int u = 0; u < NS / 1024; ++u) sk[u * 1024 + tid] = order_bits(v[u]);
    }
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    const int64_t aim = K + (K < (ROW_CAP - K) / 2 ? K : (ROW_CAP - K) / 2);
    const int64_t want = (aim * NS + n - 1) / n + 8;
    const int rank = (int)(want < NS ? want : NS);
    const uint32_t tau = radix_select32_desc(sk, NS, rank, sc32);
    __syncthreads();   // the sample is no longer read; buf collects candidates
    const float4* row4 = reinterpret_cast<const float4*>(row);
    const int64_t n4 = (n + 3) / 4;
    const int lane = tid & 63;
    for (int64_t b4 = 0; b4 < n4; b4 += 4 * bd) {
      float e[16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t j4 = b4 + u * bd + tid;
        const float4 v = j4 < n4 ? row4[j4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        e[4 * u] = v.x;
        e[4 * u + 1] = v.y;
        e[4 * u + 2] = v.z;
        e[4 * u + 3] = v.w;
      }
      bool any = false;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int64_t j = 4 * (b4 + (u >> 2) * bd + tid) + (u & 3);
        any |= j < n && order_bits(e[u]) >= tau;
      }
      if (__ballot(any) == 0ull) continue;   // uniform: most groups hold no candidate
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int64_t j = 4 * (b4 + (u >> 2) * bd + tid) + (u & 3);
        const bool take = j < n && order_bits(e[u]) >= tau;
        const uint64_t m = __ballot(take);
        if (m == 0ull) continue;
        int base = 0;
        if (lane == 0) base = atomicAdd(&s_cnt, __popcll(m));
        base = __shfl(base, 0);
        const int at = base + __popcll(m & ((1ull << lane) - 1ull));
        if (take && at < ROW_CAP) buf[at] = make_comp(e[u], (uint32_t)j);
      }
    }
    __syncthreads();
    const int cnt = s_cnt;
    if (cnt >= K && cnt <= ROW_CAP) {
      const int P2 = next_pow2(cnt);
      for (int i = cnt + tid; i < P2; i += bd) buf[i] = 0ull;
      __syncthreads();
      bitonic_sort_desc(buf, P2);
      write_topk(buf, P2, K, oi, os);
      return;
    }
    __syncthreads();
  }
  // pass 1: top 12 bits of the order key
  for (int i = tid; i < 4096; i += bd) hist[i] = 0;
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  for (int64_t j = tid; j < n; j += bd) atomicAdd(&hist[order_bits(row[j]) >> 20], 1);
  __syncthreads();
  block_find_digit(hist, 4096, K, wtmp, &s_digit, &s_above, &s_in);
  const uint32_t d1 = (uint32_t)s_digit;
  int above = s_above;
  if (above + s_in <= ROW_CAP) {
    for (int64_t j = tid; j < n; j += bd) {
      const float v = row[j];
      if ((order_bits(v) >> 20) >= d1) buf[atomicAdd(&s_cnt, 1)] = make_comp(v, (uint32_t)j);
    }
    __syncthreads();
    const int cnt = s_cnt;
    const int P2 = next_pow2(cnt);
    for (int i = cnt + tid; i < P2; i += bd) buf[i] = 0ull;
    __syncthreads();
    bitonic_sort_desc(buf, P2);
    write_topk(buf, P2, K, oi, os);
    return;
  }
  // pass 2: next 12 bits inside bin d1
  __syncthreads();
  for (int i = tid; i < 4096; i += bd) hist[i] = 0;
  __syncthreads();
  for (int64_t j = tid; j < n; j += bd) {
    const uint32_t o = order_bits(row[j]);
    if ((o >> 20) == d1) atomicAdd(&hist[(o >> 8) & 0xFFFu], 1);
  }
  __syncthreads();
  block_find_digit(hist, 4096, K - above, wtmp, &s_digit, &s_above, &s_in);
  const uint32_t p2 = (d1 << 12) | (uint32_t)s_digit;
  above += s_above;
  if (above + s_in <= ROW_CAP) {
    for (int64_t j = tid; j < n; j += bd) {
      const float v = row[j];
      if ((order_bits(v) >> 8) >= p2) buf[atomicAdd(&s_cnt, 1)] = make_comp(v, (uint32_t)j);
    }
    __syncthreads();
    const int cnt = s_cnt;
    const int P2 = next_pow2(cnt);
    for (int i = cnt + tid; i < P2; i += bd) buf[i] = 0ull;
    __syncthreads();
    bitonic_sort_desc(buf, P2);
    write_topk(buf, P2, K, oi, os);
    return;
  }
  // pass 3: last 8 bits -> exact threshold key; then ties by position
  __syncthreads();
  for (int i = tid; i < 256; i += bd) hist[i] = 0;
  __syncthreads();
  for (int64_t j = tid; j < n; j += bd) {
    const uint32_t o = order_bits(row[j]);
    if ((o >> 8) == p2) atomicAdd(&hist[o & 0xFFu], 1);
  }
  __syncthreads();
  block_find_digit(hist, 256, K - above, wtmp, &s_digit, &s_above, &s_in);
  const uint32_t thr = (p2 << 8) | (uint32_t)s_digit;
  above += s_above;   // keys strictly above thr: fewer than K
  for (int64_t j = tid; j < n; j += bd) {
    const float v = row[j];
    if (order_bits(v) > thr) buf[atomicAdd(&s_cnt, 1)] = make_comp(v, (uint32_t)j);
  }
  if (tid == 0) s_taken = 0;
  __syncthreads();
  const int need_eq = K - above;
  for (int64_t base = 0; base < n; base += bd) {
    const int taken = s_taken;
    if (taken >= need_eq) break;
    const int64_t j = base + tid;
    const float v = j < n ? row[j] : 0.0f;
    const int flag = (j < n && order_bits(v) == thr) ? 1 : 0;
    int tot;
    const int ex = block_exclusive_scan(flag, wtmp, &tot);
    if (flag && taken + ex < need_eq) buf[above + taken + ex] = make_comp(v, (uint32_t)j);
    __syncthreads();
    if (tid == 0) s_taken = taken + tot;
    __syncthreads();
  }
  const int P2 = next_pow2(K);
  for (int i = K + tid; i < P2; i += bd) buf[i] = 0ull;
  __syncthreads();
  bitonic_sort_desc(buf, P2);
  write_topk(buf, P2, K, oi, os);
}

hipError_t launch_topk_rows(const ExhParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_topk_rows, dim3(p.Tb), dim3(1024), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// representative scores: block = 4 queries, one chunk of slots
// ---------------------------------------------------------------------------
template <int DT, int D, int HT>
__global__ __launch_bounds__(256, (score_waves<DT, D, HT>())) void k_rep_score(RouteParams p, int chunk) {
  using G = Geo<DT, D>;
  using S = Stage<DT, D>;
  __shared__ float wq_s[4][HT * 32];
  __shared__ StageLds<DT, D> stage;
  __shared__ int s_r[4], s_cvis[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 31;
  const int t = blockIdx.x * 4 + wave;
  const bool active = t < p.T;
  const int tc = active ? t : p.T - 1;
  load_query_weights<HT>(wq_s[wave], p.w + (size_t)tc * p.H, p.qscale ? p.qscale + (size_t)tc * p.H : nullptr, p.H);
  const QVer v = query_version(p, tc);
  if (lane == 0) {
    s_r[wave] = active ? v.r : -1;
    s_cvis[wave] = active ? v.cvis : 0;
  }
  __syncthreads();
  // The block shares one staged pass when its queries use the same epoch (then a
  // slot's representative is the same row for all of them); otherwise each wave
  // scores its own slots.
  int r_all = -1, cmax = 0;
  bool same = true;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int rw = s_r[w];
    if (rw >= 0) {
      if (r_all < 0) r_all = rw;
      else if (rw != r_all) same = false;
      cmax = max(cmax, s_cvis[w]);
    }
  }
  const int s0 = blockIdx.y * chunk;
  float* out = p.srep + (size_t)tc * p.srep_ld;
  if (same) {
    const int s1 = min(cmax, s0 + chunk);
    if (s0 >= s1) return;
    const int own_end = active ? min(v.cvis, s1) : s0;
    const StoreView ep = epoch_store(p, r_all);
    const int split = v.split;   // the same for every query of the epoch
    QueryFrag<DT, D, HT> f;
    load_query<DT, D, HT>(f, p.q + (size_t)tc * p.H * G::RB, p.H);
    load_query_wregs<DT, D, HT>(f, wq_s[wave]);
    // slots below the split are the epoch's, the rest the seal store's: one dense run each
    auto run = [&](const uint8_t* rep, const float* rsc, int a, int b) {
      if (a >= b) return;
      score_staged<DT, D, HT, 4>(
          f, rep + (size_t)a * G::RB, DT == DT_E4M3 ? rsc + a : nullptr, b - a, stage,
          [&](int i, float x) {
            const int s = a + i;
            if (s < own_end) out[s] = x;
          });
    };
    run(ep.rep, ep.rsc, s0, min(s1, split));
    run(p.seal.rep, p.seal.rsc, max(s0, split), s1);
    return;
  }
  if (!active) return;
  const int s1 = min(v.cvis, s0 + chunk);
  if (s0 >= s1) return;
  const StoreView ep = epoch_store(p, v.r);
  QueryFrag<DT, D, HT> f;
  load_query<DT, D, HT>(f, p.q + (size_t)t * p.H * G::RB, p.H);
  load_query_wregs<DT, D, HT>(f, wq_s[wave]);
  const int nblk = (s1 - s0 + 31) >> 5;
  score_blocks<DT, D, HT, 3>(
      f, 0, 1, nblk,
      [&](int blk, uint32_t* buf, float& sc) {
        int s = s0 + blk * 32 + col;
        s = s < s1 ? s : s1 - 1;
        const bool from_epoch = s < v.split;
        load_half_row<DT, D>(buf, (from_epoch ? ep.rep : p.seal.rep) + (size_t)s * G::RB);
        sc = (DT == DT_E4M3) ? (from_epoch ? ep.rsc : p.seal.rsc)[s] : 1.0f;
      },
      [&](int blk, float x) {
        const int s = s0 + blk * 32 + col;
        if (lane < 32 && s < s1) out[s] = x;
      });
}

template <int DT, int D, int HT>
static hipError_t launch_rep_score_t(const RouteParams& p, int max_slots, hipStream_t s) {
  // slots per block: 2048 for large batches (measured best among 512 .. 8192 at 4096
  // queries); small batches split the slots finer so that about 512 blocks run (at
  // least 64 slots per block)
  const int64_t groups = (p.T + 3) / 4;
  int chunk = (int)((max_slots * groups + 511) / 512);
  chunk = chunk < 64 ? 64 : (chunk > 2048 ? 2048 : ((chunk + 63) / 64) * 64);
  dim3 grid((p.T + 3) / 4, (max_slots + chunk - 1) / chunk);
  hipLaunchKernelGGL((k_rep_score<DT, D, HT>), grid, dim3(256), 0, s, p, chunk);
  return hipGetLastError();
}

hipError_t launch_rep_score(const RouteParams& p, int dtype, int dim, int ht, int max_slots, hipStream_t s) {
  IVFTK_DISPATCH(launch_rep_score_t, dtype, dim, ht, p, max_slots, s);
}

// ---------------------------------------------------------------------------
// cluster-major scoring of the selected clusters' candidates
// ---------------------------------------------------------------------------
// Work item = one cluster and up to 16 of the queries that selected it.  The block
// gathers the cluster's member rows into LDS once (row-contiguous loads, swizzled
// like the staged scorer), then each wave scores the members against its queries
// and writes the scores to the queries' candidate rows of sbuf.  Blocks take items
// from a counter until none is left.
template <int DT, int D, int HT>
struct ClusterStage {
  static constexpr int RB = Geo<DT, D>::RB;
  static constexpr int CPR = RB / 16;
  // member rows per LDS chunk: 32 KB of rows, 32 to 256 rows
  static constexpr int CR = (32768 / RB) < 32 ? 32 : ((32768 / RB) > 256 ? 256 : 32768 / RB);
  // queries go through a per-wave LDS buffer (row-contiguous loads) when one fits in 16 KB
  static constexpr bool QLDS = HT * 32 * RB <= 16384;
  static constexpr int QCH = QLDS ? HT * 32 * CPR / 64 : 1;         // 16-byte chunks per lane
  static constexpr int QBUF = QLDS ? HT * 32 * CPR : 1;             // chunks per wave buffer
};

template <int DT, int D, int HT>
__global__ __launch_bounds__(256) void k_cluster_score(RouteParams p) {
  using G = Geo<DT, D>;
  using C = ClusterStage<DT, D, HT>;
  __shared__ u32x4 tile[C::CR * C::CPR];
  __shared__ u32x4 qbuf[4][C::QBUF];
  __shared__ float tsc[C::CR];
  __shared__ float wq_s[4][128];
  __shared__ int s_item;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31, g = (lane >> 5) & 1;
  const int nk1 = (int)(p.n_keys - 1);
  for (;;) {
    if (tid == 0) s_item = atomicAdd(&p.ctr[0], 1);
    __syncthreads();
    const int item = s_item;
    if (item >= p.ctr[1]) break;
    const int id = p.item_id[item], first = p.item_first[item], n = p.item_n[item];
    StoreView st;
    int slot;
    if (id < p.id_seal) {
      st = p.seal;
      slot = id;
    } else {
      const int e = (id - p.id_seal) / p.id_ep;
      st = p.ep[e];
      slot = id - p.id_seal - e * p.id_ep;
    }
    const int* mem = st.members + max(st.off[slot], 0);
    // members any query of the item takes (n <= 32 pairs: one per lane, wave maximum)
    int mt = lane < n ? p.pair_take[first + lane] : 0;
    for (int off = 32; off > 0; off >>= 1) mt = max(mt, __shfl_xor(mt, off));
    for (int m0 = 0; m0 < mt; m0 += C::CR) {
      const int nr = min(C::CR, mt - m0);
      __syncthreads();   // the previous chunk's readers are done
      {
        // member positions first, then all row chunks, then the LDS writes, so that
        // each thread's loads are in flight together
        constexpr int SPT = C::CR * C::CPR / 256;   // 16-byte chunks per thread
        static_assert(C::CR * C::CPR % 256 == 0 && C::CR <= 256, "chunk rows must split over the block");
        int jr[SPT];
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
          const int r = (k * 256 + tid) / C::CPR;
          jr[k] = mem[m0 + (r < nr ? r : nr - 1)];
        }
        const int js = mem[m0 + (tid < nr ? tid : nr - 1)];
        u32x4 vv[SPT];
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
          const int j = jr[k] < 0 ? 0 : (jr[k] > nk1 ? nk1 : jr[k]);
          vv[k] = *reinterpret_cast<const u32x4*>(p.keys + (size_t)j * G::RB + ((k * 256 + tid) % C::CPR) * 16);
        }
        float scl = 1.0f;
        if (DT == DT_E4M3) scl = p.kscale[js < 0 ? 0 : (js > nk1 ? nk1 : js)];
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
          const int c = k * 256 + tid;
          tile[stage_slot<C::CPR>(c / C::CPR, c % C::CPR)] = vv[k];
        }
        if (tid < C::CR) tsc[tid] = scl;
      }
      __syncthreads();
      // each wave scores pairs wave + 4j, j < np; lane j holds pair j's metadata.
      // The next pair's query rows and head weights are loaded while the current
      // pair is contracted; loads are unconditional (clamped) so that the ones in
      // flight are counted exactly.
      const int np = n > wave ? (n - wave + 3) / 4 : 0;
      int m_t = 0, m_d = 0, m_k = 0;
      if (lane < np) {
        const int pi = first + wave + 4 * lane;
        m_t = p.pair_t[pi];
        m_d = p.pair_dst[pi];
        m_k = p.pair_take[pi];
      }
      u32x4 qr[2][C::QCH];
      QueryFrag<DT, D, HT> fd[C::QLDS ? 1 : 2];   // two for direct loads (prefetch), else one
      float wv[2][2];                             // head weights of heads lane and 64 + lane
      auto fetch = [&](int j, int h) {
        const int t = __shfl(m_t, j);
        const uint8_t* q_t = p.q + (size_t)t * p.H * G::RB;
        if constexpr (C::QLDS) {
#pragma unroll
          for (int c = 0; c < C::QCH; ++c) {
            const int ci = c * 64 + lane, row = ci / C::CPR;
            const int cs = row < p.H ? ci : ci % C::CPR;   // rows past H read row 0 and are zeroed
            const u32x4 v = *reinterpret_cast<const u32x4*>(q_t + (size_t)cs * 16);
            qr[h][c] = row < p.H ? v : u32x4{0u, 0u, 0u, 0u};
          }
        } else {
          load_query<DT, D, HT>(fd[C::QLDS ? 0 : h], q_t, p.H);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int hd = u * 64 + lane;
          const size_t wi = (size_t)t * p.H + min(hd, p.H - 1);
          const float wx = p.qscale ? p.w[wi] * p.qscale[wi] : p.w[wi];
          wv[h][u] = hd < p.H ? wx : 0.0f;
        }
      };
      if (np > 0) fetch(0, 0);
      for (int j = 0; j < np; j += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int jj = j + h;
          fetch(min(jj + 1, np - 1), h ^ 1);
          if (jj < np) {
            const int t = __shfl(m_t, jj), dst = __shfl(m_d, jj), take = __shfl(m_k, jj);
            const int rows = min(take - m0, nr);
            QueryFrag<DT, D, HT>& f = fd[C::QLDS ? 0 : h];
            wq_s[wave][lane] = wv[h][0];
            wq_s[wave][64 + lane] = wv[h][1];
            if constexpr (C::QLDS) {
#pragma unroll
              for (int c = 0; c < C::QCH; ++c) {
                const int ci = c * 64 + lane;
                qbuf[wave][stage_slot<C::CPR>(ci / C::CPR, ci % C::CPR)] = qr[h][c];
              }
            }
            __builtin_amdgcn_wave_barrier();
            if constexpr (C::QLDS) {
#pragma unroll
              for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                for (int i = 0; i < G::HW / 4; ++i) {
                  const u32x4 v4 = qbuf[wave][stage_slot<C::CPR>(ht * 32 + col, g * (C::CPR / 2) + i)];
                  f.a[ht][4 * i + 0] = v4.x;
                  f.a[ht][4 * i + 1] = v4.y;
                  f.a[ht][4 * i + 2] = v4.z;
                  f.a[ht][4 * i + 3] = v4.w;
                }
            }
            load_query_wregs<DT, D, HT>(f, wq_s[wave]);
            __builtin_amdgcn_wave_barrier();
            float* out = p.sbuf + (size_t)t * p.cand_ld + dst + m0;
            for (int r0 = 0; r0 < rows; r0 += 32) {
              const int r = r0 + col;
              uint32_t bf[G::HW];
#pragma unroll
              for (int i = 0; i < G::HW / 4; ++i) {
                const u32x4 v4 = tile[stage_slot<C::CPR>(r, g * (C::CPR / 2) + i)];
                bf[4 * i + 0] = v4.x;
                bf[4 * i + 1] = v4.y;
                bf[4 * i + 2] = v4.z;
                bf[4 * i + 3] = v4.w;
              }
              const float x = score_tile<DT, D, HT>(f, bf) * tsc[r];
              if (lane < 32 && r < rows) out[r] = x;
            }
          }
        }
      }
    }
    __syncthreads();   // every thread has read s_item
  }
}

template <int DT, int D, int HT>
static hipError_t launch_cluster_score_t(const RouteParams& p, hipStream_t s) {
  int dev = 0, n_cu = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_cluster_score<DT, D, HT>, 256, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  hipLaunchKernelGGL((k_cluster_score<DT, D, HT>), dim3(n_cu * per_cu), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_cluster_score(const RouteParams& p, int dtype, int dim, int ht, hipStream_t s) {
  IVFTK_DISPATCH(launch_cluster_score_t, dtype, dim, ht, p, s);
}

}  // namespace ivftk
