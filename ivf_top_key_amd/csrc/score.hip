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

// The first K of a descending composite list of `avail` entries; missing entries
// (zero composites or past avail) are -1 / -inf.
__device__ inline void write_topk(const uint64_t* buf, int avail, int K, int* oi, float* os) {
  for (int i = threadIdx.x; i < K; i += blockDim.x) {
    const uint64_t v = i < avail ? buf[i] : 0ull;
    oi[i] = v ? (int)comp_id(v) : -1;
    if (os) os[i] = v ? comp_score(v) : -__builtin_inff();
  }
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
// query version (routed path)
// ---------------------------------------------------------------------------
struct QVer {
  int64_t n;       // prefix length
  int m;           // sealed windows inside the prefix
  int r;           // refit epoch used
  int split;       // slots below come from the epoch store
  int cvis;        // visible slots [0, cvis)
  int64_t open_lo; // open window [open_lo, n)
};

__device__ __forceinline__ QVer query_version(const RouteParams& p, int t) {
  QVer v;
  v.n = (p.qpos ? p.qpos[t] : p.q_pos0 + t) + 1;
  v.m = v.n >= p.S ? (int)((v.n - p.S) / p.W) : 0;
  v.r = p.wpr ? min(p.P, v.m / p.wpr) : 0;
  v.split = v.r * p.wpr * p.Cs;
  v.cvis = v.m * p.Cs;
  v.open_lo = (int64_t)p.S + (int64_t)v.m * p.W;
  return v;
}

__device__ __forceinline__ StoreView epoch_store(const RouteParams& p, int r) { return p.ep[r % 3]; }

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

// ---------------------------------------------------------------------------
// candidate key rows
// ---------------------------------------------------------------------------
// The three sources a query's candidate rows come from: the position-ordered keys
// (sinks and open window), the seal store's member-ordered copy and the query's
// epoch store's copy (CROW_* in params.h).  Rows are clamped below n_keys, which
// bounds every source.
// The per-lane choice of source is arithmetic on byte offsets from the first source
// (masks, no selects), which keeps the compiler from turning it into a table in
// scratch memory.
struct RowSources {
  const uint8_t* key0;
  int64_t dk1, dk2;      // key1 - key0, key2 - key0 (bytes)
  const float* scale0;
  int64_t ds1, ds2;      // scale1 - scale0, scale2 - scale0 (bytes)
};

__device__ __forceinline__ RowSources row_sources(const RouteParams& p, int r) {
  const int e = r % 3;
  const uint8_t* k2 = e == 0 ? p.ep[0].ckeys : (e == 1 ? p.ep[1].ckeys : p.ep[2].ckeys);
  const float* s2 = e == 0 ? p.ep[0].cscale : (e == 1 ? p.ep[1].cscale : p.ep[2].cscale);
  RowSources rs;
  rs.key0 = p.keys;
  rs.dk1 = (int64_t)(uintptr_t)p.seal.ckeys - (int64_t)(uintptr_t)p.keys;
  rs.dk2 = (int64_t)(uintptr_t)k2 - (int64_t)(uintptr_t)p.keys;
  rs.scale0 = p.kscale;
  rs.ds1 = (int64_t)(uintptr_t)p.seal.cscale - (int64_t)(uintptr_t)p.kscale;
  rs.ds2 = (int64_t)(uintptr_t)s2 - (int64_t)(uintptr_t)p.kscale;
  return rs;
}

template <int DT, int D>
__device__ __forceinline__ void load_cand_row(const RowSources& rs, int code, int nk1, uint32_t* buf, float& scl) {
  const int src = (int)((uint32_t)code >> CROW_SHIFT);
  int j = code & CROW_MASK;
  j = j > nk1 ? nk1 : j;
  const int64_t m1 = -(int64_t)(src == 1), m2 = -(int64_t)(src >= 2);
  const uint8_t* kb = rs.key0 + ((rs.dk1 & m1) | (rs.dk2 & m2));
  load_half_row<DT, D>(buf, kb + (size_t)j * Geo<DT, D>::RB);
  if constexpr (DT == DT_E4M3) {
    const float* sb = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(rs.scale0) +
                                                     ((rs.ds1 & m1) | (rs.ds2 & m2)));
    scl = sb[j];
  } else {
    scl = 1.0f;
  }
}

// ---------------------------------------------------------------------------
// split candidate scoring for small batches
// ---------------------------------------------------------------------------
// A batch of a few queries leaves most of the chip idle with one block per query,
// so block (t, b) scores candidates [b*CSB, (b+1)*CSB) of query t into sbuf (the
// same score tile, hence the same bits) and the final kernel only selects.
constexpr int CSB = 256;   // candidates per block

template <int DT, int D, int HT>
__global__ __launch_bounds__(256) void k_cand_score(RouteParams p) {
  using G = Geo<DT, D>;
  __shared__ float wq_s[HT * 32];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31;
  const int t = blockIdx.x;
  const int L = p.cand_len[t];
  const int i0 = blockIdx.y * CSB;
  if (i0 >= L) return;
  const int n = min(CSB, L - i0);
  const int* crow = p.cand_row + (size_t)t * p.cand_ld + i0;
  float* out = p.sbuf + (size_t)t * p.cand_ld + i0;
  const int nk1 = (int)(p.n_keys - 1);
  const RowSources rs = row_sources(p, query_version(p, t).r);
  if (wave == 0)
    load_query_weights<HT>(wq_s, p.w + (size_t)t * p.H, p.qscale ? p.qscale + (size_t)t * p.H : nullptr, p.H);
  QueryFrag<DT, D, HT> f;
  load_query<DT, D, HT>(f, p.q + (size_t)t * p.H * G::RB, p.H);
  __syncthreads();
  load_query_wregs<DT, D, HT>(f, wq_s);
  score_gather<DT, D, HT, 2>(
      f, wave, 4, (n + 31) >> 5,
      [&](int blk) -> int {
        const int i = blk * 32 + col;
        return crow[i < n ? i : n - 1];
      },
      [rs, nk1](int code, uint32_t* buf, float& scl) { load_cand_row<DT, D>(rs, code, nk1, buf, scl); },
      [&](int blk, float x) {
        const int i = blk * 32 + col;
        if (lane < 32 && i < n) out[i] = x;
      });
}

template <int DT, int D, int HT>
static hipError_t launch_cand_score_t(const RouteParams& p, int cand_cap, hipStream_t s) {
  hipLaunchKernelGGL((k_cand_score<DT, D, HT>), dim3(p.T, (cand_cap + CSB - 1) / CSB), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_cand_score(const RouteParams& p, int dtype, int dim, int ht, int cand_cap, hipStream_t s) {
  IVFTK_DISPATCH(launch_cand_score_t, dtype, dim, ht, p, cand_cap, s);
}

// ---------------------------------------------------------------------------
// candidate rescoring + top-k: one block per query
// ---------------------------------------------------------------------------
// The candidates' scores go to LDS as 32-bit order keys while the waves gather
// and score key rows (ring of row loads in flight per wave).  Then every thread
// takes its PT keys and candidate ids into registers, which frees the LDS for the
// selection: a value-binned histogram between the block's min and max score
// finds the bin holding the k-th score; entries in higher bins are placed by bin
// offset plus rank inside their bin, the cut bin is sorted exactly.  Ties at the
// k-th score go to the lowest positions; the k winners come out sorted by
// (score desc, position asc).  Degenerate cases (all scores equal, a crowded cut
// bin) use an exact radix select.
constexpr int RS_NBIN = 1024;     // value bins of the top-k histogram
constexpr int RS_TIE_CAP = 512;   // largest cut bin resolved by a local sort
constexpr int RS_THREADS = 256;        // scoring + selection blocks
constexpr int RS_SEL_THREADS = 1024;   // selection-only blocks (candidates scored beforehand)

// LDS bytes of the selection region for a candidate capacity and k (both powers of two).
__host__ __device__ constexpr size_t rescore_region_bytes(int cap_pow2, int k_pow2) {
  return (size_t)cap_pow2 * 4 > (size_t)(k_pow2 + RS_TIE_CAP) * 8 + (size_t)RS_NBIN * 8
             ? (size_t)cap_pow2 * 4
             : (size_t)(k_pow2 + RS_TIE_CAP) * 8 + (size_t)RS_NBIN * 8;
}

// NT threads per block.  With NT = RS_SEL_THREADS the block only selects: every
// candidate was scored into sbuf beforehand (small batches), and the selection's
// per-thread chains are a quarter as long, which is what a lone query waits on.
template <int DT, int D, int HT, int PT, int NT>
__global__ __launch_bounds__(NT) void k_rescore_topk(RouteParams p, int k_pow2) {
  using G = Geo<DT, D>;
  constexpr bool SELECT_ONLY = NT != RS_THREADS;
  constexpr int KPT = 4096 / NT;   // winners per thread at the largest k
  static_assert(RS_NBIN % NT == 0 && NT % 64 == 0 && NT <= 1024, "block shape");
  extern __shared__ uint64_t lds[];
  __shared__ float wq_s[HT * 32];
  __shared__ Select32Scratch sc;
  __shared__ uint32_t mm_tmp[2 * NT / 64];
  __shared__ int wtmp[16];
  __shared__ int s_cnt, s_tie, s_bstar;
  uint32_t* okey = reinterpret_cast<uint32_t*>(lds);   // scoring: [L] score keys
  uint64_t* sel = lds;                                 // selection: [k_pow2] winners
  uint64_t* tie = lds + k_pow2;                        // [RS_TIE_CAP] cut bin
  int* hist = reinterpret_cast<int*>(lds + k_pow2 + RS_TIE_CAP);   // [RS_NBIN]
  int* offs = hist + RS_NBIN;                                      // [RS_NBIN]
  const int tid = threadIdx.x, bd = NT;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, nw = bd >> 6;
  const int t = blockIdx.x;
  const int L = p.cand_len[t];
  const int* cand = p.cand_row + (size_t)t * p.cand_ld;   // gather rows; positions derived below
  const int K = p.k;
  const int nk1 = (int)(p.n_keys - 1);
  if constexpr (!SELECT_ONLY) {
  if (wave == 0)
    load_query_weights<HT>(wq_s, p.w + (size_t)t * p.H, p.qscale ? p.qscale + (size_t)t * p.H : nullptr, p.H);
  QueryFrag<DT, D, HT> f;
  load_query<DT, D, HT>(f, p.q + (size_t)t * p.H * G::RB, p.H);
  __syncthreads();
  load_query_wregs<DT, D, HT>(f, wq_s);
  // the sinks and the open window are scored here, and with cluster-major rescoring
  // the selected clusters' candidates [base_len, L) were scored into sbuf; a small
  // batch has every candidate scored into sbuf already (base_len = 0); otherwise
  // every candidate is gathered and scored here
  const QVer qv = query_version(p, t);
  const int n_sink = (int)(qv.n < p.S ? qv.n : p.S);
  const int base_len =
      p.prescored ? 0 : (p.cluster_major ? min(L, n_sink + (qv.n > qv.open_lo ? (int)(qv.n - qv.open_lo) : 0)) : L);
  const int nb = (base_len + 31) >> 5;
  const int* crow = p.cand_row + (size_t)t * p.cand_ld;
  const RowSources rs = row_sources(p, qv.r);
  // rows in flight per wave: two at 32 entries per thread keep the kernel under 168
  // VGPRs, i.e. three waves per SIMD (more loads in flight per CU than three rows
  // at two waves); at 64 entries the registers allow only two waves either way
  constexpr int RING = PT <= 32 ? 2 : 3;
  score_gather<DT, D, HT, RING>(
      f, wave, nw, nb,
      [&](int blk) -> int {
        const int i = blk * 32 + col;
        return crow[i < base_len ? i : base_len - 1];
      },
      [rs, nk1](int code, uint32_t* buf, float& scl) { load_cand_row<DT, D>(rs, code, nk1, buf, scl); },
      [&](int blk, float x) {
        const int i = blk * 32 + col;
        if (lane < 32 && i < base_len) {
          okey[i] = order_bits(x);
          if (p.dbg_cand_scores && i < p.dbg_cand_ld) p.dbg_cand_scores[(size_t)t * p.dbg_cand_ld + i] = x;
        }
      });
  {
    // eight loads in flight per thread before the first store
    const int tail_end = p.prescored ? 0 : L;   // prescored lists are read below
    for (int i0 = base_len + tid; i0 < tail_end; i0 += 8 * bd) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * bd;
        x[u] = i < L ? p.sbuf[(size_t)t * p.cand_ld + i] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * bd;
        if (i < L) {
          okey[i] = order_bits(x[u]);
          if (p.dbg_cand_scores && i < p.dbg_cand_ld) p.dbg_cand_scores[(size_t)t * p.dbg_cand_ld + i] = x[u];
        }
      }
    }
  }
  __syncthreads();
  }   // !SELECT_ONLY
  // this thread's entries: groups of four consecutive list entries, ent(u) below,
  // with their score keys and candidate positions (16-byte loads)
  auto ent = [&](int u) { return 4 * ((u >> 2) * bd + tid) + (u & 3); };
  uint32_t kv[PT];
  uint32_t cv[PT];
  // prescored: the scores come straight from sbuf into registers (no LDS pass);
  // kv holds the raw float bits until every load has been issued
  if (SELECT_ONLY || p.prescored) {
    const uint32_t* sb = reinterpret_cast<const uint32_t*>(p.sbuf + (size_t)t * p.cand_ld);
#pragma unroll
    for (int u4 = 0; u4 < PT / 4; ++u4) {
      const int i0 = 4 * (u4 * bd + tid);
      if (i0 + 3 < L) {
        const uint4 x4 = *reinterpret_cast<const uint4*>(sb + i0);
        const int4 c4 = *reinterpret_cast<const int4*>(cand + i0);
        kv[4 * u4] = x4.x, kv[4 * u4 + 1] = x4.y, kv[4 * u4 + 2] = x4.z, kv[4 * u4 + 3] = x4.w;
        cv[4 * u4] = (uint32_t)c4.x, cv[4 * u4 + 1] = (uint32_t)c4.y, cv[4 * u4 + 2] = (uint32_t)c4.z,
        cv[4 * u4 + 3] = (uint32_t)c4.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv[4 * u4 + e] = i0 + e < L ? sb[i0 + e] : 0u;
          cv[4 * u4 + e] = i0 + e < L ? (uint32_t)cand[i0 + e] : 0u;
        }
      }
    }
    float* dbs = p.dbg_cand_scores ? p.dbg_cand_scores + (size_t)t * p.dbg_cand_ld : nullptr;
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int i = ent(u);
      if (dbs && i < L && i < p.dbg_cand_ld) dbs[i] = __uint_as_float(kv[u]);
      kv[u] = i < L ? order_bits(__uint_as_float(kv[u])) : 0u;
    }
  } else if constexpr (!SELECT_ONLY) {
#pragma unroll
    for (int u4 = 0; u4 < PT / 4; ++u4) {
      const int i0 = 4 * (u4 * bd + tid);
      if (i0 + 3 < L) {
        const uint4 k4 = *reinterpret_cast<const uint4*>(okey + i0);
        const int4 c4 = *reinterpret_cast<const int4*>(cand + i0);
        kv[4 * u4 + 0] = k4.x;
        kv[4 * u4 + 1] = k4.y;
        kv[4 * u4 + 2] = k4.z;
        kv[4 * u4 + 3] = k4.w;
        cv[4 * u4 + 0] = (uint32_t)c4.x;
        cv[4 * u4 + 1] = (uint32_t)c4.y;
        cv[4 * u4 + 2] = (uint32_t)c4.z;
        cv[4 * u4 + 3] = (uint32_t)c4.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + e;
          kv[4 * u4 + e] = i < L ? okey[i] : 0u;
          cv[4 * u4 + e] = i < L ? (uint32_t)cand[i] : 0u;
        }
      }
    }
  }
  {
    // positions: source 0 rows are positions; a store copy's row j holds that store's
    // member j.  Every lane loads (source 0 reads a valid dummy word), then selects.
    const QVer qv2 = query_version(p, t);
    const int e = qv2.r % 3;
    const int* mem0 = p.cand_len + t;
    const int* mem2 = e == 0 ? p.ep[0].members : (e == 1 ? p.ep[1].members : p.ep[2].members);
    const int64_t d1 = (int64_t)(uintptr_t)p.seal.members - (int64_t)(uintptr_t)mem0;
    const int64_t d2 = (int64_t)(uintptr_t)mem2 - (int64_t)(uintptr_t)mem0;
    const int jmax = (int)max((int64_t)0, p.n_keys - 1 - p.S);
    int mv[PT];
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int src = (int)(cv[u] >> CROW_SHIFT);
      const int64_t m1 = -(int64_t)(src == 1), m2 = -(int64_t)(src >= 2);
      const int* mb = reinterpret_cast<const int*>(reinterpret_cast<const uint8_t*>(mem0) + ((d1 & m1) | (d2 & m2)));
      const int j = (int)(cv[u] & (uint32_t)CROW_MASK);
      mv[u] = mb[src == 0 ? 0 : (j < jmax ? j : jmax)];
    }
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int src = (int)(cv[u] >> CROW_SHIFT);
      cv[u] = src == 0 ? (cv[u] & (uint32_t)CROW_MASK) : (uint32_t)mv[u];
    }
  }
  if (tid == 0) {
    s_cnt = 0;
    s_tie = 0;
  }
  __syncthreads();   // the LDS region is free from here on
  int* oi = p.topk_idx + (size_t)t * K;
  float* os = p.topk_score ? p.topk_score + (size_t)t * K : nullptr;
  auto comp = [](uint32_t key, uint32_t pos) -> uint64_t { return ((uint64_t)key << 32) | (uint64_t)(~pos); };
  if (L <= K) {
    const int P2 = next_pow2(L > 0 ? L : 1);
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int i = ent(u);
      if (i < P2) sel[i] = i < L ? comp(kv[u], cv[u]) : 0ull;
    }
    __syncthreads();
    bitonic_sort_desc(sel, P2);
    write_topk(sel, L, K, oi, os);
    return;
  }
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    if (ent(u) < L) {
      mn = kv[u] < mn ? kv[u] : mn;
      mx = kv[u] > mx ? kv[u] : mx;
    }
  }
  block_minmax(mn, mx, mm_tmp);
  bool fallback = (mn == mx);
  ValBins bins;
  int bstar = 0, above = 0, in_bin = 0;
  if (!fallback) {
    bins = make_bins(mn, mx, RS_NBIN);
    for (int i = tid; i < RS_NBIN; i += bd) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PT; ++u)
      if (ent(u) < L) atomicAdd(&hist[bins(kv[u])], 1);
    __syncthreads();
    // offs[b] = entries in bins above b (descending order); the bin holding the K-th
    constexpr int per = RS_NBIN / NT;
    int sum = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) sum += hist[RS_NBIN - 1 - tid * per - q];
    int tot;
    int run = block_exclusive_scan(sum, wtmp, &tot);
#pragma unroll
    for (int q = 0; q < per; ++q) {
      const int bb = RS_NBIN - 1 - tid * per - q;
      const int c = hist[bb];
      offs[bb] = run;
      if (run < K && K <= run + c) s_bstar = bb;
      run += c;
    }
    __syncthreads();
    bstar = s_bstar;
    above = offs[bstar];
    in_bin = hist[bstar];
    fallback = in_bin > RS_TIE_CAP;
    __syncthreads();   // every thread has read hist[bstar] before hist becomes the cursors
  }
  if (!fallback) {
    // scatter: bins above the cut go to their bin's range of sel, the cut bin to tie
    for (int i = tid; i < RS_NBIN; i += bd) hist[i] = offs[i];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      if (ent(u) < L) {
        const int bb = (int)bins(kv[u]);
        if (bb > bstar) sel[atomicAdd(&hist[bb], 1)] = comp(kv[u], cv[u]);
        else if (bb == bstar) tie[atomicAdd(&s_tie, 1)] = comp(kv[u], cv[u]);
      }
    }
    const int P2 = next_pow2(in_bin);
    __syncthreads();
    if (P2 <= 64) {
      if (tid < 64) tie[tid] = wave_sort_desc(tid < in_bin ? tie[tid] : 0ull);
    } else {
      for (int i = in_bin + tid; i < P2; i += bd) tie[i] = 0ull;
      __syncthreads();
      bitonic_sort_desc(tie, P2);
    }
    // entries above the cut move to bin start + rank inside the bin (ranks are taken
    // before any entry moves), the cut bin's winners follow them
    uint64_t pv[KPT];
    int pp[KPT];
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const int i = q * bd + tid;
      pp[q] = -1;
      if (i < above) {
        const uint64_t v = sel[i];
        const int bb = (int)bins((uint32_t)(v >> 32));
        const int lo = offs[bb], hi = offs[bb - 1];
        int rank = 0;
        int j = lo;
        for (; j + 4 <= hi; j += 4) {   // four LDS reads in flight
          const uint64_t a0 = sel[j], a1 = sel[j + 1], a2 = sel[j + 2], a3 = sel[j + 3];
          rank += (a0 > v) + (a1 > v) + (a2 > v) + (a3 > v);
        }
        for (; j < hi; ++j) rank += sel[j] > v;
        pv[q] = v;
        pp[q] = lo + rank;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < KPT; ++q)
      if (pp[q] >= 0) sel[pp[q]] = pv[q];
    for (int r = tid; r < K - above; r += bd) sel[above + r] = tie[r];
    __syncthreads();
    write_topk(sel, K, K, oi, os);
    return;
  }
  // ---- fallback: exact radix select (all keys equal, or a crowded cut bin) ----
  __syncthreads();
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int i = ent(u);
    if (i < L) okey[i] = kv[u];
  }
  __syncthreads();
  const uint32_t thr = radix_select32_desc(okey, L, K, sc);
  const int need = K - sc.above;
  const int n_eq = sc.hist[thr & 255u];
  uint32_t t2 = 0u;
  __syncthreads();
  if (n_eq != need) {
    // more candidates share the k-th score than slots remain: lowest positions win
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int i = ent(u);
      if (i < L) okey[i] = (kv[u] == thr) ? ~cv[u] : 0u;
    }
    __syncthreads();
    t2 = radix_select32_desc(okey, L, need, sc);
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    if (ent(u) < L) {
      const uint32_t v = kv[u];
      if (v > thr || (v == thr && (n_eq == need || ~cv[u] >= t2))) sel[atomicAdd(&s_cnt, 1)] = comp(v, cv[u]);
    }
  }
  __syncthreads();
  for (int i = K + tid; i < k_pow2; i += bd) sel[i] = 0ull;
  __syncthreads();
  bitonic_sort_desc(sel, k_pow2);
  write_topk(sel, K, K, oi, os);
}

template <int DT, int D, int HT, int PT, int NT>
static hipError_t launch_rescore_pt(const RouteParams& p, int cap_pow2, int k_pow2, hipStream_t s) {
  const size_t lds = rescore_region_bytes(cap_pow2, k_pow2);
  hipError_t e = hipFuncSetAttribute((const void*)k_rescore_topk<DT, D, HT, PT, NT>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_rescore_topk<DT, D, HT, PT, NT>), dim3(p.T), dim3(NT), lds, s, p, k_pow2);
  return hipGetLastError();
}

template <int DT, int D, int HT>
static hipError_t launch_rescore_topk_t(const RouteParams& p, int cand_cap, hipStream_t s) {
  const int cap_pow2 = next_pow2(cand_cap);
  const int k_pow2 = next_pow2(p.k);
  if (p.prescored) {   // selection only: four times the threads, a quarter of the entries each
    if (cap_pow2 <= 8 * RS_SEL_THREADS) return launch_rescore_pt<DT, D, HT, 8, RS_SEL_THREADS>(p, cap_pow2, k_pow2, s);
    if (cap_pow2 <= 16 * RS_SEL_THREADS)
      return launch_rescore_pt<DT, D, HT, 16, RS_SEL_THREADS>(p, cap_pow2, k_pow2, s);
    return hipErrorInvalidValue;
  }
  if (cap_pow2 <= 32 * RS_THREADS) return launch_rescore_pt<DT, D, HT, 32, RS_THREADS>(p, cap_pow2, k_pow2, s);
  if (cap_pow2 <= 64 * RS_THREADS) return launch_rescore_pt<DT, D, HT, 64, RS_THREADS>(p, cap_pow2, k_pow2, s);
  return hipErrorInvalidValue;
}

hipError_t launch_rescore_topk(const RouteParams& p, int dtype, int dim, int ht, int cand_cap, hipStream_t s) {
  IVFTK_DISPATCH(launch_rescore_topk_t, dtype, dim, ht, p, cand_cap, s);
}

bool rescore_fits(int cand_cap, int k) {
  const int cap_pow2 = next_pow2(cand_cap), k_pow2 = next_pow2(k);
  // the region plus the kernel's static LDS (head weights, radix scratch, a few words)
  return cap_pow2 <= 64 * RS_THREADS && rescore_region_bytes(cap_pow2, k_pow2) + 4096 <= 163840;
}

}  // namespace ivftk
