// Indexer scoring kernels: exhaustive scores, representative scores, candidate
// rescoring with the top-k selection, and the top-k of exhaustive score rows.
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
// exhaustive scores: block = 4 waves = 4 queries, one chunk of keys
// ---------------------------------------------------------------------------
template <int DT, int D, int HT>
__global__ __launch_bounds__(256) void k_exh_score(ExhParams p) {
  using G = Geo<DT, D>;
  using S = Stage<DT, D>;
  __shared__ float wq_s[4][HT * 32];
  __shared__ u32x4 tile[2 * S::CHUNKS];
  __shared__ float tsc[2 * S::SR];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tl = blockIdx.x * 4 + wave;
  const bool active = tl < p.Tb;
  const int tc = p.t0 + (active ? tl : p.Tb - 1);   // idle waves still stage rows
  load_query_weights<HT>(wq_s[wave], p.w + (size_t)tc * p.H, p.qscale ? p.qscale + (size_t)tc * p.H : nullptr, p.H);
  // the block's rows: keys [j0, j1) with j1 bounded by its longest prefix
  const int t_last = p.t0 + min(blockIdx.x * 4 + 3, p.Tb - 1);
  const int64_t j0 = (int64_t)blockIdx.y * p.kchunk;
  const int64_t n_max = p.q_pos0 + t_last + 1;
  const int64_t j1 = (j0 + p.kchunk < n_max) ? j0 + p.kchunk : n_max;
  __syncthreads();
  if (j0 >= j1) return;
  const int64_t n_own = p.q_pos0 + tc + 1;
  const int64_t j_end = active ? (j1 < n_own ? j1 : n_own) : j0;
  QueryFrag<DT, D, HT> f;
  load_query<DT, D, HT>(f, p.q + (size_t)tc * p.H * G::RB, p.H);
  load_query_wregs<DT, D, HT>(f, wq_s[wave]);
  float* out = p.ws + (size_t)(active ? tl : 0) * p.ld;
  score_staged<DT, D, HT, 4>(
      f, (int)(j1 - j0), tile, tsc,
      [&](int i, const uint8_t*& rp, float& sc) {
        const int64_t j = j0 + i;
        rp = p.keys + (size_t)j * G::RB;
        sc = (DT == DT_E4M3) ? p.kscale[j] : 1.0f;
      },
      [&](int i, float x) {
        const int64_t j = j0 + i;
        if (lane < 32 && j < j_end) out[j] = x;
      });
}

template <int DT, int D, int HT>
static hipError_t launch_exh_score_t(const ExhParams& p, int64_t n_max, hipStream_t s) {
  dim3 grid((p.Tb + 3) / 4, (unsigned)((n_max + p.kchunk - 1) / p.kchunk));
  hipLaunchKernelGGL((k_exh_score<DT, D, HT>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_exh_score(const ExhParams& p, int dtype, int dim, int ht, int64_t n_max, hipStream_t s) {
  IVFTK_DISPATCH(launch_exh_score_t, dtype, dim, ht, p, n_max, s);
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

__device__ inline void write_topk(const uint64_t* buf, int avail, int K, int* oi, float* os) {
  for (int i = threadIdx.x; i < K; i += blockDim.x) {
    const uint64_t v = i < avail ? buf[i] : 0ull;
    oi[i] = v ? (int)comp_id(v) : -1;
    if (os) os[i] = v ? comp_score(v) : -__builtin_inff();
  }
}

__global__ __launch_bounds__(1024) void k_topk_rows(ExhParams p) {
  __shared__ uint64_t buf[ROW_CAP];
  __shared__ int hist[4096];
  __shared__ int wtmp[16];
  __shared__ int s_cnt, s_digit, s_above, s_in, s_taken;
  const int tid = threadIdx.x, bd = blockDim.x;
  const int tl = blockIdx.x, t = p.t0 + tl;
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
  v.n = p.q_pos0 + t + 1;
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
__global__ __launch_bounds__(256) void k_rep_score(RouteParams p, int chunk) {
  using G = Geo<DT, D>;
  using S = Stage<DT, D>;
  __shared__ float wq_s[4][HT * 32];
  __shared__ u32x4 tile[2 * S::CHUNKS];
  __shared__ float tsc[2 * S::SR];
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
    const int split = v.split;
    QueryFrag<DT, D, HT> f;
    load_query<DT, D, HT>(f, p.q + (size_t)tc * p.H * G::RB, p.H);
    load_query_wregs<DT, D, HT>(f, wq_s[wave]);
    score_staged<DT, D, HT, 4>(
        f, s1 - s0, tile, tsc,
        [&](int i, const uint8_t*& rp, float& sc) {
          const int s = s0 + i;
          const bool from_epoch = s < split;
          rp = (from_epoch ? ep.rep : p.seal.rep) + (size_t)s * G::RB;
          sc = (DT == DT_E4M3) ? (from_epoch ? ep.rsc : p.seal.rsc)[s] : 1.0f;
        },
        [&](int i, float x) {
          const int s = s0 + i;
          if (lane < 32 && s < own_end) out[s] = x;
        });
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
  const int chunk = 1024;
  dim3 grid((p.T + 3) / 4, (max_slots + chunk - 1) / chunk);
  hipLaunchKernelGGL((k_rep_score<DT, D, HT>), grid, dim3(256), 0, s, p, chunk);
  return hipGetLastError();
}

hipError_t launch_rep_score(const RouteParams& p, int dtype, int dim, int ht, int max_slots, hipStream_t s) {
  IVFTK_DISPATCH(launch_rep_score_t, dtype, dim, ht, p, max_slots, s);
}

// ---------------------------------------------------------------------------
// candidate rescoring + top-k: one block per query
// ---------------------------------------------------------------------------
// Scores of the candidates stay in LDS as 32-bit order keys; a 32-bit radix select
// finds the k-th score, ties at that score go to the lowest positions, and the k
// winners are sorted by (score desc, position asc).  Key rows are gathered one
// block of 32 ahead of the MFMA work so a wave always has loads in flight.
constexpr int RS_NBIN = 2048;      // linear bins of the top-k histogram
constexpr int RS_TIE_CAP = 1024;   // largest cut bin resolved by a local sort

template <int DT, int D, int HT>
__global__ __launch_bounds__(256) void k_rescore_topk(RouteParams p, int cap_pow2, int k_pow2) {
  using G = Geo<DT, D>;
  extern __shared__ uint64_t lds[];
  __shared__ float wq_s[HT * 32];
  uint64_t* sel = lds;                                                     // [k_pow2] winners
  uint64_t* tie = lds + k_pow2;                                            // [RS_TIE_CAP] cut bin
  uint32_t* okey = reinterpret_cast<uint32_t*>(lds + k_pow2 + RS_TIE_CAP);  // [cap_pow2] score keys
  __shared__ Select32Scratch sc;
  __shared__ int hist[RS_NBIN];
  __shared__ int offs[RS_NBIN];
  __shared__ uint32_t mm_tmp[16];
  __shared__ int wtmp[16];
  __shared__ int s_cnt, s_tie, s_bstar;
  const int tid = threadIdx.x, bd = blockDim.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, nw = bd >> 6;
  const int t = blockIdx.x;
  const int L = p.cand_len[t];
  const int* cand = p.cand + (size_t)t * p.cand_ld;
  const int K = p.k;
  const int nk1 = (int)(p.n_keys - 1);
  if (wave == 0)
    load_query_weights<HT>(wq_s, p.w + (size_t)t * p.H, p.qscale ? p.qscale + (size_t)t * p.H : nullptr, p.H);
  QueryFrag<DT, D, HT> f;
  load_query<DT, D, HT>(f, p.q + (size_t)t * p.H * G::RB, p.H);
  __syncthreads();
  load_query_wregs<DT, D, HT>(f, wq_s);
  const int nb = (L + 31) >> 5;
  score_blocks<DT, D, HT, 3>(
      f, wave, nw, nb,
      [&](int blk, uint32_t* buf, float& sc) {
        const int i = blk * 32 + col;
        int j = cand[i < L ? i : L - 1];
        j = j < 0 ? 0 : (j > nk1 ? nk1 : j);
        load_half_row<DT, D>(buf, p.keys + (size_t)j * G::RB);
        sc = (DT == DT_E4M3) ? p.kscale[j] : 1.0f;
      },
      [&](int blk, float x) {
        const int i = blk * 32 + col;
        if (lane < 32 && i < L) {
          okey[i] = order_bits(x);
          if (p.dbg_cand_scores && i < p.dbg_cand_ld) p.dbg_cand_scores[(size_t)t * p.dbg_cand_ld + i] = x;
        }
      });
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  int* oi = p.topk_idx + (size_t)t * K;
  float* os = p.topk_score ? p.topk_score + (size_t)t * K : nullptr;
  auto comp_of = [&](int i) -> uint64_t { return ((uint64_t)okey[i] << 32) | (uint64_t)(~(uint32_t)cand[i]); };
  auto put = [&](int idx, uint64_t v) {
    oi[idx] = (int)comp_id(v);
    if (os) os[idx] = comp_score(v);
  };
  if (L <= K) {
    const int P2 = next_pow2(L > 0 ? L : 1);
    for (int i = tid; i < P2; i += bd) sel[i] = i < L ? comp_of(i) : 0ull;
    __syncthreads();
    bitonic_sort_desc(sel, P2);
    write_topk(sel, L, K, oi, os);
    return;
  }
  // ---- linear-bin histogram over [min, max] of the score keys ----
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = tid; i < L; i += bd) {
    const uint32_t v = okey[i];
    mn = v < mn ? v : mn;
    mx = v > mx ? v : mx;
  }
  block_minmax(mn, mx, mm_tmp);
  bool fallback = (mn == mx);
  ValBins bins;
  int bstar = 0, above = 0, in_bin = 0;
  if (!fallback) {
    bins = make_bins(mn, mx, RS_NBIN);
    for (int i = tid; i < RS_NBIN; i += bd) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < L; i += bd) atomicAdd(&hist[bins(okey[i])], 1);
    __syncthreads();
    // offs[b] = entries in bins above b (descending order); the bin holding the K-th
    const int per = RS_NBIN / bd;
    int sum = 0;
    for (int q = 0; q < per; ++q) sum += hist[RS_NBIN - 1 - tid * per - q];
    int tot;
    int run = block_exclusive_scan(sum, wtmp, &tot);
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
    if (tid == 0) s_tie = 0;
    __syncthreads();
    for (int i = tid; i < L; i += bd) {
      const uint32_t v = okey[i];
      const uint32_t bb = bins(v);
      if ((int)bb > bstar) sel[atomicAdd(&hist[bb], 1)] = comp_of(i);
      else if ((int)bb == bstar) tie[atomicAdd(&s_tie, 1)] = comp_of(i);
    }
    const int P2 = next_pow2(in_bin);
    __syncthreads();
    for (int i = in_bin + tid; i < P2; i += bd) tie[i] = 0ull;
    __syncthreads();
    bitonic_sort_desc(tie, P2);
    for (int r = tid; r < K - above; r += bd) put(above + r, tie[r]);
    // entries above the cut: final index = bin start + rank inside the bin
    for (int i = tid; i < above; i += bd) {
      const uint64_t v = sel[i];
      const int bb = (int)bins((uint32_t)(v >> 32));
      const int lo = offs[bb], hi = offs[bb - 1];
      int rank = 0;
      for (int j = lo; j < hi; ++j) rank += sel[j] > v;
      put(lo + rank, v);
    }
    return;
  }
  // ---- fallback: exact radix select (all keys equal, or a crowded cut bin) ----
  const uint32_t thr = radix_select32_desc(okey, L, K, sc);
  const int above_r = sc.above;
  const int need = K - above_r;
  const int n_eq = sc.hist[thr & 255u];
  __syncthreads();
  for (int i = tid; i < L; i += bd) {
    const uint32_t v = okey[i];
    if (v > thr || (v == thr && n_eq == need)) sel[atomicAdd(&s_cnt, 1)] = comp_of(i);
  }
  __syncthreads();
  if (n_eq != need) {
    // more candidates share the k-th score than slots remain: lowest positions win
    for (int i = tid; i < L; i += bd) okey[i] = (okey[i] == thr) ? ~(uint32_t)cand[i] : 0u;
    __syncthreads();
    const uint32_t t2 = radix_select32_desc(okey, L, need, sc);
    for (int i = tid; i < L; i += bd) {
      const uint32_t v = okey[i];
      if (v != 0u && v >= t2) sel[atomicAdd(&s_cnt, 1)] = ((uint64_t)thr << 32) | (uint64_t)v;
    }
    __syncthreads();
  }
  for (int i = K + tid; i < k_pow2; i += bd) sel[i] = 0ull;
  __syncthreads();
  bitonic_sort_desc(sel, k_pow2);
  write_topk(sel, K, K, oi, os);
}

template <int DT, int D, int HT>
static hipError_t launch_rescore_topk_t(const RouteParams& p, int cand_cap, hipStream_t s) {
  const int cap_pow2 = next_pow2(cand_cap);
  const int k_pow2 = next_pow2(p.k);
  const size_t lds = (size_t)(k_pow2 + RS_TIE_CAP) * sizeof(uint64_t) + (size_t)cap_pow2 * sizeof(uint32_t);
  hipError_t e = hipFuncSetAttribute((const void*)k_rescore_topk<DT, D, HT>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_rescore_topk<DT, D, HT>), dim3(p.T), dim3(256), lds, s, p, cap_pow2, k_pow2);
  return hipGetLastError();
}

hipError_t launch_rescore_topk(const RouteParams& p, int dtype, int dim, int ht, int cand_cap, hipStream_t s) {
  IVFTK_DISPATCH(launch_rescore_topk_t, dtype, dim, ht, p, cand_cap, s);
}

}  // namespace ivftk
