// Candidate rescoring and the top-k of the routed path (templates; each format's
// instantiations are compiled in a file of their own, rescore_<format>.hip).
//
// AttentionIndex, paper-daily.com explainer, "查询时怎么挑候选？": every candidate
// (sinks, the open window, the members of the selected clusters) is scored again
// with the exact indexer score and the k best are kept.  Scores come from
// score_tile (dev.h), the tile of every other scoring path, so a (query, key) pair
// gets the same fp32 bits here as on the exhaustive path.
#pragma once

#include "cut.h"
#include "dispatch.h"
#include "launch.h"
#include "params.h"
#include "routing.h"

namespace ivftk {

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

// ---------------------------------------------------------------------------
// candidate rescoring + top-k: one block per query
// ---------------------------------------------------------------------------
// The candidates' scores go to LDS as 32-bit order keys while the waves gather
// and score key rows (ring of row loads in flight per wave).  Then every thread
// takes its PT keys and candidate row codes into registers, which frees the LDS
// for the selection: a value-binned histogram between the block's min and max
// score finds the bin holding the k-th score; entries in higher bins are placed by
// bin offset plus rank inside their bin, the cut bin is sorted exactly.  Ties at
// the k-th score go to the lowest positions; the k winners come out sorted by
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

// The cut kernel's histogram and cluster list, which the fused kernel keeps in the
// selection region before the scores arrive.
constexpr size_t CUT_REGION_BYTES = (size_t)SF_NBIN * 4 + (size_t)LIST_CAP * 8;

// LDS words of the top-k selection besides its region.
template <int NT>
struct SelWords {
  Select32Scratch sc;
  uint32_t mm_tmp[2 * NT / 64];
  int wtmp[16];
  int cnt, tie, bstar;
};

// Entry u of a thread: groups of four consecutive list entries, 4 * ((u >> 2) * NT +
// tid) + (u & 3), so that a thread's keys and codes load with 16-byte loads.
template <int NT>
__device__ __forceinline__ int sel_entry(int u) {
  return 4 * ((u >> 2) * NT + (int)threadIdx.x) + (u & 3);
}

// Gather row code (CROW_*) -> key position: source 0 rows are positions, a store
// copy's row j holds that store's member j (the seal store, or the epoch store of the
// query's epoch).  Every lane loads (source 0 reads a valid dummy word and drops it).
struct PosMap {
  const int* mem0;   // the dummy word; the members of source s sit at mem0 + d_s bytes
  int64_t d1, d2;
  int jmax;
  __device__ __forceinline__ const int* addr(uint32_t code) const {
    const int src = (int)(code >> CROW_SHIFT);
    const int64_t m1 = -(int64_t)(src == 1), m2 = -(int64_t)(src >= 2);
    const int* mb = reinterpret_cast<const int*>(reinterpret_cast<const uint8_t*>(mem0) + ((d1 & m1) | (d2 & m2)));
    const int j = (int)(code & (uint32_t)CROW_MASK);
    return mb + (src == 0 ? 0 : (j < jmax ? j : jmax));
  }
  __device__ __forceinline__ uint32_t position(uint32_t code, int loaded) const {
    return (code >> CROW_SHIFT) == 0 ? (code & (uint32_t)CROW_MASK) : (uint32_t)loaded;
  }
};

__device__ __forceinline__ PosMap pos_map(const RouteParams& p, int t) {
  const QVer qv = query_version(p, t);
  const int e = qv.r % 3;
  PosMap m;
  m.mem0 = p.cand_len + t;
  const int* mem2 = e == 0 ? p.ep[0].members : (e == 1 ? p.ep[1].members : p.ep[2].members);
  m.d1 = (int64_t)(uintptr_t)p.seal.members - (int64_t)(uintptr_t)m.mem0;
  m.d2 = (int64_t)(uintptr_t)mem2 - (int64_t)(uintptr_t)m.mem0;
  m.jmax = (int)max((int64_t)0, p.n_keys - 1 - p.S);
  return m;
}

constexpr int POS_BATCH = 8;   // positions one thread resolves with its loads in flight together

// The code source of an eager selection (the codes arrive in cv).
struct NoCodes {
  __device__ void operator()(const int (&)[POS_BATCH], uint32_t (&)[POS_BATCH]) const {}
};

// Top-k of one query's L scored candidates held in registers: kv[u] = the order key
// of entry sel_entry(u)'s score; entries >= L are ignored.  The k winners by (score
// desc, position asc) go to topk_idx / topk_score.  lds = the selection region (free
// on entry after a barrier that follows every thread's last read of it).  All NT
// threads call.
// Eager (LAZY = false): cv[u] = entry u's gather row code; every entry's position is
// resolved first.  LAZY: codes(idx, code) gives the codes of POS_BATCH list entries;
// the entries are binned and placed by their list index, and only those that can win
// (the bins at and above the one holding the k-th score: about k of the L) are then
// resolved to positions, as a dense list that every lane of the block shares.
template <int PT, int NT, bool LAZY, class Codes>
__device__ __forceinline__ void topk_select(const RouteParams& p, int t, int L, int k_pow2, uint32_t (&kv)[PT],
                                            uint32_t (&cv)[PT], Codes codes, uint64_t* lds, SelWords<NT>& sw) {
  constexpr int KPT = 4096 / NT;   // winners per thread at the largest k
  static_assert(RS_NBIN % NT == 0 && NT % 64 == 0 && NT <= 1024, "block shape");
  uint32_t* okey = reinterpret_cast<uint32_t*>(lds);   // fallback: [L] score keys
  uint64_t* sel = lds;                                 // [k_pow2] winners
  uint64_t* tie = lds + k_pow2;                        // [RS_TIE_CAP] cut bin
  int* hist = reinterpret_cast<int*>(lds + k_pow2 + RS_TIE_CAP);   // [RS_NBIN]
  int* offs = hist + RS_NBIN;                                      // [RS_NBIN]
  const int tid = threadIdx.x, bd = NT;
  const int K = p.k;
  const PosMap pm = pos_map(p, t);
  // positions of every entry, POS_BATCH at a time with their loads in flight together
  auto resolve_all = [&]() {
    if constexpr (LAZY) {
#pragma unroll
      for (int u0 = 0; u0 < PT; u0 += POS_BATCH) {
        int idx[POS_BATCH];
        uint32_t code[POS_BATCH];
#pragma unroll
        for (int c = 0; c < POS_BATCH; ++c) idx[c] = min(sel_entry<NT>(u0 + c), max(L - 1, 0));
        codes(idx, code);
#pragma unroll
        for (int c = 0; c < POS_BATCH; ++c) cv[u0 + c] = code[c];
      }
    }
    int mv[PT];
#pragma unroll
    for (int u = 0; u < PT; ++u) mv[u] = *pm.addr(cv[u]);
#pragma unroll
    for (int u = 0; u < PT; ++u) cv[u] = pm.position(cv[u], mv[u]);
  };
  // LAZY: arr[0..n) hold (score key << 32) | list index; the low word becomes ~position
  auto resolve_dense = [&](uint64_t* arr, int n) {
    for (int b0 = 0; b0 < n; b0 += NT * POS_BATCH) {
      uint64_t v[POS_BATCH];
      int idx[POS_BATCH];
      uint32_t code[POS_BATCH];
#pragma unroll
      for (int c = 0; c < POS_BATCH; ++c) {
        const int a = b0 + c * NT + tid;
        v[c] = a < n ? arr[a] : 0ull;
        idx[c] = a < n ? (int)(uint32_t)v[c] : 0;
      }
      codes(idx, code);
      int mv[POS_BATCH];
#pragma unroll
      for (int c = 0; c < POS_BATCH; ++c) mv[c] = *pm.addr(code[c]);
#pragma unroll
      for (int c = 0; c < POS_BATCH; ++c) {
        const int a = b0 + c * NT + tid;
        if (a < n) arr[a] = (v[c] & 0xFFFFFFFF00000000ull) | (uint64_t)(~pm.position(code[c], mv[c]));
      }
    }
  };
  if constexpr (!LAZY) resolve_all();
  // the low word of a placed entry: ~position, or (LAZY) the list index until resolved
  auto low = [&](int u) -> uint32_t {
    if constexpr (LAZY) return (uint32_t)sel_entry<NT>(u);
    else return ~cv[u];
  };
  if (tid == 0) {
    sw.cnt = 0;
    sw.tie = 0;
  }
  __syncthreads();   // the LDS region is free from here on
  int* oi = p.topk_idx + (size_t)t * K;
  float* os = p.topk_score ? p.topk_score + (size_t)t * K : nullptr;
  auto comp = [](uint32_t key, uint32_t pos) -> uint64_t { return ((uint64_t)key << 32) | (uint64_t)(~pos); };
  if (L <= K) {
    const int P2 = next_pow2(L > 0 ? L : 1);
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int i = sel_entry<NT>(u);
      if (i < P2) sel[i] = i < L ? (((uint64_t)kv[u] << 32) | low(u)) : 0ull;
    }
    __syncthreads();
    if constexpr (LAZY) {
      resolve_dense(sel, L);
      __syncthreads();
    }
    bitonic_sort_desc(sel, P2);
    write_topk(sel, L, K, oi, os);
    return;
  }
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    if (sel_entry<NT>(u) < L) {
      mn = kv[u] < mn ? kv[u] : mn;
      mx = kv[u] > mx ? kv[u] : mx;
    }
  }
  block_minmax(mn, mx, sw.mm_tmp);
  bool fallback = (mn == mx);
  ValBins bins;
  int bstar = 0, above = 0, in_bin = 0;
  if (!fallback) {
    bins = make_bins(mn, mx, RS_NBIN);
    for (int i = tid; i < RS_NBIN; i += bd) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PT; ++u)
      if (sel_entry<NT>(u) < L) atomicAdd(&hist[bins(kv[u])], 1);
    __syncthreads();
    // offs[b] = entries in bins above b (descending order); the bin holding the K-th
    constexpr int per = RS_NBIN / NT;
    int sum = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) sum += hist[RS_NBIN - 1 - tid * per - q];
    int tot;
    int run = block_exclusive_scan(sum, sw.wtmp, &tot);
#pragma unroll
    for (int q = 0; q < per; ++q) {
      const int bb = RS_NBIN - 1 - tid * per - q;
      const int c = hist[bb];
      offs[bb] = run;
      if (run < K && K <= run + c) sw.bstar = bb;
      run += c;
    }
    __syncthreads();
    bstar = sw.bstar;
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
      if (sel_entry<NT>(u) < L) {
        const int bb = (int)bins(kv[u]);
        const uint64_t v = ((uint64_t)kv[u] << 32) | low(u);
        if (bb > bstar) sel[atomicAdd(&hist[bb], 1)] = v;
        else if (bb == bstar) tie[atomicAdd(&sw.tie, 1)] = v;
      }
    }
    const int P2 = next_pow2(in_bin);
    __syncthreads();
    if constexpr (LAZY) {
      resolve_dense(sel, above);
      resolve_dense(tie, in_bin);
      __syncthreads();
    }
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
  if constexpr (LAZY) resolve_all();
  __syncthreads();
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int i = sel_entry<NT>(u);
    if (i < L) okey[i] = kv[u];
  }
  __syncthreads();
  const uint32_t thr = radix_select32_desc(okey, L, K, sw.sc);
  const int need = K - sw.sc.above;
  const int n_eq = sw.sc.hist[thr & 255u];
  uint32_t t2 = 0u;
  __syncthreads();
  if (n_eq != need) {
    // more candidates share the k-th score than slots remain: lowest positions win
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int i = sel_entry<NT>(u);
      if (i < L) okey[i] = (kv[u] == thr) ? ~cv[u] : 0u;
    }
    __syncthreads();
    t2 = radix_select32_desc(okey, L, need, sw.sc);
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    if (sel_entry<NT>(u) < L) {
      const uint32_t v = kv[u];
      if (v > thr || (v == thr && (n_eq == need || ~cv[u] >= t2))) sel[atomicAdd(&sw.cnt, 1)] = comp(v, cv[u]);
    }
  }
  __syncthreads();
  for (int i = K + tid; i < k_pow2; i += bd) sel[i] = 0ull;
  __syncthreads();
  bitonic_sort_desc(sel, k_pow2);
  write_topk(sel, K, K, oi, os);
}

// Candidate list through memory: the cut kernel (route.hip) wrote each candidate's
// gather row code to cand_row.  NT threads per block.  With NT = RS_SEL_THREADS the
// block only selects: every candidate was scored into sbuf beforehand (small
// batches), and the selection's per-thread chains are a quarter as long, which is
// what a lone query waits on.  lds = the selection region; wq_s holds HT * 32 floats.
// All threads of the block call.
template <int DT, int D, int HT, int PT, int NT>
__device__ inline void rescore_query(const RouteParams& p, int t, int k_pow2, uint64_t* lds, float* wq_s,
                                     SelWords<NT>& sw) {
  using G = Geo<DT, D>;
  constexpr bool SELECT_ONLY = NT != RS_THREADS;
  uint32_t* okey = reinterpret_cast<uint32_t*>(lds);   // scoring: [L] score keys
  const int tid = threadIdx.x, bd = NT;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, nw = bd >> 6;
  const int L = p.cand_len[t];
  const int* cand = p.cand_row + (size_t)t * p.cand_ld;   // gather rows; positions derived below
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
  // this thread's entries with their score keys and row codes (16-byte loads)
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
      const int i = sel_entry<NT>(u);
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
  topk_select<PT, NT, false>(p, t, L, k_pow2, kv, cv, NoCodes{}, lds, sw);
}

template <int DT, int D, int HT, int PT, int NT>
__global__ __launch_bounds__(NT) void k_rescore_topk(RouteParams p, int k_pow2) {
  extern __shared__ uint64_t lds[];
  __shared__ float wq_s[HT * 32];
  __shared__ SelWords<NT> sw;
  rescore_query<DT, D, HT, PT, NT>(p, blockIdx.x, k_pow2, lds, wq_s, sw);
}

// ---------------------------------------------------------------------------
// cut + rescoring + top-k in one block per query (query-major batches)
// ---------------------------------------------------------------------------
// The cut of cut.h runs first, with its histogram and cluster list in the
// selection region; it leaves the ranked clusters' prefix sums in LDS, and the
// gather row code of candidate i follows from them: the sinks [0, n_sink), the open
// window, then the members of the ranked clusters in order (cluster s's member c at
// list index base_len + pre[s] + c is row seg[s] + pre[s] + c of its store's
// member-ordered copy).  No candidate list goes through memory.  A query whose
// cluster list overflows is appended to the overflow list (ovf) and left to
// k_route_overflow, which runs after this kernel.
//
// Largest s < n with pre[s] <= c (pre ascending, pre[0] = 0 <= c, n >= 1).
__device__ __forceinline__ int seg_search(const int* pre, int n, int c) {
  int s = 0;
  for (int step = 1 << (31 - __builtin_clz((unsigned)n)); step > 0; step >>= 1)
    if (s + step < n && pre[s + step] <= c) s += step;
  return s;
}

template <int DT, int D, int HT, int PT>
__global__ __launch_bounds__(RS_THREADS) void k_route_rescore(RouteParams p, int k_pow2) {
  using G = Geo<DT, D>;
  constexpr int NT = RS_THREADS;
  extern __shared__ uint64_t lds[];
  __shared__ float wq_s[HT * 32];
  __shared__ SelWords<NT> sw;
  __shared__ CutWords cw;
  __shared__ int pre[LIST_CAP + 1];
  __shared__ uint32_t seg[LIST_CAP];   // first member's row code of ranked cluster s, minus pre[s]
  uint32_t* okey = reinterpret_cast<uint32_t*>(lds);   // scoring: [L] score keys
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31, nw = NT >> 6;
  const int t = blockIdx.x;
  const QVer qv = query_version(p, t);
  const StoreView ep = epoch_store(p, qv.r);
  const int n_sink = (int)(qv.n < p.S ? qv.n : p.S);
  const int n_open = qv.n > qv.open_lo ? (int)(qv.n - qv.open_lo) : 0;
  const int base_len = n_sink + n_open;
  const uint32_t open_d = (uint32_t)(qv.open_lo - n_sink);   // open-window entry i: position open_d + i
  if (wave == 0)
    load_query_weights<HT>(wq_s, p.w + (size_t)t * p.H, p.qscale ? p.qscale + (size_t)t * p.H : nullptr, p.H);
  if (p.dbg_version && tid == 0) {
    p.dbg_version[4 * t + 0] = qv.r;
    p.dbg_version[4 * t + 1] = qv.m;
    p.dbg_version[4 * t + 2] = qv.cvis;
    p.dbg_version[4 * t + 3] = (int)qv.open_lo;
  }
  const int room = p.budget - base_len;
  int nsel = 0, used = 0;
  if (room > 0 && qv.cvis > 0) {
    int* hist = reinterpret_cast<int*>(lds);
    uint64_t* list = lds + SF_NBIN / 2;
    const int cap = p.list_cap > 0 ? min(p.list_cap, LIST_CAP) : LIST_CAP;
    const CutResult cr = cut_clusters<NT>(p, p.srep + (size_t)t * p.srep_ld, qv.cvis, qv.split, ep, room, cap, hist,
                                          list, pre, reinterpret_cast<int*>(seg), sw.wtmp, sw.mm_tmp, cw);
    if (cr.nsel < 0) {
      if (tid == 0) p.ovf[2 + atomicAdd(&p.ovf[0], 1)] = t;
      return;
    }
    nsel = cr.nsel;
    used = cr.used;
    if (p.dbg_order) {
      for (int i = tid; i < nsel && i < p.dbg_order_cap; i += NT) {
        p.dbg_order[(size_t)t * p.dbg_order_cap + i] = (int)comp_id(list[i]);
        if (p.dbg_take) p.dbg_take[(size_t)t * p.dbg_order_cap + i] = min(pre[i + 1], used) - pre[i];
      }
    }
    for (int i = tid; i < nsel; i += NT) seg[i] = cut_row_tag((int)seg[i], qv.r) - (uint32_t)pre[i];
  }
  const int L = base_len + used;
  if (tid == 0) {
    p.cand_len[t] = L;
    if (p.dbg_n_order) p.dbg_n_order[t] = nsel;
  }
  __syncthreads();   // seg is complete; the histogram and the list are no longer read
  // row code of list entry i < L; s = the cluster of the previous entry looked up by
  // this lane (entries are looked up in ascending order), updated
  auto code_at = [&](int i, int& s) -> uint32_t {
    if (i < base_len) return i < n_sink ? (uint32_t)i : open_d + (uint32_t)i;
    const int c = i - base_len;
    while (s + 1 < nsel && pre[s + 1] <= c) ++s;
    return seg[s] + (uint32_t)c;
  };
  if (p.write_cand) {   // positions for the debug read-back
    int* cand = p.cand + (size_t)t * p.cand_ld;
    for (int i = tid; i < L; i += NT) {
      int s = i >= base_len ? seg_search(pre, nsel, i - base_len) : 0;
      const uint32_t code = code_at(i, s);
      const int src = (int)(code >> CROW_SHIFT), j = (int)(code & (uint32_t)CROW_MASK);
      cand[i] = src == 0 ? j : (src == 1 ? p.seal.members : ep.members)[j];
    }
  }
  {
    const int nk1 = (int)(p.n_keys - 1);
    QueryFrag<DT, D, HT> f;
    load_query<DT, D, HT>(f, p.q + (size_t)t * p.H * G::RB, p.H);
    load_query_wregs<DT, D, HT>(f, wq_s);
    const RowSources rs = row_sources(p, qv.r);
    constexpr int RING = PT <= 32 ? 2 : 3;
    int cur = 0;
    score_gather<DT, D, HT, RING>(
        f, wave, nw, (L + 31) >> 5,
        [&](int blk) -> int {
          const int i = blk * 32 + col;
          return (int)code_at(i < L ? i : L - 1, cur);
        },
        [rs, nk1](int code, uint32_t* buf, float& scl) { load_cand_row<DT, D>(rs, code, nk1, buf, scl); },
        [&](int blk, float x) {
          const int i = blk * 32 + col;
          if (lane < 32 && i < L) {
            okey[i] = order_bits(x);
            if (p.dbg_cand_scores && i < p.dbg_cand_ld) p.dbg_cand_scores[(size_t)t * p.dbg_cand_ld + i] = x;
          }
        });
  }
  __syncthreads();
  uint32_t kv[PT];
  uint32_t cv[PT];   // written by the selection where it needs every entry's position
#pragma unroll
  for (int u4 = 0; u4 < PT / 4; ++u4) {
    const int i0 = 4 * (u4 * NT + tid);
    if (i0 + 3 < L) {
      const uint4 k4 = *reinterpret_cast<const uint4*>(okey + i0);
      kv[4 * u4 + 0] = k4.x;
      kv[4 * u4 + 1] = k4.y;
      kv[4 * u4 + 2] = k4.z;
      kv[4 * u4 + 3] = k4.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) kv[4 * u4 + e] = i0 + e < L ? okey[i0 + e] : 0u;
    }
  }
  // row codes of POS_BATCH list entries (each < L): the sinks and the open window
  // directly, cluster members through a binary search over the prefix sums, the
  // batch's searches stepping together
  auto codes = [&](const int (&idx)[POS_BATCH], uint32_t (&code)[POS_BATCH]) {
    int sx[POS_BATCH];
#pragma unroll
    for (int c = 0; c < POS_BATCH; ++c) sx[c] = 0;
    if (nsel > 0) {
      for (int step = 1 << (31 - __builtin_clz((unsigned)nsel)); step > 0; step >>= 1) {
#pragma unroll
        for (int c = 0; c < POS_BATCH; ++c) {
          const int cc = idx[c] - base_len;
          if (cc >= 0 && sx[c] + step < nsel && pre[sx[c] + step] <= cc) sx[c] += step;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < POS_BATCH; ++c) {
      const int i = idx[c];
      code[c] = i < base_len ? (i < n_sink ? (uint32_t)i : open_d + (uint32_t)i) : seg[sx[c]] + (uint32_t)(i - base_len);
    }
  };
  topk_select<PT, NT, true>(p, t, L, k_pow2, kv, cv, codes, lds, sw);
}

// The queries k_route_rescore appended to the overflow list: the full cut
// (select_full, candidate rows through memory) and then the list-based rescoring,
// one query at a time per block, blocks striding over the list.  The block that
// finishes last clears the list for the next call.
constexpr int OVF_BLOCKS = 256;

template <int DT, int D, int HT, int PT>
__global__ __launch_bounds__(RS_THREADS) void k_route_overflow(RouteParams p, int slot_pow2, int k_pow2) {
  extern __shared__ uint64_t lds[];   // the full cut's composites and sizes, then the selection region
  __shared__ FullCutShared fc;
  __shared__ float wq_s[HT * 32];
  __shared__ SelWords<RS_THREADS> sw;
  __shared__ int s_n;
  if (threadIdx.x == 0) s_n = __hip_atomic_load(&p.ovf[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int n = s_n;
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const int t = p.ovf[2 + i];
    select_full(p, t, slot_pow2, lds, fc);
    __syncthreads();   // the candidate rows and count are written
    rescore_query<DT, D, HT, PT, RS_THREADS>(p, t, k_pow2, lds, wq_s, sw);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    __threadfence();
    if (atomicAdd(&p.ovf[1], 1) == (int)gridDim.x - 1) {
      p.ovf[0] = 0;
      p.ovf[1] = 0;
    }
  }
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

// LDS region of the fused kernel: the selection region, at least the cut's.
__host__ __device__ constexpr size_t route_rescore_region_bytes(int cap_pow2, int k_pow2) {
  return rescore_region_bytes(cap_pow2, k_pow2) > CUT_REGION_BYTES ? rescore_region_bytes(cap_pow2, k_pow2)
                                                                    : CUT_REGION_BYTES;
}

template <int DT, int D, int HT, int PT>
static hipError_t launch_route_rescore_pt(const RouteParams& p, int cap_pow2, int k_pow2, hipStream_t s) {
  const size_t lds = route_rescore_region_bytes(cap_pow2, k_pow2);
  hipError_t e = hipFuncSetAttribute((const void*)k_route_rescore<DT, D, HT, PT>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_route_rescore<DT, D, HT, PT>), dim3(p.T), dim3(RS_THREADS), lds, s, p, k_pow2);
  return hipGetLastError();
}

template <int DT, int D, int HT>
static hipError_t launch_route_rescore_t(const RouteParams& p, int cand_cap, hipStream_t s) {
  const int cap_pow2 = next_pow2(cand_cap);
  const int k_pow2 = next_pow2(p.k);
  // at 64 entries per thread the cut's registers on top of the selection's leave one
  // wave per SIMD; such lists take the two-kernel path (route_rescore_max_cands)
  if (cap_pow2 <= 32 * RS_THREADS) return launch_route_rescore_pt<DT, D, HT, 32>(p, cap_pow2, k_pow2, s);
  return hipErrorInvalidValue;
}

template <int DT, int D, int HT>
static hipError_t launch_route_overflow_t(const RouteParams& p, int cand_cap, int max_slots, hipStream_t s) {
  const int cap_pow2 = next_pow2(cand_cap);
  const int k_pow2 = next_pow2(p.k);
  const int slot_pow2 = next_pow2(max_slots > 0 ? max_slots : 1);
  if (cap_pow2 > 32 * RS_THREADS) return hipErrorInvalidValue;
  const size_t cut = (size_t)slot_pow2 * (sizeof(uint64_t) + sizeof(int));
  const size_t sel = rescore_region_bytes(cap_pow2, k_pow2);
  const size_t lds = cut > sel ? cut : sel;
  hipError_t e = hipFuncSetAttribute((const void*)k_route_overflow<DT, D, HT, 32>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_route_overflow<DT, D, HT, 32>), dim3(OVF_BLOCKS), dim3(RS_THREADS), lds, s, p, slot_pow2,
                     k_pow2);
  return hipGetLastError();
}

// The launchers of one format (defined in rescore_<format>.hip).
#define IVFTK_RESCORE_LAUNCHERS(SUF, DISPATCH)                                                              \
  hipError_t launch_cand_score_##SUF(const RouteParams& p, int dim, int ht, int cand_cap, hipStream_t s) {   \
    DISPATCH(launch_cand_score_t, dim, ht, p, cand_cap, s)                                                  \
    return hipErrorInvalidValue;                                                                            \
  }                                                                                                         \
  hipError_t launch_rescore_topk_##SUF(const RouteParams& p, int dim, int ht, int cand_cap, hipStream_t s) { \
    DISPATCH(launch_rescore_topk_t, dim, ht, p, cand_cap, s)                                                \
    return hipErrorInvalidValue;                                                                            \
  }                                                                                                         \
  hipError_t launch_route_rescore_##SUF(const RouteParams& p, int dim, int ht, int cand_cap, hipStream_t s) { \
    DISPATCH(launch_route_rescore_t, dim, ht, p, cand_cap, s)                                               \
    return hipErrorInvalidValue;                                                                            \
  }                                                                                                         \
  hipError_t launch_route_overflow_##SUF(const RouteParams& p, int dim, int ht, int cand_cap, int max_slots,  \
                                         hipStream_t s) {                                                   \
    DISPATCH(launch_route_overflow_t, dim, ht, p, cand_cap, max_slots, s)                                   \
    return hipErrorInvalidValue;                                                                            \
  }

#define IVFTK_RESCORE_DECLARE(SUF)                                                                         \
  hipError_t launch_cand_score_##SUF(const RouteParams& p, int dim, int ht, int cand_cap, hipStream_t s);   \
  hipError_t launch_rescore_topk_##SUF(const RouteParams& p, int dim, int ht, int cand_cap, hipStream_t s); \
  hipError_t launch_route_rescore_##SUF(const RouteParams& p, int dim, int ht, int cand_cap, hipStream_t s);  \
  hipError_t launch_route_overflow_##SUF(const RouteParams& p, int dim, int ht, int cand_cap, int max_slots,  \
                                         hipStream_t s);

IVFTK_RESCORE_DECLARE(f32)
IVFTK_RESCORE_DECLARE(bf16)
IVFTK_RESCORE_DECLARE(e4m3)

}  // namespace ivftk
