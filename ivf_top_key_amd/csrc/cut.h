// The cluster cut of the routed path, for one query per block.
//
// AttentionIndex, paper-daily.com explainer, "查询时怎么挑候选？": the visible
// clusters are ranked by representative score, high to low (equal scores: lower
// slot first), and whole clusters are taken in that order until the candidate
// budget left after the sinks and the open window is used up; the cluster that does
// not fit is truncated.
//
// One pass builds a histogram of the live clusters' scores (linear value bins
// between the smallest and the largest score) weighted by cluster size; a suffix
// scan finds the bin in which the running member count reaches the free budget;
// only the clusters in that bin or above are listed and sorted exactly by (score
// desc, slot asc), and prefix sums of their sizes place each cluster in the
// candidate list.  A list longer than LIST_CAP (many clusters crowded into the top
// bins, e.g. equal scores) is left to the full radix-select kernel.
#pragma once

#include "dev.h"
#include "params.h"
#include "routing.h"

namespace ivftk {

constexpr int LIST_CAP = 1024;   // clusters listed at or above the cut bin, at most
constexpr int SF_NBIN = 2048;    // value bins of the cut histogram
constexpr int SF_SLOTS = 8192;   // routed slots at most (checked when an index is created)

// Bin holding the need-th unit counted from the top bin down (hist = units per bin);
// written to *o_digit by the thread that finds it.  All threads call.
__device__ inline void find_bin_desc(const int* hist, int nbins, int need, int* wtmp, int* o_digit) {
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
        break;
      }
      acc += hist[d];
    }
  }
  __syncthreads();
}

// LDS words of one cut besides the arrays.
struct CutWords {
  int digit, cnt, nsel;
};

// Result of cut_clusters: nsel selected clusters (list[0..nsel) in rank order) whose
// first `used` members (in rank order) are candidates; nsel = -1 when the list
// would exceed `cap` (the query goes to the full kernel).
struct CutResult {
  int nsel;
  int used;
};

// Ranks and cuts the visible slots [0, cvis) of one query: slots below `split` come
// from the epoch store `ep`, the rest from the seal store; srep = the query's
// representative scores, room = free budget (> 0), cap <= LIST_CAP.
// On return (after a barrier): list[i] = (score key << 32) | ~slot of the i-th
// ranked cluster, pre[i] = members ranked before it (pre[nsel] = the listed total),
// moff[i] = its first member index (epoch store if >= 0, else the seal store at
// ~moff[i]).  hist must hold SF_NBIN ints, list LIST_CAP composites, pre LIST_CAP + 1
// and moff LIST_CAP ints; wtmp one int per wave, mm_tmp two per wave.  NT threads,
// each holding SF_SLOTS / NT slots.
template <int NT>
__device__ inline CutResult cut_clusters(const RouteParams& p, const float* srep, int cvis, int split,
                                         const StoreView& ep, int room, int cap, int* hist, uint64_t* list, int* pre,
                                         int* moff, int* wtmp, uint32_t* mm_tmp, CutWords& cw) {
  constexpr int PT = SF_SLOTS / NT;
  static_assert(SF_SLOTS % NT == 0 && NT <= 1024, "block shape");
  const int tid = threadIdx.x;
  // this thread's slots s = u * NT + tid: score order key and size (0 = dead or not
  // visible).  The loads are unconditional (slots past the visible ones read the
  // last visible slot and are masked afterwards) so that all of them are in flight
  // together.
  uint32_t ks[PT];
  int szs[PT];
  float scs[PT];
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int s = min(u * NT + tid, cvis - 1);
    szs[u] = (s < split ? ep.size : p.seal.size)[s];
    scs[u] = srep[s];
  }
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const bool vis = u * NT + tid < cvis;
    ks[u] = vis ? order_bits(scs[u]) : 0u;
    szs[u] = vis ? szs[u] : 0;
  }
  for (int i = tid; i < SF_NBIN; i += NT) hist[i] = 0;
  if (tid == 0) {
    cw.cnt = 0;
    cw.digit = 0;
    cw.nsel = 0;
  }
  // value bins over [min, max] of the live clusters' scores
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    if (szs[u] > 0) {
      mn = ks[u] < mn ? ks[u] : mn;
      mx = ks[u] > mx ? ks[u] : mx;
    }
  }
  block_minmax(mn, mx, mm_tmp);
  const ValBins bins = make_bins(mn, mx < mn ? mn : mx, SF_NBIN);
  int bn[PT];
  int mine = 0;
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    bn[u] = (int)bins(ks[u]);
    if (szs[u] > 0) {
      atomicAdd(&hist[bn[u]], szs[u]);
      mine += szs[u];
    }
  }
  int total;
  block_exclusive_scan(mine, wtmp, &total);
  // total <= room: every live cluster is taken (bin 0 and up)
  if (total > room) find_bin_desc(hist, SF_NBIN, room, wtmp, &cw.digit);
  const uint32_t cut_bin = (uint32_t)cw.digit;
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    if (szs[u] > 0 && (uint32_t)bn[u] >= cut_bin) {
      const int i = atomicAdd(&cw.cnt, 1);
      if (i < LIST_CAP) list[i] = ((uint64_t)ks[u] << 32) | (uint64_t)(~(uint32_t)(u * NT + tid));
    }
  }
  __syncthreads();
  const int cnt = cw.cnt;
  if (cnt > cap) return CutResult{-1, 0};
  if (cnt <= 64) {
    if (tid < 64) list[tid] = wave_sort_desc(tid < cnt ? list[tid] : 0ull);
    __syncthreads();
  } else {
    const int P2 = next_pow2(cnt);
    for (int i = cnt + tid; i < P2; i += NT) list[i] = 0ull;
    __syncthreads();
    bitonic_sort_desc(list, P2);
  }
  // prefix sums of member counts in rank order; pre[cnt] = total of the list
  int run = 0;
  for (int b0 = 0; b0 < cnt; b0 += NT) {
    const int i = b0 + tid;
    int sz = 0, mo = 0;
    if (i < cnt) {
      const int s = (int)comp_id(list[i]);
      const bool from_epoch = s < split;
      sz = (from_epoch ? ep.size : p.seal.size)[s];
      const int off = max((from_epoch ? ep.off : p.seal.off)[s], 0);
      mo = from_epoch ? off : ~off;
    }
    int tot;
    const int ex = block_exclusive_scan(sz, wtmp, &tot);
    if (i < cnt) {
      pre[i] = run + ex;
      moff[i] = mo;
    }
    run += tot;
    __syncthreads();
  }
  if (tid == 0) pre[cnt] = run;
  const int used = min(room, run);
  for (int i = tid; i < cnt; i += NT)
    if (pre[i] < used && (i == cnt - 1 || pre[i + 1] >= used)) cw.nsel = i + 1;
  __syncthreads();
  return CutResult{cw.nsel, used};
}

// Gather row code of the first member of ranked cluster i (see CROW_SHIFT): the
// member-ordered copy of the epoch store of epoch r, or of the seal store.
__device__ __forceinline__ uint32_t cut_row_tag(int mo, int r) {
  return mo >= 0 ? (((uint32_t)(2 + r % 3) << CROW_SHIFT) | (uint32_t)mo) : ((1u << CROW_SHIFT) | (uint32_t)~mo);
}

// Unified id of visible slot `slot` for a query of version v (see RouteParams).
__device__ __forceinline__ int unified_id(const RouteParams& p, const QVer& v, int slot) {
  return slot < v.split ? p.id_seal + (v.r % 3) * p.id_ep + slot : slot;
}

// Records the query's selected clusters (rank order) for the cluster-major
// rescoring and counts one selection per cluster id.  first[i] = the list index of
// cluster i's first candidate.  All threads call.
__device__ inline void record_selection(const RouteParams& p, const QVer& v, int t, const uint64_t* comp,
                                        const int* pre, int base_len, int nsel) {
  if (!p.cluster_major) return;
  int* sid = p.sel_id + (size_t)t * p.sel_ld;
  int* sdst = p.sel_dst + (size_t)t * p.sel_ld;
  for (int i = threadIdx.x; i < nsel; i += blockDim.x) {
    const int id = unified_id(p, v, (int)comp_id(comp[i]));
    sid[i] = id;
    sdst[i] = base_len + pre[i];
    atomicAdd(&p.pc_cnt[id], 1);
  }
  if (threadIdx.x == 0) p.n_sel[t] = nsel;
}

// LDS words of select_full besides its region.
struct FullCutShared {
  SelectScratch sc;
  int wtmp[16];
  int total, nsel;
};

// The cut of one query without a list limit: every visible cluster's composite
// (score key, ~slot) and size in LDS, a weighted radix select over the composites
// finds the cluster at which the running member count reaches the free budget, the
// selected clusters are compacted (stably), sorted and prefix-summed, and each
// candidate's gather row (CROW_*) goes to cand_row, its count to cand_len.
// lds must hold slot_pow2 composites and slot_pow2 ints (slot_pow2 >= the visible
// slots, a power of two).  All threads of the block call.
__device__ inline void select_full(const RouteParams& p, int t, int slot_pow2, uint64_t* lds, FullCutShared& sh) {
  uint64_t* comp = lds;                                   // [slot_pow2]
  int* wt = reinterpret_cast<int*>(lds + slot_pow2);      // [slot_pow2]: sizes, later prefix sums
  SelectScratch& sc = sh.sc;
  int* wtmp = sh.wtmp;
  int& s_total = sh.total;
  int& s_nsel = sh.nsel;
  const int tid = threadIdx.x, bd = blockDim.x;
  const QVer v = query_version(p, t);
  const StoreView ep = p.ep[v.r % 3];
  int* cand = p.cand + (size_t)t * p.cand_ld;
  int* crow = p.cand_row + (size_t)t * p.cand_ld;

  // sinks [0, min(S, n)) then the open window [open_lo, n); their keys are gathered
  // from the position-ordered keys
  const int n_sink = (int)(v.n < p.S ? v.n : p.S);
  const int n_open = v.n > v.open_lo ? (int)(v.n - v.open_lo) : 0;
  const int base_len = n_sink + n_open;
  for (int i = tid; i < base_len; i += bd) {
    const int pos = i < n_sink ? i : (int)(v.open_lo + (i - n_sink));
    if (p.write_cand) cand[i] = pos;
    crow[i] = pos;
  }
  if (p.dbg_version && tid == 0) {
    p.dbg_version[4 * t + 0] = v.r;
    p.dbg_version[4 * t + 1] = v.m;
    p.dbg_version[4 * t + 2] = v.cvis;
    p.dbg_version[4 * t + 3] = (int)v.open_lo;
  }
  const int room = p.budget - base_len;
  if (room <= 0 || v.cvis == 0) {
    if (tid == 0) {
      p.cand_len[t] = base_len;
      if (p.cluster_major) p.n_sel[t] = 0;
      if (p.dbg_n_order) p.dbg_n_order[t] = 0;
    }
    return;
  }

  // composites and sizes of the visible slots; empty slots get key 0
  const float* srep = p.srep + (size_t)t * p.srep_ld;
  int alive_total = 0;
  for (int s = tid; s < slot_pow2; s += bd) {
    uint64_t c = 0;
    int sz = 0;
    if (s < v.cvis) {
      sz = (s < v.split ? ep.size : p.seal.size)[s];
      if (sz > 0) c = make_comp(srep[s], (uint32_t)s);
    }
    comp[s] = c;
    wt[s] = sz;
    alive_total += sz;
  }
  int total;
  block_exclusive_scan(alive_total, wtmp, &total);
  const uint64_t thr = (total <= room) ? 1ull : radix_select_desc(comp, wt, v.cvis, room, sc);

  // stable in-place compaction of the selected clusters (comp >= thr, nonzero)
  if (tid == 0) s_nsel = 0;
  __syncthreads();
  for (int b0 = 0; b0 < v.cvis; b0 += bd) {
    const int i = b0 + tid;
    const uint64_t c = i < v.cvis ? comp[i] : 0ull;
    const int flag = (c != 0 && c >= thr) ? 1 : 0;
    int tot;
    const int ex = block_exclusive_scan(flag, wtmp, &tot);
    const int base = s_nsel;
    __syncthreads();
    if (flag) comp[base + ex] = c;
    __syncthreads();
    if (tid == 0) s_nsel = base + tot;
    __syncthreads();
  }
  const int nsel = s_nsel;
  const int P2 = next_pow2(nsel);
  for (int i = nsel + tid; i < P2; i += bd) comp[i] = 0ull;
  __syncthreads();
  bitonic_sort_desc(comp, P2);

  // prefix sums of member counts in rank order
  int chunk_base = 0;
  for (int b0 = 0; b0 < nsel; b0 += bd) {
    const int i = b0 + tid;
    int sz = 0;
    if (i < nsel) {
      const int s = (int)comp_id(comp[i]);
      sz = (s < v.split ? ep.size : p.seal.size)[s];
    }
    int tot;
    const int ex = block_exclusive_scan(sz, wtmp, &tot);
    if (i < nsel) wt[i] = chunk_base + ex;
    chunk_base += tot;
    __syncthreads();
  }
  if (tid == 0) s_total = chunk_base;
  __syncthreads();
  const int used = min(room, s_total);
  record_selection(p, v, t, comp, wt, base_len, nsel);

  // fill: candidate c -> cluster i with wt[i] <= c < wt[i+1]
  for (int c = tid; c < used; c += bd) {
    int lo = 0, hi = nsel - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (wt[mid] <= c) lo = mid; else hi = mid - 1;
    }
    const int s = (int)comp_id(comp[lo]);
    const bool from_epoch = s < v.split;
    const int off = max((from_epoch ? ep.off : p.seal.off)[s], 0);
    const int j = off + (c - wt[lo]);
    if (p.write_cand) cand[base_len + c] = (from_epoch ? ep.members : p.seal.members)[j];
    crow[base_len + c] = ((from_epoch ? 2 + v.r % 3 : 1) << CROW_SHIFT) | j;
  }
  if (p.dbg_order) {
    for (int i = tid; i < nsel && i < p.dbg_order_cap; i += bd) {
      const int s = (int)comp_id(comp[i]);
      const int sz = (s < v.split ? ep.size : p.seal.size)[s];
      p.dbg_order[(size_t)t * p.dbg_order_cap + i] = s;
      if (p.dbg_take) p.dbg_take[(size_t)t * p.dbg_order_cap + i] = min(sz, room - wt[i]);
    }
  }
  if (tid == 0) {
    p.cand_len[t] = base_len + used;
    if (p.dbg_n_order) p.dbg_n_order[t] = nsel;
  }
}


}  // namespace ivftk
