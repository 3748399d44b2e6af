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

}  // namespace ivftk
