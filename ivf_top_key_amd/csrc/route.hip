// Cluster ranking, cut and candidate fill for the routed path (one block per query).
//
// AttentionIndex, paper-daily.com explainer, "查询时怎么挑候选？": clusters are
// ranked by representative score, high to low; the first few keys (sinks) and the
// open window take fixed slots; the remaining slots take every member of the
// clusters in rank order and the last cluster that does not fit is truncated.
// Ranking ties go to the lower slot id; a truncated cluster gives its lowest
// positions (members are stored in ascending position).
//
// The cut is a weighted radix select over composite keys (score bits, ~slot) with
// the cluster sizes as weights: it finds the cluster at which the running member
// count first reaches the free budget without sorting every visible cluster.  Only
// the selected clusters are sorted, and the fill writes their members with one
// binary search per candidate slot.
#include "cut.h"
#include "dev.h"
#include "launch.h"
#include "params.h"
#include "routing.h"

namespace ivftk {

// Full version (select_full in cut.h): every visible cluster in LDS, weighted radix
// select over composite keys.  Runs only for queries the fast kernel handed over
// (redo[t] = 1).
__global__ __launch_bounds__(256) void k_route_select(RouteParams p, int slot_pow2) {
  if (p.redo[blockIdx.x] == 0) return;
  extern __shared__ uint64_t lds[];
  __shared__ FullCutShared sh;
  select_full(p, blockIdx.x, slot_pow2, lds, sh);
}

// Fast version (cut_clusters in cut.h): a size-weighted value histogram finds the
// bin holding the cut and only the clusters at or above it are sorted; a query whose
// list would exceed LIST_CAP is left to the full kernel above.
constexpr int SF_THREADS = 512;       // threads per query in large batches
constexpr int SF_SMALL_BATCH = 64;    // batches this small leave most CUs idle: a block of
constexpr int SF_SMALL_THREADS = 1024;   // 1024 threads per query halves the per-thread chains

// NT threads per block; each thread holds SF_SLOTS / NT slots.
template <int NT>
__global__ __launch_bounds__(NT) void k_route_select_fast(RouteParams p) {
  __shared__ int hist[SF_NBIN];
  __shared__ uint64_t list[LIST_CAP];
  __shared__ int pre[LIST_CAP + 1];
  __shared__ int moff[LIST_CAP];   // first member index; epoch store if >= 0, else seal store at ~moff
  __shared__ int wtmp[16];
  __shared__ uint32_t mm_tmp[2 * NT / 64];
  __shared__ CutWords cw;
  const int tid = threadIdx.x, bd = NT;
  const int wave = tid >> 6, lane = tid & 63, nw = bd >> 6;
  const int t = blockIdx.x;
  const QVer v = query_version(p, t);
  const StoreView ep = p.ep[v.r % 3];
  int* cand = p.cand + (size_t)t * p.cand_ld;
  int* crow = p.cand_row + (size_t)t * p.cand_ld;
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
      p.redo[t] = 0;
      if (p.cluster_major) p.n_sel[t] = 0;
      if (p.dbg_n_order) p.dbg_n_order[t] = 0;
    }
    return;
  }
  const float* srep = p.srep + (size_t)t * p.srep_ld;
  const int cap = p.list_cap > 0 ? min(p.list_cap, LIST_CAP) : LIST_CAP;
  const CutResult cr = cut_clusters<NT>(p, srep, v.cvis, v.split, ep, room, cap, hist, list, pre, moff, wtmp, mm_tmp, cw);
  if (cr.nsel < 0) {
    if (tid == 0) p.redo[t] = 1;
    return;
  }
  const int nsel = cr.nsel, used = cr.used;
  record_selection(p, v, t, list, pre, base_len, nsel);
  // fill: one wave per selected cluster copies its first `take` members, four
  // clusters per step; the loads are unconditional (clamped inside the cluster) so
  // that all of a step's loads are in flight before its stores
  for (int i0 = wave; i0 < nsel; i0 += 4 * nw) {
    int start[4], take[4], rtag[4];
    const int* src[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int i = i0 + h * nw;
      const bool on = i < nsel;
      start[h] = on ? pre[i] : 0;
      take[h] = on ? min(pre[i + 1], used) - start[h] : 0;
      const int mo = on ? moff[i] : ~0;
      src[h] = mo >= 0 ? ep.members + mo : p.seal.members + ~mo;
      // gather row of member m: (store copy << CROW_SHIFT) | (first member index + m)
      rtag[h] = mo >= 0 ? (((2 + v.r % 3) << CROW_SHIFT) | mo) : ((1 << CROW_SHIFT) | ~mo);
    }
    const int most = max(max(take[0], take[1]), max(take[2], take[3]));
    for (int m0 = 0; m0 < most; m0 += 128) {
      if (p.write_cand) {   // positions only for the debug read-back
        int val[4][2];
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int r = 0; r < 2; ++r) val[h][r] = src[h][max(0, min(m0 + r * 64 + lane, take[h] - 1))];
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int m = m0 + r * 64 + lane;
            if (m < take[h]) cand[base_len + start[h] + m] = val[h][r];
          }
      }
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int m = m0 + r * 64 + lane;
          if (m < take[h]) crow[base_len + start[h] + m] = rtag[h] + m;
        }
    }
  }
  if (p.dbg_order) {
    for (int i = tid; i < nsel && i < p.dbg_order_cap; i += bd) {
      const int s = (int)comp_id(list[i]);
      p.dbg_order[(size_t)t * p.dbg_order_cap + i] = s;
      if (p.dbg_take) p.dbg_take[(size_t)t * p.dbg_order_cap + i] = min(pre[i + 1], used) - pre[i];
    }
  }
  if (tid == 0) {
    p.cand_len[t] = base_len + used;
    p.redo[t] = 0;
    if (p.dbg_n_order) p.dbg_n_order[t] = nsel;
  }
}

// ---------------------------------------------------------------------------
// grouping of (query, cluster) selections by cluster for the cluster-major rescoring
// ---------------------------------------------------------------------------
constexpr int CS_PAIRS = 32;   // selections per work item of the cluster-major scorer

__global__ void k_pairs_zero(RouteParams p) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < p.n_ids; i += gridDim.x * blockDim.x) p.pc_cnt[i] = 0;
}

// One block: exclusive scan of the per-id counts into pair offsets (left in pc_cnt
// as scatter cursors) and the work items (id, first pair, pairs) in id order.
__global__ __launch_bounds__(1024) void k_pairs_scan(RouteParams p) {
  __shared__ int wtmp[16];
  const int tid = threadIdx.x, bd = blockDim.x;
  const int per = (p.n_ids + bd - 1) / bd;
  const int i0 = min(tid * per, p.n_ids), i1 = min(i0 + per, p.n_ids);
  int cnt = 0, nit = 0;
  for (int i = i0; i < i1; ++i) {
    const int c = p.pc_cnt[i];
    cnt += c;
    nit += (c + CS_PAIRS - 1) / CS_PAIRS;
  }
  int tot_pairs, tot_items;
  int start = block_exclusive_scan(cnt, wtmp, &tot_pairs);
  int item = block_exclusive_scan(nit, wtmp, &tot_items);
  for (int i = i0; i < i1; ++i) {
    const int c = p.pc_cnt[i];
    for (int j = 0; j * CS_PAIRS < c; ++j, ++item) {
      if (item < p.item_cap) {
        p.item_id[item] = i;
        p.item_first[item] = start + j * CS_PAIRS;
        p.item_n[item] = min(CS_PAIRS, c - j * CS_PAIRS);
      }
    }
    p.pc_cnt[i] = start;
    start += c;
  }
  if (tid == 0) {
    p.ctr[0] = 0;
    p.ctr[1] = (int)min((int64_t)tot_items, p.item_cap);
  }
}

// One block per query: its selections go to their cluster's range of the pair arrays.
__global__ __launch_bounds__(256) void k_pairs_scatter(RouteParams p) {
  const int t = blockIdx.x;
  const int n = p.n_sel[t];
  const int* sid = p.sel_id + (size_t)t * p.sel_ld;
  const int* sdst = p.sel_dst + (size_t)t * p.sel_ld;
  const int end = p.cand_len[t];
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int id = sid[i], dst = sdst[i];
    const int nx = i + 1 < n ? sdst[i + 1] : end;
    const int pos = atomicAdd(&p.pc_cnt[id], 1);
    p.pair_t[pos] = t;
    p.pair_dst[pos] = dst;
    p.pair_take[pos] = nx - dst;
  }
}

hipError_t launch_pairs_zero(const RouteParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_pairs_zero, dim3((p.n_ids + 1023) / 1024), dim3(1024), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_pairs_group(const RouteParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_pairs_scan, dim3(1), dim3(1024), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_pairs_scatter, dim3(p.T), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_route_select(const RouteParams& p, int max_slots, hipStream_t s) {
  if (p.T <= SF_SMALL_BATCH)
    hipLaunchKernelGGL(k_route_select_fast<SF_SMALL_THREADS>, dim3(p.T), dim3(SF_SMALL_THREADS), 0, s, p);
  else
    hipLaunchKernelGGL(k_route_select_fast<SF_THREADS>, dim3(p.T), dim3(SF_THREADS), 0, s, p);
  hipError_t e0 = hipGetLastError();
  if (e0 != hipSuccess) return e0;
  const int slot_pow2 = next_pow2(max_slots > 0 ? max_slots : 1);
  const size_t lds = (size_t)slot_pow2 * (sizeof(uint64_t) + sizeof(int));
  hipError_t e = hipFuncSetAttribute((const void*)k_route_select, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_route_select, dim3(p.T), dim3(256), lds, s, p, slot_pow2);
  return hipGetLastError();
}

}  // namespace ivftk
