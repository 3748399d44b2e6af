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
#include "dev.h"
#include "launch.h"
#include "params.h"

namespace ivftk {

struct QV {
  int64_t n;
  int m, r, split, cvis;
  int64_t open_lo;
};

__device__ __forceinline__ QV qversion(const RouteParams& p, int t) {
  QV v;
  v.n = (p.qpos ? p.qpos[t] : p.q_pos0 + t) + 1;
  v.m = v.n >= p.S ? (int)((v.n - p.S) / p.W) : 0;
  v.r = p.wpr ? min(p.P, v.m / p.wpr) : 0;
  v.split = v.r * p.wpr * p.Cs;
  v.cvis = v.m * p.Cs;
  v.open_lo = (int64_t)p.S + (int64_t)v.m * p.W;
  return v;
}

// Unified id of visible slot `slot` for a query of version v (see RouteParams).
__device__ __forceinline__ int unified_id(const RouteParams& p, const QV& v, int slot) {
  return slot < v.split ? p.id_seal + (v.r % 3) * p.id_ep + slot : slot;
}

// Records the query's selected clusters (rank order) for the cluster-major
// rescoring and counts one selection per cluster id.  first[i] = the list index of
// cluster i's first candidate.  All threads call.
__device__ inline void record_selection(const RouteParams& p, const QV& v, int t, const uint64_t* comp,
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

// Full version: every visible cluster in LDS, weighted radix select over composite
// keys.  Runs only for queries the fast kernel handed over (redo[t] = 1).
__global__ __launch_bounds__(256) void k_route_select(RouteParams p, int slot_pow2) {
  if (p.redo[blockIdx.x] == 0) return;
  extern __shared__ uint64_t lds[];
  uint64_t* comp = lds;                                   // [slot_pow2]
  int* wt = reinterpret_cast<int*>(lds + slot_pow2);      // [slot_pow2]: sizes, later prefix sums
  __shared__ SelectScratch sc;
  __shared__ int wtmp[16];
  __shared__ int s_total, s_nsel;
  const int tid = threadIdx.x, bd = blockDim.x;
  const int t = blockIdx.x;
  const QV v = qversion(p, t);
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

// Fast version: one pass builds a 4096-bin histogram of the live clusters' score
// keys (linear bins between the smallest and largest key), weighted by cluster
// size; the bin holding the cut is found by a suffix scan, and only clusters in
// that bin or above (the selected ones plus the cut bin's other members) are
// gathered and sorted exactly.  If that list would exceed LIST_CAP the query is
// left to the full kernel.
constexpr int LIST_CAP = 1024;
constexpr int SF_NBIN = 2048;   // value bins of the cluster-cut histogram

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

constexpr int SF_SLOTS = 8192;        // routed slots at most (checked when an index is created)
constexpr int SF_THREADS = 512;       // threads per query in large batches
constexpr int SF_SMALL_BATCH = 64;    // batches this small leave most CUs idle: a block of
constexpr int SF_SMALL_THREADS = 1024;   // 1024 threads per query halves the per-thread chains

// NT threads per block; each thread holds SF_SLOTS / NT slots.
template <int NT>
__global__ __launch_bounds__(NT) void k_route_select_fast(RouteParams p) {
  constexpr int SF_PT = SF_SLOTS / NT;
  static_assert(SF_SLOTS % NT == 0 && NT <= 1024, "block shape");
  __shared__ int hist[SF_NBIN];
  __shared__ uint64_t list[LIST_CAP];
  __shared__ int pre[LIST_CAP + 1];
  __shared__ int moff[LIST_CAP];   // first member index; epoch store if >= 0, else seal store at ~moff
  __shared__ int wtmp[16];
  __shared__ uint32_t mm_tmp[2 * NT / 64];
  __shared__ int s_digit, s_cnt, s_nsel;
  const int tid = threadIdx.x, bd = NT;
  const int wave = tid >> 6, lane = tid & 63, nw = bd >> 6;
  const int t = blockIdx.x;
  const QV v = qversion(p, t);
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
  // this thread's slots s = u * bd + tid: score order key and size (0 = dead or not
  // visible).  The loads are unconditional (slots past the visible ones read the
  // last visible slot and are masked afterwards) so that all of them are in flight
  // together.
  uint32_t ks[SF_PT];
  int szs[SF_PT];
  float scs[SF_PT];
#pragma unroll
  for (int u = 0; u < SF_PT; ++u) {
    const int s = min(u * bd + tid, v.cvis - 1);
    szs[u] = (s < v.split ? ep.size : p.seal.size)[s];
    scs[u] = srep[s];
  }
#pragma unroll
  for (int u = 0; u < SF_PT; ++u) {
    const bool vis = u * bd + tid < v.cvis;
    ks[u] = vis ? order_bits(scs[u]) : 0u;
    szs[u] = vis ? szs[u] : 0;
  }
  for (int i = tid; i < SF_NBIN; i += bd) hist[i] = 0;
  if (tid == 0) {
    s_cnt = 0;
    s_digit = 0;
    s_nsel = 0;
  }
  // value bins over [min, max] of the live clusters' scores
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int u = 0; u < SF_PT; ++u) {
    if (szs[u] > 0) {
      mn = ks[u] < mn ? ks[u] : mn;
      mx = ks[u] > mx ? ks[u] : mx;
    }
  }
  block_minmax(mn, mx, mm_tmp);
  const ValBins bins = make_bins(mn, mx < mn ? mn : mx, SF_NBIN);
  int bn[SF_PT];
  int mine = 0;
#pragma unroll
  for (int u = 0; u < SF_PT; ++u) {
    bn[u] = (int)bins(ks[u]);
    if (szs[u] > 0) {
      atomicAdd(&hist[bn[u]], szs[u]);
      mine += szs[u];
    }
  }
  int total;
  block_exclusive_scan(mine, wtmp, &total);
  // total <= room: every live cluster is taken (bin 0 and up)
  if (total > room) find_bin_desc(hist, SF_NBIN, room, wtmp, &s_digit);
  const uint32_t cut_bin = (uint32_t)s_digit;
#pragma unroll
  for (int u = 0; u < SF_PT; ++u) {
    if (szs[u] > 0 && (uint32_t)bn[u] >= cut_bin) {
      const int i = atomicAdd(&s_cnt, 1);
      if (i < LIST_CAP) list[i] = ((uint64_t)ks[u] << 32) | (uint64_t)(~(uint32_t)(u * bd + tid));
    }
  }
  __syncthreads();
  const int cnt = s_cnt;
  if (cnt > (p.list_cap > 0 ? min(p.list_cap, LIST_CAP) : LIST_CAP)) {
    if (tid == 0) p.redo[t] = 1;
    return;
  }
  if (cnt <= 64) {
    if (tid < 64) list[tid] = wave_sort_desc(tid < cnt ? list[tid] : 0ull);
    __syncthreads();
  } else {
    const int P2 = next_pow2(cnt);
    for (int i = cnt + tid; i < P2; i += bd) list[i] = 0ull;
    __syncthreads();
    bitonic_sort_desc(list, P2);
  }
  // prefix sums of member counts in rank order; pre[cnt] = total of the list
  int run = 0;
  for (int b0 = 0; b0 < cnt; b0 += bd) {
    const int i = b0 + tid;
    int sz = 0, mo = 0;
    if (i < cnt) {
      const int s = (int)comp_id(list[i]);
      const bool from_epoch = s < v.split;
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
  for (int i = tid; i < cnt; i += bd)
    if (pre[i] < used && (i == cnt - 1 || pre[i + 1] >= used)) s_nsel = i + 1;
  __syncthreads();
  const int nsel = s_nsel;
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
