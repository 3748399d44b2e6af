// Host runtime behind the C ABI in include/ivftk.h: argument and state checks,
// device memory owned by an index, version bookkeeping, streams and events.
//
// Index layout in device memory (all allocated at idx_create):
//   keys [max_keys, d] in the key format, k_scale [max_keys] (E4M3);
//   seal store, one entry per sealed-window cluster, slot s = w*C + c: size, offset,
//     members (window w's keys at [w*W, (w+1)*W), grouped by cluster), fp32
//     centroid, representative and its scale;
//   three epoch stores (a ring: the published epoch, the one before it, and a refit
//     in flight) with slots [0, r*Q), members [0, r*R), centroids, representatives,
//     and the centroid drift of the epoch's update;
//   per-key bound state (assigned slot, upper and lower distance bound) and the
//     refit work list; per-tile slot counts for the stable member placement;
//   routing scratch: representative scores [max_queries, slots] and candidate
//     lists [max_queries, cand_cap].
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "ivftk.h"
#include "launch.h"

using namespace ivftk;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int elem_bytes(int dt) { return dt == IDX_F32 ? 4 : (dt == IDX_BF16 ? 2 : 1); }

bool dim_supported(int dt, int d) {
  if (dt == IDX_F32) return d == 32 || d == 64 || d == 128;
  if (dt == IDX_BF16 || dt == IDX_E4M3) return d == 64 || d == 128;
  return false;
}

int head_tiles(int H) { return H <= 32 ? 1 : (H <= 64 ? 2 : 4); }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct EpochStore {
  int* size = nullptr;
  int* off = nullptr;
  int* members = nullptr;
  float* cent = nullptr;
  float* lrep = nullptr;
  uint8_t* rep = nullptr;
  float* rsc = nullptr;
  float* drift = nullptr;
  float* drift_max = nullptr;
  uint8_t* ckeys = nullptr;   // [members, RB] keys in member order
  float* cscale = nullptr;    // [members] their scales (E4M3)
};

constexpr int TILE = 1024;
constexpr int CS_PAIRS_HOST = 32;   // selections per work item of the cluster-major scorer
constexpr size_t LDS_BYTES = 163840;

}  // namespace

// Batches of at most this many queries score their candidates with blocks that split
// each query's list (the final kernel then only selects); larger batches use one
// block per query for both.
constexpr int kSplitQueries = 64;

struct idx_index {
  idx_config cfg{};
  int device = 0;
  int Cs = 0, wpr = 0, Q = 0, RB = 0, HT = 1;
  int64_t max_windows = 0, slot_cap = 0, member_cap = 0;
  int64_t ep_slot_cap = 0, ep_member_cap = 0;
  int cand_cap = 0;
  int n_tiles_cap = 0;
  uint8_t* keys = nullptr;
  float* kscale = nullptr;
  int *sl_size = nullptr, *sl_off = nullptr, *sl_members = nullptr;
  float* sl_cent = nullptr;
  float* sl_lrep = nullptr;
  float* enc = nullptr;      // learned-representative weights (packed), used when has_enc
  bool has_enc = false;
  uint8_t* sl_rep = nullptr;
  float* sl_rsc = nullptr;
  uint8_t* sl_ckeys = nullptr;   // [member_cap, RB] sealed keys in member order
  float* sl_cscale = nullptr;    // [member_cap] their scales (E4M3)
  int* cand_row = nullptr;       // [max_queries, cand_cap] gather rows of the candidates
  EpochStore ep[3];
  int* assign = nullptr;
  float* ub = nullptr;
  float* lb = nullptr;
  int* work = nullptr;
  int* work_count = nullptr;
  int* tile_cnt = nullptr;
  uint16_t* cbf = nullptr;       // refit screening: bf16 warm centroids, norms, tile maxima
  float* cnrm = nullptr;
  unsigned* tile_cmax = nullptr;
  int* ovf = nullptr;
  int* ovf_count = nullptr;
  uint32_t* hkey = nullptr;      // refit certification: drift keys, listed slots, their count, rest drift
  int* hlist = nullptr;
  int* nlist = nullptr;
  float* rest_drift = nullptr;
  float* srep = nullptr;
  int* cand = nullptr;
  int* cand_len = nullptr;
  int* redo = nullptr;
  int* route_ovf = nullptr;      // [max_queries + 2] overflow list of the fused cut + rescoring
  int64_t* qpos = nullptr;   // positions of a decode batch (idx_route_topk_pos)
  // cluster-major rescoring: selections per query, pairs grouped by cluster, work items
  int64_t sel_cap = 0, pair_cap = 0, item_cap = 0;
  int n_ids = 0;
  int *sel_id = nullptr, *sel_dst = nullptr, *n_sel = nullptr, *pc_cnt = nullptr;
  int *pair_t = nullptr, *pair_dst = nullptr, *pair_take = nullptr;
  int *item_id = nullptr, *item_first = nullptr, *item_n = nullptr, *ctr = nullptr;
  float* sbuf = nullptr;
  std::vector<void*> allocs;
  hipStream_t fill_stream = nullptr;   // idx_create's stream: new memory is zero-filled on it
  int64_t bytes = 0;
  int64_t n_keys = 0;
  int sealed = 0;
  int computed = 0;
  int published = 0;
  int imported = 0;          // epoch installed by idx_import_version (no refit bound state)
  int lost = 0;              // newest epoch whose ring store a later refit or import reused
  hipEvent_t ev_main = nullptr, ev_refit = nullptr;
  bool poisoned = false;

  template <typename T>
  bool alloc(T** p, int64_t count) {
    *p = nullptr;
    if (count <= 0) return true;
    void* v = nullptr;
    const size_t b = (size_t)count * sizeof(T);
    if (hipMalloc(&v, b) != hipSuccess) return false;
    if (hipMemsetAsync(v, 0, b, fill_stream) != hipSuccess) {
      (void)hipFree(v);
      return false;
    }
    allocs.push_back(v);
    bytes += (int64_t)b;
    *p = static_cast<T*>(v);
    return true;
  }

  void release() {
    for (void* p : allocs) (void)hipFree(p);
    allocs.clear();
    if (ev_main) (void)hipEventDestroy(ev_main);
    if (ev_refit) (void)hipEventDestroy(ev_refit);
    ev_main = ev_refit = nullptr;
  }

  StoreView seal_view() const {
    return StoreView{sl_size, sl_off, sl_members, sl_cent, sl_rep, sl_rsc, sl_ckeys, sl_cscale};
  }
  StoreView epoch_view(int r) const {
    if (r <= 0) return StoreView{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    const EpochStore& e = ep[r % 3];
    return StoreView{e.size, e.off, e.members, e.cent, e.rep, e.rsc, e.ckeys, e.cscale};
  }
};

namespace {

int device_error(idx_index* ix, hipError_t e, const char* what) {
  if (ix) ix->poisoned = true;
  return fail(IDX_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Oldest refit epoch whose store still holds it: the ring keeps three stores, and a
// refit or import of epoch r reuses the store of epoch r - 3 (also when that refit
// is later abandoned).
int oldest_held(const idx_index* ix) { return std::max(std::max(1, ix->computed - 2), ix->lost + 1); }

int check_handle(const idx_index* ix) {
  if (!ix) return fail(IDX_EINVAL, "null index handle");
  if (ix->poisoned) return fail(IDX_ESTATE, "index handle is poisoned by an earlier device error");
  return IDX_OK;
}

}  // namespace

extern "C" {

const char* idx_last_error(void) { return g_err.c_str(); }

int idx_create(const idx_config* cfg, void* stream, idx_index** out) {
  g_err.clear();
  if (!cfg || !out) return fail(IDX_EINVAL, "null config or output pointer");
  *out = nullptr;
  const idx_config c = *cfg;
  if (c.dtype < IDX_F32 || c.dtype > IDX_E4M3) return fail(IDX_EINVAL, "unknown dtype %d", c.dtype);
  if (c.heads < 1 || c.heads > 128) return fail(IDX_EINVAL, "heads must be 1..128 (got %d)", c.heads);
  if (!dim_supported(c.dtype, c.dim)) return fail(IDX_ENOTIMPL, "dim %d not built for dtype %d", c.dim, c.dtype);
  if (c.n_sink < 0) return fail(IDX_EINVAL, "n_sink must be >= 0");
  if (c.window < 2 || c.window > 1024) return fail(IDX_EINVAL, "window must be 2..1024");
  if (c.cluster_size < 1 || c.window % c.cluster_size) return fail(IDX_EINVAL, "window must be a multiple of cluster_size");
  const int Cs = c.window / c.cluster_size;
  if (Cs != 1 && Cs != 2 && Cs != 4 && Cs != 8) return fail(IDX_ENOTIMPL, "clusters per window must be 1, 2, 4 or 8 (got %d)", Cs);
  if ((int64_t)c.window * Cs > 8192) return fail(IDX_EINVAL, "window * clusters per window must be <= 8192");
  if (c.seal_cap < 1 || (int64_t)c.seal_cap * Cs < c.window) return fail(IDX_EINVAL, "seal_cap * clusters per window must be >= window");
  if (c.seal_iters < 1 || c.seal_iters > 64) return fail(IDX_EINVAL, "seal_iters must be 1..64");
  if (c.refit_every < 0 || (c.refit_every && c.refit_every % c.window)) return fail(IDX_EINVAL, "refit_every must be 0 or a multiple of window");
  if (c.max_queries < 1) return fail(IDX_EINVAL, "max_queries must be >= 1");
  if (c.max_k < 1 || c.max_k > 4096) return fail(IDX_EINVAL, "max_k must be 1..4096");
  if (c.max_budget < c.max_k) return fail(IDX_EINVAL, "max_budget must be >= max_k");
  if (c.rescore_mode < IDX_RESCORE_AUTO || c.rescore_mode > IDX_RESCORE_CLUSTER)
    return fail(IDX_EINVAL, "rescore_mode must be IDX_RESCORE_AUTO, _QUERY or _CLUSTER");
  if (c.cluster_mode != IDX_CLUSTERS_CONTENT && c.cluster_mode != IDX_CLUSTERS_POSITIONAL)
    return fail(IDX_EINVAL, "cluster_mode must be IDX_CLUSTERS_CONTENT or IDX_CLUSTERS_POSITIONAL");
  if (c.cluster_mode == IDX_CLUSTERS_POSITIONAL && c.refit_every != 0)
    return fail(IDX_EINVAL, "positional blocks are never refitted: refit_every must be 0");
  if (c.max_keys < 1 || c.max_keys > (int64_t)1 << 29) return fail(IDX_EINVAL, "max_keys must be 1..2^29");

  idx_index* ix = new (std::nothrow) idx_index();
  if (!ix) return fail(IDX_ENOMEM, "host allocation failed");
  ix->cfg = c;
  ix->fill_stream = (hipStream_t)stream;
  (void)hipGetDevice(&ix->device);
  ix->Cs = Cs;
  ix->wpr = c.refit_every ? c.refit_every / c.window : 0;
  ix->Q = ix->wpr * Cs;
  ix->RB = c.dim * elem_bytes(c.dtype);
  ix->HT = head_tiles(c.heads);
  ix->max_windows = c.max_keys > c.n_sink ? (c.max_keys - c.n_sink) / c.window : 0;
  ix->slot_cap = ix->max_windows * Cs;
  ix->member_cap = ix->max_windows * c.window;
  const int64_t max_refits = ix->wpr ? ix->max_windows / ix->wpr : 0;
  ix->ep_slot_cap = max_refits * ix->Q;
  ix->ep_member_cap = max_refits * ix->wpr * (int64_t)c.window;
  ix->cand_cap = (int)round_up(std::max<int64_t>(c.max_budget, (int64_t)c.n_sink + c.window), 32);
  ix->n_tiles_cap = (int)((ix->member_cap + TILE - 1) / TILE);
  if (ix->slot_cap > 8192) {
    const long long slots = (long long)ix->slot_cap;
    delete ix;
    return fail(IDX_ECAPACITY, "max_keys allows %lld clusters; at most 8192 are routed", slots);
  }
  if (!rescore_fits(ix->cand_cap, c.max_k)) {
    delete ix;
    return fail(IDX_ECAPACITY, "max(budget, n_sink + window) and max_k do not fit one rescoring block");
  }
  ix->sel_cap = std::min<int64_t>(ix->cand_cap, std::max<int64_t>(ix->slot_cap, 1));
  ix->pair_cap = (int64_t)c.max_queries * ix->sel_cap;
  ix->n_ids = (int)(ix->slot_cap + (ix->wpr ? 3 * ix->ep_slot_cap : 0));
  ix->item_cap = ix->pair_cap / CS_PAIRS_HOST + ix->n_ids;
  bool ok = ix->alloc(&ix->keys, c.max_keys * ix->RB) &&
            (c.dtype != IDX_E4M3 || ix->alloc(&ix->kscale, c.max_keys)) &&
            ix->alloc(&ix->sl_size, ix->slot_cap) && ix->alloc(&ix->sl_off, ix->slot_cap) &&
            ix->alloc(&ix->sl_members, ix->member_cap) && ix->alloc(&ix->sl_cent, ix->slot_cap * c.dim) &&
            ix->alloc(&ix->sl_rep, ix->slot_cap * ix->RB) && ix->alloc(&ix->sl_rsc, ix->slot_cap) &&
            ix->alloc(&ix->sl_lrep, ix->slot_cap * c.dim) && ix->alloc(&ix->enc, encoder_floats(c.dim)) &&
            ix->alloc(&ix->srep, (int64_t)c.max_queries * std::max<int64_t>(ix->slot_cap, 1)) &&
            ix->alloc(&ix->cand, (int64_t)c.max_queries * ix->cand_cap) &&
            ix->alloc(&ix->cand_row, (int64_t)c.max_queries * ix->cand_cap) &&
            ix->alloc(&ix->sl_ckeys, ix->member_cap * ix->RB) &&
            (c.dtype != IDX_E4M3 || ix->alloc(&ix->sl_cscale, ix->member_cap)) &&
            ix->alloc(&ix->cand_len, c.max_queries) && ix->alloc(&ix->redo, c.max_queries) &&
            ix->alloc(&ix->route_ovf, (int64_t)c.max_queries + 2) && ix->alloc(&ix->qpos, c.max_queries);
  if (ok && c.rescore_mode == IDX_RESCORE_CLUSTER)
    ok = ix->alloc(&ix->sel_id, (int64_t)c.max_queries * ix->sel_cap) &&
            ix->alloc(&ix->sel_dst, (int64_t)c.max_queries * ix->sel_cap) && ix->alloc(&ix->n_sel, c.max_queries) &&
            ix->alloc(&ix->pc_cnt, std::max(ix->n_ids, 1)) && ix->alloc(&ix->pair_t, ix->pair_cap) &&
            ix->alloc(&ix->pair_dst, ix->pair_cap) && ix->alloc(&ix->pair_take, ix->pair_cap) &&
            ix->alloc(&ix->item_id, ix->item_cap) && ix->alloc(&ix->item_first, ix->item_cap) &&
            ix->alloc(&ix->item_n, ix->item_cap) && ix->alloc(&ix->ctr, 2) &&
            ix->alloc(&ix->sbuf, (int64_t)c.max_queries * ix->cand_cap);
  else if (ok)
    ok = ix->alloc(&ix->sbuf, (int64_t)std::min(c.max_queries, kSplitQueries) * ix->cand_cap);
  if (ok && ix->wpr) {
    for (int i = 0; i < 3 && ok; ++i) {
      EpochStore& e = ix->ep[i];
      ok = ix->alloc(&e.size, ix->ep_slot_cap) && ix->alloc(&e.off, ix->ep_slot_cap) &&
           ix->alloc(&e.members, ix->ep_member_cap) && ix->alloc(&e.cent, ix->ep_slot_cap * c.dim) &&
           ix->alloc(&e.ckeys, ix->ep_member_cap * ix->RB) &&
           (c.dtype != IDX_E4M3 || ix->alloc(&e.cscale, ix->ep_member_cap)) &&
           ix->alloc(&e.lrep, ix->ep_slot_cap * c.dim) &&
           ix->alloc(&e.rep, ix->ep_slot_cap * ix->RB) && ix->alloc(&e.rsc, ix->ep_slot_cap) &&
           ix->alloc(&e.drift, ix->ep_slot_cap) && ix->alloc(&e.drift_max, 1);
    }
    ok = ok && ix->alloc(&ix->assign, c.max_keys) && ix->alloc(&ix->ub, c.max_keys) &&
         ix->alloc(&ix->lb, c.max_keys) && ix->alloc(&ix->work, c.max_keys) && ix->alloc(&ix->work_count, 1) &&
         ix->alloc(&ix->tile_cnt, (int64_t)ix->n_tiles_cap * std::max<int64_t>(ix->ep_slot_cap, 1)) &&
         ix->alloc(&ix->cbf, 2 * std::max<int64_t>(ix->ep_slot_cap, 1) * c.dim) &&
         ix->alloc(&ix->cnrm, std::max<int64_t>(ix->ep_slot_cap, 1)) &&
         ix->alloc(&ix->tile_cmax, std::max<int64_t>((ix->ep_slot_cap + 31) / 32, 1)) &&
         ix->alloc(&ix->ovf, c.max_keys) && ix->alloc(&ix->ovf_count, 1) &&
         ix->alloc(&ix->hkey, std::max<int64_t>(ix->ep_slot_cap, 1)) &&
         ix->alloc(&ix->hlist, std::max<int64_t>(ix->ep_slot_cap, 1)) && ix->alloc(&ix->nlist, 1) &&
         ix->alloc(&ix->rest_drift, 1);
  }
  if (!ok) {
    (void)hipStreamSynchronize(ix->fill_stream);
    ix->release();
    delete ix;
    return fail(IDX_ENOMEM, "device allocation failed");
  }
  if (hipEventCreateWithFlags(&ix->ev_main, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&ix->ev_refit, hipEventDisableTiming) != hipSuccess ||
      hipStreamSynchronize(ix->fill_stream) != hipSuccess) {
    (void)hipDeviceSynchronize();
    ix->release();
    delete ix;
    return fail(IDX_EDEVICE, "event creation or zero fill failed");
  }
  *out = ix;
  return IDX_OK;
}

int idx_destroy(idx_index* ix) {
  g_err.clear();
  if (!ix) return IDX_OK;
  (void)hipSetDevice(ix->device);
  (void)hipDeviceSynchronize();
  ix->release();
  delete ix;
  return IDX_OK;
}

int idx_get_info(const idx_index* ix, idx_info* out) {
  g_err.clear();
  if (!ix || !out) return fail(IDX_EINVAL, "null argument");
  out->n_keys = ix->n_keys;
  out->sealed_windows = ix->sealed;
  out->computed_epoch = ix->computed;
  out->published_epoch = ix->published;
  out->clusters_per_window = ix->Cs;
  out->slots_per_epoch = ix->Q;
  out->device_bytes = ix->bytes;
  return IDX_OK;
}

int idx_build_seal(idx_index* ix, const void* keys, const float* k_scale, int64_t n, void* stream) {
  g_err.clear();
  if (int e = check_handle(ix)) return e;
  const idx_config& c = ix->cfg;
  if (n < 0) return fail(IDX_EINVAL, "n must be >= 0");
  if (n == 0) return IDX_OK;
  if (!keys) return fail(IDX_EINVAL, "null keys");
  if (c.dtype == IDX_E4M3 && !k_scale) return fail(IDX_EINVAL, "E4M3 keys need k_scale");
  if (ix->n_keys + n > c.max_keys)
    return fail(IDX_ECAPACITY, "inserting %lld keys after %lld exceeds max_keys %lld", (long long)n,
                (long long)ix->n_keys, (long long)c.max_keys);
  (void)hipSetDevice(ix->device);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(ix->keys + (size_t)ix->n_keys * ix->RB, keys, (size_t)n * ix->RB,
                                hipMemcpyDefault, s);
  if (e == hipSuccess && c.dtype == IDX_E4M3)
    e = hipMemcpyAsync(ix->kscale + ix->n_keys, k_scale, (size_t)n * sizeof(float), hipMemcpyDefault, s);
  if (e != hipSuccess) return device_error(ix, e, "key copy");
  ix->n_keys += n;
  const int64_t full = ix->n_keys > c.n_sink ? (ix->n_keys - c.n_sink) / c.window : 0;
  const int new_windows = (int)(full - ix->sealed);
  if (new_windows > 0) {
    SealParams p{};
    p.keys = ix->keys;
    p.kscale = ix->kscale;
    p.S = c.n_sink;
    p.W = c.window;
    p.Cs = ix->Cs;
    p.cap = c.seal_cap;
    p.positional = c.cluster_mode == IDX_CLUSTERS_POSITIONAL;
    p.iters = p.positional ? 1 : c.seal_iters;
    p.w0 = ix->sealed;
    p.size = ix->sl_size;
    p.off = ix->sl_off;
    p.members = ix->sl_members;
    p.cent = ix->sl_cent;
    p.lrep = ix->sl_lrep;
    p.rep = ix->sl_rep;
    p.rsc = ix->sl_rsc;
    e = launch_seal(p, c.dtype, c.dim, new_windows, s);
    if (e == hipSuccess)
      e = launch_copy_member_rows(ix->sl_members, (int64_t)ix->sealed * c.window, full * (int64_t)c.window, ix->keys,
                                  ix->kscale, ix->n_keys, ix->RB, ix->sl_ckeys, ix->sl_cscale, s);
    if (e == hipSuccess && ix->has_enc) {
      EncParams ep{};
      ep.keys = ix->keys;
      ep.kscale = ix->kscale;
      ep.n_keys = ix->n_keys;
      ep.st = ix->seal_view();
      ep.w = ix->enc;
      ep.lrep = ix->sl_lrep;
      ep.rep = ix->sl_rep;
      ep.rsc = ix->sl_rsc;
      ep.slot0 = ix->sealed * ix->Cs;
      ep.n_slots = (int)(new_windows * ix->Cs);
      e = launch_encode(ep, c.dtype, c.dim, s);
    }
    if (e != hipSuccess) return device_error(ix, e, "seal launch");
    ix->sealed = (int)full;
  }
  return IDX_OK;
}

int idx_refit(idx_index* ix, void* stream, void* side_stream, int32_t* launched) {
  g_err.clear();
  if (int e = check_handle(ix)) return e;
  if (launched) *launched = 0;
  const idx_config& c = ix->cfg;
  if (!ix->wpr) return IDX_OK;
  if (ix->computed != ix->published) return IDX_OK;               // previous refit not published yet
  const int r = ix->computed + 1;
  if (ix->sealed < r * ix->wpr) return IDX_OK;                      // boundary not sealed past
  (void)hipSetDevice(ix->device);
  hipStream_t s = (hipStream_t)stream, side = (hipStream_t)side_stream;
  hipError_t e = hipEventRecord(ix->ev_main, s);
  if (e == hipSuccess) e = hipStreamWaitEvent(side, ix->ev_main, 0);
  if (e != hipSuccess) return device_error(ix, e, "refit stream ordering");
  RefitParams p{};
  p.keys = ix->keys;
  p.kscale = ix->kscale;
  p.n_keys = ix->n_keys;
  p.S = c.n_sink;
  p.r = r;
  p.Q = ix->Q;
  p.B_prev = (int64_t)c.n_sink + (int64_t)(r - 1) * c.refit_every;
  p.B_r = (int64_t)c.n_sink + (int64_t)r * c.refit_every;
  const StoreView pv = ix->epoch_view(r - 1);
  p.prev = pv;
  p.prev_drift = r >= 2 ? ix->ep[(r - 1) % 3].drift : nullptr;
  p.seal = ix->seal_view();
  p.assign = ix->assign;
  p.ub = ix->ub;
  p.lb = ix->lb;
  p.work = ix->work;
  p.work_count = ix->work_count;
  EpochStore& out = ix->ep[r % 3];
  p.size = out.size;
  p.off = out.off;
  p.members = out.members;
  p.cent = out.cent;
  p.lrep = out.lrep;
  p.rep = out.rep;
  p.rsc = out.rsc;
  p.drift = out.drift;
  p.drift_max = out.drift_max;
  p.tile_cnt = ix->tile_cnt;
  p.cbf = ix->cbf;
  p.cnrm = ix->cnrm;
  p.tile_cmax = ix->tile_cmax;
  p.ovf = ix->ovf;
  p.ovf_count = ix->ovf_count;
  p.brute_ovf = 0;
  p.hkey = ix->hkey;
  p.hlist = ix->hlist;
  p.nlist = ix->nlist;
  p.rest_drift = ix->rest_drift;
  p.tile = TILE;
  p.n_tiles = (int)((p.B_r - p.S + TILE - 1) / TILE);
  e = launch_refit(p, c.dtype, c.dim, side);
  if (e == hipSuccess)
    e = launch_copy_member_rows(out.members, 0, p.B_r - p.S, ix->keys, ix->kscale, ix->n_keys, ix->RB, out.ckeys,
                                out.cscale, side);
  if (e == hipSuccess && ix->has_enc) {
    EncParams ep{};
    ep.keys = ix->keys;
    ep.kscale = ix->kscale;
    ep.n_keys = ix->n_keys;
    ep.st = StoreView{out.size, out.off, out.members, out.cent, out.rep, out.rsc, out.ckeys, out.cscale};
    ep.w = ix->enc;
    ep.lrep = out.lrep;
    ep.rep = out.rep;
    ep.rsc = out.rsc;
    ep.slot0 = 0;
    ep.n_slots = r * ix->Q;
    e = launch_encode(ep, c.dtype, c.dim, side);
  }
  if (e == hipSuccess) e = hipEventRecord(ix->ev_refit, side);
  if (e != hipSuccess) return device_error(ix, e, "refit launch");
  ix->computed = r;
  ix->lost = std::max(ix->lost, r - 3);
  ix->imported = 0;
  if (launched) *launched = 1;
  return IDX_OK;
}

int idx_publish(idx_index* ix, void* stream, int32_t* published) {
  g_err.clear();
  if (int e = check_handle(ix)) return e;
  if (ix->computed > ix->published) {
    (void)hipSetDevice(ix->device);
    hipError_t e = hipStreamWaitEvent((hipStream_t)stream, ix->ev_refit, 0);
    if (e != hipSuccess) return device_error(ix, e, "publish wait");
    ix->published = ix->computed;
  }
  if (published) *published = ix->published;
  return IDX_OK;
}

int idx_abandon_refit(idx_index* ix, void* stream, int32_t* abandoned) {
  g_err.clear();
  if (int e = check_handle(ix)) return e;
  if (abandoned) *abandoned = 0;
  if (ix->computed == ix->published) return IDX_OK;
  (void)hipSetDevice(ix->device);
  // the store the refit writes is the one the next launch (or import) of the same
  // epoch writes again: order everything later on the main stream after it
  const hipError_t e = hipStreamWaitEvent((hipStream_t)stream, ix->ev_refit, 0);
  if (e != hipSuccess) return device_error(ix, e, "abandon wait");
  if (abandoned) *abandoned = ix->computed;
  ix->computed = ix->published;
  ix->imported = 0;
  return IDX_OK;
}

// Shared body of idx_route_topk (positions == nullptr: q_pos0 + t) and
// idx_route_topk_pos (host positions, copied to the index's device buffer).
static int route_common(idx_index* ix, const void* q, const float* q_scale, const float* w, int64_t q_pos0,
                        const int64_t* positions, int32_t T, int32_t k, int32_t budget, int32_t* topk_idx,
                        float* topk_score, const idx_route_debug* dbg, void* stream) {
  g_err.clear();
  if (int e = check_handle(ix)) return e;
  const idx_config& c = ix->cfg;
  if (!q || !w || !topk_idx) return fail(IDX_EINVAL, "null q, w or topk_idx");
  if (c.dtype == IDX_E4M3 && !q_scale) return fail(IDX_EINVAL, "E4M3 queries need q_scale");
  if (T < 1) return fail(IDX_EINVAL, "T must be >= 1");
  if (T > c.max_queries) return fail(IDX_ECAPACITY, "T %d exceeds max_queries %d", T, c.max_queries);
  if (k < 1 || k > c.max_k) return fail(IDX_ECAPACITY, "k %d outside 1..max_k %d", k, c.max_k);
  if (budget < k) return fail(IDX_EINVAL, "budget %d < k %d", budget, k);
  if (budget > c.max_budget) return fail(IDX_ECAPACITY, "budget %d exceeds max_budget %d", budget, c.max_budget);
  int64_t pmin = q_pos0, pmax = q_pos0 + T - 1;
  if (positions) {
    pmin = pmax = positions[0];
    for (int32_t t = 1; t < T; ++t) {
      pmin = std::min(pmin, positions[t]);
      pmax = std::max(pmax, positions[t]);
    }
  }
  if (pmin < 0) return fail(IDX_EINVAL, "query positions must be >= 0");
  if (pmax >= ix->n_keys)
    return fail(IDX_ECAUSAL, "query position %lld has no inserted key (%lld keys)", (long long)pmax,
                (long long)ix->n_keys);
  const int P = ix->published;
  auto windows_in = [&](int64_t n) -> int {
    return n >= c.n_sink ? (int)((n - c.n_sink) / c.window) : 0;
  };
  if (ix->wpr) {
    // epochs used by this call: r_t = min(P, m_t / wpr) is monotone in the position,
    // so the smallest position uses the oldest epoch; every epoch used must still be
    // held (the ring keeps three stores and a refit in flight overwrites the oldest)
    const int r0 = std::min(P, windows_in(pmin + 1) / ix->wpr);
    const int r1 = std::min(P, windows_in(pmax + 1) / ix->wpr);
    const int oldest = oldest_held(ix);
    const int lo = std::max(r0, 1);
    if (r1 >= 1 && lo < oldest)
      return fail(IDX_ESTATE, "queries at %lld..%lld need epoch %d; epochs below %d are no longer held",
                  (long long)pmin, (long long)pmax, lo, oldest);
  }
  (void)hipSetDevice(ix->device);
  hipStream_t s = (hipStream_t)stream;
  RouteParams p{};
  p.keys = ix->keys;
  p.kscale = ix->kscale;
  p.q = static_cast<const uint8_t*>(q);
  p.qscale = c.dtype == IDX_E4M3 ? q_scale : nullptr;
  p.w = w;
  p.n_keys = ix->n_keys;
  p.H = c.heads;
  p.T = T;
  p.q_pos0 = q_pos0;
  p.qpos = nullptr;
  p.k = k;
  p.budget = budget;
  p.S = c.n_sink;
  p.W = c.window;
  p.Cs = ix->Cs;
  p.wpr = ix->wpr;
  p.P = P;
  for (int i = 0; i < 3; ++i) {
    const EpochStore& e = ix->ep[i];
    p.ep[i] = StoreView{e.size, e.off, e.members, e.cent, e.rep, e.rsc, e.ckeys, e.cscale};
  }
  p.seal = ix->seal_view();
  p.srep = ix->srep;
  p.srep_ld = std::max<int64_t>(ix->slot_cap, 1);
  p.cand = ix->cand;
  p.cand_row = ix->cand_row;
  p.write_cand = (dbg && dbg->cand) ? 1 : 0;
  p.cand_ld = ix->cand_cap;
  p.cand_len = ix->cand_len;
  p.redo = ix->redo;
  p.ovf = ix->route_ovf;
  p.topk_idx = topk_idx;
  p.topk_score = topk_score;
  p.cluster_major = c.rescore_mode == IDX_RESCORE_CLUSTER;
  p.id_seal = (int)ix->slot_cap;
  p.id_ep = (int)ix->ep_slot_cap;
  p.n_ids = ix->n_ids;
  p.sel_id = ix->sel_id;
  p.sel_dst = ix->sel_dst;
  p.n_sel = ix->n_sel;
  p.sel_ld = ix->sel_cap;
  p.pc_cnt = ix->pc_cnt;
  p.pair_t = ix->pair_t;
  p.pair_dst = ix->pair_dst;
  p.pair_take = ix->pair_take;
  p.item_id = ix->item_id;
  p.item_first = ix->item_first;
  p.item_n = ix->item_n;
  p.item_cap = ix->item_cap;
  p.ctr = ix->ctr;
  p.sbuf = ix->sbuf;
  p.prescored = (!p.cluster_major && T <= kSplitQueries) ? 1 : 0;
  if (dbg) {
    p.dbg_order = dbg->order;
    p.dbg_take = dbg->order_take;
    p.dbg_order_cap = dbg->order_cap;
    p.dbg_n_order = dbg->n_order;
    p.dbg_version = dbg->version;
    p.list_cap = dbg->list_cap;
    p.dbg_cand_scores = dbg->cand_scores;
    p.dbg_cand_ld = dbg->cand_cap;
  }
  const int max_slots = windows_in(pmax + 1) * ix->Cs;
  if (positions) {
    hipError_t ec = hipMemcpyAsync(ix->qpos, positions, (size_t)T * sizeof(int64_t), hipMemcpyHostToDevice, s);
    if (ec != hipSuccess) return device_error(ix, ec, "position copy");
    p.qpos = ix->qpos;
  }
  hipEvent_t* ev = (dbg && dbg->events) ? reinterpret_cast<hipEvent_t*>(dbg->events) : nullptr;
  hipError_t e = hipSuccess;
  auto mark = [&](int i) {
    if (ev && ev[i] && e == hipSuccess) e = hipEventRecord(ev[i], s);
  };
  // AUTO with a large batch: cut, rescoring and top-k in one kernel; a query whose
  // cluster list overflows goes through the full cut kernel and the rescoring kernel
  // (both return at once for every other query)
  const int call_cap = (int)round_up(std::max<int64_t>(budget, (int64_t)c.n_sink + c.window), 32);
  const bool fused = c.rescore_mode == IDX_RESCORE_AUTO && !p.cluster_major && !p.prescored &&
                     call_cap <= route_rescore_max_cands();
  mark(0);
  if (max_slots > 0 && e == hipSuccess) e = launch_rep_score(p, c.dtype, c.dim, ix->HT, max_slots, s);
  mark(1);
  mark(2);
  if (fused) {
    if (e == hipSuccess) e = launch_route_rescore(p, c.dtype, c.dim, ix->HT, call_cap, s);
  } else {
    if (p.cluster_major && e == hipSuccess) e = launch_pairs_zero(p, s);
    if (e == hipSuccess) e = launch_route_select(p, max_slots, s);
    if (p.cluster_major && e == hipSuccess) e = launch_pairs_group(p, s);
  }
  mark(3);
  mark(4);
  if (p.cluster_major && e == hipSuccess) e = launch_cluster_score(p, c.dtype, c.dim, ix->HT, s);
  if (p.prescored && e == hipSuccess) e = launch_cand_score(p, c.dtype, c.dim, ix->HT, call_cap, s);
  mark(5);
  mark(6);
  if (fused) {
    if (e == hipSuccess) e = launch_route_overflow(p, c.dtype, c.dim, ix->HT, call_cap, max_slots, s);
  } else {
    if (e == hipSuccess) e = launch_rescore_topk(p, c.dtype, c.dim, ix->HT, call_cap, s);
  }
  mark(7);
  if (e != hipSuccess) return device_error(ix, e, "route launch");
  if (dbg) {
    if (dbg->cand && dbg->cand_cap > 0) {
      const size_t wcols = (size_t)std::min(dbg->cand_cap, ix->cand_cap);
      e = hipMemcpy2DAsync(dbg->cand, (size_t)dbg->cand_cap * 4, ix->cand, (size_t)ix->cand_cap * 4, wcols * 4, T,
                           hipMemcpyDeviceToDevice, s);
    }
    if (e == hipSuccess && dbg->cand_len)
      e = hipMemcpyAsync(dbg->cand_len, ix->cand_len, (size_t)T * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && dbg->rep_scores && dbg->rep_cap > 0 && max_slots > 0) {
      const size_t wcols = (size_t)std::min<int64_t>(dbg->rep_cap, p.srep_ld);
      e = hipMemcpy2DAsync(dbg->rep_scores, (size_t)dbg->rep_cap * 4, ix->srep, (size_t)p.srep_ld * 4, wcols * 4, T,
                           hipMemcpyDeviceToDevice, s);
    }
    if (e != hipSuccess) return device_error(ix, e, "route debug copy");
  }
  return IDX_OK;
}

int idx_route_topk(idx_index* ix, const void* q, const float* q_scale, const float* w, int64_t q_pos0, int32_t T,
                   int32_t k, int32_t budget, int32_t* topk_idx, float* topk_score, const idx_route_debug* dbg,
                   void* stream) {
  if (q_pos0 < 0) {
    g_err.clear();
    return fail(IDX_EINVAL, "q_pos0 must be >= 0");
  }
  return route_common(ix, q, q_scale, w, q_pos0, nullptr, T, k, budget, topk_idx, topk_score, dbg, stream);
}

int idx_route_topk_pos(idx_index* ix, const void* q, const float* q_scale, const float* w, const int64_t* positions,
                       int32_t T, int32_t k, int32_t budget, int32_t* topk_idx, float* topk_score,
                       const idx_route_debug* dbg, void* stream) {
  if (!positions) {
    g_err.clear();
    return fail(IDX_EINVAL, "null positions");
  }
  return route_common(ix, q, q_scale, w, 0, positions, T, k, budget, topk_idx, topk_score, dbg, stream);
}

}  // extern "C"

// Score rows of idx_exhaustive_topk_noalloc: one array per GPU, set up when the code
// object is loaded and held until the process ends.  Host code never names it: its
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) float scratch[IDX_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (nullptr + message on failure).
float* scratch_on_current_device(int* dev_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    fail(IDX_EDEVICE, "no usable current device");
    return nullptr;
  }
  *dev_out = dev;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(IDX_EDEVICE, "scratch address on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  return g_scratch_ptr[dev];
}

// Checks shared by both exhaustive entry points (no device work).
int exhaustive_check(const void* keys, const float* k_scale, int64_t n_keys, int32_t dtype, int32_t heads, int32_t dim,
                     const void* q, const float* q_scale, const float* w, int64_t q_pos0, int32_t T, int32_t k,
                     int32_t* topk_idx) {
  if (dtype < IDX_F32 || dtype > IDX_E4M3) return fail(IDX_EINVAL, "unknown dtype %d", dtype);
  if (heads < 1 || heads > 128) return fail(IDX_EINVAL, "heads must be 1..128");
  if (!dim_supported(dtype, dim)) return fail(IDX_ENOTIMPL, "dim %d not built for dtype %d", dim, dtype);
  if (!keys || !q || !w || !topk_idx) return fail(IDX_EINVAL, "null pointer argument");
  if (dtype == IDX_E4M3 && (!k_scale || !q_scale)) return fail(IDX_EINVAL, "E4M3 needs k_scale and q_scale");
  if (T < 1) return fail(IDX_EINVAL, "T must be >= 1");
  if (k < 1 || k > 4096) return fail(IDX_EINVAL, "k must be 1..4096");
  if (q_pos0 < 0) return fail(IDX_EINVAL, "q_pos0 must be >= 0");
  if (q_pos0 + T > n_keys) return fail(IDX_ECAUSAL, "query position beyond n_keys");
  if (q_pos0 + T > INT32_MAX) return fail(IDX_EINVAL, "positions must fit in int32");
  return IDX_OK;
}

// Layout of an exhaustive workspace (byte offsets from its start, 256-aligned):
//   [failed list: 1 + Tb ints][sample rows][sample scales]            per call
//   [sample scores: Tb x sld][tau: Tb][count: Tb][survivors: Tb x caps]  per pass
// The fallback's score rows reuse everything from the sample scores on.
struct ExhPlan {
  int stride = 64, soff = 32, caps = 8192, aim = 0;
  int64_t ns = 0, sld = 0, ld = 0;
  int64_t off_skeys = 0, off_sscale = 0, off_srow = 0, off_tau = 0, off_cnt = 0, off_surv = 0, end = 0;
};

int64_t align256(int64_t x) { return round_up(x, 256); }

// n_all: the longest prefix of the call; rb: bytes per key row; Tb: rows per pass.
ExhPlan exh_plan(int64_t n_all, int k, int rb, int64_t Tb) {
  ExhPlan pl;
  pl.stride = (int)std::max<int64_t>(64, (n_all + 16383) / 16384);   // at most 16384 sample keys
  pl.soff = pl.stride / 2;
  pl.caps = k > 2048 ? 16384 : 8192;
  pl.aim = (int)std::min<int64_t>(std::max<int64_t>(2ll * k, 32ll * pl.stride), pl.caps / 2);
  pl.ns = n_all > pl.soff ? (n_all - pl.soff + pl.stride - 1) / pl.stride : 0;
  pl.sld = round_up(std::max<int64_t>(pl.ns, 1), 64);
  pl.ld = round_up(n_all, 64);
  pl.off_skeys = align256((1 + Tb) * 4);
  pl.off_sscale = pl.off_skeys + align256(pl.ns * rb);
  pl.off_srow = pl.off_sscale + align256(pl.ns * 4);
  pl.off_tau = pl.off_srow + align256(Tb * pl.sld * 4);
  pl.off_cnt = pl.off_tau + align256(Tb * 4);
  pl.off_surv = pl.off_cnt + align256(Tb * 4);
  pl.end = std::max(pl.off_surv + Tb * pl.caps * 8, pl.off_srow + pl.ld * 4);   // room for one fallback row
  return pl;
}

// Bytes a pass of Tb rows needs (the sizes the workspace query promises cover every
// format and k: 512-byte rows, 16384 survivors).
int64_t exh_bytes(int64_t n_all, int k, int rb, int64_t Tb) { return exh_plan(n_all, k, rb, Tb).end; }

// The exhaustive passes: as many queries per pass as `ws_bytes` hold (exh_plan).  After
// each pass the call reads how many rows need the fallback (a wait on the stream);
// those run through materialized score rows, as many at a time as the workspace
// holds.
int exhaustive_passes(const void* keys, const float* k_scale, int32_t dtype, int32_t heads, int32_t dim, const void* q,
                      const float* q_scale, const float* w, int64_t q_pos0, int32_t T, int32_t k, int32_t* topk_idx,
                      float* topk_score, void* ws, int64_t ws_bytes, hipStream_t s) {
  const int64_t n_all = q_pos0 + T;
  const int rb = dim * elem_bytes(dtype);
  int64_t Tb_max = T;
  while (Tb_max > 1 && exh_bytes(n_all, k, rb, Tb_max) > ws_bytes) Tb_max = std::max<int64_t>(1, Tb_max / 2);
  if (exh_bytes(n_all, k, rb, Tb_max) > ws_bytes)
    return fail(IDX_EINVAL, "workspace too small: %lld bytes, need >= %lld", (long long)ws_bytes,
                (long long)exh_bytes(n_all, k, rb, 1));
  while (Tb_max < T && exh_bytes(n_all, k, rb, Tb_max + 1) <= ws_bytes) ++Tb_max;   // grow back after halving
  const ExhPlan pl = exh_plan(n_all, k, rb, Tb_max);
  uint8_t* const wb = static_cast<uint8_t*>(ws);
  int* const failed = reinterpret_cast<int*>(wb);
  const int HT = head_tiles(heads);
  auto dev_fail = [&](hipError_t e) { return fail(IDX_EDEVICE, "exhaustive launch: %s", hipGetErrorString(e)); };

  ExhParams p{};
  p.keys = static_cast<const uint8_t*>(keys);
  p.kscale = dtype == IDX_E4M3 ? k_scale : nullptr;
  p.q = static_cast<const uint8_t*>(q);
  p.qscale = dtype == IDX_E4M3 ? q_scale : nullptr;
  p.w = w;
  p.H = heads;
  p.q_pos0 = q_pos0;
  p.kchunk = 8192;
  p.k = k;
  p.topk_idx = topk_idx;
  p.topk_score = topk_score;
  p.stride = pl.stride;
  p.soff = pl.soff;
  p.skeys = wb + pl.off_skeys;
  p.sscale = reinterpret_cast<const float*>(wb + pl.off_sscale);
  p.srow = reinterpret_cast<float*>(wb + pl.off_srow);
  p.sld = pl.sld;
  p.aim = pl.aim;
  p.tau = reinterpret_cast<uint32_t*>(wb + pl.off_tau);
  p.cnt = reinterpret_cast<int*>(wb + pl.off_cnt);
  p.surv = reinterpret_cast<uint64_t*>(wb + pl.off_surv);
  p.caps = pl.caps;
  p.failed = failed;
  std::vector<int> rows;
  for (int t0 = 0; t0 < T; t0 += (int)Tb_max) {
    p.t0 = t0;
    p.Tb = (int)std::min<int64_t>(Tb_max, T - t0);
    p.tlist = nullptr;
    const int64_t n_batch = q_pos0 + t0 + p.Tb;
    const int64_t ns_batch = n_batch > pl.soff ? (n_batch - pl.soff + pl.stride - 1) / pl.stride : 0;
    // the sample rows are gathered again each pass: a fallback overwrites nothing
    // before them, but one pass's gather covers only its own prefixes
    hipError_t e = launch_exh_gather(p, rb, ns_batch, s);
    if (e == hipSuccess && ns_batch > 0) e = launch_exh_score(p, EXH_SAMPLE, dtype, dim, HT, ns_batch, s);
    if (e == hipSuccess) e = launch_exh_threshold(p, s);
    if (e == hipSuccess) e = launch_exh_score(p, EXH_STREAM, dtype, dim, HT, n_batch, s);
    if (e == hipSuccess) e = launch_exh_finalize(p, s);
    if (e != hipSuccess) return dev_fail(e);
    int n_failed = 0;
    e = hipMemcpyAsync(&n_failed, failed, sizeof(int), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return dev_fail(e);
    if (n_failed <= 0) continue;
    // ---- fallback: the listed rows through materialized score rows, in position order ----
    rows.assign(n_failed, 0);
    e = hipMemcpy(rows.data(), failed + 1, (size_t)n_failed * sizeof(int), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return dev_fail(e);
    std::sort(rows.begin(), rows.end());
    e = hipMemcpy(failed + 1, rows.data(), (size_t)n_failed * sizeof(int), hipMemcpyHostToDevice);
    if (e != hipSuccess) return dev_fail(e);
    const int per = (int)std::max<int64_t>(1, (ws_bytes - pl.off_srow) / (pl.ld * 4));
    ExhParams f = p;
    f.ws = reinterpret_cast<float*>(wb + pl.off_srow);
    f.ld = pl.ld;
    for (int r0 = 0; r0 < n_failed; r0 += per) {
      f.tlist = failed + 1 + r0;
      f.Tb = std::min(per, n_failed - r0);
      const int64_t n_rows = q_pos0 + t0 + rows[r0 + f.Tb - 1] + 1;
      e = launch_exh_score(f, EXH_ROWS, dtype, dim, HT, n_rows, s);
      if (e == hipSuccess) e = launch_topk_rows(f, s);
      if (e != hipSuccess) return dev_fail(e);
    }
  }
  return IDX_OK;
}

}  // namespace

extern "C" {

int64_t idx_exhaustive_workspace_bytes(int64_t n_keys, int32_t T) {
  if (n_keys < 1 || T < 1) return 0;
  return exh_bytes(n_keys, 4096, 512, T);
}

int idx_exhaustive_topk(const void* keys, const float* k_scale, int64_t n_keys, int32_t dtype, int32_t heads,
                        int32_t dim, const void* q, const float* q_scale, const float* w, int64_t q_pos0, int32_t T,
                        int32_t k, int32_t* topk_idx, float* topk_score, void* workspace, int64_t workspace_bytes,
                        void* stream) {
  g_err.clear();
  if (int e = exhaustive_check(keys, k_scale, n_keys, dtype, heads, dim, q, q_scale, w, q_pos0, T, k, topk_idx))
    return e;
  if (!workspace) return fail(IDX_EINVAL, "null pointer argument");
  return exhaustive_passes(keys, k_scale, dtype, heads, dim, q, q_scale, w, q_pos0, T, k, topk_idx, topk_score,
                           workspace, workspace_bytes, (hipStream_t)stream);
}

int idx_exhaustive_topk_noalloc(const void* keys, const float* k_scale, int64_t n_keys, int32_t dtype, int32_t heads,
                                int32_t dim, const void* q, const float* q_scale, const float* w, int64_t q_pos0,
                                int32_t T, int32_t k, int32_t* topk_idx, float* topk_score, void* stream) {
  g_err.clear();
  if (int e = exhaustive_check(keys, k_scale, n_keys, dtype, heads, dim, q, q_scale, w, q_pos0, T, k, topk_idx))
    return e;
  const int64_t need = exh_bytes(q_pos0 + T, k, dim * elem_bytes(dtype), 1);
  if (need > (int64_t)IDX_NOALLOC_SCRATCH_BYTES)
    return fail(IDX_ECAPACITY, "a pass over %lld keys needs %lld bytes, more than the %lld-byte scratch array",
                (long long)(q_pos0 + T), (long long)need, (long long)IDX_NOALLOC_SCRATCH_BYTES);
  int dev = 0;
  float* ws = scratch_on_current_device(&dev);
  if (!ws) return IDX_EDEVICE;
  return exhaustive_passes(keys, k_scale, dtype, heads, dim, q, q_scale, w, q_pos0, T, k, topk_idx, topk_score, ws,
                           (int64_t)IDX_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream);
}

int64_t idx_encoder_floats(int32_t dim) {
  if (dim != 32 && dim != 64 && dim != 128) return -1;
  return encoder_floats(dim);
}

int idx_set_encoder(idx_index* ix, const float* weights, void* stream) {
  g_err.clear();
  if (int e = check_handle(ix)) return e;
  if (ix->computed != ix->published) return fail(IDX_ESTATE, "a refit is in flight; publish it first");
  if (!weights) {
    ix->has_enc = false;
    return IDX_OK;
  }
  (void)hipSetDevice(ix->device);
  const hipError_t e = hipMemcpyAsync(ix->enc, weights, (size_t)encoder_floats(ix->cfg.dim) * sizeof(float),
                                      hipMemcpyDeviceToDevice, (hipStream_t)stream);
  if (e != hipSuccess) return device_error(ix, e, "encoder copy");
  ix->has_enc = true;
  return IDX_OK;
}

int idx_export(idx_index* ix, int32_t which, idx_export_buf* buf) {
  g_err.clear();
  if (int e = check_handle(ix)) return e;
  if (!buf) return fail(IDX_EINVAL, "null export buffer");
  const idx_config& c = ix->cfg;
  const int *size, *off, *members;
  const float *cent, *rsc, *lrep;
  const uint8_t* rep;
  int64_t n_slots, n_members;
  if (which == -1) {
    n_slots = (int64_t)ix->sealed * ix->Cs;
    n_members = (int64_t)ix->sealed * c.window;
    size = ix->sl_size; off = ix->sl_off; members = ix->sl_members;
    cent = ix->sl_cent; rep = ix->sl_rep; rsc = ix->sl_rsc; lrep = ix->sl_lrep;
  } else {
    if (which < 1 || which > ix->computed || which < oldest_held(ix))
      return fail(IDX_ESTATE, "epoch %d is not held (computed %d)", which, ix->computed);
    n_slots = (int64_t)which * ix->Q;
    n_members = (int64_t)which * ix->wpr * c.window;
    const EpochStore& e = ix->ep[which % 3];
    size = e.size; off = e.off; members = e.members; cent = e.cent; rep = e.rep; rsc = e.rsc; lrep = e.lrep;
  }
  buf->n_slots = (int32_t)n_slots;
  buf->n_members = (int32_t)n_members;
  (void)hipSetDevice(ix->device);
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return device_error(ix, e, "export wait");
  auto cp = [&](void* dst, const void* src, size_t bytes) {
    if (dst && bytes && e == hipSuccess) e = hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
  };
  cp(buf->sizes, size, (size_t)n_slots * 4);
  cp(buf->offsets, off, (size_t)n_slots * 4);
  cp(buf->members, members, (size_t)n_members * 4);
  cp(buf->centroids, cent, (size_t)n_slots * c.dim * 4);
  cp(buf->reps, rep, (size_t)n_slots * ix->RB);
  cp(buf->rep_scale, rsc, (size_t)n_slots * 4);
  cp(buf->rep_f32, lrep, (size_t)n_slots * c.dim * 4);
  buf->n_screened = -1;
  buf->n_brute = -1;
  buf->n_bound_keys = 0;
  if (which >= 1 && which == ix->computed && ix->imported != which) {
    int wc = 0, oc = 0;
    cp(&wc, ix->work_count, 4);
    cp(&oc, ix->ovf_count, 4);
    const int64_t nb = (int64_t)which * c.refit_every;
    buf->n_screened = (int64_t)c.refit_every + wc;
    buf->n_brute = oc;
    buf->n_bound_keys = nb;
    cp(buf->assign, ix->assign + c.n_sink, (size_t)nb * 4);
    cp(buf->ub, ix->ub + c.n_sink, (size_t)nb * 4);
    cp(buf->lb, ix->lb + c.n_sink, (size_t)nb * 4);
  }
  if (e != hipSuccess) return device_error(ix, e, "export copy");
  return IDX_OK;
}

int idx_export_version(idx_index* ix, int64_t prefix_len, int32_t* epoch, int32_t* windows, idx_export_buf* buf) {
  g_err.clear();
  if (int e = check_handle(ix)) return e;
  if (!buf) return fail(IDX_EINVAL, "null export buffer");
  if (prefix_len < 1) return fail(IDX_EINVAL, "prefix_len must be >= 1");
  if (prefix_len > ix->n_keys)
    return fail(IDX_ECAUSAL, "prefix_len %lld exceeds the %lld inserted keys", (long long)prefix_len,
                (long long)ix->n_keys);
  const idx_config& c = ix->cfg;
  const int m = prefix_len >= c.n_sink ? (int)((prefix_len - c.n_sink) / c.window) : 0;
  const int r = ix->wpr ? std::min(ix->published, m / ix->wpr) : 0;
  if (r >= 1 && r < oldest_held(ix))
    return fail(IDX_ESTATE, "prefix %lld routes over epoch %d, which is no longer held", (long long)prefix_len, r);
  if (epoch) *epoch = r;
  if (windows) *windows = m;
  const int64_t n_slots = (int64_t)m * ix->Cs, n_members = (int64_t)m * c.window;
  const int64_t e_slots = (int64_t)r * ix->Q, e_members = (int64_t)r * c.refit_every;
  buf->n_slots = (int32_t)n_slots;
  buf->n_members = (int32_t)n_members;
  buf->n_screened = -1;
  buf->n_brute = -1;
  buf->n_bound_keys = 0;
  (void)hipSetDevice(ix->device);
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return device_error(ix, e, "export wait");
  const EpochStore* es = r >= 1 ? &ix->ep[r % 3] : nullptr;
  // slots [0, e_slots) and members [0, e_members) from the epoch, the rest from the
  // seal store; a seal slot's offset already counts the members of the windows
  // before it, e_members of them being the epoch's
  auto cp = [&](void* dst, const void* ep_src, const void* sl_src, int64_t n_ep, int64_t n_all, size_t unit) {
    if (!dst || e != hipSuccess) return;
    uint8_t* d = static_cast<uint8_t*>(dst);
    if (n_ep > 0) e = hipMemcpy(d, ep_src, (size_t)n_ep * unit, hipMemcpyDeviceToHost);
    if (e == hipSuccess && n_all > n_ep)
      e = hipMemcpy(d + (size_t)n_ep * unit, static_cast<const uint8_t*>(sl_src) + (size_t)n_ep * unit,
                    (size_t)(n_all - n_ep) * unit, hipMemcpyDeviceToHost);
  };
  const size_t dbytes = (size_t)c.dim * 4;
  cp(buf->sizes, es ? es->size : nullptr, ix->sl_size, e_slots, n_slots, 4);
  cp(buf->offsets, es ? es->off : nullptr, ix->sl_off, e_slots, n_slots, 4);
  cp(buf->members, es ? es->members : nullptr, ix->sl_members, e_members, n_members, 4);
  cp(buf->centroids, es ? es->cent : nullptr, ix->sl_cent, e_slots, n_slots, dbytes);
  cp(buf->reps, es ? es->rep : nullptr, ix->sl_rep, e_slots, n_slots, (size_t)ix->RB);
  cp(buf->rep_scale, es ? es->rsc : nullptr, ix->sl_rsc, e_slots, n_slots, 4);
  cp(buf->rep_f32, es ? es->lrep : nullptr, ix->sl_lrep, e_slots, n_slots, dbytes);
  if (e != hipSuccess) return device_error(ix, e, "export copy");
  return IDX_OK;
}

int idx_import_version(idx_index* ix, int64_t prefix_len, const idx_import_buf* buf, void* stream) {
  g_err.clear();
  if (int e = check_handle(ix)) return e;
  if (!buf) return fail(IDX_EINVAL, "null import buffer");
  const idx_config& c = ix->cfg;
  if (!ix->wpr) return fail(IDX_EINVAL, "the index has no refit epochs (refit_every = 0)");
  if (ix->computed != ix->published) return fail(IDX_ESTATE, "a refit is in flight; publish or abandon it first");
  const int r = ix->computed + 1;
  const int64_t S = c.n_sink, B = S + (int64_t)r * c.refit_every;
  if (prefix_len != B)
    return fail(IDX_EINVAL, "prefix_len %lld is not the boundary %lld of the next epoch %d", (long long)prefix_len,
                (long long)B, r);
  if (B > ix->n_keys)
    return fail(IDX_ECAUSAL, "epoch %d covers keys below %lld; only %lld are inserted", r, (long long)B,
                (long long)ix->n_keys);
  if (ix->sealed < r * ix->wpr) return fail(IDX_ESTATE, "keys below %lld are not sealed yet", (long long)B);
  const int64_t ns = (int64_t)r * ix->Q;
  if (buf->n_slots != ns) return fail(IDX_EINVAL, "epoch %d has %lld slots (got %d)", r, (long long)ns, buf->n_slots);
  if (!buf->sizes || !buf->members || !buf->centroids || !buf->reps)
    return fail(IDX_EINVAL, "null sizes, members, centroids or reps");
  if (c.dtype == IDX_E4M3 && !buf->rep_scale) return fail(IDX_EINVAL, "E4M3 representatives need rep_scale");
  const int64_t nm = B - S;
  std::vector<int> off((size_t)ns), assign_h((size_t)nm, -1);
  int64_t total = 0;
  for (int64_t s = 0; s < ns; ++s) {
    const int sz = buf->sizes[s];
    if (sz < 0 || total + sz > nm)
      return fail(IDX_EINVAL, "slot %lld: size %d; the members must cover keys [%lld, %lld) exactly once",
                  (long long)s, sz, (long long)S, (long long)B);
    off[(size_t)s] = (int)total;
    int64_t prev = -1;
    for (int i = 0; i < sz; ++i) {
      const int64_t pos = buf->members[total + i];
      if (pos >= B)
        return fail(IDX_ECAUSAL, "slot %lld: member %lld lies at or beyond the version's prefix %lld", (long long)s,
                    (long long)pos, (long long)B);
      if (pos < S) return fail(IDX_EINVAL, "slot %lld: member %lld is a sink or negative", (long long)s, (long long)pos);
      if (pos <= prev) return fail(IDX_EINVAL, "slot %lld: members must be strictly ascending", (long long)s);
      if (assign_h[(size_t)(pos - S)] >= 0)
        return fail(IDX_EINVAL, "key %lld is a member of slots %d and %lld", (long long)pos,
                    assign_h[(size_t)(pos - S)], (long long)s);
      assign_h[(size_t)(pos - S)] = (int)s;
      prev = pos;
    }
    total += sz;
  }
  if (total != nm) return fail(IDX_EINVAL, "the members cover %lld of the %lld keys of [%lld, %lld)", (long long)total,
                               (long long)nm, (long long)S, (long long)B);
  const int d = c.dim;
  for (int64_t i = 0; i < ns * d; ++i)
    if (!std::isfinite(buf->centroids[i]) || (buf->rep_f32 && !std::isfinite(buf->rep_f32[i])))
      return fail(IDX_EINVAL, "slot %lld: centroid or representative is not finite", (long long)(i / d));
  if (c.dtype == IDX_E4M3) {
    const uint8_t* codes = static_cast<const uint8_t*>(buf->reps);
    for (int64_t s = 0; s < ns; ++s) {
      const float sc = buf->rep_scale[s];
      if (!(sc > 0.0f) || !std::isfinite(sc)) return fail(IDX_EINVAL, "slot %lld: rep_scale must be finite and > 0", (long long)s);
      for (int i = 0; i < d; ++i)
        if ((codes[s * d + i] & 0x7F) == 0x7F) return fail(IDX_EINVAL, "slot %lld: E4M3 NaN code", (long long)s);
    }
  } else if (c.dtype == IDX_F32) {
    const float* v = static_cast<const float*>(buf->reps);
    for (int64_t i = 0; i < ns * d; ++i)
      if (!std::isfinite(v[i])) return fail(IDX_EINVAL, "slot %lld: representative is not finite", (long long)(i / d));
  } else {
    const uint16_t* v = static_cast<const uint16_t*>(buf->reps);
    for (int64_t i = 0; i < ns * d; ++i)
      if ((v[i] & 0x7F80u) == 0x7F80u) return fail(IDX_EINVAL, "slot %lld: representative is not finite", (long long)(i / d));
  }
  (void)hipSetDevice(ix->device);
  hipStream_t s = (hipStream_t)stream;
  // the target store (epoch r - 3's) may still be read by routes enqueued earlier
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipEventSynchronize(ix->ev_refit);
  if (e != hipSuccess) return device_error(ix, e, "import wait");
  EpochStore& out = ix->ep[r % 3];
  std::vector<float> ones((size_t)ns, 1.0f), zeros((size_t)ns, 0.0f), ub_h((size_t)nm, HUGE_VALF),
      lb_h((size_t)nm, 0.0f);
  const float zero = 0.0f;
  auto h2d = [&](void* dst, const void* src, size_t bytes) {
    if (e == hipSuccess && bytes) e = hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice);
  };
  h2d(out.size, buf->sizes, (size_t)ns * 4);
  h2d(out.off, off.data(), (size_t)ns * 4);
  h2d(out.members, buf->members, (size_t)nm * 4);
  h2d(out.cent, buf->centroids, (size_t)ns * d * 4);
  h2d(out.lrep, buf->rep_f32 ? buf->rep_f32 : buf->centroids, (size_t)ns * d * 4);
  h2d(out.rep, buf->reps, (size_t)ns * ix->RB);
  h2d(out.rsc, c.dtype == IDX_E4M3 ? buf->rep_scale : ones.data(), (size_t)ns * 4);
  // no bounds: the next refit finds every key uncertified (lower bound 0) and
  // compares it with every centre; the centres did not move
  h2d(out.drift, zeros.data(), (size_t)ns * 4);
  h2d(out.drift_max, &zero, 4);
  h2d(ix->assign + S, assign_h.data(), (size_t)nm * 4);
  h2d(ix->ub + S, ub_h.data(), (size_t)nm * 4);
  h2d(ix->lb + S, lb_h.data(), (size_t)nm * 4);
  if (e == hipSuccess)
    e = launch_copy_member_rows(out.members, 0, nm, ix->keys, ix->kscale, ix->n_keys, ix->RB, out.ckeys, out.cscale, s);
  if (e == hipSuccess) e = hipEventRecord(ix->ev_refit, s);
  if (e != hipSuccess) return device_error(ix, e, "import copy");
  ix->computed = r;
  ix->lost = std::max(ix->lost, r - 3);
  ix->imported = r;
  return IDX_OK;
}

}  // extern "C"
