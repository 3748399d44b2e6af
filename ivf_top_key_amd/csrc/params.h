// Kernel parameter blocks shared by the host runtime and the kernels.
#pragma once

#include <stdint.h>

namespace ivftk {

// One set of clusters in device memory, indexed by slot id.
//   size[s]      members of slot s (0 = empty: never ranked, never a warm start)
//   off[s]       index of the slot's first member in `members`
//   members[]    key positions, ascending within a slot
//   cent[s*d]    fp32 centroid; rep[s*RB] representative in the key format;
//   rsc[s]       representative scale (E4M3), 1 otherwise
//   ckeys[j*RB]  the key of members[j] (a copy in member order, so a cluster's keys
//                are contiguous); cscale[j] its scale (E4M3), null otherwise
struct StoreView {
  const int* size;
  const int* off;
  const int* members;
  const float* cent;
  const uint8_t* rep;
  const float* rsc;
  const uint8_t* ckeys;
  const float* cscale;
};

// Candidate rows for the rescoring gathers: (source << CROW_SHIFT) | row, source 0 =
// the position-ordered keys (row = position), 1 = the seal store's member-ordered
// copy, 2 + e = epoch store e's copy (row = index into that store's members).
constexpr int CROW_SHIFT = 29;
constexpr int CROW_MASK = (1 << CROW_SHIFT) - 1;

// Everything the routed path needs.  Query t sits at position qpos[t] when qpos is
// set (a decode batch), at q_pos0 + t otherwise; its
// version is computed on the device from (S, W, Cs, wpr, P): m = windows inside
// the prefix, epoch r = min(P, m / wpr), slots [0, r*wpr*Cs) come from epoch r's
// store and slots [r*wpr*Cs, m*Cs) from the seal store.
struct RouteParams {
  const uint8_t* keys;
  const float* kscale;
  const uint8_t* q;
  const float* qscale;
  const float* w;
  int64_t n_keys;      // keys inserted (positions read from index data are clamped below it)
  int H;
  int T;
  int64_t q_pos0;
  const int64_t* qpos; // [T] positions of a decode batch, or null
  int k;
  int budget;
  int S, W, Cs, wpr, P;
  StoreView ep[3];     // epoch r lives in ep[r % 3] (the host checks every epoch used is held)
  StoreView seal;
  float* srep;         // [T, srep_ld] representative scores
  int64_t srep_ld;
  int* cand;           // [T, cand_ld] candidate positions
  int* cand_row;       // [T, cand_ld] the row each candidate's key is gathered from (CROW_*)
  int write_cand;      // 1: the cut also writes the candidate positions to cand (debug
                       // read-back); the rescoring derives positions from cand_row
  int64_t cand_ld;
  int* cand_len;       // [T]
  int* redo;           // [T]: 1 when the fast cut kernel left the query to the full one
  int* ovf;            // [2 + T]: overflow list of the fused cut + rescoring kernel:
                       // [0] entries, [1] finished blocks of the overflow kernel,
                       // [2..] query indices; zero entries between calls
  int* topk_idx;       // [T, k]
  float* topk_score;   // [T, k] or null
  // optional debug outputs (null when unused)
  int* dbg_order;
  int* dbg_take;
  int dbg_order_cap;
  int* dbg_n_order;
  int* dbg_version;
  int list_cap;        // > 0: smaller cluster-list capacity of the fast cut kernel (tests)
  float* dbg_cand_scores;  // [T, dbg_cand_ld]
  int dbg_cand_ld;
  // Cluster-major rescoring (cluster_major = 1; otherwise the final kernel gathers
  // and scores every candidate).  A cluster is named by a unified id: ids
  // [0, id_seal) are seal slots, id_seal + e * id_ep + s is slot s of epoch store e.
  int cluster_major;
  int id_seal, id_ep, n_ids;
  int* sel_id;         // [T, sel_ld] ids of the query's selected clusters in rank order
  int* sel_dst;        // [T, sel_ld] list index of each selected cluster's first candidate
  int* n_sel;          // [T]
  int64_t sel_ld;
  int* pc_cnt;         // [n_ids] selections per id, then the scatter cursors
  int* pair_t;         // [pair_cap] (query, list index, members taken), grouped by id
  int* pair_dst;
  int* pair_take;
  int* item_id;        // [item_cap] work items: up to CS_PAIRS pairs of one id
  int* item_first;
  int* item_n;
  int64_t item_cap;
  int* ctr;            // [2] next work item, number of work items
  float* sbuf;         // [T, cand_ld] scores of the cluster candidates
  // Small batches: every candidate was scored into sbuf by blocks that split each
  // query's list (prescored = 1); the final kernel then only selects.
  int prescored;
};

struct ExhParams {
  const uint8_t* keys;
  const float* kscale;
  const uint8_t* q;
  const float* qscale;
  const float* w;
  int H;
  int64_t q_pos0;
  int t0;              // first query of this pass
  int Tb;              // query rows in this pass
  const int* tlist;    // row tl is query t0 + tlist[tl] (null: t0 + tl)
  float* ws;           // [Tb, ld] scores (materialized rows)
  int64_t ld;
  int kchunk;          // keys per block of the score kernel
  int k;
  int* topk_idx;       // [T, k] (row t0 + tl)
  float* topk_score;
  // streamed selection
  int stride, soff;    // sample: keys soff, soff + stride, soff + 2 stride, ...
  const uint8_t* skeys;   // the sample's rows, dense
  const float* sscale;
  float* srow;         // [Tb, sld] sample scores
  int64_t sld;
  int aim;             // survivors a threshold aims at
  uint32_t* tau;       // [Tb] order-key threshold
  int* cnt;            // [Tb] scores at or above tau (all of them, also past caps)
  uint64_t* surv;      // [Tb, caps] composites of the survivors
  int caps;
  int* failed;         // [1 + Tb]: count, then the rows the fallback handles
};

// Seal of windows [w0, w0 + gridDim.x).
struct SealParams {
  const uint8_t* keys;
  const float* kscale;
  int S, W, Cs, cap, iters;
  int positional;     // 1: cluster i of a window = its keys [i*W/Cs, (i+1)*W/Cs), one pass
  int w0;
  int* size;          // seal store, indexed by slot w*Cs + c
  int* off;
  int* members;       // [windows * W], window w's members at [w*W, (w+1)*W)
  float* cent;
  float* lrep;        // representative before quantization (= centroid; an encoder may replace it)
  uint8_t* rep;
  float* rsc;
};

// One refit: epoch r from slots [0, r*Q) (prev epoch for s < (r-1)*Q, seal store
// otherwise) over keys [S, B_r), B_r = S + r*R.
struct RefitParams {
  const uint8_t* keys;
  const float* kscale;
  int64_t n_keys;
  int S, r, Q;
  int64_t B_prev;      // S + (r-1)*R : keys below carry bounds from epoch r-1
  int64_t B_r;         // S + r*R
  StoreView prev;      // epoch r-1 (size/cent used; valid when r >= 2)
  const float* prev_drift;      // [slots of r-1]: centroid movement of epoch r-1's update
  StoreView seal;
  // per-key state, indexed by position
  int* assign;
  float* ub;
  float* lb;
  // work list of keys that need all centroids
  int* work;
  int* work_count;
  // output epoch store
  int* size;
  int* off;
  int* members;
  float* cent;
  float* lrep;         // representative before quantization (= centroid; an encoder may replace it)
  uint8_t* rep;
  float* rsc;
  float* drift;
  float* drift_max;
  // tile histogram scratch [n_tiles, Q*r]
  int* tile_cnt;
  int tile;            // keys per tile
  int n_tiles;
  // screening of the work keys with bf16 matrix products (see refit.hip)
  uint16_t* cbf;       // [2, r*Q, d] split bf16 copies (hi, lo) of the warm centroids
  float* cnrm;         // [r*Q] squared norm of each warm centroid, -1 for empty slots
  unsigned* tile_cmax; // [ceil(r*Q / 32)] largest squared norm per 32-slot tile (float bits)
  int* ovf;            // keys whose candidate list overflowed: exact brute force
  int* ovf_count;
  int brute_ovf;       // 1: the brute-force kernel takes its keys from ovf
  // certification of the keys of epoch r-1 (see refit.hip)
  uint32_t* hkey;      // [(r-1)*Q] selection keys of the old slots' drifts, then each old
                       // slot's place in hlist (0xFFFFFFFF: not listed)
  int* hlist;          // [r*Q] listed slots: the most-moved old slots, then the new ones
  int* nlist;          // device scalar: listed slots
  float* rest_drift;   // device scalar: largest drift of an unlisted live old slot
};

// Learned representatives of slots [slot0, slot0 + n_slots) of one store.
struct EncParams {
  const uint8_t* keys;
  const float* kscale;
  int64_t n_keys;
  StoreView st;        // size, off, members, cent of the store
  const float* w;      // packed encoder weights
  float* lrep;         // [slots, d] out: representative before quantization
  uint8_t* rep;        // [slots, RB] out: representative in the key format
  float* rsc;          // [slots] out: its scale
  int slot0, n_slots;
};

}  // namespace ivftk
