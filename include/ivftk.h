/*
 * ivftk.h — C ABI of the causal IVF-routed indexer top-k library (AMD MI355X, gfx950).
 *
 * What it computes (AttentionIndex: Accelerating Learned Sparse Attention with a
 * Causal Inverted-File Index, Park & Hwu, arXiv:2611.02508; pages cited by site and
 * section):
 *
 *   Indexer score (paper-daily.com explainer, "它到底在解决什么问题？" and
 *   "代表向量为什么要学？"): for query token t with H heads and key j,
 *       s(t, j) = sum_h w[t,h] * ReLU(q[t,h] . k[j]).
 *   With E4M3 storage, q[t,h] = codes * q_scale[t,h] and k[j] = codes * k_scale[j];
 *   both scales must be finite and > 0, so they factor out of the ReLU.
 *
 *   Exhaustive selection (same page, "它到底在解决什么问题？"): every key j <= p of
 *   the query at position p is scored and the top k are kept.
 *
 *   Routed selection (same page, "查询时怎么挑候选？"): the query scores every
 *   visible cluster representative with the same formula, ranks the clusters,
 *   fills a candidate budget with the sink keys and the whole open window, then the
 *   members of clusters in rank order, truncating the last one, scores the
 *   candidates exactly and keeps the top k.
 *
 *   Index maintenance (same page, "索引怎么边算边建？"; kurate.org assessment,
 *   "Core Contribution" item 1): keys are inserted into an open window; every W
 *   keys are sealed into W/cluster_size clusters by size-capped k-means; every R
 *   tokens the whole sealed prefix is refitted (one assignment + update round,
 *   warm-started from the previous centres plus the new seal centres, with
 *   upper/lower distance bounds) on a second stream; every seal and refit is a
 *   version, and a query only sees versions whose keys all lie in its prefix.
 *
 * Conventions shared by every call:
 *   - Return value: IDX_OK (0) or a negative idx_status.  On error nothing has been
 *     enqueued and idx_last_error() gives a message (thread-local, valid until the
 *     next call on the same thread).  No call aborts and no C++ exception crosses
 *     this boundary.
 *   - "device" pointers are HIP device memory (e.g. torch CUDA tensors under ROCm);
 *     "host" pointers are ordinary CPU memory.  Every array is dense and row-major.
 *   - Streams are hipStream_t passed as void* (NULL = the default stream).  Calls
 *     validate on the host, enqueue work on the given stream(s) and return without
 *     waiting, except idx_create, idx_destroy, idx_export, idx_export_version and
 *     idx_import_version, which wait.
 *   - Caller-owned inputs must stay valid until the stream has passed the enqueued
 *     work; caller-owned outputs are written by that work.
 *   - An index handle is used from one host thread at a time, with one main stream
 *     that orders all its calls (routes, seals, publication).
 *   - Key storage formats (idx_dtype): IDX_F32 = fp32; IDX_BF16 = bf16 (2 bytes);
 *     IDX_E4M3 = OCP 8-bit E4M3 (e4m3fn, 1 byte, largest finite 448) with an fp32
 *     scale per key and per (query, head).  Codes 0x7F/0xFF (NaN) must not occur.
 *   - A row of d elements takes d * element_size bytes; queries are [T, H, d].
 *   - Top-k outputs hold key positions sorted by (score descending, position
 *     ascending); fewer than k candidates pad with position -1 and score -inf.
 */
#ifndef IVFTK_H
#define IVFTK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct idx_index idx_index;

typedef enum { IDX_F32 = 0, IDX_BF16 = 1, IDX_E4M3 = 2 } idx_dtype;

typedef enum {
  IDX_OK = 0,
  IDX_EINVAL = -1,      /* bad argument, shape, dtype or pointer                       */
  IDX_ENOMEM = -2,      /* device allocation failed at idx_create                      */
  IDX_EDEVICE = -3,     /* a HIP call failed; the handle is poisoned                   */
  IDX_ECAUSAL = -4,     /* a query position whose key has not been inserted            */
  IDX_ESTATE = -5,      /* call not allowed in this state (poisoned, epoch retired...) */
  IDX_ECAPACITY = -6,   /* more keys than max_keys, or a size above a create-time max  */
  IDX_ENOTIMPL = -7     /* shape or format this build does not provide                 */
} idx_status;

/* Index configuration, fixed at idx_create.  All device memory of the index is
 * allocated there from these numbers; no later call allocates. */
typedef struct {
  int32_t heads;         /* H, indexer heads per query: 1..128                                 */
  int32_t dim;           /* d: F32 32, 64 or 128; BF16 and E4M3 64 or 128                      */
  int32_t dtype;         /* idx_dtype of keys, queries and cluster representatives           */
  int32_t n_sink;        /* S: keys [0, S) are always candidates and never clustered (>= 0)  */
  int32_t window;        /* W: keys sealed per window, 2..1024                                 */
  int32_t cluster_size;  /* W / cluster_size clusters per seal, window*(W/cluster_size) <= 8192 */
  int32_t seal_cap;      /* most keys one seal cluster may hold; cap * clusters >= W           */
  int32_t seal_iters;    /* Lloyd iterations per seal, 1..64                                   */
  int32_t refit_every;   /* R: refit after every R/W seals; multiple of W; 0 = never           */
  int32_t max_queries;   /* largest T of one idx_route_topk call                               */
  int32_t max_budget;    /* largest budget of one idx_route_topk call (max(budget, S+W) <= 16384) */
  int32_t max_k;         /* largest k of one idx_route_topk call (<= 4096)                     */
  int32_t rescore_mode;  /* how idx_route_topk scores the selected clusters' candidates:
                            IDX_RESCORE_AUTO, IDX_RESCORE_QUERY or IDX_RESCORE_CLUSTER      */
  int32_t cluster_mode;  /* IDX_CLUSTERS_CONTENT (size-capped k-means seal + refits) or
                            IDX_CLUSTERS_POSITIONAL (position blocks; refit_every must be 0) */
  int64_t max_keys;      /* capacity in keys (positions 0 .. max_keys-1), 1 .. 2^29; also at most
                            8192 clusters may ever be routed: (max_keys - S) / W sealed windows
                            times W / cluster_size clusters each must be <= 8192 (at W = 1024
                            and cluster_size = 128: max_keys < S + 1025 * 1024), else ECAPACITY */
} idx_config;

/* Candidate rescoring of idx_route_topk.  All give bit-identical results.
 *   QUERY:   each query gathers and scores all of its candidates' key rows; the
 *            cluster cut writes each candidate's gather row to device memory first.
 *   CLUSTER: the (query, cluster) selections are grouped by cluster; each selected
 *            cluster's key rows are read once and scored against every query that
 *            selected it (pays off when many queries of a call share clusters).
 *   AUTO:    QUERY with the cut in the rescoring kernel for calls of more than 64
 *            queries whose max(budget, n_sink + window) is at most 8192 (the ranked
 *            clusters stay in on-chip memory, no candidate list goes through device
 *            memory), QUERY otherwise; the fastest on the measured workloads (1M-key
 *            E4M3 prefill chunk of 4096 queries). */
enum { IDX_RESCORE_AUTO = 0, IDX_RESCORE_QUERY = 1, IDX_RESCORE_CLUSTER = 2 };

/* How sealed windows are grouped.
 *   CONTENT:    size-capped k-means (the method of the pages).
 *   POSITIONAL: window w's cluster i is the contiguous block of cluster_size keys
 *               [S + w*W + i*cluster_size, ...), represented by its mean: the
 *               position-block grouping of the comparison method the paper-daily
 *               explainer calls HiSA ("它到底在解决什么问题？"), routed by the same
 *               kernels as a baseline. */
enum { IDX_CLUSTERS_CONTENT = 0, IDX_CLUSTERS_POSITIONAL = 1 };

/* Snapshot of the host-side index state (no device wait). */
typedef struct {
  int64_t n_keys;            /* keys inserted so far                                  */
  int32_t sealed_windows;    /* m: windows [0, m) sealed                              */
  int32_t computed_epoch;    /* newest refit epoch launched (0 = none)                */
  int32_t published_epoch;   /* newest refit epoch visible to queries (0 = none)      */
  int32_t clusters_per_window;
  int32_t slots_per_epoch;   /* Q = (R/W) * clusters_per_window                       */
  int64_t device_bytes;      /* device memory owned by the index                      */
} idx_info;

/* Optional debug outputs of idx_route_topk: all device pointers, each may be NULL.
 * Rows are per query; cand/order rows have cand_cap/order_cap entries. */
typedef struct {
  int32_t* cand;         /* [T, cand_cap]: candidate positions in fill order            */
  int32_t cand_cap;
  int32_t* cand_len;     /* [T]: candidates of each query                               */
  int32_t* order;        /* [T, order_cap]: clusters (slot ids) used, in rank order     */
  int32_t* order_take;   /* [T, order_cap]: members taken from each (last may be cut)   */
  int32_t order_cap;
  int32_t* n_order;      /* [T]: clusters used (entries beyond order_cap not written)   */
  float* rep_scores;     /* [T, rep_cap]: representative score of each visible slot     */
  int32_t rep_cap;
  int32_t* version;      /* [T, 4]: epoch r, sealed windows m, visible slots, open start */
  void** events;         /* host array of 8 hipEvent_t, recorded in pairs around the four
                            stages: representative scores; cluster cut + fill + grouping of
                            the selections by cluster (or, when AUTO fuses them, cut,
                            rescoring and top-k in one kernel); cluster-by-cluster or split
                            candidate scores; candidate scores + top-k (fused: only the
                            queries whose cut went to the full kernel).  A NULL entry is
                            not recorded (each record costs a few microseconds of stream
                            time)                                                          */
  int32_t list_cap;      /* > 0: cap the short cluster list of the fast cut (in the cut
                            kernel or the fused cut + rescoring kernel) at this size, so
                            the full radix-select cut takes over sooner (testing)          */
  float* cand_scores;    /* [T, cand_cap]: exact score of each candidate, fill order      */
} idx_route_debug;

/* Host buffers for idx_export.  Pass NULL arrays to read only the counts. */
typedef struct {
  int32_t n_slots;       /* out: slots in the exported set                              */
  int32_t n_members;     /* out: member entries                                         */
  int32_t* sizes;        /* [n_slots]: members per slot (0 = empty, never routed)       */
  int32_t* offsets;      /* [n_slots]: index of the slot's first member in `members`    */
  int32_t* members;      /* [n_members]: key positions, ascending within each slot      */
  float* centroids;      /* [n_slots, d] fp32                                           */
  void* reps;            /* [n_slots, d] representatives in the key format              */
  float* rep_scale;      /* [n_slots] (1.0 unless E4M3)                                 */
  float* rep_f32;        /* [n_slots, d]: representative before quantization (the
                            centroid, or the learned representative with an encoder)     */
  /* Refit statistics and per-key bound state, filled only when `which` is the newest
   * computed epoch e (its refit is the last one launched; the state is overwritten by
   * the next refit).  Otherwise the counts are -1 / 0 and the arrays are untouched. */
  int64_t n_screened;    /* out: keys refit e compared with every warm centroid: its R new
                            keys plus the older keys whose bounds did not certify them    */
  int64_t n_brute;       /* out: of those, keys whose screening list overflowed and that
                            the fixed-order brute force assigned                          */
  int64_t n_bound_keys;  /* out: keys with bound state, positions [S, S + e*R)            */
  int32_t* assign;       /* [n_bound_keys]: warm-centroid slot each key was assigned to   */
  float* ub;             /* [n_bound_keys]: upper bound on the distance to that centroid  */
  float* lb;             /* [n_bound_keys]: lower bound on the distance to every other
                            live warm centroid (+inf when there is none)                 */
} idx_export_buf;

/* Host buffers for idx_import_version: a cluster set built by the caller (a test
 * fixture, or an epoch saved with idx_export_version to rebuild an index).  All
 * pointers are host memory, read during the call only. */
typedef struct {
  int32_t n_slots;          /* slots of the set: e * slots_per_epoch for the imported epoch e    */
  const int32_t* sizes;     /* [n_slots]: members per slot (0 = empty slot, never routed)       */
  const int32_t* members;   /* [sum of sizes]: key positions slot by slot in slot order,
                               strictly ascending within a slot                                 */
  const float* centroids;   /* [n_slots, d] fp32: the centres the next refit starts from         */
  const void* reps;         /* [n_slots, d] representatives in the key format (what is scored)  */
  const float* rep_scale;   /* [n_slots] fp32 scales, finite and > 0 (E4M3); NULL otherwise     */
  const float* rep_f32;     /* [n_slots, d] representative before quantization, or NULL
                               (= centroids); only read back by the exports                    */
} idx_import_buf;

/* Create an index on the current HIP device; *out receives the handle.  Every
 * device allocation of the index happens here (W, the clusters per seal and R are
 * the maintenance parameters of the paper-daily explainer, "索引怎么边算边建？"
 * items 2 and 3); the memory is zero-filled on `stream`, and the call returns once
 * that work is done.
 * Errors: EINVAL / ENOTIMPL for the config fields above, ECAPACITY for the cluster
 * ceiling at max_keys or budgets too large for one rescoring block, ENOMEM when a
 * device allocation fails, EDEVICE when the fill fails. */
int idx_create(const idx_config* cfg, void* stream, idx_index** out);

/* Wait for all work of the device, free everything.  NULL is accepted. */
int idx_destroy(idx_index* ix);

/* Message for the last failing call on this thread ("" if none). */
const char* idx_last_error(void);

int idx_get_info(const idx_index* ix, idx_info* out);

/* Insert n keys at positions [n_keys, n_keys + n) and seal every window that fills.
 * Insert and seal are items 1 and 2 of the paper-daily explainer, "索引怎么边算边建？"
 * (a new key is searchable at once through the open window; every W keys are
 * grouped and appended, older clusters untouched); the seal's size-capped k-means
 * is from the kurate.org assessment, "Core Contribution" item 1.
 *   keys:    device [n, d] in the index dtype; copied, free once the stream passes.
 *   k_scale: device [n] fp32 (> 0) for E4M3, NULL otherwise.
 * Each sealed window runs `seal_iters` Lloyd iterations with the size-capped greedy
 * assignment in exact-order fp32 and appends its clusters (slots w*C .. w*C+C-1);
 * a query sees them once its prefix holds the whole window.
 * Errors: EINVAL (pointers, n < 0), ECAPACITY (n_keys + n > max_keys). */
int idx_build_seal(idx_index* ix, const void* keys, const float* k_scale, int64_t n, void* stream);

/* Launch the next refit if one is due (paper-daily explainer, "索引怎么边算边建？"
 * item 3 and the paragraph after it: every R tokens the whole prefix is regrouped,
 * warm-started, with per-key distance bounds, one round, on another stream; kurate.org
 * assessment, "Core Contribution" item 1).  Due means: sealed windows >= (e+1)*R/W
 * for the next epoch e+1, and the previous epoch has been published.  Refit e+1 covers keys
 * [S, S + (e+1)*R): it starts from the centroids of slots [0, (e+1)*Q) (epoch e plus
 * the newer seal clusters), assigns every covered key to its nearest centroid (ties
 * to the lower slot; Hamerly-style bounds skip keys whose cluster is certified), and
 * replaces each centroid by the exact-order mean of its members.  Work runs on
 * side_stream after everything already enqueued on `stream`.
 *   launched: host out, 1 if a refit was launched, else 0. */
int idx_refit(idx_index* ix, void* stream, void* side_stream, int32_t* launched);

/* Make the launched refit visible: `stream` waits for it; later routes may use the
 * new epoch for queries whose prefix holds all of its keys (the versioning rule of
 * the paper-daily explainer, "索引怎么边算边建？", last paragraph).  published: host
 * out, the newest visible epoch (may be NULL).  A launched refit that is never
 * published is never seen by any query.
 * Errors: ESTATE (poisoned handle). */
int idx_publish(idx_index* ix, void* stream, int32_t* published);

/* Abandon a launched, unpublished refit: it never becomes visible, routes keep
 * using the published epoch, and the next idx_refit computes the same epoch again.
 * `stream` is ordered after the abandoned work (it may still be running on the side
 * stream when this returns).  This is the failure path of a refit whose result must
 * not be used (a caller that detects a fault on its side stream, or a test hook).
 * abandoned: host out, the epoch given up (0 if no refit was in flight; may be NULL).
 * Errors: ESTATE (poisoned handle), EDEVICE. */
int idx_abandon_refit(idx_index* ix, void* stream, int32_t* abandoned);

/* Learned representatives (paper-daily explainer, "代表向量为什么要学？"): clusters
 * keep their distance-based members and centroid, and the representative that
 * queries score becomes mean + alpha * tanh(Wb ReLU(Wa z + ba) + bb) with
 * z = [mean, log n, mean and max over members of W2 ReLU(W1 x + b1) + b2] (128
 * hidden units).  weights: device array of idx_encoder_floats(dim) fp32 values,
 * packed W1 [128, d], b1 [128], W2 [128, 128], b2 [128], Wa [128, d + 257],
 * ba [128], Wb [d, 128], bb [d], alpha; copied on `stream`.  Applies to clusters
 * created by later seals and refits; NULL returns to mean representatives.
 * Errors: ESTATE while a refit is launched but not yet published. */
int64_t idx_encoder_floats(int32_t dim);   /* -1 for an unsupported dim */
int idx_set_encoder(idx_index* ix, const float* weights, void* stream);

/* Routed top-k for T queries at positions q_pos0 .. q_pos0 + T - 1 (paper-daily
 * explainer, "查询时怎么挑候选？": score each cluster representative with the
 * indexer formula, rank high to low, fill the budget with the first keys and the
 * not-yet-grouped keys, then all members of clusters in rank order, truncating the
 * last, score the candidates exactly and keep the top k; the version of each query
 * follows "索引怎么边算边建？", last paragraph).
 *   q:       device [T, H, d] in the index dtype.
 *   q_scale: device [T, H] fp32 (> 0) for E4M3, NULL otherwise.
 *   w:       device [T, H] fp32 head weights (any sign).
 *   k <= budget <= max_budget, k <= max_k, T <= max_queries.
 *   topk_idx: device [T, k] int32 out; topk_score: device [T, k] fp32 out or NULL.
 *   dbg:     host struct of optional device outputs, or NULL.
 * Per query at position p: the version is the newest published epoch whose keys
 * all lie below S + m*W (m = windows inside the prefix) plus the seal clusters of
 * later windows < m; candidates are sinks [0, S), the open window [S + m*W, p] and
 * ranked cluster members until `budget` is reached (sinks and open window count
 * against the budget but are always taken whole).
 * Errors: ECAUSAL (q_pos0 + T > n_keys), ESTATE (a query needs an epoch that is no
 * longer held: the three newest computed epochs are held, two while a refit is in
 * flight), EINVAL / ECAPACITY for sizes. */
int idx_route_topk(idx_index* ix, const void* q, const float* q_scale, const float* w, int64_t q_pos0,
                   int32_t T, int32_t k, int32_t budget, int32_t* topk_idx, float* topk_score,
                   const idx_route_debug* dbg, void* stream);

/* Routed top-k for a decode batch: query t is the token at positions[t] (host array
 * of T int64, any order, repeats allowed) and sees keys 0 .. positions[t].  This is
 * the generation phase of the paper-daily explainer ("它到底在解决什么问题？" and the
 * limitations paragraph on decoding): each generated token's key is inserted with
 * idx_build_seal (n = 1 per step) and its query routed against the same index.
 * Everything else as idx_route_topk.  The positions are read during the call
 * (copied to device memory on `stream`).
 * Errors: EINVAL (null positions or a negative one), ECAUSAL (a position >= n_keys),
 * ESTATE, EINVAL / ECAPACITY as idx_route_topk. */
int idx_route_topk_pos(idx_index* ix, const void* q, const float* q_scale, const float* w,
                       const int64_t* positions, int32_t T, int32_t k, int32_t budget, int32_t* topk_idx,
                       float* topk_score, const idx_route_debug* dbg, void* stream);

/* Exhaustive selection, the method's baseline and the reference answer for recall
 * (paper-daily explainer, "它到底在解决什么问题？": the indexer scores every earlier
 * key and keeps the top k).
 * Workspace bytes idx_exhaustive_topk needs to handle `T` queries in one pass, for
 * every format and every k: per query one row of sample scores (one key in 64 of
 * the prefix, at most 16384) and a list of up to 16384 survivors, plus the sample's
 * rows and room for one full fp32 score row. */
int64_t idx_exhaustive_workspace_bytes(int64_t n_keys, int32_t T);

/* Exhaustive top-k (stateless): query t at position q_pos0 + t scores keys
 * [0, q_pos0 + t] of `keys` and keeps the top k (score descending, ties to the lower
 * position; a prefix shorter than k pads with -1 / -inf).
 *   keys: device [n_keys, d]; k_scale: device [n_keys] for E4M3 else NULL;
 *   q, q_scale, w as in idx_route_topk; q_pos0 + T <= n_keys, q_pos0 + T < 2^31;
 *   1 <= k <= 4096.
 *   workspace: device scratch of workspace_bytes >= idx_exhaustive_workspace_bytes(n_keys, 1);
 *   queries are processed in as many passes as the workspace requires.
 * No score row is written in the common case: a sample of the keys sets a threshold
 * per query, the full pass keeps only the scores at or above it, and those are
 * sorted.  A query whose survivors are fewer than min(k, prefix) or more than the
 * survivor list holds (heavy exact ties, for instance) is redone through a full
 * score row.  The call waits for `stream` once per pass, to read how many queries
 * need that.  Scores are bit-identical to the rescoring of idx_route_topk for the
 * same (q, k). */
int idx_exhaustive_topk(const void* keys, const float* k_scale, int64_t n_keys, int32_t dtype, int32_t heads,
                        int32_t dim, const void* q, const float* q_scale, const float* w, int64_t q_pos0,
                        int32_t T, int32_t k, int32_t* topk_idx, float* topk_score, void* workspace,
                        int64_t workspace_bytes, void* stream);

/* idx_exhaustive_topk for callers that cannot allocate device memory (tight serving
 * loops, harnesses that forbid hipMalloc): the same kernels and the same results,
 * bit for bit, with the workspace kept in a device array that the library holds on
 * every GPU it runs on, IDX_NOALLOC_SCRATCH_BYTES per GPU, until the process ends.
 * The call allocates nothing; like idx_exhaustive_topk it waits for `stream` once
 * per pass.  Queries run in passes of as many as the array holds.  Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller.
 * Errors: as idx_exhaustive_topk, and ECAPACITY when one query's pass exceeds the
 * array (prefixes beyond about 31 million keys: the fallback's full fp32 score row
 * is the largest part); EDEVICE if the array's address cannot be obtained. */
#define IDX_NOALLOC_SCRATCH_BYTES (128ll << 20)
int idx_exhaustive_topk_noalloc(const void* keys, const float* k_scale, int64_t n_keys, int32_t dtype,
                                int32_t heads, int32_t dim, const void* q, const float* q_scale, const float* w,
                                int64_t q_pos0, int32_t T, int32_t k, int32_t* topk_idx, float* topk_score,
                                void* stream);

/* Copy one cluster store to host memory (waits for the device).
 *   which = -1: every sealed window's clusters (slots [0, m*C)), members grouped
 *               per window in slot order;
 *   which = e >= 1: refit epoch e (must be one of the last three computed), slots
 *               [0, e*Q).
 * Call once with NULL arrays to read n_slots / n_members, then with buffers.
 * Errors: EINVAL (null buf), ESTATE (epoch not held), EDEVICE. */
int idx_export(idx_index* ix, int32_t which, idx_export_buf* buf);

/* Copy the version a query whose prefix holds `prefix_len` keys routes over (the
 * versioning rule of the paper-daily explainer, "索引怎么边算边建？", last
 * paragraph) to host memory: the clusters of slots [0, m*C), where m sealed
 * windows lie inside the prefix; slots below e*Q come from its epoch e (the newest
 * published epoch whose keys all lie in the prefix), the others from the seal
 * store.  Members are slot by slot; offsets index into `members`.  The refit fields
 * of buf are not filled (counts -1 / 0).  Waits for the device.
 *   epoch, windows: host out (may be NULL): e and m.
 * Call once with NULL arrays to read n_slots / n_members, then with buffers.
 * Errors: EINVAL (null buf, prefix_len < 1), ECAUSAL (prefix_len > inserted keys),
 * ESTATE (its epoch is no longer held), EDEVICE. */
int idx_export_version(idx_index* ix, int64_t prefix_len, int32_t* epoch, int32_t* windows, idx_export_buf* buf);

/* Install a caller-built cluster set as the next refit epoch e = computed + 1 in
 * place of running that refit, for test fixtures (hand-computed indexes) and to
 * restore an exported epoch.  prefix_len must be e's boundary S + e*R; the keys
 * below it must be inserted and sealed, and no refit may be in flight.  The set
 * must hold e*Q slots whose members cover every key of [S, prefix_len) exactly
 * once.  Representatives are used as given (no encoder runs).  The epoch is then
 * like a computed one: idx_publish makes it visible, and the next refit starts
 * from its centroids and compares every key with every centre (the imported set
 * carries no distance bounds).  The data is copied before the call returns; the
 * member-ordered key copy is built on `stream`.
 * Errors: EINVAL (shape, order, duplicate or missing member, bad scale or code,
 * prefix_len not the boundary, refit_every = 0), ECAUSAL (a member at or beyond
 * prefix_len, which would let a query see a key outside its prefix; or prefix_len
 * beyond the inserted keys), ESTATE (a refit in flight, keys not sealed yet),
 * EDEVICE. */
int idx_import_version(idx_index* ix, int64_t prefix_len, const idx_import_buf* buf, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* IVFTK_H */
