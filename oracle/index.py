"""Causal IVF index over indexer keys, with routing and the exhaustive baseline.

Test infrastructure: the CPU oracle.  Sources, all from the paper-daily.com
explainer of AttentionIndex unless noted:

* "查询时怎么挑候选？" (query time): each query scores every cluster
  representative with the indexer formula and ranks clusters high to low.
  The first few keys (sinks) and the not-yet-clustered keys take fixed slots;
  the remaining slots take all members of clusters in rank order, and the
  last cluster that does not fit is truncated.  The indexer then scores the
  candidates and the top k go on to sparse attention.
* "索引怎么边算边建？" (build while computing): (1) insert: a new key joins the
  open window and is a candidate at once; (2) seal: every W keys are
  clustered and appended, older clusters untouched; before the first seal
  queries score exhaustively; (3) refit every R tokens: start from the
  previous centres, add new centres from recent keys, one round of
  assignment plus update.  Every seal or refit makes a new version; a query
  uses a version only when its own prefix holds every key of that version.
* kurate.org assessment, "Core Contribution" item 1: windows are sealed with
  size-capped k-means, and seals and refits are published as versions; a query
  may use a version only if every key it was built from lies in the query's
  prefix.

Readings where the pages are silent (each is a constructor argument or stated
here):
* S sink keys at positions [0, S) are never clustered; windows are
  [S + wW, S + (w+1)W).
* A query at position p sees keys j <= p (its own key included).
* Cluster ids ("slots") are canonical: epoch r (the r-th refit) owns slots
  [0, r*Q) with Q = (R/W) * (W/cluster_size); the clusters of sealed window w
  own slots [w*C_w, (w+1)*C_w) with C_w = W/cluster_size.  Refit r starts from
  the centroids of slots [0, r*Q): epoch r-1's clusters and the seal clusters
  of the windows it has not absorbed yet (those seal centroids are the "new
  centres from recent keys").  A slot with no member is empty ("dead"): it is
  never ranked, never carried into a later warm start, and stays dead.
* The budget counts the sinks and the open window, which are always taken
  whole; clusters fill max(0, budget - |sinks| - |open|) slots.  Ranking ties
  go to the lower slot; a truncated cluster gives its lowest positions.
* Refit r covers the sealed keys [S, B_r), B_r = S + r*R.  The query at
  position p uses the newest published epoch r with B_r <= S + m*W where
  m = floor((p + 1 - S) / W) is the number of windows inside its prefix, plus
  the seal clusters of windows [r*R/W, m); its open window is [S + m*W, p].
* Top-k order: score descending, then position ascending; fewer than k
  candidates pad with position -1 and score -inf.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import codec
from .encoder import encode
from .kmeans import mean_exact, nearest, seal_blocks, seal_window, sqdist_exact
from .score import indexer_scores


class CausalityError(ValueError):
    """A query asked for a key position that has not been inserted."""


@dataclass
class OracleConfig:
    heads: int
    dim: int
    dtype: str
    n_sink: int = 4
    window: int = 1024
    cluster_size: int = 128
    seal_cap: int = 256
    seal_iters: int = 10
    refit_every: int = 16384           # 0 = never refit
    positional: bool = False           # clusters = contiguous blocks (no k-means, no refit)
    encoder: object = None             # learned-representative weights (oracle.encoder), or None

    def __post_init__(self):
        if self.positional and self.refit_every:
            raise ValueError("positional blocks are never refitted (refit_every must be 0)")
        if self.window % self.cluster_size:
            raise ValueError("window must be a multiple of cluster_size")
        if self.refit_every and self.refit_every % self.window:
            raise ValueError("refit_every must be a multiple of window")
        if self.seal_cap * self.n_clusters < self.window:
            raise ValueError("seal_cap * clusters per window must cover the window")

    @property
    def n_clusters(self) -> int:          # clusters per sealed window
        return self.window // self.cluster_size

    @property
    def windows_per_refit(self) -> int:
        return self.refit_every // self.window if self.refit_every else 0

    @property
    def slots_per_refit(self) -> int:
        return self.windows_per_refit * self.n_clusters


@dataclass
class Cluster:
    slot: int
    members: np.ndarray            # int64 key positions, ascending
    centroid: np.ndarray           # fp32 [d]
    rep_raw: np.ndarray            # representative in the key format
    rep_scale: np.float32          # E4M3 scale (1.0 otherwise)
    rep_value: np.ndarray = field(default=None)   # float64 value used for scoring

    @property
    def alive(self) -> bool:
        return self.members.size > 0


def make_cluster(slot: int, members: np.ndarray, centroid: np.ndarray, dtype: str, rep=None) -> Cluster:
    """rep: the representative before quantization (default: the centroid)."""
    raw, sc = codec.quantize_rep(centroid if rep is None else np.asarray(rep, dtype=np.float32), dtype)
    value = codec.decode_codes(raw, dtype).astype(np.float64) * np.float64(sc)
    return Cluster(slot, np.asarray(members, dtype=np.int64), np.asarray(centroid, np.float32).copy(),
                   raw, np.float32(sc), value)


def fill_budget(base: np.ndarray, ranked: list, budget: int):
    """Candidate list for one query.

    base: sinks then open window (always taken whole).  ranked: clusters in
    rank order.  Members of each cluster are added whole while room remains;
    the cluster that does not fit gives its first (lowest-position) members.
    Returns (cand int64 array, used list of (slot, take)).
    """
    cand = [np.asarray(base, dtype=np.int64)]
    room = budget - len(base)
    used = []
    for c in ranked:
        if room <= 0:
            break
        take = min(c.members.size, room)
        cand.append(c.members[:take])
        used.append((c.slot, take))
        room -= take
    return np.concatenate(cand), used


def topk_sorted(cand: np.ndarray, scores: np.ndarray, k: int):
    """Top k of (score desc, position asc), padded with -1 / -inf."""
    order = np.lexsort((cand, -scores))[:k]
    idx = np.full(k, -1, dtype=np.int64)
    sc = np.full(k, -np.inf, dtype=np.float64)
    idx[:order.size] = cand[order]
    sc[:order.size] = scores[order]
    return idx, sc


def query_values(q_raw, q_scale, dtype: str) -> np.ndarray:
    """Stored queries [T, H, d] -> float64 values (E4M3: codes times the (t, h) scale)."""
    v = codec.decode_codes(q_raw, dtype).astype(np.float64)
    if dtype == "e4m3":
        v = v * np.asarray(q_scale, dtype=np.float64)[..., None]
    return v


def key_values(k_raw, k_scale, dtype: str) -> np.ndarray:
    """Stored keys [N, d] -> float64 values for scoring (exact)."""
    v = codec.decode_codes(k_raw, dtype).astype(np.float64)
    if dtype == "e4m3":
        v = v * np.asarray(k_scale, dtype=np.float64)[:, None]
    return v


def exhaustive_topk(kv: np.ndarray, qv: np.ndarray, w: np.ndarray, q_pos0: int, k: int,
                    block: int = 16):
    """Score every key j <= p for the query at position p = q_pos0 + t; keep the top k.

    kv [N, d] float64, qv [T, H, d] float64, w [T, H].  This is the selection
    the indexer makes without any index (paper-daily explainer, "它到底在解决什么
    问题？") and the reference answer for recall.
    """
    T = qv.shape[0]
    idx = np.full((T, k), -1, dtype=np.int64)
    sc = np.full((T, k), -np.inf, dtype=np.float64)
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        n_hi = q_pos0 + t1
        if n_hi > kv.shape[0]:
            raise CausalityError("query position beyond the inserted keys")
        s = indexer_scores(qv[t0:t1], w[t0:t1], kv[:n_hi])
        for t in range(t0, t1):
            n = q_pos0 + t + 1
            idx[t], sc[t] = topk_sorted(np.arange(n, dtype=np.int64), s[t - t0, :n], k)
    return idx, sc


class OracleIndex:
    """The index state: keys, sealed windows, refit epochs, published epoch."""

    def __init__(self, cfg: OracleConfig):
        self.cfg = cfg
        d = cfg.dim
        self.raw = np.zeros((0, d), dtype={"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}[cfg.dtype])
        self.k_scale = np.zeros(0, dtype=np.float32)
        self.X = np.zeros((0, d), dtype=np.float32)      # fp32 keys for clustering
        self.kv = np.zeros((0, d), dtype=np.float64)     # exact keys for scoring
        self.seals = []          # per sealed window: list of n_clusters Cluster
        self.epochs = {0: []}    # epoch r -> list of Cluster for slots [0, r*Q)
        self.computed = 0        # newest epoch computed
        self.published = 0       # newest epoch visible to queries

    # ---- insert + seal --------------------------------------------------
    @property
    def n_keys(self) -> int:
        return self.X.shape[0]

    def append(self, k_raw, k_scale=None):
        """Insert keys at the next positions; seal every window that fills."""
        cfg = self.cfg
        k_raw = np.asarray(k_raw).reshape(-1, cfg.dim).astype(self.raw.dtype)
        n = k_raw.shape[0]
        if cfg.dtype == "e4m3":
            ks = np.asarray(k_scale, dtype=np.float32).reshape(n)
        else:
            ks = np.ones(n, dtype=np.float32)
        self.raw = np.concatenate([self.raw, k_raw])
        self.k_scale = np.concatenate([self.k_scale, ks])
        self.X = np.concatenate([self.X, codec.dequantize(k_raw, ks, cfg.dtype)])
        self.kv = np.concatenate([self.kv, key_values(k_raw, ks, cfg.dtype)])
        while cfg.n_sink + (len(self.seals) + 1) * cfg.window <= self.n_keys:
            self._seal(len(self.seals))

    def _seal(self, w: int):
        cfg = self.cfg
        lo = cfg.n_sink + w * cfg.window
        X = self.X[lo:lo + cfg.window]
        if cfg.positional:
            assign, C, _ = seal_blocks(X, cfg.n_clusters)
        else:
            assign, C, _ = seal_window(X, cfg.n_clusters, cfg.seal_cap, cfg.seal_iters)
        clusters = []
        for i in range(cfg.n_clusters):
            members = lo + np.nonzero(assign == i)[0]
            clusters.append(make_cluster(w * cfg.n_clusters + i, members, C[i], cfg.dtype,
                                         self._learned(members, C[i])))
        self.seals.append(clusters)

    def _learned(self, members, centroid):
        """Learned representative (float32) when an encoder is set, else None (the mean)."""
        if self.cfg.encoder is None or len(members) == 0:
            return None
        return encode(self.X[np.asarray(members, dtype=np.int64)], centroid, self.cfg.encoder).astype(np.float32)

    # ---- refit + publish ------------------------------------------------
    def refit_due(self) -> bool:
        wpr = self.cfg.windows_per_refit
        return wpr > 0 and len(self.seals) >= (self.computed + 1) * wpr

    def boundary(self, r: int) -> int:
        """B_r: keys [S, B_r) are covered by epoch r."""
        return self.cfg.n_sink + r * self.cfg.refit_every

    def warm_start(self, r: int) -> list:
        """Slots [0, r*Q) that refit r starts from: epoch r-1, then the seal
        clusters of windows [(r-1)*R/W, r*R/W)."""
        wpr = self.cfg.windows_per_refit
        warm = list(self.epochs[r - 1])
        for w in range((r - 1) * wpr, r * wpr):
            warm.extend(self.seals[w])
        return warm

    def refit(self) -> int:
        """Compute the next epoch (one assignment + update round). Returns r."""
        if not self.refit_due():
            raise RuntimeError("no refit boundary has been sealed past")
        cfg = self.cfg
        r = self.computed + 1
        warm = self.warm_start(r)
        alive = [c for c in warm if c.alive]
        lo, hi = cfg.n_sink, self.boundary(r)
        X = self.X[lo:hi]
        C = np.stack([c.centroid for c in alive]) if alive else np.zeros((0, cfg.dim), np.float32)
        a = nearest(sqdist_exact(X, C))                   # brute force, ties -> lower slot
        owner = np.array([c.slot for c in alive], dtype=np.int64)[a]
        epoch = []
        for c in warm:
            members = lo + np.nonzero(owner == c.slot)[0] if c.alive else np.zeros(0, np.int64)
            if members.size:
                cent = mean_exact(self.X[members])
            else:
                cent = c.centroid
            epoch.append(make_cluster(c.slot, members, cent, cfg.dtype, self._learned(members, cent)))
        self.epochs[r] = epoch
        self.computed = r
        return r

    def publish(self):
        self.published = self.computed

    def install_epoch(self, clusters: list) -> int:
        """Take a cluster set built elsewhere as the next epoch r, in place of
        computing refit r (test fixtures; the library's import of a version).
        clusters: one Cluster per slot [0, r*Q), slot order.  The set must cover
        the keys [S, B_r) exactly once, none at or beyond B_r.  Returns r."""
        if not self.refit_due():
            raise RuntimeError("no refit boundary has been sealed past")
        r = self.computed + 1
        lo, hi = self.cfg.n_sink, self.boundary(r)
        if [c.slot for c in clusters] != list(range(r * self.cfg.slots_per_refit)):
            raise ValueError("one cluster per slot of the epoch, in slot order")
        allm = np.sort(np.concatenate([c.members for c in clusters]))
        if allm.size and allm.max() >= hi:
            raise CausalityError("a member lies beyond the epoch's prefix")
        if not np.array_equal(allm, np.arange(lo, hi)):
            raise ValueError("the members must cover the epoch's keys exactly once")
        self.epochs[r] = list(clusters)
        self.computed = r
        return r

    # ---- versions --------------------------------------------------------
    def version_of(self, n: int):
        """(epoch r, windows m) seen by a query whose prefix has n keys."""
        cfg = self.cfg
        m = max(0, (n - cfg.n_sink) // cfg.window) if n >= cfg.n_sink else 0
        m = min(m, len(self.seals))
        wpr = cfg.windows_per_refit
        r = min(self.published, m // wpr) if wpr else 0
        return r, m

    def visible(self, n: int) -> list:
        r, m = self.version_of(n)
        out = [c for c in self.epochs[r] if c.alive]
        for w in range(r * self.cfg.windows_per_refit, m):
            out.extend(c for c in self.seals[w] if c.alive)
        return out

    def base_candidates(self, n: int) -> np.ndarray:
        cfg = self.cfg
        _, m = self.version_of(n)
        sinks = np.arange(min(cfg.n_sink, n), dtype=np.int64)
        openw = np.arange(cfg.n_sink + m * cfg.window, n, dtype=np.int64) if n > cfg.n_sink else \
            np.zeros(0, np.int64)
        return np.concatenate([sinks, openw])

    # ---- routing --------------------------------------------------------
    def route(self, q_raw, q_scale, w, q_pos0: int, k: int, budget: int, debug: bool = False):
        """Routed top-k for queries at positions q_pos0 .. q_pos0+T-1."""
        T = np.asarray(q_raw).shape[0]
        return self.route_at(q_raw, q_scale, w, q_pos0 + np.arange(T), k, budget, debug)

    def route_at(self, q_raw, q_scale, w, positions, k: int, budget: int, debug: bool = False):
        """Routed top-k for queries at arbitrary positions (a decode batch: query t is
        the token at positions[t] and sees keys 0 .. positions[t])."""
        cfg = self.cfg
        qv = query_values(q_raw, q_scale, cfg.dtype)
        w = np.asarray(w, dtype=np.float64)
        T = qv.shape[0]
        positions = np.asarray(positions, dtype=np.int64)
        if positions.shape != (T,):
            raise ValueError("one position per query")
        if T and (positions.min() < 0 or positions.max() >= self.n_keys):
            raise CausalityError("query position beyond the inserted keys")
        idx = np.full((T, k), -1, dtype=np.int64)
        sc = np.full((T, k), -np.inf, dtype=np.float64)
        dbg = []
        for t in range(T):
            n = int(positions[t]) + 1
            vis = self.visible(n)
            base = self.base_candidates(n)
            if vis:
                reps = np.stack([c.rep_value for c in vis])
                srep = indexer_scores(qv[t:t + 1], w[t:t + 1], reps)[0]
                slots = np.array([c.slot for c in vis], dtype=np.int64)
                order = np.lexsort((slots, -srep))            # score desc, slot asc
                ranked = [vis[i] for i in order]
            else:
                srep = np.zeros(0)
                slots = np.zeros(0, np.int64)
                ranked = []
            cand, used = fill_budget(base, ranked, budget)
            s = indexer_scores(qv[t:t + 1], w[t:t + 1], self.kv[cand])[0]
            idx[t], sc[t] = topk_sorted(cand, s, k)
            if debug:
                r, m = self.version_of(n)
                dbg.append(dict(n=n, epoch=r, windows=m, slots=slots, srep=srep, used=used,
                                cand=cand, cand_scores=s, base_len=base.size,
                                sizes={c.slot: c.members.size for c in vis}))
        return (idx, sc, dbg) if debug else (idx, sc)

    def exhaustive(self, q_raw, q_scale, w, q_pos0: int, k: int):
        qv = query_values(q_raw, q_scale, self.cfg.dtype)
        return exhaustive_topk(self.kv, qv, np.asarray(w, np.float64), q_pos0, k)
