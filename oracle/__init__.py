"""CPU oracle for causal IVF-routed indexer top-k selection (test infrastructure).

A plain, slow, obviously correct numpy implementation of what the GPU library
computes.  It exists to check the library: only the tests, the smoke check and
the benchmark's CPU-baseline leg may import it.  It shares no code with the HIP
path and imports nothing from the product package.

Sources (AttentionIndex: Accelerating Learned Sparse Attention with a Causal
Inverted-File Index, Park & Hwu, arXiv:2611.02508; cited by page and section):

* paper-daily.com explainer, section "它到底在解决什么问题？" (the problem):
  the DSA indexer scores every prefix key and keeps the top k.
* same page, "查询时怎么挑候选？" (query time): score cluster representatives,
  rank clusters, fill the budget (fixed slots for the first keys and the open
  window, then whole clusters in rank order, truncate the last), rescore the
  candidates, take the top k.
* same page, "索引怎么边算边建？" (build while computing): insert, seal every W
  keys, refit every R tokens from the previous centres with bounds, versioned
  publication.
* same page, "代表向量为什么要学？" (why learn representatives): the score is a
  weighted sum over heads of ReLU'd inner products, so a cluster mean does not
  score like its members (worked example with members -2 and 2).
* kurate.org assessment, "Core Contribution": size-capped k-means at seal,
  warm-started refits with Elkan/Hamerly-style bounds, versioned publication.

Modules: codec (stored formats), score (fp64 indexer score), kmeans
(exact-order fp32 seal/refit arithmetic), encoder (learned representatives),
index (versions, routing, exhaustive baseline), recall.
"""
from . import codec, score, kmeans, encoder, index, recall  # noqa: F401
from .index import OracleConfig, OracleIndex, exhaustive_topk, fill_budget  # noqa: F401
