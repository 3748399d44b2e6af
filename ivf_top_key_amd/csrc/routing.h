// Device helpers of the routed path shared by its kernels: the version a query
// routes over and the sources its candidates' key rows are gathered from.
#pragma once

#include "dev.h"
#include "params.h"

namespace ivftk {

// ---------------------------------------------------------------------------
// query version (routed path)
// ---------------------------------------------------------------------------
struct QVer {
  int64_t n;       // prefix length
  int m;           // sealed windows inside the prefix
  int r;           // refit epoch used
  int split;       // slots below come from the epoch store
  int cvis;        // visible slots [0, cvis)
  int64_t open_lo; // open window [open_lo, n)
};

__device__ __forceinline__ QVer query_version(const RouteParams& p, int t) {
  QVer v;
  v.n = (p.qpos ? p.qpos[t] : p.q_pos0 + t) + 1;
  v.m = v.n >= p.S ? (int)((v.n - p.S) / p.W) : 0;
  v.r = p.wpr ? min(p.P, v.m / p.wpr) : 0;
  v.split = v.r * p.wpr * p.Cs;
  v.cvis = v.m * p.Cs;
  v.open_lo = (int64_t)p.S + (int64_t)v.m * p.W;
  return v;
}

__device__ __forceinline__ StoreView epoch_store(const RouteParams& p, int r) { return p.ep[r % 3]; }

// ---------------------------------------------------------------------------
// candidate key rows
// ---------------------------------------------------------------------------
// The three sources a query's candidate rows come from: the position-ordered keys
// (sinks and open window), the seal store's member-ordered copy and the query's
// epoch store's copy (CROW_* in params.h).  Rows are clamped below n_keys, which
// bounds every source.
// The per-lane choice of source is arithmetic on byte offsets from the first source
// (masks, no selects), which keeps the compiler from turning it into a table in
// scratch memory.
struct RowSources {
  const uint8_t* key0;
  int64_t dk1, dk2;      // key1 - key0, key2 - key0 (bytes)
  const float* scale0;
  int64_t ds1, ds2;      // scale1 - scale0, scale2 - scale0 (bytes)
};

__device__ __forceinline__ RowSources row_sources(const RouteParams& p, int r) {
  const int e = r % 3;
  const uint8_t* k2 = e == 0 ? p.ep[0].ckeys : (e == 1 ? p.ep[1].ckeys : p.ep[2].ckeys);
  const float* s2 = e == 0 ? p.ep[0].cscale : (e == 1 ? p.ep[1].cscale : p.ep[2].cscale);
  RowSources rs;
  rs.key0 = p.keys;
  rs.dk1 = (int64_t)(uintptr_t)p.seal.ckeys - (int64_t)(uintptr_t)p.keys;
  rs.dk2 = (int64_t)(uintptr_t)k2 - (int64_t)(uintptr_t)p.keys;
  rs.scale0 = p.kscale;
  rs.ds1 = (int64_t)(uintptr_t)p.seal.cscale - (int64_t)(uintptr_t)p.kscale;
  rs.ds2 = (int64_t)(uintptr_t)s2 - (int64_t)(uintptr_t)p.kscale;
  return rs;
}

template <int DT, int D>
__device__ __forceinline__ void load_cand_row(const RowSources& rs, int code, int nk1, uint32_t* buf, float& scl) {
  const int src = (int)((uint32_t)code >> CROW_SHIFT);
  int j = code & CROW_MASK;
  j = j > nk1 ? nk1 : j;
  const int64_t m1 = -(int64_t)(src == 1), m2 = -(int64_t)(src >= 2);
  const uint8_t* kb = rs.key0 + ((rs.dk1 & m1) | (rs.dk2 & m2));
  load_half_row<DT, D>(buf, kb + (size_t)j * Geo<DT, D>::RB);
  if constexpr (DT == DT_E4M3) {
    const float* sb = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(rs.scale0) +
                                                     ((rs.ds1 & m1) | (rs.ds2 & m2)));
    scl = sb[j];
  } else {
    scl = 1.0f;
  }
}

}  // namespace ivftk
