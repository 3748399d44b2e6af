// Host-side launchers of the kernels (each returns the launch status).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "params.h"

namespace ivftk {

enum { EXH_ROWS = 0, EXH_SAMPLE = 1, EXH_STREAM = 2 };
hipError_t launch_exh_score(const ExhParams& p, int mode, int dtype, int dim, int ht, int64_t n_max, hipStream_t s);
hipError_t launch_topk_rows(const ExhParams& p, hipStream_t s);
hipError_t launch_exh_gather(const ExhParams& p, int rb, int64_t ns, hipStream_t s);
hipError_t launch_exh_threshold(const ExhParams& p, hipStream_t s);
hipError_t launch_exh_finalize(const ExhParams& p, hipStream_t s);
hipError_t launch_rep_score(const RouteParams& p, int dtype, int dim, int ht, int max_slots, hipStream_t s);
hipError_t launch_route_select(const RouteParams& p, int max_slots, hipStream_t s);
hipError_t launch_pairs_zero(const RouteParams& p, hipStream_t s);
hipError_t launch_pairs_group(const RouteParams& p, hipStream_t s);
hipError_t launch_cluster_score(const RouteParams& p, int dtype, int dim, int ht, hipStream_t s);
hipError_t launch_cand_score(const RouteParams& p, int dtype, int dim, int ht, int cand_cap, hipStream_t s);
hipError_t launch_rescore_topk(const RouteParams& p, int dtype, int dim, int ht, int cand_cap, hipStream_t s);
// Cut, rescoring and top-k fused (query-major batches); queries whose cluster list
// overflows go to the overflow list, which launch_route_overflow then serves (and
// leaves empty).
hipError_t launch_route_rescore(const RouteParams& p, int dtype, int dim, int ht, int cand_cap, hipStream_t s);
hipError_t launch_route_overflow(const RouteParams& p, int dtype, int dim, int ht, int cand_cap, int max_slots,
                                 hipStream_t s);
// Largest candidate capacity of one call that the fused kernel takes.
int route_rescore_max_cands();
// True if one rescoring block holds cand_cap candidates and k winners.
bool rescore_fits(int cand_cap, int k);
hipError_t launch_seal(const SealParams& p, int dtype, int dim, int n_windows, hipStream_t s);
hipError_t launch_copy_member_rows(const int* members, int64_t j0, int64_t j1, const uint8_t* keys,
                                   const float* kscale, int64_t n_keys, int rb, uint8_t* ckeys, float* cscale,
                                   hipStream_t s);
hipError_t launch_refit(const RefitParams& p, int dtype, int dim, hipStream_t s);
hipError_t launch_encode(const EncParams& p, int dtype, int dim, hipStream_t s);
int64_t encoder_floats(int dim);

}  // namespace ivftk
