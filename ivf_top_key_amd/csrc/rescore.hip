// Format dispatch of the rescoring launchers (rescore.h) and the capacity check.
#include "rescore.h"

namespace ivftk {

#define IVFTK_RESCORE_BY_FORMAT(NAME, ...)                 \
  switch (dtype) {                                       \
    case DT_F32: return NAME##_f32(__VA_ARGS__);         \
    case DT_BF16: return NAME##_bf16(__VA_ARGS__);       \
    case DT_E4M3: return NAME##_e4m3(__VA_ARGS__);       \
    default: return hipErrorInvalidValue;                \
  }

hipError_t launch_cand_score(const RouteParams& p, int dtype, int dim, int ht, int cand_cap, hipStream_t s) {
  IVFTK_RESCORE_BY_FORMAT(launch_cand_score, p, dim, ht, cand_cap, s)
}

hipError_t launch_rescore_topk(const RouteParams& p, int dtype, int dim, int ht, int cand_cap, hipStream_t s) {
  IVFTK_RESCORE_BY_FORMAT(launch_rescore_topk, p, dim, ht, cand_cap, s)
}

hipError_t launch_route_rescore(const RouteParams& p, int dtype, int dim, int ht, int cand_cap, hipStream_t s) {
  IVFTK_RESCORE_BY_FORMAT(launch_route_rescore, p, dim, ht, cand_cap, s)
}

hipError_t launch_route_overflow(const RouteParams& p, int dtype, int dim, int ht, int cand_cap, int max_slots,
                                 hipStream_t s) {
  IVFTK_RESCORE_BY_FORMAT(launch_route_overflow, p, dim, ht, cand_cap, max_slots, s)
}

int route_rescore_max_cands() { return 32 * RS_THREADS; }

bool rescore_fits(int cand_cap, int k) {
  const int cap_pow2 = next_pow2(cand_cap), k_pow2 = next_pow2(k);
  // the region plus the kernels' static LDS: head weights and selection words, and in
  // the fused kernel the cut's words and its ranked clusters' prefix sums and rows
  const size_t fixed = 4096 + (size_t)(2 * LIST_CAP + 1) * 4;
  return cap_pow2 <= 64 * RS_THREADS && route_rescore_region_bytes(cap_pow2, k_pow2) + fixed <= 163840;
}

}  // namespace ivftk
