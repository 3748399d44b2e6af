// Rescoring kernels instantiated for one key format (bf16).
#include "rescore.h"

namespace ivftk {

IVFTK_RESCORE_LAUNCHERS(bf16, IVFTK_DISPATCH_BF16)

}  // namespace ivftk
