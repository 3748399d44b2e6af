// Rescoring kernels instantiated for one key format (f32).
#include "rescore.h"

namespace ivftk {

IVFTK_RESCORE_LAUNCHERS(f32, IVFTK_DISPATCH_F32)

}  // namespace ivftk
