// Rescoring kernels instantiated for one key format (e4m3).
#include "rescore.h"

namespace ivftk {

IVFTK_RESCORE_LAUNCHERS(e4m3, IVFTK_DISPATCH_E4M3)

}  // namespace ivftk
