// fa_bwd.hip -- recompute-based backward kernels (placeholder until the kernels land).
#include "fa_internal.h"

namespace fa {

hipError_t launch_bwd(fa_dtype, int, bool, BwdArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace fa
