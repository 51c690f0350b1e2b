// fa_bwd.hip — backward kernels (placeholder until the kernels land).
#include "fa_internal.h"
namespace fa {
hipError_t launch_bwd(const BwdArgs&) { return hipErrorNotSupported; }
}  // namespace fa
