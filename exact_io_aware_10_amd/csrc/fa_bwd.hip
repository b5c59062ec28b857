// placeholder until the backward kernels land
#include "fa_internal.h"
namespace fa {
hipError_t launch_bwd(const BwdArgs&, int, bool, bool, bool, hipStream_t) { return hipErrorNotSupported; }
}
