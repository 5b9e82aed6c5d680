// fa_bwd_mfma.hip -- attention backward on the CDNA4 matrix cores.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

bool bwd_mfma_supported(int, int64_t, int64_t) { return false; }

hipError_t launch_bwd_mfma(const BwdArgs &) { return hipErrorInvalidValue; }

}  // namespace fa
