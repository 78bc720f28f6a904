// Backward kernels (placeholder until the dK/dV and dQ passes land).
#include "sdpa_internal.h"

namespace sdpa07 {
hipError_t launch_bwd(const BwdParams&, Dt, int, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace sdpa07
