// Backward kernels (placeholder until the adjoint kernels land).
#include "kda_common.hpp"
#include "kda_kernels.h"

namespace kda {
hipError_t launch_state_rebuild(const FwdArgs&, int64_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_chunk(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_reduce(const BwdArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kda
