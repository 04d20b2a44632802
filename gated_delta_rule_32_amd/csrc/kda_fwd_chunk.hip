// Chunked MFMA forward (placeholder).
#include "kda_common.hpp"
#include "kda_kernels.h"

namespace kda {
hipError_t launch_fwd_chunk(const FwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kda
