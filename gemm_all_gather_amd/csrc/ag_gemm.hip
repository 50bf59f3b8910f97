// Fused GEMM + multi-destination store (placeholder until the MFMA kernel lands).
#include <hip/hip_runtime.h>

#include "ag_internal.h"

namespace ag {

hipError_t launch_gemm(const GemmLaunch&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ag
