// Backward ring step, bf16 inputs, on gfx950 MFMA (placeholder until the MFMA kernels land).
#include "ra_internal.h"

namespace ra {

hipError_t launch_bwd_bf16(const BwdArgs&, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ra
