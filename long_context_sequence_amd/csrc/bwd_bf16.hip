// Backward ring step (bf16): not implemented yet.
#include "kernels.hpp"

namespace cpa {
hipError_t launch_bwd_bf16(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace cpa
