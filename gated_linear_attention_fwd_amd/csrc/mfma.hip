// mfma.hip -- bf16 matrix-core kernels (placeholder until the MFMA path lands).
#include "common.hpp"
#include "plan.hpp"

namespace gla {
bool mfma_supports(int) { return false; }
hipError_t launch_kv_mfma(const Plan &, const KvArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_readout_mfma(const Plan &, const ReadoutArgs &, hipStream_t) {
  return hipErrorInvalidValue;
}
}  // namespace gla
