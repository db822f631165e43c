// grouped_gemm.hip -- placeholder until the MoE grouped GEMM lands.
#include "kernels.hpp"
namespace w4a16 {
hipError_t launch_grouped_gemm(const uint16_t*, const uint32_t*, const uint16_t*, const int32_t*, uint16_t*, int,
                               int, int, int, int, const DeviceInfo&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace w4a16
