// gemm.hip -- placeholder until the MFMA GEMM lands.
#include "kernels.hpp"
namespace w4a16 {
size_t gemm_workspace_bytes(int64_t, int64_t, int64_t, int, const DeviceInfo&) { return 0; }
hipError_t launch_gemm(const uint16_t*, const uint32_t*, const uint16_t*, uint16_t*, int, int, int, int, void*,
                       const DeviceInfo&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_grouped_gemm(const uint16_t*, const uint32_t*, const uint16_t*, const int32_t*, uint16_t*, int,
                               int, int, int, int, const DeviceInfo&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace w4a16
