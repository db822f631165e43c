// stub_launchers.cpp -- host-only stand-ins for the device launchers, so the C
// ABI's host code (validation, dispatch, packing) links into a plain g++
// executable built with AddressSanitizer and UndefinedBehaviorSanitizer.
// Every launcher reports "no device"; nothing here touches a GPU.
#include "../../w4a16_int4_weight_linear_amd/csrc/kernels.hpp"

namespace w4a16 {

GemvPlan gemv_plan(int, int, int, int, const DeviceInfo&, bool) { return GemvPlan{}; }
int64_t gemv_max_k(int, int, const DeviceInfo&) { return 0; }
hipError_t launch_gemv(const uint16_t*, const uint32_t*, const uint16_t*, uint16_t*, int, int, int, int,
                       const GemvPlan&, const DeviceInfo&, hipStream_t) { return hipErrorNoDevice; }
bool gemv_mfma_plan(int, int, int, int, const DeviceInfo&, int*, size_t*, bool) { return false; }
hipError_t launch_gemv_mfma(const uint16_t*, const uint32_t*, const uint16_t*, uint16_t*, int, int, int, int, int,
                            size_t, const DeviceInfo&, hipStream_t, bool) { return hipErrorNoDevice; }
bool gemm_skinny_fits(int, int, int, const DeviceInfo&) { return false; }
hipError_t launch_gemm_skinny(const uint16_t*, const uint32_t*, const uint16_t*, uint16_t*, int, int, int, int,
                              const DeviceInfo&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_swiglu_skinny(const uint16_t*, const uint32_t*, const uint16_t*, uint16_t*, int, int, int, int,
                                const DeviceInfo&, hipStream_t) { return hipErrorNoDevice; }
size_t gemm_workspace_bytes(int64_t, int64_t, int64_t, int, const DeviceInfo&) { return 0; }
hipError_t gemm_scratch(const DeviceInfo&, void**, size_t*) { return hipErrorNoDevice; }
size_t gemm_workspace_flags_offset(int64_t, int64_t, int64_t, const DeviceInfo&) { return 0; }
hipError_t launch_gemm(const uint16_t*, const uint32_t*, const uint16_t*, uint16_t*, int, int, int, int, void*,
                       const DeviceInfo&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_grouped_gemm(const uint16_t*, const uint32_t*, const uint16_t*, const int32_t*, uint16_t*, int,
                               int, int, int, int, const DeviceInfo&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_grouped_gemm_gather(const uint16_t*, const int32_t*, int, const uint32_t*, const uint16_t*,
                                      const int32_t*, uint16_t*, int, int, int, int, int, const DeviceInfo&,
                                      hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_grouped_gemm_swiglu(const uint16_t*, const int32_t*, int, const uint32_t*, const uint16_t*,
                                      const int32_t*, uint16_t*, int, int, int, int, int, const DeviceInfo&,
                                      hipStream_t) { return hipErrorNoDevice; }
size_t moe_route_lds(int experts) { return (size_t)experts * 4; }
hipError_t launch_moe_route(const int32_t*, int, int, int, int32_t*, int32_t*, int32_t*, const DeviceInfo&,
                            hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_moe_combine(const uint16_t*, const int32_t*, const float*, uint16_t*, int, int, int, int,
                              hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_zero_fill(uint16_t*, size_t, hipStream_t) { return hipErrorNoDevice; }
int probe_sink_words(const DeviceInfo& dev) { return dev.num_cu * 8; }
hipError_t launch_stream_read(const void*, size_t, uint32_t*, const DeviceInfo&, hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace w4a16
