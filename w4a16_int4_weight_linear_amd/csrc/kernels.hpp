// kernels.hpp -- host-side launchers of the gfx950 W4A16 kernels.
//
// The launchers take already-validated arguments (api.cpp checks every
// argument before calling them) and return the HIP error of the launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

struct DeviceInfo {
  int device = 0;
  int num_cu = 0;
  size_t max_lds = 0;  // bytes of LDS one workgroup may allocate
};

// Cached per-device facts of the current device.
hipError_t current_device_info(DeviceInfo* out);

// ---- decode GEMV (gemv.hip) ----
struct GemvPlan {
  int blocks = 0, rows_base = 0, rows_extra = 0;   // workgroups; row units per workgroup (+1 for the first rows_extra)
  size_t lds = 0;       // bytes of LDS per workgroup
  bool ok = false;      // false: the activations and scales do not fit in LDS
  bool gated = false;   // SwiGLU pairs: row units are (gate, up) row pairs, y gets n / 2 columns
};
// Launch plan (work split and LDS size) for an m x k by n x k problem; gated:
// the n weight rows interleave gate and up rows and y[m, n / 2] = SiLU(gate) * up.
GemvPlan gemv_plan(int m, int n, int k, int group, const DeviceInfo& dev, bool gated = false);
// Largest k (a multiple of group) that has a feasible plan for every n.
int64_t gemv_max_k(int m, int group, const DeviceInfo& dev);
hipError_t launch_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y,
                       int m, int n, int k, int group, const GemvPlan& plan, const DeviceInfo& dev,
                       hipStream_t stream);

// ---- batched decode GEMV on MFMA, 2 <= m <= 4 (gemv_mfma.hip) ----
// Workgroup count and LDS bytes; false if the activations do not fit in LDS.
// gated: the n weight rows interleave SwiGLU gate and up rows and y[m, n / 2] = SiLU(gate) * up.
bool gemv_mfma_plan(int m, int n, int k, int group, const DeviceInfo& dev, int* blocks, size_t* lds,
                    bool gated = false);
hipError_t launch_gemv_mfma(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int m,
                            int n, int k, int group, int blocks, size_t lds, const DeviceInfo& dev,
                            hipStream_t stream, bool gated = false);

// ---- 5 <= m <= 16 rows, weight-streaming on MFMA (gemm_skinny.hip) ----
bool gemm_skinny_fits(int m, int n, int k, const DeviceInfo& dev);
hipError_t launch_gemm_skinny(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int m,
                              int n, int k, int group, const DeviceInfo& dev, hipStream_t stream);
// y [m, n_out] = SiLU(gate) * up, packed/scales holding 2 n_out interleaved rows (1 <= m <= 16).
hipError_t launch_swiglu_skinny(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y,
                                int m, int n_out, int k, int group, const DeviceInfo& dev, hipStream_t stream);

// ---- prefill GEMM (gemm.hip) ----
// The workspace starts with a status word (non-zero after a stream-K fix-up
// gave up waiting), padded to kWorkspaceHeader bytes; the partial tiles follow.
constexpr size_t kWorkspaceHeader = 256;
size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int group, const DeviceInfo& dev);
// The allocation-free entry point's workspace: this device's copy of the
// library's static scratch array (looked up once per device) and its size.
hipError_t gemm_scratch(const DeviceInfo& dev, void** ptr, size_t* bytes);
// Byte offset of the flags and counters (3 * workgroups uint32) in a workspace.
size_t gemm_workspace_flags_offset(int64_t m, int64_t n, int64_t k, const DeviceInfo& dev);
hipError_t launch_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y,
                       int m, int n, int k, int group, void* workspace, const DeviceInfo& dev,
                       hipStream_t stream);

// ---- MoE grouped GEMM (grouped_gemm.hip) ----
hipError_t launch_grouped_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                               const int32_t* offsets, uint16_t* y, int experts, int rows, int n, int k,
                               int group, const DeviceInfo& dev, hipStream_t stream);

// Gather variant: row r of the product reads row pair_token[r] of x [tokens, k].
hipError_t launch_grouped_gemm_gather(const uint16_t* x, const int32_t* pair_token, int tokens,
                                      const uint32_t* packed, const uint16_t* scales, const int32_t* offsets,
                                      uint16_t* y, int experts, int rows, int n, int k, int group,
                                      const DeviceInfo& dev, hipStream_t stream);

// SwiGLU variant: packed/scales hold 2 n_out interleaved (gate, up) rows per expert;
// y [rows, n_out] = SiLU(gate) * up.  pair_token may be null (x sorted, x_rows = rows).
hipError_t launch_grouped_gemm_swiglu(const uint16_t* x, const int32_t* pair_token, int x_rows,
                                      const uint32_t* packed, const uint16_t* scales, const int32_t* offsets,
                                      uint16_t* y, int experts, int rows, int n_out, int k, int group,
                                      const DeviceInfo& dev, hipStream_t stream);

// ---- MoE routing and combine (moe.hip) ----
size_t moe_route_lds(int experts);
hipError_t launch_moe_route(const int32_t* ids, int pairs, int topk, int experts, int32_t* offsets,
                            int32_t* pair_token, int32_t* pair_row, const DeviceInfo& dev, hipStream_t stream);
hipError_t launch_moe_combine(const uint16_t* y_pairs, const int32_t* pair_row, const float* weights, uint16_t* out,
                              int tokens, int topk, int n, int rows, hipStream_t stream);

// ---- streaming-read HBM probe (probe.hip) ----
int probe_sink_words(const DeviceInfo& dev);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, const DeviceInfo& dev,
                              hipStream_t stream);

// ---- y = 0 (the empty sum, k == 0) ----
hipError_t launch_zero_fill(uint16_t* y, size_t count, hipStream_t stream);

}  // namespace w4a16
