// api.cpp -- the C ABI of include/w4a16.h: argument validation, per-device
// facts, and dispatch to the gfx950 kernels.
//
// Every check runs on the host before anything is launched, in a fixed order
// (group, shape, null, alignment, size limits, device), so a CPU-only process
// can exercise every validation error without touching a GPU.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "../../include/w4a16.h"
#include "kernels.hpp"

namespace w4a16 {

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];
hipError_t g_dev_err[kMaxDevices];
}  // namespace

hipError_t current_device_info(DeviceInfo* out) {
  int d = 0;
  hipError_t e = hipGetDevice(&d);
  if (e != hipSuccess) return e;
  if (d < 0 || d >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_dev_once[d], [d] {
    DeviceInfo info;
    info.device = d;
    int cu = 0, lds = 0;
    hipError_t err = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, d);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, d);
    info.num_cu = cu;
    info.max_lds = (size_t)lds;
    g_dev[d] = info;
    g_dev_err[d] = err;
  });
  if (g_dev_err[d] != hipSuccess) return g_dev_err[d];
  *out = g_dev[d];
  return hipSuccess;
}

}  // namespace w4a16

namespace {

using w4a16::DeviceInfo;

bool valid_group(int32_t g) { return g == 32 || g == 128; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Activations, packed weights and scales are addressed with 32-bit buffer
// offsets below 2^31 (an offset of 2^31 marks an out-of-range load).
constexpr int64_t kMaxBufferBytes = (int64_t)1 << 31;
constexpr int64_t kMaxDim = (int64_t)1 << 30;
// Experts the routing kernel counts in LDS (one int per expert beside 4 KB).
constexpr int32_t kMaxRouteExperts = 32768;

// A bank of `experts` packed [n, k/8] weight tensors stays below the buffer
// limit (n, k <= 2^30 already; the product is bounded before it is formed).
bool bank_fits(int64_t experts, int64_t n, int64_t k) {
  const int64_t per = n * (k / 2);
  if (per >= kMaxBufferBytes) return false;
  return per == 0 || experts < kMaxBufferBytes / per;
}

int common_dense_checks(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y,
                        int64_t m, int64_t n, int64_t k, int32_t group) {
  if (!valid_group(group)) return W4A16_ERR_GROUP;
  if (m < 0 || n < 0 || k < 0 || k % group) return W4A16_ERR_SHAPE;
  if (m > kMaxDim || n > kMaxDim || k > kMaxDim) return W4A16_ERR_SHAPE;
  if (m == 0 || n == 0) return -1;  // no-op
  if (!y) return W4A16_ERR_NULL;
  if (k > 0 && (!x || !packed || !scales)) return W4A16_ERR_NULL;
  if (!aligned(y, 16) || (k > 0 && (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2))))
    return W4A16_ERR_ALIGN;
  if (n * (k / 2) >= kMaxBufferBytes) return W4A16_ERR_SHAPE;
  if (2 * m * k >= kMaxBufferBytes || 2 * m * n >= kMaxBufferBytes) return W4A16_ERR_SHAPE;
  return W4A16_OK;
}

w4a16_status status_of(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP; }
w4a16_status as_status(int s) { return static_cast<w4a16_status>(s); }

// Which kernels w4a16_gemm runs: up to 32 rows the product is a weight stream
// (m <= 4: the decode GEMV kernels while their plan fits; 5..32: the
// weight-streaming MFMA kernel, one pass per 16 rows); otherwise the tiled GEMM,
// the only one that uses the workspace.
// Fewest activation rows that the decode GEMV runs on the MFMA kernel (below: the
// per-lane dot-product kernel).
#ifndef W4A16_MFMA_MIN_ROWS
#define W4A16_MFMA_MIN_ROWS 2
#endif
constexpr int64_t kMfmaMinRows = W4A16_MFMA_MIN_ROWS;

enum class GemmPath { kGemv, kSkinny, kTiled };

GemmPath gemm_path(int64_t m, int64_t n, int64_t k, int32_t group, const DeviceInfo& dev) {
  if (m <= 4) {
    int mb = 0;
    size_t mlds = 0;
    if (m >= kMfmaMinRows && w4a16::gemv_mfma_plan((int)m, (int)n, (int)k, group, dev, &mb, &mlds)) return GemmPath::kGemv;
    if (w4a16::gemv_plan((int)m, (int)n, (int)k, group, dev).ok) return GemmPath::kGemv;
  }
  if (m <= 32 && w4a16::gemm_skinny_fits((int)(m < 16 ? m : 16), (int)n, (int)k, dev)) return GemmPath::kSkinny;
  return GemmPath::kTiled;
}

// The weight-streaming kernel, one pass per 16 rows (k > 0, arguments checked).
int skinny_passes(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int64_t m,
                  int64_t n, int64_t k, int32_t group, const DeviceInfo& dev, hipStream_t st) {
  for (int64_t m0 = 0; m0 < m; m0 += 16) {
    const int mm = (int)(m - m0 < 16 ? m - m0 : 16);
    const hipError_t e = w4a16::launch_gemm_skinny(x + m0 * k, packed, scales, y + m0 * n, mm, (int)n, (int)k,
                                                   group, dev, st);
    if (e != hipSuccess) return W4A16_ERR_HIP;
  }
  return W4A16_OK;
}

// The decode GEMV kernels for 1 <= m <= 4 (k > 0, arguments already checked).
// Returns -1 when no GEMV plan fits this k (the activations do not fit in LDS).
int gemv_dispatch(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int64_t m,
                  int64_t n, int64_t k, int32_t group, const DeviceInfo& dev, hipStream_t st) {
  // Two to four activation rows: the MFMA kernel (faster there; measured 12% at two
  // rows), while its activations fit in LDS; else the per-lane kernel.
  int mb = 0;
  size_t mlds = 0;
  if (m >= kMfmaMinRows && w4a16::gemv_mfma_plan((int)m, (int)n, (int)k, group, dev, &mb, &mlds))
    return status_of(w4a16::launch_gemv_mfma(x, packed, scales, y, (int)m, (int)n, (int)k, group, mb, mlds, dev, st));
  const w4a16::GemvPlan plan = w4a16::gemv_plan((int)m, (int)n, (int)k, group, dev);
  if (!plan.ok) return -1;
  return status_of(w4a16::launch_gemv(x, packed, scales, y, (int)m, (int)n, (int)k, group, plan, dev, st));
}

}  // namespace

extern "C" {

int w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

const char* w4a16_status_str(int status) {
  switch (status) {
    case W4A16_OK: return "W4A16_OK";
    case W4A16_ERR_NULL: return "W4A16_ERR_NULL: a required pointer is NULL";
    case W4A16_ERR_SHAPE: return "W4A16_ERR_SHAPE: invalid or unsupported sizes";
    case W4A16_ERR_GROUP: return "W4A16_ERR_GROUP: group size must be 32 or 128";
    case W4A16_ERR_ALIGN: return "W4A16_ERR_ALIGN: pointer misaligned";
    case W4A16_ERR_WORKSPACE: return "W4A16_ERR_WORKSPACE: workspace missing or too small";
    case W4A16_ERR_HIP: return "W4A16_ERR_HIP: HIP runtime error";
    case W4A16_ERR_RANGE: return "W4A16_ERR_RANGE: value out of range";
    case W4A16_ERR_TIMEOUT: return "W4A16_ERR_TIMEOUT: a split-K fix-up gave up waiting; outputs were written as NaN";
    default: return "W4A16: unknown status";
  }
}

int64_t w4a16_gemv_max_k(int64_t m, int32_t group) {
  if (m < 1 || m > 4 || !valid_group(group)) return 0;
  DeviceInfo dev;
  if (w4a16::current_device_info(&dev) != hipSuccess) return 0;
  return w4a16::gemv_max_k((int)m, group, dev);
}

w4a16_status w4a16_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int64_t m,
               int64_t n, int64_t k, int32_t group, w4a16_stream_t stream) {
  if (valid_group(group) && m > 4) return W4A16_ERR_SHAPE;
  int c = common_dense_checks(x, packed, scales, y, m, n, k, group);
  if (c < 0) return W4A16_OK;
  if (c != W4A16_OK) return as_status(c);
  DeviceInfo dev;
  if (w4a16::current_device_info(&dev) != hipSuccess) return W4A16_ERR_HIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (k == 0) return status_of(w4a16::launch_zero_fill(y, (size_t)(m * n), st));
  const int r = gemv_dispatch(x, packed, scales, y, m, n, k, group, dev, st);
  if (r >= 0) return as_status(r);
  // k too long for the LDS-staged decode kernels: the weight-streaming kernel
  // stages the activations in chunks and takes any k
  if (!w4a16::gemm_skinny_fits((int)m, (int)n, (int)k, dev)) return W4A16_ERR_SHAPE;
  return as_status(skinny_passes(x, packed, scales, y, m, n, k, group, dev, st));
}

size_t w4a16_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t group) {
  if (!valid_group(group) || m <= 0 || n <= 0 || k <= 0 || k % group) return 0;
  if (m > kMaxDim || n > kMaxDim || k > kMaxDim) return 0;
  DeviceInfo dev;
  if (w4a16::current_device_info(&dev) != hipSuccess) return 0;
  if (gemm_path(m, n, k, group, dev) != GemmPath::kTiled) return 0;
  return w4a16::gemm_workspace_bytes(m, n, k, group, dev);
}

w4a16_status w4a16_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int64_t m,
               int64_t n, int64_t k, int32_t group, void* workspace, size_t workspace_bytes,
               w4a16_stream_t stream) {
  int c = common_dense_checks(x, packed, scales, y, m, n, k, group);
  if (c < 0) return W4A16_OK;
  if (c != W4A16_OK) return as_status(c);
  if (workspace && !aligned(workspace, 16)) return W4A16_ERR_ALIGN;
  DeviceInfo dev;
  if (w4a16::current_device_info(&dev) != hipSuccess) return W4A16_ERR_HIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (k == 0) return status_of(w4a16::launch_zero_fill(y, (size_t)(m * n), st));
  const GemmPath path = gemm_path(m, n, k, group, dev);
  if (path == GemmPath::kGemv) {
    const int r = gemv_dispatch(x, packed, scales, y, m, n, k, group, dev, st);
    return as_status(r < 0 ? W4A16_ERR_SHAPE : r);   // not reached: gemm_path checked the plan
  }
  // one pass per 16 rows (two passes beat the 128-row GEMM tiles up to 32 rows)
  if (path == GemmPath::kSkinny) return as_status(skinny_passes(x, packed, scales, y, m, n, k, group, dev, st));
  const size_t need = w4a16::gemm_workspace_bytes(m, n, k, group, dev);
  if (need && (!workspace || workspace_bytes < need)) return W4A16_ERR_WORKSPACE;
  return status_of(w4a16::launch_gemm(x, packed, scales, y, (int)m, (int)n, (int)k, group,
                                      need ? workspace : nullptr, dev, st));
}

w4a16_status w4a16_gemm_noalloc(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y,
                                int64_t m, int64_t n, int64_t k, int32_t group, w4a16_stream_t stream) {
  int c = common_dense_checks(x, packed, scales, y, m, n, k, group);
  if (c < 0) return W4A16_OK;
  if (c != W4A16_OK) return as_status(c);
  DeviceInfo dev;
  if (w4a16::current_device_info(&dev) != hipSuccess) return W4A16_ERR_HIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (k == 0) return status_of(w4a16::launch_zero_fill(y, (size_t)(m * n), st));
  const GemmPath path = gemm_path(m, n, k, group, dev);
  if (path == GemmPath::kGemv) {
    const int r = gemv_dispatch(x, packed, scales, y, m, n, k, group, dev, st);
    return as_status(r < 0 ? W4A16_ERR_SHAPE : r);
  }
  if (path == GemmPath::kSkinny) return as_status(skinny_passes(x, packed, scales, y, m, n, k, group, dev, st));
  const size_t need = w4a16::gemm_workspace_bytes(m, n, k, group, dev);
  if (need == 0)
    return status_of(w4a16::launch_gemm(x, packed, scales, y, (int)m, (int)n, (int)k, group, nullptr, dev, st));
  // the library's own scratch: this device's copy, looked up once (no allocation)
  void* ws = nullptr;
  size_t cap = 0;
  if (w4a16::gemm_scratch(dev, &ws, &cap) != hipSuccess) return W4A16_ERR_HIP;
  if (need > cap) return W4A16_ERR_WORKSPACE;
  // the previous call's flags and counters may remain (a fix-up that gave up):
  // clear them with a fill kernel (no memset node if the caller captures this)
  const size_t off = w4a16::gemm_workspace_flags_offset(m, n, k, dev);
  uint16_t* flags = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + off);
  const hipError_t e = w4a16::launch_zero_fill(flags, (need - off) / 2, st);
  if (e != hipSuccess) return W4A16_ERR_HIP;
  return status_of(w4a16::launch_gemm(x, packed, scales, y, (int)m, (int)n, (int)k, group, ws, dev, st));
}

w4a16_status w4a16_gemm_workspace_status(void* workspace, size_t workspace_bytes, w4a16_stream_t stream) {
  if (!workspace) return W4A16_ERR_NULL;
  if (!aligned(workspace, 16)) return W4A16_ERR_ALIGN;
  if (workspace_bytes < w4a16::kWorkspaceHeader) return W4A16_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint32_t word = 0;
  const uint32_t zero = 0;
  // synchronous: read the word after the stream's earlier work, then clear it
  if (hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, st) != hipSuccess) return W4A16_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return W4A16_ERR_HIP;
  if (word != 0) {
    if (hipMemcpyAsync(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice, st) != hipSuccess) return W4A16_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return W4A16_ERR_HIP;
    return W4A16_ERR_TIMEOUT;
  }
  return W4A16_OK;
}

w4a16_status w4a16_gemv_swiglu(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int64_t m,
                      int64_t n, int64_t k, int32_t group, w4a16_stream_t stream) {
  if (valid_group(group) && m > 16) return W4A16_ERR_SHAPE;
  if (n > kMaxDim / 2) return W4A16_ERR_SHAPE;
  // the weights have 2n rows; y has n columns (checked as part of the 2n-column bound)
  int c = common_dense_checks(x, packed, scales, y, m, 2 * n, k, group);
  if (c < 0) return W4A16_OK;
  if (c != W4A16_OK) return as_status(c);
  DeviceInfo dev;
  if (w4a16::current_device_info(&dev) != hipSuccess) return W4A16_ERR_HIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (k == 0) return status_of(w4a16::launch_zero_fill(y, (size_t)(m * n), st));   // SiLU(0) * 0
  // Up to four rows: the decode GEMV kernels with the gate/up epilogue (two to
  // four rows on MFMA, as for the plain product), while the activations fit in LDS.
  int mb = 0;
  size_t mlds = 0;
  if (m >= kMfmaMinRows && m <= 4 && w4a16::gemv_mfma_plan((int)m, (int)(2 * n), (int)k, group, dev, &mb, &mlds, true))
    return status_of(w4a16::launch_gemv_mfma(x, packed, scales, y, (int)m, (int)(2 * n), (int)k, group, mb, mlds,
                                             dev, st, true));
  if (m <= 4) {
    const w4a16::GemvPlan plan = w4a16::gemv_plan((int)m, (int)(2 * n), (int)k, group, dev, true);
    if (plan.ok)
      return status_of(w4a16::launch_gemv(x, packed, scales, y, (int)m, (int)(2 * n), (int)k, group, plan, dev, st));
  }
  if (!w4a16::gemm_skinny_fits(5, (int)(2 * n), (int)k, dev)) return W4A16_ERR_SHAPE;
  return status_of(w4a16::launch_swiglu_skinny(x, packed, scales, y, (int)m, (int)n, (int)k, group, dev, st));
}

w4a16_status w4a16_grouped_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const int32_t* offsets,
                       uint16_t* y, int32_t num_experts, int64_t rows, int64_t n, int64_t k, int32_t group,
                       w4a16_stream_t stream) {
  if (!valid_group(group)) return W4A16_ERR_GROUP;
  if (num_experts < 0 || rows < 0 || n < 0 || k < 0 || k % group) return W4A16_ERR_SHAPE;
  if (rows > kMaxDim || n > kMaxDim || k > kMaxDim) return W4A16_ERR_SHAPE;
  if (rows == 0 || n == 0) return W4A16_OK;
  if (num_experts == 0) return W4A16_ERR_SHAPE;  // rows exist but no expert owns them
  if (!y || !offsets) return W4A16_ERR_NULL;
  if (k > 0 && (!x || !packed || !scales)) return W4A16_ERR_NULL;
  if (!aligned(y, 16) || !aligned(offsets, 4) ||
      (k > 0 && (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2))))
    return W4A16_ERR_ALIGN;
  if (!bank_fits(num_experts, n, k)) return W4A16_ERR_SHAPE;
  if (2 * rows * k >= kMaxBufferBytes || 2 * rows * n >= kMaxBufferBytes) return W4A16_ERR_SHAPE;
  DeviceInfo dev;
  if (w4a16::current_device_info(&dev) != hipSuccess) return W4A16_ERR_HIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (k == 0) return status_of(w4a16::launch_zero_fill(y, (size_t)(rows * n), st));
  return status_of(w4a16::launch_grouped_gemm(x, packed, scales, offsets, y, num_experts, (int)rows, (int)n,
                                              (int)k, group, dev, st));
}

w4a16_status w4a16_grouped_gemm_gather(const uint16_t* x, const int32_t* pair_token, const uint32_t* packed,
                              const uint16_t* scales, const int32_t* offsets, uint16_t* y, int32_t num_experts,
                              int64_t rows, int64_t tokens, int64_t n, int64_t k, int32_t group,
                              w4a16_stream_t stream) {
  if (!valid_group(group)) return W4A16_ERR_GROUP;
  if (num_experts < 0 || rows < 0 || tokens < 0 || n < 0 || k < 0 || k % group) return W4A16_ERR_SHAPE;
  if (rows > kMaxDim || tokens > kMaxDim || n > kMaxDim || k > kMaxDim) return W4A16_ERR_SHAPE;
  if (rows == 0 || n == 0) return W4A16_OK;
  if (num_experts == 0) return W4A16_ERR_SHAPE;
  if (!y || !offsets) return W4A16_ERR_NULL;
  if (k > 0 && (!x || !packed || !scales || !pair_token)) return W4A16_ERR_NULL;
  if (!aligned(y, 16) || !aligned(offsets, 4) ||
      (k > 0 && (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(pair_token, 4))))
    return W4A16_ERR_ALIGN;
  if (!bank_fits(num_experts, n, k)) return W4A16_ERR_SHAPE;
  if (2 * tokens * k >= kMaxBufferBytes || 2 * rows * n >= kMaxBufferBytes) return W4A16_ERR_SHAPE;
  DeviceInfo dev;
  if (w4a16::current_device_info(&dev) != hipSuccess) return W4A16_ERR_HIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (k == 0) return status_of(w4a16::launch_zero_fill(y, (size_t)(rows * n), st));
  return status_of(w4a16::launch_grouped_gemm_gather(x, pair_token, (int)tokens, packed, scales, offsets, y,
                                                     num_experts, (int)rows, (int)n, (int)k, group, dev, st));
}

w4a16_status w4a16_grouped_gemm_swiglu(const uint16_t* x, const int32_t* pair_token, const uint32_t* packed,
                                       const uint16_t* scales, const int32_t* offsets, uint16_t* y,
                                       int32_t num_experts, int64_t rows, int64_t tokens, int64_t n, int64_t k,
                                       int32_t group, w4a16_stream_t stream) {
  if (!valid_group(group)) return W4A16_ERR_GROUP;
  if (num_experts < 0 || rows < 0 || tokens < 0 || n < 0 || k < 0 || k % group) return W4A16_ERR_SHAPE;
  if (rows > kMaxDim || tokens > kMaxDim || n > kMaxDim / 2 || k > kMaxDim) return W4A16_ERR_SHAPE;
  if (rows == 0 || n == 0) return W4A16_OK;
  if (num_experts == 0) return W4A16_ERR_SHAPE;
  if (!y || !offsets) return W4A16_ERR_NULL;
  if (k > 0 && (!x || !packed || !scales)) return W4A16_ERR_NULL;
  if (!aligned(y, 16) || !aligned(offsets, 4) ||
      (k > 0 && (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2) ||
                 (pair_token && !aligned(pair_token, 4)))))
    return W4A16_ERR_ALIGN;
  const int64_t x_rows = pair_token ? tokens : rows;   // without pair_token, x is the sorted rows
  if (!bank_fits(num_experts, 2 * n, k)) return W4A16_ERR_SHAPE;
  if (2 * x_rows * k >= kMaxBufferBytes || 2 * rows * n >= kMaxBufferBytes) return W4A16_ERR_SHAPE;
  DeviceInfo dev;
  if (w4a16::current_device_info(&dev) != hipSuccess) return W4A16_ERR_HIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (k == 0) return status_of(w4a16::launch_zero_fill(y, (size_t)(rows * n), st));   // SiLU(0) * 0
  return status_of(w4a16::launch_grouped_gemm_swiglu(x, pair_token, (int)x_rows, packed, scales, offsets, y,
                                                     num_experts, (int)rows, (int)n, (int)k, group, dev, st));
}

w4a16_status w4a16_moe_route(const int32_t* topk_ids, int64_t tokens, int32_t topk, int32_t num_experts, int32_t* offsets,
                    int32_t* pair_token, int32_t* pair_row, w4a16_stream_t stream) {
  if (tokens < 0 || topk < 1 || num_experts < 1 || num_experts > kMaxRouteExperts) return W4A16_ERR_SHAPE;
  if (tokens > kMaxDim || tokens * topk >= ((int64_t)1 << 31)) return W4A16_ERR_SHAPE;
  if (!offsets) return W4A16_ERR_NULL;
  if (tokens > 0 && (!topk_ids || !pair_token || !pair_row)) return W4A16_ERR_NULL;
  if (!aligned(offsets, 4) || (tokens > 0 && (!aligned(topk_ids, 4) || !aligned(pair_token, 4) ||
                                              !aligned(pair_row, 4))))
    return W4A16_ERR_ALIGN;
  DeviceInfo dev;
  if (w4a16::current_device_info(&dev) != hipSuccess) return W4A16_ERR_HIP;
  if (w4a16::moe_route_lds(num_experts) > dev.max_lds) return W4A16_ERR_SHAPE;
  return status_of(w4a16::launch_moe_route(topk_ids, (int)(tokens * topk), topk, num_experts, offsets, pair_token,
                                           pair_row, dev, reinterpret_cast<hipStream_t>(stream)));
}

w4a16_status w4a16_moe_combine(const uint16_t* y_pairs, const int32_t* pair_row, const float* weights, uint16_t* out,
                      int64_t tokens, int32_t topk, int64_t rows, int64_t n, w4a16_stream_t stream) {
  if (tokens < 0 || topk < 1 || rows < 0 || n < 0) return W4A16_ERR_SHAPE;
  if (tokens > kMaxDim || rows > kMaxDim || n > kMaxDim || tokens * topk >= ((int64_t)1 << 31)) return W4A16_ERR_SHAPE;
  if (2 * rows * n >= kMaxBufferBytes || 2 * tokens * n >= kMaxBufferBytes) return W4A16_ERR_SHAPE;
  if (tokens == 0 || n == 0) return W4A16_OK;
  if (!out || !pair_row || !weights || (rows > 0 && !y_pairs)) return W4A16_ERR_NULL;
  if (!aligned(out, 16) || !aligned(pair_row, 4) || !aligned(weights, 4) || (rows > 0 && !aligned(y_pairs, 16)))
    return W4A16_ERR_ALIGN;
  DeviceInfo dev;
  if (w4a16::current_device_info(&dev) != hipSuccess) return W4A16_ERR_HIP;
  return status_of(w4a16::launch_moe_combine(y_pairs, pair_row, weights, out, (int)tokens, topk, (int)n, (int)rows,
                                             reinterpret_cast<hipStream_t>(stream)));
}

int64_t w4a16_hbm_read_probe_sink_words(void) {
  DeviceInfo dev;
  if (w4a16::current_device_info(&dev) != hipSuccess) return 0;
  return w4a16::probe_sink_words(dev);
}

w4a16_status w4a16_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                                  w4a16_stream_t stream) {
  if (bytes % 1024) return W4A16_ERR_SHAPE;
  if (bytes == 0) return W4A16_OK;
  if (!buf || !sink) return W4A16_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return W4A16_ERR_ALIGN;
  DeviceInfo dev;
  if (w4a16::current_device_info(&dev) != hipSuccess) return W4A16_ERR_HIP;
  if (sink_words < (size_t)w4a16::probe_sink_words(dev)) return W4A16_ERR_SHAPE;
  // each wave addresses its own range with 32-bit offsets
  if (bytes / (size_t)w4a16::probe_sink_words(dev) >= (size_t)1 << 30) return W4A16_ERR_SHAPE;
  return status_of(w4a16::launch_stream_read(buf, bytes, sink, dev, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
