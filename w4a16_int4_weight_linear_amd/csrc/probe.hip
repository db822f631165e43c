// probe.hip -- streaming-read HBM probe: the same-box denominator of the
// weight-streaming kernels.
//
// The infr page (Validated models & performance) measures decode GEMVs as a
// fraction of DRAM peak; the published peak (8 TB/s) is not what one launch can
// read, so the benchmark also reports what a plain read of the same bytes
// achieves here.  The probe reads a buffer once with the access pattern of the
// decode GEMV and nothing else: one 512-thread workgroup per CU, each owning a
// contiguous range, each wave one sequential stream of 1 KiB load instructions
// (16 bytes per lane, non-temporal), four in flight.  Every loaded word is
// folded into one XOR per wave and stored to `sink`, so no load can be dropped.
#include "device.hpp"
#include "kernels.hpp"
#include "launch.hpp"
#include "wave_stamps.hpp"

W4A16_STAMP_STORAGE(w4a16_wave_stamps_probe)

namespace w4a16 {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeWaves = kProbeThreads / 64;
constexpr int kInFlight = 4;

__global__ void __launch_bounds__(kProbeThreads)
stream_read_kernel(const uint8_t* __restrict__ buf, uint64_t items, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  W4A16_STAMP_DECL;   // timeline stamps (profiling build only)
  W4A16_STAMP(0);
  // items (1 KiB each) of this workgroup, then of this wave
  const uint64_t g0 = items * blockIdx.x / gridDim.x, g1 = items * (blockIdx.x + 1) / gridDim.x;
  const uint64_t w0 = g0 + (g1 - g0) * wave / kProbeWaves, w1 = g0 + (g1 - g0) * (wave + 1) / kProbeWaves;
  const uint32_t n = (uint32_t)(w1 - w0);
  // one descriptor per wave covering its own range (below 2^31 bytes per wave)
  const __amdgpu_buffer_rsrc_t r = make_rsrc(buf + (w0 << 10), n << 10);
  const uint32_t voff = (uint32_t)lane * 16u;
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 v[kInFlight];
#pragma unroll
  for (int u = 0; u < kInFlight; ++u)
    v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
        r, voff, (uint32_t)u < n ? (uint32_t)u << 10 : kOutOfRange, kStream));
  for (uint32_t i = 0; i < n; i += kInFlight) {
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      acc ^= v[u];
#ifdef W4A16_WAVE_STAMPS
      if (u == 0 && i == 0) {
        asm volatile("" ::"v"(acc.x));   // the first item has arrived
        W4A16_STAMP(2);
      }
#endif
      const uint32_t nx = i + kInFlight + (uint32_t)u;
      v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          r, voff, nx < n ? nx << 10 : kOutOfRange, kStream));
    }
  }
  W4A16_STAMP(3);
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  // fold the wave's lanes (any order: XOR)
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x ^= (uint32_t)__shfl_xor((int)x, d);
  if (lane == 0) sink[blockIdx.x * kProbeWaves + wave] = x;
  W4A16_STAMP(5);
  W4A16_STAMP_FLUSH(wave);
}

}  // namespace

int probe_sink_words(const DeviceInfo& dev) { return dev.num_cu * kProbeWaves; }

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, const DeviceInfo& dev,
                              hipStream_t stream) {
  const uint64_t items = bytes >> 10;
  if (items == 0) return hipSuccess;
  return launch_kernel(stream_read_kernel, dim3((unsigned)dev.num_cu), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint8_t*>(buf), items, sink);
}

}  // namespace w4a16
