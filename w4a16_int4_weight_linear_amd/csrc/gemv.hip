// gemv.hip -- decode GEMV (1 <= M <= 4) of the W4A16 int4 weight-only layer on gfx950.
//
// y[m, n] = sum_k x[m, k] * s[n, k / g] * q[n, k]: the per-token decode step of
// the W4A16 models on the LLM170 CUDA/W4A16 page (tg column, M = 1; np4 column,
// M = 4).  The infr page (Validated models & performance) puts such decode
// GEMVs at the DRAM bandwidth wall, so the kernel is written to stream the
// packed weights once at full HBM rate and to keep arithmetic off the critical
// path:
//
// * Work split: one 64-lane wavefront owns a contiguous run of output rows
//   (rows are dealt to waves so counts differ by at most one); for a row, lane
//   l covers the 16-weight pieces p = l, l+64, l+128, ... so every load
//   instruction reads 512 contiguous bytes of one row (8-byte loads; K = 5120
//   and K = 17408 give exactly 5 and 17 pieces per lane).  All M activation
//   rows are applied to each weight piece, so the weights are read once for
//   all rows.
// * Weights and scales come through buffer loads marked non-temporal, issued
//   a fixed number of pieces ahead of use (a software pipeline over the
//   wave's flattened (row, piece) sequence); loads past the end fall outside
//   the buffer and return zero without touching memory.
// * Activations are staged once per workgroup in LDS, pre-arranged so that a
//   lane's four reads per word line up with the nibble pairs below, together
//   with per-piece activation sums.
// * Dequantisation in registers without conversion instructions: masking a
//   packed word with 0x000F000F leaves the nibbles k = 8j and 8j+4 in the two
//   fp16 halves as the subnormals u * 2^-24 (exact); 0x00F000F0 leaves
//   k = 8j+1, 8j+5 as (16 u) * 2^-24; the same two masks on the word shifted
//   right by 8 give k = 8j+2, 8j+6 and 8j+3, 8j+7.  The fp16 pair dot product
//   (fp32 accumulate) takes these directly.  The code offset is folded in
//   once per piece: sum x (u - 8) = sum x u - 8 sum x, with sum x read from LDS.
// * The group scale is applied once per piece in fp32, the lanes' partial
//   sums are combined with DPP row operations plus four lane reads, and the
//   fp32 result is rounded once to fp16.
//
// For integer x, codes and power-of-two scales every step above is exact, so
// such inputs give bit-exact results regardless of summation order.
#include <atomic>

#include "device.hpp"
#include "kernels.hpp"

namespace w4a16 {
namespace {

constexpr int kGemvThreads = 256;   // 4 wavefronts per workgroup
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kPrefetch = 16;       // pieces in flight per wave (2 loads each)

template <int M>
struct XSumSlots { static constexpr int value = (M == 1) ? 1 : (M == 2 ? 2 : 4); };

// LDS layout: xs[m][word j in {0,1}][piece p] of 16 bytes holding the fp16
// pairs (x[8j'], x[8j'+4]), (x[8j'+2], x[8j'+6]), (x[8j'+1], x[8j'+5]),
// (x[8j'+3], x[8j'+7]) of word j' = 2p + j; then xsum[p][slot] = -8 * 2^-20 *
// (sum of the piece's 16 activations of row slot), in fp32.
template <int M>
__global__ void __launch_bounds__(kGemvThreads)
gemv_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
            const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
            int n, int k, int gshift, int waves_total, int rows_base, int rows_extra) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int XS = XSumSlots<M>::value;
  const int P = k >> 4;              // 16-weight pieces per row
  const int PPL = (P + 63) >> 6;     // pieces per lane per row
  u32x4* xs = reinterpret_cast<u32x4*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + (size_t)M * 2 * P * 16);

  const int lane = threadIdx.x & 63;
  // wave index, made explicitly wave-uniform so the row bookkeeping lives in SGPRs
  const int gw = blockIdx.x * kGemvWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nrows = gw < waves_total ? rows_base + (gw < rows_extra ? 1 : 0) : 0;
  const int r0 = gw * rows_base + min(gw, rows_extra);
  const int r_end = r0 + nrows;
  const int total = nrows * PPL;

  const __amdgpu_buffer_rsrc_t wres = make_rsrc(packed, (uint32_t)((size_t)n * (size_t)P * 8u));
  const int spr = P >> gshift;       // scales per row
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(scales, (uint32_t)((size_t)n * (size_t)spr * 2u));

  u32x2 wb[kPrefetch];
  uint32_t sb[kPrefetch];
  int iss_row = r0, iss_i = 0;

  auto issue = [&](int slot) {
    const int p = lane + (iss_i << 6);
    const bool live = (iss_row < r_end) && (p < P);
    const uint32_t wo = live ? (uint32_t)(iss_row * P + p) * 8u : kOutOfRange;
    const uint32_t so = live ? (uint32_t)(iss_row * spr + (p >> gshift)) * 2u : kOutOfRange;
    wb[slot] = __builtin_amdgcn_raw_buffer_load_b64(wres, wo, 0, kStream);
    sb[slot] = __builtin_amdgcn_raw_buffer_load_b16(sres, so, 0, kStream);
    if (++iss_i == PPL) { iss_i = 0; ++iss_row; }
  };

  // Start the weight stream before staging the activations so the two
  // latencies overlap.
#pragma unroll
  for (int j = 0; j < kPrefetch; ++j) issue(j);

  // Stage x: one thread per (row slot m, piece p).
  for (int idx = threadIdx.x; idx < M * P; idx += kGemvThreads) {
    const int m = idx / P;
    const int p = idx - m * P;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)m * k + (size_t)p * 16);
    const u32x4 a = src[0];
    const u32x4 b = src[1];
    const uint32_t one2 = 0x3C003C00u;  // fp16 pair (1, 1)
    float s = dot2(a.x, one2, 0.f);
    s = dot2(a.y, one2, s);
    s = dot2(a.z, one2, s);
    s = dot2(a.w, one2, s);
    s = dot2(b.x, one2, s);
    s = dot2(b.y, one2, s);
    s = dot2(b.z, one2, s);
    s = dot2(b.w, one2, s);
    // a = x[16p .. 16p+7] as pairs (0,1),(2,3),(4,5),(6,7); regroup to the
    // nibble pairing (0,4),(2,6),(1,5),(3,7).
    u32x4 pa, pb;
    pa.x = (a.x & 0xFFFFu) | (a.z << 16);
    pa.y = (a.y & 0xFFFFu) | (a.w << 16);
    pa.z = (a.x >> 16) | (a.z & 0xFFFF0000u);
    pa.w = (a.y >> 16) | (a.w & 0xFFFF0000u);
    pb.x = (b.x & 0xFFFFu) | (b.z << 16);
    pb.y = (b.y & 0xFFFFu) | (b.w << 16);
    pb.z = (b.x >> 16) | (b.z & 0xFFFF0000u);
    pb.w = (b.y >> 16) | (b.w & 0xFFFF0000u);
    xs[(m * 2 + 0) * P + p] = pa;
    xs[(m * 2 + 1) * P + p] = pb;
    xsum[p * XS + m] = s * -0x1p-17f;   // -8 * 2^-20 * sum
  }
  if (M == 3) {
    for (int p = threadIdx.x; p < P; p += kGemvThreads) xsum[p * XS + 3] = 0.f;
  }
  __syncthreads();

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;
  int con_row = r0, con_i = 0;

  for (int base = 0; base < total; base += kPrefetch) {
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      if (base + j < total) {
        const int p = lane + (con_i << 6);
        const bool live = p < P;
        const int pc = live ? p : 0;
        const float s = half_bits_to_float(sb[j]);
        const uint32_t w0 = wb[j].x, w1 = wb[j].y;
        const uint32_t l0 = w0 & 0x000F000Fu, h0 = w0 & 0x00F000F0u;
        const uint32_t l0b = (w0 >> 8) & 0x000F000Fu, h0b = (w0 >> 8) & 0x00F000F0u;
        const uint32_t l1 = w1 & 0x000F000Fu, h1 = w1 & 0x00F000F0u;
        const uint32_t l1b = (w1 >> 8) & 0x000F000Fu, h1b = (w1 >> 8) & 0x00F000F0u;
        float xsv[XS];
        if constexpr (XS == 1) {
          xsv[0] = xsum[pc];
        } else if constexpr (XS == 2) {
          const float2 v = reinterpret_cast<const float2*>(xsum)[pc];
          xsv[0] = v.x; xsv[1] = v.y;
        } else {
          const f32x4 v = reinterpret_cast<const f32x4*>(xsum)[pc];
          xsv[0] = v.x; xsv[1] = v.y; xsv[2] = v.z; xsv[3] = v.w;
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const u32x4 xa = xs[(m * 2 + 0) * P + pc];
          const u32x4 xb = xs[(m * 2 + 1) * P + pc];
          float lo = dot2(xa.x, l0, 0.f);
          lo = dot2(xa.y, l0b, lo);
          lo = dot2(xb.x, l1, lo);
          lo = dot2(xb.y, l1b, lo);
          float hi = dot2(xa.z, h0, xsv[m]);
          hi = dot2(xa.w, h0b, hi);
          hi = dot2(xb.z, h1, hi);
          hi = dot2(xb.w, h1b, hi);
          const float t = live ? __builtin_fmaf(lo, 16.f, hi) : 0.f;  // 2^-20 * sum x (u - 8)
          acc[m] = __builtin_fmaf(s, t, acc[m]);
        }
        if (con_i == PPL - 1) {
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const float v = wave_sum(acc[m]) * 0x1p20f;
            if (lane == m) y[(size_t)m * n + con_row] = float_to_half_bits(v);
            acc[m] = 0.f;
          }
        }
        if (++con_i == PPL) { con_i = 0; ++con_row; }
      }
      issue(j);
    }
  }
}

template <int M>
hipError_t launch_gemv_m(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y,
                         int n, int k, int group, const DeviceInfo& dev, hipStream_t stream) {
  const size_t lds = gemv_lds_bytes(M, k);
  static std::atomic<uint64_t> attr_set{0};   // one bit per device
  const uint64_t bit = 1ull << (dev.device & 63);
  if (!(attr_set.load(std::memory_order_acquire) & bit)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<M>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int waves_total = n < dev.num_cu * kGemvWaves ? n : dev.num_cu * kGemvWaves;
  const int blocks = (waves_total + kGemvWaves - 1) / kGemvWaves;
  const int gshift = group == 128 ? 3 : 1;   // log2(group / 16)
  hipLaunchKernelGGL(gemv_kernel<M>, dim3(blocks), dim3(kGemvThreads), lds, stream, x, packed, scales, y, n,
                     k, gshift, waves_total, n / waves_total, n % waves_total);
  return hipGetLastError();
}

}  // namespace

size_t gemv_lds_bytes(int64_t m, int64_t k) {
  const int64_t P = k / 16;
  const int64_t xs_slots = m == 1 ? 1 : (m == 2 ? 2 : 4);
  return (size_t)(m * 2 * P * 16 + P * xs_slots * 4);
}

hipError_t launch_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int m,
                       int n, int k, int group, const DeviceInfo& dev, hipStream_t stream) {
  switch (m) {
    case 1: return launch_gemv_m<1>(x, packed, scales, y, n, k, group, dev, stream);
    case 2: return launch_gemv_m<2>(x, packed, scales, y, n, k, group, dev, stream);
    case 3: return launch_gemv_m<3>(x, packed, scales, y, n, k, group, dev, stream);
    case 4: return launch_gemv_m<4>(x, packed, scales, y, n, k, group, dev, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a16
