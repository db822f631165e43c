// gemv.hip -- decode GEMV (1 <= M <= 4) of the W4A16 int4 weight-only layer on gfx950.
//
// y[m, n] = sum_k x[m, k] * s[n, k / g] * q[n, k]: the per-token decode step of
// the W4A16 models on the LLM170 CUDA/W4A16 page (tg column, M = 1; np4 column,
// M = 4).  The infr page (Validated models & performance) puts such decode
// GEMVs at the DRAM bandwidth wall, so the kernel streams the packed weights
// once, at full HBM rate, and keeps the per-byte instruction count low:
//
// * Work split: each 64-lane wavefront owns a contiguous run of output rows
//   (counts differ by at most one across waves); the four waves of a
//   workgroup own consecutive runs.  For a row, lane l covers the 32-weight
//   chunks c = l, l+64, l+128, ...: every load is one 16-byte packed chunk per
//   lane, 1 KiB contiguous per wave.  R rows (1 or 2) are processed together so
//   each activation read from LDS serves R rows.
// * The weights come through buffer loads marked non-temporal, issued a fixed
//   number of chunks ahead of use (a software pipeline over the wave's
//   flattened (row group, chunk) sequence).  The row offset goes in the scalar
//   offset field, so a load costs no vector address arithmetic; loads past the
//   end use an offset outside the buffer and return zero without touching
//   memory.
// * Once per workgroup, the activations (pre-arranged to line up with the
//   nibble pairs below), their per-chunk sums and the group scales of the
//   workgroup's rows are staged in LDS.
// * Dequantisation in registers without conversion instructions: masking a
//   packed word with 0x000F000F leaves the nibbles k = 8j and 8j+4 in the two
//   fp16 halves as the subnormals u * 2^-24 (exact); 0x00F000F0 leaves
//   k = 8j+1, 8j+5 as (16 u) * 2^-24; the same two masks on the word shifted
//   right by 8 give k = 8j+2, 8j+6 and 8j+3, 8j+7.  The fp16 pair dot product
//   (fp32 accumulate) takes these directly.  The code offset is folded in once
//   per chunk: sum x (u - 8) = sum x u - 8 sum x, with sum x read from LDS.
// * The group scale is applied once per chunk in fp32, lane partial sums are
//   combined with DPP row operations plus four lane reads, and the fp32 result
//   is rounded once to fp16.
//
// For integer x, codes and power-of-two scales every step above is exact, so
// such inputs give bit-exact results regardless of summation order.
#include <atomic>

#include "device.hpp"
#include "kernels.hpp"

namespace w4a16 {
namespace {

// Launch shape.  Defaults are the measured best on MI355X; the macros only
// exist so a sweep can rebuild the library with other values.
#ifndef W4A16_GEMV_LOADS_IN_FLIGHT
#define W4A16_GEMV_LOADS_IN_FLIGHT 8
#endif
#ifndef W4A16_GEMV_WAVES_PER_CU
#define W4A16_GEMV_WAVES_PER_CU 8
#endif
constexpr int kGemvThreads = 512;   // 8 wavefronts per workgroup
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kLoadsInFlight = W4A16_GEMV_LOADS_IN_FLIGHT;   // 16-byte loads per lane
constexpr int kWavesPerCU = W4A16_GEMV_WAVES_PER_CU;
constexpr uint32_t kScaleSlack = 256;   // staged past the workgroup's last scale

template <int M>
struct XSumSlots { static constexpr int value = (M == 1) ? 1 : (M == 2 ? 2 : 4); };

// Rows processed together: two when the activation reads from LDS would
// otherwise outrun LDS bandwidth (M >= 3).
template <int M>
struct RowsTogether { static constexpr int value = M >= 3 ? 2 : 1; };

struct GemvLayout {
  uint32_t xs, xsum, sc, total;   // byte offsets of the LDS regions, and the size
};

__host__ __device__ inline GemvLayout gemv_layout(int m, int chunks, int spr, int rows_wg) {
  const int xs_slots = m == 1 ? 1 : (m == 2 ? 2 : 4);
  const uint32_t padded = (uint32_t)((chunks + 63) & ~63);   // whole items of 64 chunks
  GemvLayout l;
  l.xs = 0;
  l.xsum = padded * (uint32_t)m * 64u;
  l.sc = l.xsum + padded * (uint32_t)xs_slots * 4u;
  l.total = l.sc + (((uint32_t)rows_wg * (uint32_t)spr * 2u + 15u) & ~15u) + 32u + kScaleSlack;
  return l;
}

// LDS layout (chunk c = 32 consecutive k of a row; item i = c / 64, lane = c % 64):
//   xs[i][m][j][lane] : 16 bytes = for word j of chunk c, the fp16 pairs
//              (x[8j], x[8j+4]), (x[8j+2], x[8j+6]), (x[8j+1], x[8j+5]),
//              (x[8j+3], x[8j+7]) of activation row m (lanes read consecutive
//              16-byte slots: no bank conflicts, offsets are immediates);
//   xsum[c][slot] : -8 * 2^-20 * (sum of the chunk's 32 activations of row slot), fp32;
//   sc : a 16-byte-aligned copy of the scales of the workgroup's rows (plus slack).
template <int M>
__global__ void __launch_bounds__(kGemvThreads)
gemv_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
            const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
            int n, int k, int gshift, int waves_total, int rows_base, int rows_extra) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int XS = XSumSlots<M>::value;
  constexpr int R = RowsTogether<M>::value;
  constexpr int U = kLoadsInFlight / R;          // items (row group, chunk index) in flight
  const int C = k >> 5;                          // 32-weight chunks per row
  const int IPR = (C + 63) >> 6;                 // chunks per lane per row
  const int spr = C >> gshift;                   // scales per row
  const bool ragged = (C & 63) != 0;

  const int lane = threadIdx.x & 63;
  // wave index, made explicitly wave-uniform so the row bookkeeping lives in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto row_start = [&](int w) { return w * rows_base + (w < rows_extra ? w : rows_extra); };
  const int wg_first = blockIdx.x * kGemvWaves;
  const int gw = wg_first + wave;
  const int r0 = row_start(gw);
  const int nrows = gw < waves_total ? rows_base + (gw < rows_extra ? 1 : 0) : 0;
  const int wg_r0 = row_start(wg_first);
  const int wg_last = wg_first + kGemvWaves < waves_total ? wg_first + kGemvWaves : waves_total;
  const int wg_rows = row_start(wg_last) - wg_r0;
  const GemvLayout L = gemv_layout(M, C, spr, kGemvWaves * (rows_base + 1));

  const int groups = (nrows + R - 1) / R;        // row groups of this wave
  const int total = groups * IPR;                // items

  const uint32_t row_bytes = (uint32_t)k >> 1;
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(packed, (uint32_t)n * row_bytes);
  const uint32_t voff_full = (uint32_t)lane * 16u;
  const bool lane_live_last = !ragged || (lane + ((IPR - 1) << 6)) < C;
  const uint32_t voff_last = lane_live_last ? voff_full : kOutOfRange;

  u32x4 wb[U][R];
  int iss_g = 0, iss_i = 0;
  auto issue = [&](int slot) {
    const uint32_t voff = (iss_i == IPR - 1) ? voff_last : voff_full;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int rl = iss_g * R + j;
      const uint32_t soff = (iss_g < groups && rl < nrows)
                                ? (uint32_t)(r0 + rl) * row_bytes + ((uint32_t)iss_i << 10)
                                : kOutOfRange;
      wb[slot][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, voff, soff, kStream));
    }
    if (++iss_i == IPR) { iss_i = 0; ++iss_g; }
  };

  // Start the weight stream before staging, so the latencies overlap.
#pragma unroll
  for (int u = 0; u < U; ++u) issue(u);

  // Stage the scales of this workgroup's rows: a 16-byte-aligned window of the
  // scale array, loaded whole (reads past the array return zero).
  const uint32_t sc_begin = (uint32_t)wg_r0 * (uint32_t)spr * 2u;
  const uint32_t sc_a0 = sc_begin & ~15u;
  const uint32_t sc_chunks = (sc_begin - sc_a0 + (uint32_t)wg_rows * (uint32_t)spr * 2u + kScaleSlack + 15u) >> 4;
  const uint32_t sc_bytes = (uint32_t)n * (uint32_t)spr * 2u;
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(scales, sc_bytes);
  // Stage x in batches of two (chunk, row slot) pairs per thread, loads first.
  const int pairs = C * M;
  const uint32_t one2 = 0x3C003C00u;  // fp16 pair (1, 1)
  for (int b0 = threadIdx.x; b0 < pairs || (b0 == (int)threadIdx.x && (uint32_t)threadIdx.x < sc_chunks);
       b0 += 2 * kGemvThreads) {
    u32x4 a[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int idx = b0 + h * kGemvThreads;
      if (idx < pairs) {
        const int c = idx / M, m = idx - (idx / M) * M;
        const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)m * k + (size_t)c * 32);
#pragma unroll
        for (int w = 0; w < 4; ++w) a[h][w] = src[w];
      }
    }
    u32x4 sv[2];
    const bool first = b0 == (int)threadIdx.x;
    if (first) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t t = threadIdx.x + h * kGemvThreads;
        sv[h] = load16_tail(sres, t < sc_chunks ? sc_a0 + t * 16u : kOutOfRange, sc_bytes);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int idx = b0 + h * kGemvThreads;
      if (idx < pairs) {
        const int c = idx / M, m = idx - (idx / M) * M;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const u32x4 v = a[h][w];      // x[32c+8w .. +7] as pairs (0,1),(2,3),(4,5),(6,7)
          s = dot2(v.x, one2, s);
          s = dot2(v.y, one2, s);
          s = dot2(v.z, one2, s);
          s = dot2(v.w, one2, s);
          u32x4 p;                      // regrouped to (0,4),(2,6),(1,5),(3,7)
          p.x = (v.x & 0xFFFFu) | (v.z << 16);
          p.y = (v.y & 0xFFFFu) | (v.w << 16);
          p.z = (v.x >> 16) | (v.z & 0xFFFF0000u);
          p.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
          const uint32_t off = (uint32_t)((((c >> 6) * M + m) * 4 + w) * 1024 + (c & 63) * 16);
          *reinterpret_cast<u32x4*>(smem + L.xs + off) = p;
        }
        reinterpret_cast<float*>(smem + L.xsum)[c * XS + m] = s * -0x1p-17f;   // -8 * 2^-20 * sum
      }
    }
    if (first) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t t = threadIdx.x + h * kGemvThreads;
        if (t < sc_chunks) *reinterpret_cast<u32x4*>(smem + L.sc + t * 16u) = sv[h];
      }
    }
  }
  for (uint32_t t = threadIdx.x + 2 * kGemvThreads; t < sc_chunks; t += kGemvThreads) {
    *reinterpret_cast<u32x4*>(smem + L.sc + t * 16u) = load16_tail(sres, sc_a0 + t * 16u, sc_bytes);
  }
  if (M == 3) {
    for (int c = threadIdx.x; c < C; c += kGemvThreads) reinterpret_cast<float*>(smem + L.xsum)[c * XS + 3] = 0.f;
  }
  __syncthreads();

  float acc[R][M];
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[j][m] = 0.f;

  const uint32_t xs_lane = L.xs + (uint32_t)lane * 16u;
  const uint32_t xsum_lane = L.xsum + (uint32_t)lane * (uint32_t)(XS * 4);
  const uint32_t sc_lane = L.sc + (sc_begin - sc_a0) + ((uint32_t)lane >> gshift) * 2u;
  int con_g = 0, con_i = 0;

  for (int base = 0; base < total; base += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u < total) {
        const bool last = con_i == IPR - 1;
        const bool live = !last || lane_live_last;
        const uint8_t* xp = smem + xs_lane + (uint32_t)con_i * (uint32_t)(M * 4096);
        float xsv[XS];
        {
          const uint8_t* sp = smem + xsum_lane + ((uint32_t)con_i << 6) * (uint32_t)(XS * 4);
          if constexpr (XS == 1) {
            xsv[0] = *reinterpret_cast<const float*>(sp);
          } else if constexpr (XS == 2) {
            const float2 v = *reinterpret_cast<const float2*>(sp);
            xsv[0] = v.x; xsv[1] = v.y;
          } else {
            const f32x4 v = *reinterpret_cast<const f32x4*>(sp);
            xsv[0] = v.x; xsv[1] = v.y; xsv[2] = v.z; xsv[3] = v.w;
          }
        }
        u32x4 xv[M][4];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int w = 0; w < 4; ++w) xv[m][w] = *reinterpret_cast<const u32x4*>(xp + (m * 4 + w) * 1024);
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const int rl = min(con_g * R + j, nrows - 1);         // row index within the wave
          const uint32_t sofs = sc_lane + (uint32_t)(r0 + rl - wg_r0) * (uint32_t)spr * 2u
                                + ((((uint32_t)con_i << 6) >> gshift) << 1);
          const float s = half_bits_to_float(*reinterpret_cast<const uint16_t*>(smem + sofs));
          float lo[M], hi[M];
#pragma unroll
          for (int m = 0; m < M; ++m) { lo[m] = 0.f; hi[m] = xsv[m]; }
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t q = w == 0 ? wb[u][j].x : (w == 1 ? wb[u][j].y : (w == 2 ? wb[u][j].z : wb[u][j].w));
            const uint32_t q8 = q >> 8;
            const uint32_t a = q & 0x000F000Fu, b = q8 & 0x000F000Fu;
            const uint32_t c = q & 0x00F000F0u, d = q8 & 0x00F000F0u;
#pragma unroll
            for (int m = 0; m < M; ++m) {
              lo[m] = dot2(xv[m][w].x, a, lo[m]);
              lo[m] = dot2(xv[m][w].y, b, lo[m]);
              hi[m] = dot2(xv[m][w].z, c, hi[m]);
              hi[m] = dot2(xv[m][w].w, d, hi[m]);
            }
          }
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const float t = live ? __builtin_fmaf(lo[m], 16.f, hi[m]) : 0.f;   // 2^-20 sum x (u - 8)
            acc[j][m] = __builtin_fmaf(s, t, acc[j][m]);
          }
        }
        if (last) {
#pragma unroll
          for (int j = 0; j < R; ++j) {
            const int rl = con_g * R + j;
#pragma unroll
            for (int m = 0; m < M; ++m) {
              const float v = wave_sum(acc[j][m]) * 0x1p20f;
              if (lane == m && rl < nrows) y[(size_t)m * n + r0 + rl] = float_to_half_bits(v);
              acc[j][m] = 0.f;
            }
          }
        }
        if (++con_i == IPR) { con_i = 0; ++con_g; }
      }
      issue(u);
    }
  }
}

template <int M>
hipError_t launch_gemv_m(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y,
                         int n, int k, int group, const GemvPlan& plan, const DeviceInfo& dev,
                         hipStream_t stream) {
  static std::atomic<uint64_t> attr_set{0};   // one bit per device
  const uint64_t bit = 1ull << (dev.device & 63);
  if (!(attr_set.load(std::memory_order_acquire) & bit)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<M>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int gshift = group == 128 ? 2 : 0;   // log2(group / 32)
  const int blocks = (plan.waves_total + kGemvWaves - 1) / kGemvWaves;
  (void)hipGetLastError();   // drop an error left by an earlier HIP call of the process
  hipLaunchKernelGGL(gemv_kernel<M>, dim3(blocks), dim3(kGemvThreads), plan.lds, stream, x, packed, scales, y, n,
                     k, gshift, plan.waves_total, plan.rows_base, plan.rows_extra);
  return hipGetLastError();
}

size_t plan_lds(int m, int n, int k, int group, int waves_total) {
  const int C = k / 32;
  const int spr = C / (group / 32);
  const int rows_base = n / waves_total, rows_extra = n % waves_total;
  return gemv_layout(m, C, spr, kGemvWaves * (rows_base + (rows_extra ? 1 : 0))).total;
}

}  // namespace

GemvPlan gemv_plan(int m, int n, int k, int group, const DeviceInfo& dev) {
  GemvPlan p;
  int waves_total = n < dev.num_cu * kWavesPerCU ? n : dev.num_cu * kWavesPerCU;
  // More waves (fewer rows, so fewer staged scales, each) until the LDS fits.
  while (waves_total < n && plan_lds(m, n, k, group, waves_total) > dev.max_lds) {
    waves_total = waves_total * 2 < n ? waves_total * 2 : n;
  }
  p.waves_total = waves_total;
  p.rows_base = n / waves_total;
  p.rows_extra = n % waves_total;
  p.lds = plan_lds(m, n, k, group, waves_total);
  p.ok = p.lds <= dev.max_lds;
  return p;
}

int64_t gemv_max_k(int m, int group, const DeviceInfo& dev) {
  // Fewest rows a workgroup can be given: one per wave.
  int64_t best = 0;
  for (int64_t k = group; k <= (int64_t)1 << 22; k += group) {
    const int C = (int)(k / 32);
    if (gemv_layout(m, C, C / (group / 32), kGemvWaves).total > dev.max_lds) break;
    best = k;
  }
  return best;
}

hipError_t launch_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int m,
                       int n, int k, int group, const GemvPlan& plan, const DeviceInfo& dev, hipStream_t stream) {
  switch (m) {
    case 1: return launch_gemv_m<1>(x, packed, scales, y, n, k, group, plan, dev, stream);
    case 2: return launch_gemv_m<2>(x, packed, scales, y, n, k, group, plan, dev, stream);
    case 3: return launch_gemv_m<3>(x, packed, scales, y, n, k, group, plan, dev, stream);
    case 4: return launch_gemv_m<4>(x, packed, scales, y, n, k, group, plan, dev, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a16
