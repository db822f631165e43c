// grouped_gemm.hip -- MoE grouped GEMM of the W4A16 int4 weight-only layer on gfx950.
//
// The routed-expert layers of the 35B-A3B MoE model on the LLM170 CUDA/W4A16
// page (g32): x holds one row per (token, expert) pair, sorted by expert, and
// the rows offsets[e] .. offsets[e+1]-1 are multiplied by expert e's packed
// weights.  With a few rows per expert (16 on average for 512 tokens routed
// top-8 over 256 experts) the work is bound by streaming the experts' weights
// from HBM, not by the matrix cores, so the kernel is organised around the
// weight stream:
//
// * One 512-thread workgroup per (expert, band of 256 output columns); each
//   of its eight wavefronts owns 32 columns (two 16-column MFMA blocks).  An
//   expert that received no rows is skipped without reading its weights.
// * Each lane streams 16-byte packed chunks (32 consecutive k of one column,
//   one group of 32 or a quarter of a group of 128, so one scale per chunk)
//   a few K chunks ahead of use, and dequantises them in registers exactly as
//   the dense GEMM does (nibble -> fp16 code -> times the group scale).
// * The expert's activation rows are staged through LDS in K chunks of 128,
//   32 rows at a time (two 16-row MFMA blocks, v_mfma_f32_16x16x32_f16); more
//   rows loop over further 32-row passes.
// * Row offsets are read on the device, so the host never synchronises.
#include "device.hpp"
#include "kernels.hpp"
#include "mfma_operands.hpp"

namespace w4a16 {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int BN = 256;                 // output columns per workgroup
constexpr int kWaveN = BN / kWaves;     // 32 columns per wave
constexpr int kNB = kWaveN / 16;        // 16-column MFMA blocks per wave
constexpr int BMP = 32;                 // rows per pass
constexpr int kMB = BMP / 16;
constexpr int KC = 128;                 // k per chunk
constexpr int kAPitch = KC * 2 + 16;    // bytes per LDS row (padded)
constexpr int kATile = BMP * kAPitch;
constexpr int kDepth = 4;               // weight chunks in flight

__global__ void __launch_bounds__(kThreads)
grouped_gemm_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
                    const uint16_t* __restrict__ scales, const int32_t* __restrict__ offsets,
                    uint16_t* __restrict__ y, int N, int K, int gshift, int tiles_n, int rows_total) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2 * kATile];

  const int e = blockIdx.x / tiles_n;
  const int tn = blockIdx.x - e * tiles_n;
  const int row0 = __builtin_amdgcn_readfirstlane(offsets[e]);
  const int rows = __builtin_amdgcn_readfirstlane(offsets[e + 1]) - row0;
  if (rows <= 0) return;                 // no tokens routed here: nothing to read

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane >> 4;              // K quarter of the MFMA operands
  const int li = lane & 15;
  const int nw = tn * BN + wave * kWaveN;

  const int KCH = (K + KC - 1) / KC;
  const uint32_t row_w = (uint32_t)K >> 1;                      // packed bytes per weight row
  const uint32_t spr = (uint32_t)K >> (5 + gshift);            // scales per weight row
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(packed + (size_t)e * N * (K >> 3), (uint32_t)N * row_w);
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(scales + (size_t)e * N * spr, (uint32_t)N * spr * 2u);
  const uint32_t kbytes = (uint32_t)K * 2u;
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(x, (uint32_t)rows_total * kbytes);

  auto load_w = [&](int c, u32x4 (&w)[kNB], uint32_t (&s)[kNB]) {
    const int k = c * KC + lq * 32;
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const int n = nw + b * 16 + li;
      const bool ok = c < KCH && n < N && k < K;
      const uint32_t woff = ok ? (uint32_t)n * row_w + (uint32_t)k / 2u : kOutOfRange;
      const uint32_t soff = ok ? ((uint32_t)n * spr + ((uint32_t)k >> (5 + gshift))) * 2u : kOutOfRange;
      w[b] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, woff, 0, kStream));
      s[b] = __builtin_amdgcn_raw_buffer_load_b16(sres, soff, 0, 0);
    }
  };
  // one 16-byte group of 8 activations per thread: 32 rows x 16 groups
  const int a_row = tid >> 4, a_grp = tid & 15;
  auto load_x = [&](int pass_row0, int c) -> u32x4 {
    const int r = pass_row0 + a_row;
    const int k = c * KC + a_grp * 8;
    const uint32_t off = (r < rows && k < K) ? (uint32_t)(row0 + r) * kbytes + (uint32_t)k * 2u : kOutOfRange;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0));
  };

  for (int p0 = 0; p0 < rows; p0 += BMP) {
    f32x4 acc[kMB][kNB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
      for (int b = 0; b < kNB; ++b) acc[i][b] = f32x4{};

    u32x4 wq[kDepth][kNB];
    uint32_t ws[kDepth][kNB];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) load_w(d, wq[d], ws[d]);
    u32x4 xa = load_x(p0, 0);
    *reinterpret_cast<u32x4*>(As + a_row * kAPitch + a_grp * 16) = permute_a(xa);
    __syncthreads();

    for (int cb = 0; cb < KCH; cb += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int c = cb + d;
        if (c < KCH) {
          const bool more = c + 1 < KCH;
          if (more) xa = load_x(p0, c + 1);
          const uint8_t* at = As + (c & 1) * kATile;
#pragma unroll
          for (int s = 0; s < KC / 32; ++s) {
            f16x8 bop[kNB];
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
              const uint32_t q = s == 0 ? wq[d][b].x : (s == 1 ? wq[d][b].y : (s == 2 ? wq[d][b].z : wq[d][b].w));
              const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)ws[d][b]);
              bop[b] = dequant_word(q, f16x2{sv, sv});
            }
#pragma unroll
            for (int i = 0; i < kMB; ++i) {
              const u32x4 av = *reinterpret_cast<const u32x4*>(at + (i * 16 + li) * kAPitch + (4 * lq + s) * 16);
              const f16x8 aop = __builtin_bit_cast(f16x8, av);
#pragma unroll
              for (int b = 0; b < kNB; ++b)
                acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[b], acc[i][b], 0, 0, 0);
            }
          }
          load_w(c + kDepth, wq[d], ws[d]);   // refill this slot (past the end: no memory access)
          if (more) *reinterpret_cast<u32x4*>(As + ((c + 1) & 1) * kATile + a_row * kAPitch + a_grp * 16) =
              permute_a(xa);
          __syncthreads();
        }
      }
    }

    // lane holds column li of each block, rows 4 * lq + r
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const int n = nw + b * 16 + li;
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < kMB; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = p0 + i * 16 + 4 * lq + r;
          if (m < rows) y[(size_t)(row0 + m) * N + n] = float_to_half_bits(acc[i][b][r]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_grouped_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                               const int32_t* offsets, uint16_t* y, int experts, int rows, int n, int k,
                               int group, const DeviceInfo&, hipStream_t stream) {
  const int tiles_n = (n + BN - 1) / BN;
  const int gshift = group == 128 ? 2 : 0;
  (void)hipGetLastError();   // drop an error left by an earlier HIP call of the process
  hipLaunchKernelGGL(grouped_gemm_kernel, dim3(experts * tiles_n), dim3(kThreads), 0, stream, x, packed, scales,
                     offsets, y, n, k, gshift, tiles_n, rows);
  return hipGetLastError();
}

}  // namespace w4a16
