// gemm.hip -- prefill GEMM of the W4A16 int4 weight-only layer on gfx950 (fp16 MFMA).
//
// y[m, n] = sum_k x[m, k] * s[n, k / g] * q[n, k] for any M: the prompt
// (prefill) phase of the W4A16 models on the LLM170 CUDA/W4A16 page (pp512,
// pp1024, pp4096 columns).  Here the layer is a dense contraction, so it runs
// on the matrix cores: v_mfma_f32_32x32x16_f16, fp16 inputs, fp32 accumulation.
//
// * Tiles: a 256-thread workgroup owns a 128 x 256 output tile; each of its
//   four wavefronts owns 128 x 64 (4 x 2 MFMA blocks of 32 x 32, 128 fp32
//   accumulators per lane).
// * Activations (the MFMA A operand) are staged through LDS, 128 x 64 per
//   K step, double buffered, padded rows (no bank conflicts), and rearranged
//   on the way in so each lane's 16-byte read lines up with the nibble order
//   of the dequantised weights.
// * Weights (the B operand) never touch LDS: each lane loads one 16-byte
//   packed chunk (32 consecutive k of one output column) per 32-column block
//   and K step straight from memory, one K step ahead of use, and dequantises
//   it in registers: nibble pairs (u_j, u_j+4) are or-ed into the fp16
//   pattern 0x6400 (1024 + u, exact), 1032 is subtracted (the code q, exact)
//   and the group scale multiplied in (one rounding).  A 32-weight chunk never
//   straddles a group of 32 or 128, so one scale serves the whole chunk.
// * The MFMA's K order inside an 8-element slice is free as long as A and B
//   agree; both use the order k = 0,4,1,5,2,6,3,7 of each packed word.
// * Workgroups are mapped so each of the 8 XCDs (private L2 each) works on a
//   contiguous band of output columns: every packed weight is fetched from
//   HBM by one XCD only.
//
// For integer activations, codes and power-of-two scales every product and
// partial sum is exact, so such inputs give bit-exact results.
#include "device.hpp"
#include "kernels.hpp"
#include "mfma_operands.hpp"

namespace w4a16 {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 256, BK = 64;
constexpr int kWaveN = 64;                  // output columns per wave
constexpr int kMB = BM / 32, kNB = kWaveN / 32;
constexpr int kAPitch = BK * 2 + 16;        // bytes per LDS row of the A tile (padded)
constexpr int kATile = BM * kAPitch;        // bytes per A buffer

__global__ void __launch_bounds__(kThreads)
gemm_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
            const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
            int M, int N, int K, int gshift, int tiles_m, int tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2 * kATile];

  // XCD-aware tile order: dispatch deals workgroups to the 8 XCDs round
  // robin; give each XCD a contiguous range of tiles, column-band major.
  const int bid = blockIdx.x;
  const int q8 = tiles >> 3, r8 = tiles & 7;
  const int xcd = bid & 7, local = bid >> 3;
  const int tile = xcd * q8 + (xcd < r8 ? xcd : r8) + local;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;            // K half of the MFMA operands
  const int li = lane & 31;

  const int KT = (K + BK - 1) / BK;
  const uint32_t kbytes = (uint32_t)K * 2u;
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(x, (uint32_t)M * kbytes);
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(packed, (uint32_t)N * ((uint32_t)K >> 1));
  const uint32_t spr = (uint32_t)K >> (5 + gshift);   // scales per row
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(scales, (uint32_t)N * spr * 2u);

  // ---- A tile loader: 1024 chunks of 8 fp16 per K step, 4 per thread.
  auto load_a = [&](int kt, u32x4 (&ra)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + j * kThreads;
      const int row = c >> 3, cg = c & 7;
      const int k = kt * BK + cg * 8;
      const uint32_t off = (m0 + row < M && k < K) ? (uint32_t)(m0 + row) * kbytes + (uint32_t)k * 2u : kOutOfRange;
      ra[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0));
    }
  };
  auto store_a = [&](int buf, const u32x4 (&ra)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + j * kThreads;
      const int row = c >> 3, cg = c & 7;
      *reinterpret_cast<u32x4*>(As + buf * kATile + row * kAPitch + cg * 16) = permute_a(ra[j]);
    }
  };

  // ---- B loader: per 32-column block, one 16-byte chunk and one scale.
  const int nw = n0 + wave * kWaveN;
  auto load_b = [&](int kt, u32x4 (&rb)[kNB], uint32_t (&rs)[kNB]) {
    const int k = kt * BK + h * 32;
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const int n = nw + b * 32 + li;
      const bool ok = n < N && k < K;
      const uint32_t woff = ok ? (uint32_t)n * ((uint32_t)K >> 1) + (uint32_t)k / 2u : kOutOfRange;
      const uint32_t soff = ok ? ((uint32_t)n * spr + ((uint32_t)k >> (5 + gshift))) * 2u : kOutOfRange;
      rb[b] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, woff, 0, kStream));
      rs[b] = __builtin_amdgcn_raw_buffer_load_b16(sres, soff, 0, 0);
    }
  };

  f32x16 acc[kMB][kNB];
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int b = 0; b < kNB; ++b) acc[i][b] = f32x16{};

  u32x4 ra[4];
  u32x4 rb[kNB], rb_next[kNB];
  uint32_t rs[kNB], rs_next[kNB];
  load_a(0, ra);
  load_b(0, rb, rs);
  store_a(0, ra);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      load_a(kt + 1, ra);
      load_b(kt + 1, rb_next, rs_next);
    }
    const uint8_t* at = As + buf * kATile;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      f16x8 bop[kNB];
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        const uint32_t q = s == 0 ? rb[b].x : (s == 1 ? rb[b].y : (s == 2 ? rb[b].z : rb[b].w));
        const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)rs[b]);
        bop[b] = dequant_word(q, f16x2{sv, sv});
      }
#pragma unroll
      for (int i = 0; i < kMB; ++i) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(at + (i * 32 + li) * kAPitch + (4 * h + s) * 16);
        const f16x8 aop = __builtin_bit_cast(f16x8, av);
#pragma unroll
        for (int b = 0; b < kNB; ++b)
          acc[i][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, bop[b], acc[i][b], 0, 0, 0);
      }
    }
    if (more) {
      store_a(buf ^ 1, ra);
#pragma unroll
      for (int b = 0; b < kNB; ++b) { rb[b] = rb_next[b]; rs[b] = rs_next[b]; }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds column li of each block, rows 8*(r/4) + 4*h + r%4.
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int n = nw + b * 32 + li;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M) y[(size_t)m * N + n] = float_to_half_bits(acc[i][b][r]);
      }
    }
  }
}

}  // namespace

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t, int, const DeviceInfo&) { return 0; }

hipError_t launch_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int m,
                       int n, int k, int group, void*, const DeviceInfo&, hipStream_t stream) {
  const int tiles_m = (m + BM - 1) / BM;
  const int tiles_n = (n + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n;
  const int gshift = group == 128 ? 2 : 0;
  hipLaunchKernelGGL(gemm_kernel, dim3(tiles), dim3(kThreads), 0, stream, x, packed, scales, y, m, n, k, gshift,
                     tiles_m, tiles);
  return hipGetLastError();
}

}  // namespace w4a16
