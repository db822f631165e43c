// gemv_mfma.hip -- batched decode GEMV (2 <= M <= 4) of the W4A16 int4 layer on fp16 MFMA.
//
// y[m, n] = sum_k x[m, k] * s[n, k / g] * q[n, k] for a few activation rows:
// the np4 column of the LLM170 CUDA/W4A16 page's benchmark tables, where the
// rows of a decode batch share one pass over the weights.  The per-lane dot
// product kernel (gemv.hip) reads 32 activations per activation row from LDS
// for every 32 weights, so at M = 4 LDS bandwidth, not HBM, sets its speed.
// Here the contraction runs on v_mfma_f32_16x16x32_f16 with the weights as the
// A operand (16 weight rows x 32 k) and the activations as the B operand
// (16 columns, of which the first M are real): one 16-byte activation fragment
// now serves 16 weight rows.
//
// * Work split as in the per-lane kernel: each workgroup owns a contiguous
//   range of weight rows (range sizes differ by at most one row).  The range is
//   covered by 16-row blocks; a unit of work is (block, line) where a line is
//   256 k, i.e. 128 bytes of every row.  The workgroup's eight waves take the
//   units round robin and keep one fp32 accumulator tile per block.
// * Weight loads cover whole 128-byte lines (8 rows x 128 bytes per load
//   instruction), go through a per-wave LDS tile into operand layout, and are
//   dequantised in registers (nibble -> fp16 code -> times the group scale).
//   kDepth units are in flight ahead of use.
// * The activations (M rows, all of K) are staged in LDS once per workgroup.
// * At the end the eight waves' accumulators meet in LDS and are added in wave
//   order (deterministic), rounded once to fp16 and stored.
#include <atomic>
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"
#include "launch.hpp"
#include "mfma_operands.hpp"

namespace w4a16 {
namespace {

#ifndef W4A16_GEMVM_DEPTH
#define W4A16_GEMVM_DEPTH 1
#endif
#ifndef W4A16_GEMVM_WG_PER_CU
#define W4A16_GEMVM_WG_PER_CU 2
#endif
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBlocks = 4;                   // 16-row blocks per workgroup
constexpr int KL = 256;                         // k per line: 128 bytes of a weight row
constexpr int kDepth = W4A16_GEMVM_DEPTH;       // units in flight ahead of use
static_assert(kDepth == 1, "the unit loop refills its single ring slot");
constexpr int kTileWave = 16 * 128;             // per-wave transpose tile [16 rows][128 B]
constexpr int kTileBytes = kWaves * kTileWave;

// Staged activation rows are padded with zeros to whole lines (the operand
// reads of a line's last chunk reach its end), plus 16 bytes so consecutive
// rows start on different banks.
__host__ __device__ inline uint32_t x_pitch(int k) { return (uint32_t)((k + KL - 1) / KL) * KL * 2u + 16u; }
// LDS: [activations M x pitch][tiles]; the end-of-kernel partial sums reuse the front.
__host__ inline size_t lds_bytes(int m, int k, int blocks) {
  const size_t main = (size_t)m * x_pitch(k) + kTileBytes;
  (void)blocks;
  const size_t red = (size_t)kWaves * kMaxBlocks * 1024;   // [wave][block][lane] partial tiles
  return main > red ? main : red;
}

// GATED: the N weight rows interleave the gate and up rows of a SwiGLU pair;
// workgroups own whole pairs (rows_base / rows_extra count pairs) and
// y[m, N / 2] = SiLU(gate) * up.
template <int M, int G, bool ALIGNED, bool GATED>
__global__ void __launch_bounds__(kThreads)
gemv_mfma_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
                 const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
                 int N, int K, int rows_base, int rows_extra) {
  constexpr int kUnit = GATED ? 2 : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane >> 4;
  const int li = lane & 15;

  const int blk = blockIdx.x;
  const int nr = kUnit * (rows_base + (blk < rows_extra ? 1 : 0));
  const int r0 = kUnit * (blk * rows_base + (blk < rows_extra ? blk : rows_extra));
  const int nb = (nr + 15) >> 4;                  // 16-row blocks (<= kMaxBlocks, checked on the host)
  const int lines = (K + KL - 1) / KL;
  const int units = nb * lines;

  const uint32_t row_w = (uint32_t)K >> 1;
  const uint32_t spr = (uint32_t)(K / G);
  // descriptors cover exactly the workgroup's rows: rows past the range read zero
  const __amdgpu_buffer_rsrc_t wres =
      make_rsrc(reinterpret_cast<const uint8_t*>(packed) + (size_t)r0 * row_w, (uint32_t)nr * row_w);
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(scales + (size_t)r0 * spr, (uint32_t)nr * spr * 2u);
  const uint32_t xp = x_pitch(K);

  // ---- whole-line loads: instruction i reads rows 8 i .. 8 i + 7 of the block ----
  uint32_t woff[2];
  int klim[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int q = (lane & 7) ^ ((r >> 1) & 7);
    woff[i] = (uint32_t)r * row_w + 16u * (uint32_t)q;
    klim[i] = K - 32 * q;
  }
  // The whole offset is in the vector offset, so the descriptor's range check
  // covers it: rows past the workgroup's range read zero.
  auto load_raw = [&](int b, int s, int i) -> u32x4 {
    const uint32_t off = KL * s < klim[i] ? woff[i] + 16u * (uint32_t)b * row_w + 128u * (uint32_t)s : kOutOfRange;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, off, 0, kStream));
  };
  uint8_t* tile = smem + (size_t)M * xp + wave * kTileWave;
  uint8_t* tile_w = tile + 16 * lane;
  const uint32_t swz = (uint32_t)((li >> 1) & 7);
  const uint8_t* tile_r0 = tile + li * 128 + 16 * ((uint32_t)lq ^ swz);
  const uint8_t* tile_r1 = tile + li * 128 + 16 * ((uint32_t)(4 + lq) ^ swz);

  // ---- scales of operand column li of block b ----
  const uint32_t scol = (uint32_t)li * spr * 2u;
  auto srow = [&](int b) { return scol + 16u * (uint32_t)b * spr * 2u; };
  auto load_s32 = [&](int b, int s) -> u32x4 {       // G = 32 aligned: groups 8 s .. 8 s + 7
    const uint32_t off = 8 * s < (int)spr ? srow(b) + 16u * (uint32_t)s : kOutOfRange;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sres, off, 0, 0));
  };
  auto load_s128 = [&](int b, int s) -> uint32_t {   // G = 128 aligned: groups 2 s, 2 s + 1
    const uint32_t off = 2 * s < (int)spr ? srow(b) + 4u * (uint32_t)s : kOutOfRange;
    return __builtin_amdgcn_raw_buffer_load_b32(sres, off, 0, 0);
  };
  auto load_s16 = [&](int b, int s, int h) -> uint32_t {   // any alignment: k = 256 s + 128 h + 32 lq
    const int k = KL * s + 128 * h + 32 * lq;
    const uint32_t off = k < K ? srow(b) + 2u * (uint32_t)(k / G) : kOutOfRange;
    return __builtin_amdgcn_raw_buffer_load_b16(sres, off, 0, 0);
  };

  struct Slot {
    u32x4 raw[2];
    u32x4 s32;
    uint32_t s128;
    uint32_t s16[2];
  };
  Slot ring[kDepth];
  auto issue = [&](int u, Slot& sl) {
    const int b = u < units ? u / lines : 0;
    const int s = u < units ? u - b * lines : lines;   // past the end: s = lines, no memory access
    sl.raw[0] = load_raw(b, s, 0);
    sl.raw[1] = load_raw(b, s, 1);
    if constexpr (ALIGNED && G == 32) sl.s32 = load_s32(b, s);
    if constexpr (ALIGNED && G == 128) sl.s128 = load_s128(b, s);
    if constexpr (!ALIGNED) { sl.s16[0] = load_s16(b, s, 0); sl.s16[1] = load_s16(b, s, 1); }
  };
#pragma unroll
  for (int d = 0; d < kDepth; ++d) issue(wave + kWaves * d, ring[d]);

  // ---- stage the activations (all of K, nibble-pair order within each 8; zeros to the line end) ----
  // Batches of kXBatch loads per thread are issued before any is written, so
  // the staging costs one memory latency per batch rather than one per piece.
  const int row_pieces = lines * (KL / 8);
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  constexpr int kXBatch = 8;
  for (int p0 = tid; p0 < M * row_pieces; p0 += kXBatch * kThreads) {
    u32x4 v[kXBatch];
#pragma unroll
    for (int j = 0; j < kXBatch; ++j) {
      const int p = p0 + j * kThreads;
      const int m = p / row_pieces;
      const int c = p - m * row_pieces;
      const bool ok = p < M * row_pieces && c < (K >> 3);
      v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          xres, ok ? ((uint32_t)m * (uint32_t)K + (uint32_t)c * 8u) * 2u : kOutOfRange, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < kXBatch; ++j) {
      const int p = p0 + j * kThreads;
      const int m = p / row_pieces;
      const int c = p - m * row_pieces;
      if (p < M * row_pieces) *reinterpret_cast<u32x4*>(smem + (size_t)m * xp + (size_t)c * 16) = permute_a(v[j]);
    }
  }
  __syncthreads();

  f32x4 acc[kMaxBlocks];
#pragma unroll
  for (int b = 0; b < kMaxBlocks; ++b) acc[b] = f32x4{};
  const uint32_t sel_lq = (uint32_t)(2 * lq) * 0x00010001u + (uint32_t)(2 * lq + 1) * 0x01000100u;
  // B operand: activation row li mod M (lanes li >= M give output columns that
  // are never stored; their duplicate addresses cost no extra LDS bandwidth)
  const uint8_t* xfrag = smem + (size_t)(li % M) * xp + 64 * lq;

  // One unit (block b, line s) from ring slot `sl` into the accumulator tile `a`.
  auto unit = [&](int b, int s, Slot& sl, f32x4& a, int u_next) {
    *reinterpret_cast<u32x4*>(tile_w) = sl.raw[0];
    *reinterpret_cast<u32x4*>(tile_w + 1024) = sl.raw[1];
    const u32x4 wq0 = *reinterpret_cast<const u32x4*>(tile_r0);
    const u32x4 wq1 = *reinterpret_cast<const u32x4*>(tile_r1);
    f16x2 sv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if constexpr (!ALIGNED) {
        const _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)sl.s16[h]);
        sv[h] = f16x2{v, v};
      } else if constexpr (G == 32) {
        sv[h] = h ? __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(sl.s32.w, sl.s32.z, sel_lq))
                  : __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(sl.s32.y, sl.s32.x, sel_lq));
      } else {
        sv[h] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(sl.s128, sl.s128, h ? 0x03020302u : 0x01000100u));
      }
    }
    issue(u_next, sl);   // refill the slot (past the end: no memory access)
    const uint8_t* xb = xfrag + 512 * s;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 wv = h ? wq1 : wq0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f16x8 xf = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(xb + 256 * h + 16 * w));
        const uint32_t q = w == 0 ? wv.x : (w == 1 ? wv.y : (w == 2 ? wv.z : wv.w));
        a = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant_word(q, sv[h]), xf, a, 0, 0, 0);
      }
    }
  };
  // The wave's units in order (u = wave, wave + 8, ...), grouped by block so
  // each block's tile is a fixed register set.
  int u = wave;
#pragma unroll
  for (int bb = 0; bb < kMaxBlocks; ++bb) {
    for (; u < units && u < (bb + 1) * lines; u += kWaves) unit(bb, u - bb * lines, ring[0], acc[bb], u + kWaves);
  }

  // ---- combine the waves' partial tiles in wave order, round once, store ----
  __syncthreads();                                 // activations and tiles no longer read
  f32x4* red = reinterpret_cast<f32x4*>(smem);     // [wave][block][lane]
#pragma unroll
  for (int bb = 0; bb < kMaxBlocks; ++bb)
    if (bb < nb) red[(wave * kMaxBlocks + bb) * 64 + lane] = acc[bb];
  __syncthreads();
  if (wave < nb && li < M) {
    f32x4 t = red[wave * 64 + lane];
    for (int w = 1; w < kWaves; ++w) t += red[(w * kMaxBlocks + wave) * 64 + lane];
    // lane holds weight rows 4 lq .. 4 lq + 3 of block `wave` for activation row li
    if constexpr (GATED) {
      // r0 and nr are even, so rows 4 lq + j, 4 lq + j + 1 are one (gate, up) pair
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const int rr = 16 * wave + 4 * lq + j;
        const float g = t[j];
        if (rr < nr) y[(size_t)li * (N >> 1) + ((r0 + rr) >> 1)] = float_to_half_bits(g / (1.f + __expf(-g)) * t[j + 1]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = 16 * wave + 4 * lq + j;
        if (rr < nr) y[(size_t)li * N + r0 + rr] = float_to_half_bits(t[j]);
      }
    }
  }
}

template <int M, int G, bool ALIGNED, bool GATED>
hipError_t launch_m(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int n, int k,
                    int blocks, size_t lds, const DeviceInfo& dev, hipStream_t stream) {
  static std::atomic<uint64_t> attr_set{0};   // one bit per device
  const uint64_t bit = 1ull << (dev.device & 63);
  auto kern = gemv_mfma_kernel<M, G, ALIGNED, GATED>;
  if (!(attr_set.load(std::memory_order_acquire) & bit)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int units = GATED ? n / 2 : n;
  return launch_kernel(kern, dim3(blocks), dim3(kThreads), lds, stream, x, packed, scales, y, n, k, units / blocks,
                       units % blocks);
}

template <int M, bool GATED>
hipError_t launch_g(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int n, int k,
                    int group, int blocks, size_t lds, const DeviceInfo& dev, hipStream_t stream) {
  const int spr = k / group;
  // one vector load per row brings a line's scales when every scale row is
  // 16-byte (g32) or 4-byte (g128) aligned in memory
  const uintptr_t sp = reinterpret_cast<uintptr_t>(scales);
  if (group == 32)
    return spr % 8 == 0 && (sp & 15) == 0
               ? launch_m<M, 32, true, GATED>(x, packed, scales, y, n, k, blocks, lds, dev, stream)
               : launch_m<M, 32, false, GATED>(x, packed, scales, y, n, k, blocks, lds, dev, stream);
  return spr % 2 == 0 && (sp & 3) == 0
             ? launch_m<M, 128, true, GATED>(x, packed, scales, y, n, k, blocks, lds, dev, stream)
             : launch_m<M, 128, false, GATED>(x, packed, scales, y, n, k, blocks, lds, dev, stream);
}

}  // namespace

bool gemv_mfma_plan(int m, int n, int k, const DeviceInfo& dev, int* blocks, size_t* lds, bool gated) {
  if (m < 2 || m > 4 || n <= 0 || k <= 0) return false;
  // Rows are handed out in units: single rows, or (gate, up) row pairs.
  const int unit = gated ? 2 : 1;
  if (n % unit) return false;
  const int units = n / unit;
  // Two workgroups per CU, more if a workgroup would exceed kMaxBlocks row blocks.
  int g = W4A16_GEMVM_WG_PER_CU * dev.num_cu;
  if ((int64_t)g * 16 > n) g = (n + 15) / 16;
  const int per = 16 * kMaxBlocks / unit;
  if ((int64_t)g * per < units) g = (units + per - 1) / per;
  if (g > units) g = units;
  const int rows_max = unit * (units / g + (units % g ? 1 : 0));
  const size_t bytes = lds_bytes(m, k, (rows_max + 15) / 16);
  if (bytes > dev.max_lds) return false;
  *blocks = g;
  *lds = bytes;
  return true;
}

hipError_t launch_gemv_mfma(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int m,
                            int n, int k, int group, int blocks, size_t lds, const DeviceInfo& dev,
                            hipStream_t stream, bool gated) {
  if (gated) {
    switch (m) {
      case 2: return launch_g<2, true>(x, packed, scales, y, n, k, group, blocks, lds, dev, stream);
      case 3: return launch_g<3, true>(x, packed, scales, y, n, k, group, blocks, lds, dev, stream);
      case 4: return launch_g<4, true>(x, packed, scales, y, n, k, group, blocks, lds, dev, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (m) {
    case 2: return launch_g<2, false>(x, packed, scales, y, n, k, group, blocks, lds, dev, stream);
    case 3: return launch_g<3, false>(x, packed, scales, y, n, k, group, blocks, lds, dev, stream);
    case 4: return launch_g<4, false>(x, packed, scales, y, n, k, group, blocks, lds, dev, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a16
