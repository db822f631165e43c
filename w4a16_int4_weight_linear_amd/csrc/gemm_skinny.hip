// gemm_skinny.hip -- W4A16 product for up to 16 rows per pass on fp16 MFMA (weight-streaming).
//
// A decode step batching 5-32 sequences (the pages' continuous batching; the
// caller makes one pass per 16 rows) is still a pass over the weights: at M = 16 and 4-bit weights there are 8 FLOP per weight
// byte, far below the MFMA/HBM ridge.  The 128 x 256 tiles of the prefill GEMM
// compute mostly padding there and spread only N / 256 tiles over the CUs, so
// this kernel streams the weights once, one workgroup per CU:
//
// * Each workgroup (one per CU) owns a contiguous range of weight rows (sizes
//   differ by at most one row), covered by 16-row blocks.  A unit of work is
//   (block, line), a line being 256 k = 128 bytes of every row of the block.
// * The activations (up to 16 rows) no longer fit in LDS whole, so they are
//   staged in chunks of 8 lines (2048 k), double buffered, one barrier per
//   chunk; the next chunk is loaded into registers while the current one is
//   used.  Within a chunk the units go round robin to the 8 waves (balanced
//   except in a partial last chunk).
// * Weight loads cover whole 128-byte lines and go through a per-wave LDS tile
//   into operand layout, dequantised in registers; the weights are the A
//   operand of v_mfma_f32_16x16x32_f16 and the 16 activation rows (zero past M)
//   the B operand.
// * The eight waves' accumulator tiles are added in wave order in LDS
//   (deterministic) and rounded once to fp16.
// * The same kernel serves the fused gate/up projection of a SwiGLU feed-forward
//   (gemv_swiglu): the epilogue applies SiLU to the gate row and multiplies by
//   the up row before the single rounding, so the 2 x M x N intermediate never
//   reaches HBM.
#include <atomic>

#include "device.hpp"
#include "kernels.hpp"
#include "launch.hpp"
#include "mfma_operands.hpp"

namespace w4a16 {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBlocks = 6;                    // 16-row blocks per workgroup (96 rows)
constexpr int KL = 256;                          // k per line
constexpr int kChunkLines = 8;                   // lines per staged activation chunk
constexpr int KCH = KL * kChunkLines;            // 2048 k per chunk
constexpr int kRows = 16;                        // activation rows staged (B operand columns)
constexpr int kXPitch = KCH * 2 + 16;            // bytes per staged row: rows shift by 4 banks
constexpr int kXBuf = kRows * kXPitch;
constexpr int kXPieces = kRows * KCH / 8 / kThreads;   // 16-byte pieces per thread and chunk
constexpr int kTileWave = 16 * 128;
constexpr int kTileBase = 2 * kXBuf;
constexpr int kGroupsPerChunk = KCH / 128;        // 128-k groups per staged chunk
constexpr int kXSumBuf = kRows * kGroupsPerChunk * 4;   // biased activation sums of one chunk (g128 path)
constexpr int kXSumBase = kTileBase + kWaves * kTileWave;
constexpr int kLds = kXSumBase + 2 * kXSumBuf;
static_assert(kXPieces == 8, "staging assumes eight pieces per thread");
static_assert(kLds <= 160 * 1024, "LDS");
static_assert(kWaves * kMaxBlocks * 1024 <= kLds, "the final partial tiles reuse the LDS");

// SWIGLU: the 2 n weight rows interleave gate (even) and up (odd) rows of n
// outputs; workgroup ranges are whole pairs and the epilogue writes
// y[m, i] = SiLU(gate_i) * up_i (fp32, rounded once) instead of both rows.
template <int G, bool ALIGNED, bool SWIGLU>
__global__ void __launch_bounds__(kThreads)
gemm_skinny_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
                   const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
                   int M, int N, int K, int rows_base, int rows_extra) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane >> 4;
  const int li = lane & 15;
  // Group 128 with aligned scales: every MFMA's 32 k lie in one group (k =
  // 128 h + 32 lq + 8 w + j for MFMA (h, w)), so the codes enter it without
  // conversion (one AND-OR per pair, see kBiasPair) and the scale is applied once
  // per group to the MFMA results; otherwise each word is dequantised with its
  // scale before the MFMA.
  constexpr bool kEnc = G == 128 && ALIGNED;

  // rows_base / rows_extra count whole rows, or whole (gate, up) row pairs
  constexpr int kUnit = SWIGLU ? 2 : 1;
  const int blk = blockIdx.x;
  const int nr = kUnit * (rows_base + (blk < rows_extra ? 1 : 0));
  const int r0 = kUnit * (blk * rows_base + (blk < rows_extra ? blk : rows_extra));
  const int nb = (nr + 15) >> 4;                   // <= kMaxBlocks (the host sizes the grid)
  const int lines = (K + KL - 1) / KL;
  const int chunks = (lines + kChunkLines - 1) / kChunkLines;

  const uint32_t row_w = (uint32_t)K >> 1;
  const uint32_t spr = (uint32_t)(K / G);
  const __amdgpu_buffer_rsrc_t wres =
      make_rsrc(reinterpret_cast<const uint8_t*>(packed) + (size_t)r0 * row_w, (uint32_t)nr * row_w);
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(scales + (size_t)r0 * spr, (uint32_t)nr * spr * 2u);
  const uint32_t kbytes = (uint32_t)K * 2u;
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(x, (uint32_t)M * kbytes);

  // ---- whole-line weight loads: instruction i reads rows 8 i .. 8 i + 7 of the block ----
  uint32_t woff[2];
  int klim[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int q = (lane & 7) ^ ((r >> 1) & 7);
    woff[i] = (uint32_t)r * row_w + 16u * (uint32_t)q;
    klim[i] = K - 32 * q;
  }
  // the whole offset is in the vector offset, so the range check covers it
  auto load_raw = [&](int b, int s, int i) -> u32x4 {
    const uint32_t off = KL * s < klim[i] ? woff[i] + 16u * (uint32_t)b * row_w + 128u * (uint32_t)s : kOutOfRange;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, off, 0, kStream));
  };
  uint8_t* tile = smem + kTileBase + wave * kTileWave;
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

  // ---- unit order: chunk by chunk; inside chunk c, unit j -> (block j % nb, line 8 c + j / nb),
  // units j = wave, wave + 8, ... to this wave.  The cursor (chunk, block, line in chunk) advances
  // by additions only: j + 8 is block + 8 % nb, line + 8 / nb, with a carry (no division per unit).
  auto chunk_lines = [&](int c) { return min(kChunkLines, lines - kChunkLines * c); };
  const int b0 = wave % nb, l0 = wave / nb;         // the wave's first unit of every chunk
  const int db = kWaves % nb, dl = kWaves / nb;
  struct Cursor {
    int c, b, l, lc;                                // chunk, block, line in the chunk, lines in the chunk
  };
  // the wave's first unit in chunk u.c or a later one (u.c == chunks: none left)
  auto first_unit = [&](Cursor& u) {
    for (; u.c < chunks; ++u.c) {
      u.lc = chunk_lines(u.c);
      u.b = b0;
      u.l = l0;
      if (l0 < u.lc) return;
    }
  };
  auto next_unit = [&](Cursor& u) {
    u.b += db;
    u.l += dl;
    if (u.b >= nb) {
      u.b -= nb;
      ++u.l;
    }
    if (u.l >= u.lc) {
      ++u.c;
      first_unit(u);
    }
  };
  struct Slot {
    u32x4 raw[2];
    u32x4 s32;
    uint32_t s128;
    uint32_t s16[2];
  };
  auto issue = [&](const Cursor& u, Slot& sl) {
    const bool ok = u.c < chunks;
    const int b = ok ? u.b : 0;
    const int s = ok ? kChunkLines * u.c + u.l : lines;   // past the end: no memory access
    sl.raw[0] = load_raw(b, s, 0);
    sl.raw[1] = load_raw(b, s, 1);
    if constexpr (ALIGNED && G == 32) sl.s32 = load_s32(b, s);
    if constexpr (ALIGNED && G == 128) sl.s128 = load_s128(b, s);
    if constexpr (!ALIGNED) { sl.s16[0] = load_s16(b, s, 0); sl.s16[1] = load_s16(b, s, 1); }
  };

  // ---- activation chunks: thread -> row tid / 32, pieces (tid % 32) + 32 p ----
  const int xr = tid >> 5;
  const int xq = tid & 31;
  const bool xrow_ok = xr < M;
  auto load_x = [&](int c, u32x4 (&v)[kXPieces]) {
#pragma unroll
    for (int p = 0; p < kXPieces; ++p) {
      const int k = KCH * c + 8 * (xq + 32 * p);
      const uint32_t off = (xrow_ok && k < K) ? (uint32_t)xr * kbytes + 2u * (uint32_t)k : kOutOfRange;
      v[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0));
    }
  };
  auto store_x = [&](int c, const u32x4 (&v)[kXPieces]) {
    uint8_t* dst = smem + (c & 1) * kXBuf + xr * kXPitch + xq * 16;
#pragma unroll
    for (int p = 0; p < kXPieces; ++p) *reinterpret_cast<u32x4*>(dst + 512 * p) = permute_a(v[p]);
    if constexpr (kEnc) {
      // the biased sum of every 128-k group of the row: its 16 pieces are one
      // 16-lane DPP row (pieces xq + 32 p, xq = lane mod 32)
      float* xs = reinterpret_cast<float*>(smem + kXSumBase + (c & 1) * kXSumBuf) + xr * kGroupsPerChunk;
#pragma unroll
      for (int p = 0; p < kXPieces; ++p) {
        float t = dot2(v[p].x, kBiasPair, 0.f);
        t = dot2(v[p].y, kBiasPair, t);
        t = dot2(v[p].z, kBiasPair, t);
        t = dot2(v[p].w, kBiasPair, t);
        t = dpp_add<0xB1>(t);    // quad_perm [1,0,3,2]
        t = dpp_add<0x4E>(t);    // quad_perm [2,3,0,1]
        t = dpp_add<0x124>(t);   // row_ror:4
        t = dpp_add<0x128>(t);   // row_ror:8
        if ((xq & 15) == 0) xs[2 * p + (xq >> 4)] = t;
      }
    }
  };

  Slot sl;
  Cursor iu = {0, 0, 0, 0};                         // this wave's next unit to issue
  first_unit(iu);
  issue(iu, sl);
  u32x4 xv[kXPieces];
  load_x(0, xv);
  store_x(0, xv);
  if (chunks > 1) load_x(1, xv);
  __syncthreads();

  f32x4 acc[kMaxBlocks];
#pragma unroll
  for (int b = 0; b < kMaxBlocks; ++b) acc[b] = f32x4{};
  const uint32_t sel_lq = (uint32_t)(2 * lq) * 0x00010001u + (uint32_t)(2 * lq + 1) * 0x01000100u;
  const uint8_t* xfrag = smem + li * kXPitch + 64 * lq;
  // encoded path: masks and exponents in registers, so each pair of codes is one v_and_or_b32
  const uint32_t m_lo = __builtin_amdgcn_readfirstlane(0x000F000Fu), m_hi = __builtin_amdgcn_readfirstlane(0x00F000F0u);
  uint32_t e_even = 0x14001400u, e_odd = 0x04000400u;   // fp16 exponent fields 5 and 1, both halves
  asm volatile("" : "+v"(e_even), "+v"(e_odd));

  // One unit in flight per wave (a second one measured no faster).
  for (int c = 0; c < chunks; ++c) {
    const uint8_t* xc = xfrag + (c & 1) * kXBuf;
    const uint8_t* xsc = smem + kXSumBase + (c & 1) * kXSumBuf;   // biased sums of chunk c
    Cursor cu = {c, b0, l0, chunk_lines(c)};        // this wave's units of chunk c
    for (; cu.l < cu.lc; cu.b += db, cu.l += dl, cu.b >= nb ? (cu.b -= nb, ++cu.l) : 0) {
      const int b = cu.b;
      const int sl_line = cu.l;                     // line within the chunk
      *reinterpret_cast<u32x4*>(tile_w) = sl.raw[0];
      *reinterpret_cast<u32x4*>(tile_w + 1024) = sl.raw[1];
      const u32x4 wq0 = *reinterpret_cast<const u32x4*>(tile_r0);
      const u32x4 wq1 = *reinterpret_cast<const u32x4*>(tile_r1);
      // encoded path: the scales (groups 2 s, 2 s + 1) of the lane's output rows
      // 4 lq + r, held by lanes 4 lq + r (each lane loaded its operand row li's)
      uint32_t srow[4];
      if constexpr (kEnc) {
#pragma unroll
        for (int r = 0; r < 4; ++r) srow[r] = (uint32_t)__shfl((int)sl.s128, 4 * lq + r);
      }
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
      next_unit(iu);
      issue(iu, sl);                                // the wave's next unit (past the end: no memory access)
      const uint8_t* xb = xc + 512 * sl_line;
      f32x4 part = f32x4{};
      if constexpr (kEnc) {
        // the biased sums of the lane's activation row li for the line's two groups
        const float2 bsum = *reinterpret_cast<const float2*>(xsc + li * (kGroupsPerChunk * 4) + 8 * sl_line);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 wv = h ? wq1 : wq0;
          f32x4 t = f32x4{};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const f16x8 xf = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(xb + 256 * h + 16 * w));
            const uint32_t q = w == 0 ? wv.x : (w == 1 ? wv.y : (w == 2 ? wv.z : wv.w));
            const uint32_t q8 = q >> 8;
            // pairs (0,4), (2,6), (1,5), (3,7): the activations' slice order
            const u32x4 a = u32x4{(q & m_lo) | e_even, (q8 & m_lo) | e_even, (q & m_hi) | e_odd, (q8 & m_hi) | e_odd};
            t = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), xf, t, 0, 0, 0);
          }
          const float b = h ? bsum.y : bsum.x;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float s = half_bits_to_float(h ? srow[r] >> 16 : srow[r] & 0xFFFFu);
            part[r] = __builtin_fmaf(s, t[r] - b, part[r]);
          }
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 wv = h ? wq1 : wq0;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const f16x8 xf = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(xb + 256 * h + 16 * w));
            const uint32_t q = w == 0 ? wv.x : (w == 1 ? wv.y : (w == 2 ? wv.z : wv.w));
            part = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant_word(q, sv[h]), xf, part, 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int bb = 0; bb < kMaxBlocks; ++bb)
        if (bb == b) acc[bb] += part;
    }
    if (c + 1 < chunks) {
      store_x(c + 1, xv);
      if (c + 2 < chunks) load_x(c + 2, xv);
      __syncthreads();
    }
  }

  // ---- combine the waves' partial tiles in wave order, round once, store ----
  __syncthreads();                                  // activations and tiles no longer read
  f32x4* red = reinterpret_cast<f32x4*>(smem);      // [wave][block][lane]
#pragma unroll
  for (int bb = 0; bb < kMaxBlocks; ++bb)
    if (bb < nb) red[(wave * kMaxBlocks + bb) * 64 + lane] = acc[bb];
  __syncthreads();
  if (wave < nb && li < M) {
    f32x4 t = red[wave * 64 + lane];
    for (int w = 1; w < kWaves; ++w) t += red[(w * kMaxBlocks + wave) * 64 + lane];
    if constexpr (kEnc) t *= 0x1p20f;    // the codes' 2^-20
    // lane holds weight rows 4 lq .. 4 lq + 3 of block `wave` for activation row li
    if constexpr (SWIGLU) {
      // rows r0 + rr (gate) and r0 + rr + 1 (up) for even rr: output (r0 + rr) / 2
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const int rr = 16 * wave + 4 * lq + j;
        if (rr < nr) {
          const float g = t[j];
          const float v = g / (1.0f + __expf(-g)) * t[j + 1];
          y[(size_t)li * (N >> 1) + ((r0 + rr) >> 1)] = float_to_half_bits(v);
        }
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

template <int G, bool ALIGNED, bool SWIGLU>
hipError_t launch_ga(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int m, int n,
                     int k, int blocks, int units, hipStream_t stream) {
  return launch_kernel(gemm_skinny_kernel<G, ALIGNED, SWIGLU>, dim3(blocks), dim3(kThreads), 0, stream, x, packed,
                       scales, y, m, n, k, units / blocks, units % blocks);
}

// n weight rows in units of `unit` rows (2: gate/up pairs); returns the grid.
int skinny_grid(int n, int unit, const DeviceInfo& dev) {
  // One workgroup per CU (the LDS allows no more), more if a range would exceed
  // kMaxBlocks row blocks; at least 16 rows per workgroup.
  const int units = n / unit;
  const int lo = 16 / unit, hi = 16 * kMaxBlocks / unit;
  int g = dev.num_cu;
  if ((int64_t)g * lo > units) g = (units + lo - 1) / lo;
  if ((int64_t)g * hi < units) g = (units + hi - 1) / hi;
  return g;
}

template <bool SWIGLU>
hipError_t launch_s(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int m, int n,
                    int k, int group, const DeviceInfo& dev, hipStream_t stream) {
  const int unit = SWIGLU ? 2 : 1;
  const int g = skinny_grid(n, unit, dev);
  const int units = n / unit;
  const int spr = k / group;
  // one vector load per row brings a line's scales when every scale row is
  // 16-byte (g32) or 4-byte (g128) aligned in memory
  const uintptr_t sp = reinterpret_cast<uintptr_t>(scales);
  if (group == 32)
    return spr % 8 == 0 && (sp & 15) == 0 ? launch_ga<32, true, SWIGLU>(x, packed, scales, y, m, n, k, g, units, stream)
                                          : launch_ga<32, false, SWIGLU>(x, packed, scales, y, m, n, k, g, units, stream);
  return spr % 2 == 0 && (sp & 3) == 0 ? launch_ga<128, true, SWIGLU>(x, packed, scales, y, m, n, k, g, units, stream)
                                       : launch_ga<128, false, SWIGLU>(x, packed, scales, y, m, n, k, g, units, stream);
}

}  // namespace

bool gemm_skinny_fits(int m, int n, int k, const DeviceInfo& dev) {
  (void)k;   // any k: the activations are staged in chunks
  return m >= 1 && m <= kRows && n > 0 && dev.max_lds >= (size_t)kLds;
}

hipError_t launch_gemm_skinny(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int m,
                              int n, int k, int group, const DeviceInfo& dev, hipStream_t stream) {
  return launch_s<false>(x, packed, scales, y, m, n, k, group, dev, stream);
}

hipError_t launch_swiglu_skinny(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y,
                                int m, int n_out, int k, int group, const DeviceInfo& dev, hipStream_t stream) {
  return launch_s<true>(x, packed, scales, y, m, 2 * n_out, k, group, dev, stream);
}

}  // namespace w4a16
