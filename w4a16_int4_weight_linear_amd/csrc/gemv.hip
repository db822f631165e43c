// gemv.hip -- decode GEMV (1 <= M <= 4) of the W4A16 int4 weight-only layer on gfx950.
//
// y[m, n] = sum_k x[m, k] * s[n, k / g] * q[n, k]: the per-token decode step of
// the W4A16 models on the LLM170 CUDA/W4A16 page (tg column, M = 1; np4 column,
// M = 4).  The infr page (Validated models & performance) puts such decode
// GEMVs at the DRAM bandwidth wall, so the kernel streams the packed weights
// once, at full HBM rate, and keeps the per-byte instruction count low:
//
// * Work split: one workgroup per CU, each owning a contiguous block of rows
//   (block sizes differ by at most one row).  Rows are contiguous in memory, so
//   the block is one run of bytes; it is cut into 1 KiB items (one 16-byte load
//   per lane, 64 chunks of 32 weights), and the items are divided evenly among
//   the workgroup's eight wavefronts regardless of row boundaries.  Every wave
//   thus reads one sequential stream (which HBM serves faster than interleaved
//   streams), no lane idles at a row's ragged end, and all waves stream the
//   same number of bytes.
// * Lane l of item u holds chunk 64u + l of the block.  The chunk's group
//   scale index is simply (64u + l) / (g / 32), so the scale address advances
//   uniformly; the chunk's position in its row (for the activations) advances by
//   64 and wraps at the row length, one compare per item.  An item that contains
//   a row end splits its lanes between the two rows (a wave-uniform test); the
//   finished row is reduced across lanes at once.
// * Rows cut between waves: each wave leaves the wave-reduced partial sums of
//   its first and last row in LDS; after one workgroup barrier, one lane per
//   wave boundary adds the partials of the row that boundary cuts, in wave
//   order (deterministic), reading them all at once.  Finished rows collect in
//   LDS and the whole workgroup writes them to y after a second barrier, so the
//   loop itself issues no global stores.  (The workgroup cannot end before its
//   slowest wave anyway; combining after a barrier keeps the slowest wave's
//   path after its loop to a few LDS round trips.)
// * The weights come through buffer loads marked non-temporal, issued a fixed
//   number of items ahead of use.  The item offset goes in the scalar offset
//   field, so a load costs no vector address arithmetic; loads past the end use
//   an offset outside the buffer and return zero without touching memory.
// * Once per workgroup, the activations (pre-arranged to line up with the
//   nibble pairs below), their per-chunk sums and the group scales of the
//   workgroup's rows are staged in LDS.  Their global loads are issued before
//   the first weight loads, so waiting for them does not wait for (and drain)
//   the weight stream.  In the main loop the LDS reads of the next item are
//   issued before the current item's arithmetic (M <= 2).
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
// * Gated variant (the SwiGLU gate/up pair of an FFN): the weight rows
//   interleave gate and up rows, workgroups own whole row pairs, and after the
//   rows are finished one workgroup barrier lets every pair be read back from
//   LDS and written as SiLU(gate) * up, rounded once to fp16.
//
// For integer x, codes and power-of-two scales every step above is exact, so
// such inputs give bit-exact results regardless of summation order.
#include <atomic>

#include "device.hpp"
#include "kernels.hpp"
#include "launch.hpp"
#include "wave_stamps.hpp"

W4A16_STAMP_STORAGE(w4a16_wave_stamps_gemv)

namespace w4a16 {
namespace {

// Launch shape.  Defaults are the measured best on MI355X; the macros only
// exist so a sweep can rebuild the library with other values.
#ifndef W4A16_GEMV_LOADS_IN_FLIGHT
#define W4A16_GEMV_LOADS_IN_FLIGHT 4
#endif
#ifndef W4A16_GEMV_THREADS
#define W4A16_GEMV_THREADS 512
#endif
constexpr int kGemvThreads = W4A16_GEMV_THREADS;
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kLoadsInFlight = W4A16_GEMV_LOADS_IN_FLIGHT;   // 16-byte loads per lane
#ifndef W4A16_GEMV_SKEW
#define W4A16_GEMV_SKEW 100
#endif
constexpr int kGemvSkew = W4A16_GEMV_SKEW;   // in 1/1024
constexpr uint32_t kScaleSlack = 256;   // staged past the workgroup's last scale
constexpr int kPartSlots = 4;           // floats per partial slot: M <= 4

template <int M>
struct XSumSlots { static constexpr int value = (M == 1) ? 1 : (M == 2 ? 2 : 4); };

struct GemvLayout {
  uint32_t xs, sc, part, res, total;   // byte offsets of the LDS regions, and the size
};

__host__ __device__ inline GemvLayout gemv_layout(int m, int chunks, int spr, int rows_wg) {
  GemvLayout l;
  l.xs = 0;
  l.sc = (uint32_t)chunks * (uint32_t)(4 * m + 1) * 16u;
  l.part = l.sc + (((uint32_t)rows_wg * (uint32_t)spr * 2u + 15u) & ~15u) + 32u + kScaleSlack;
  l.res = l.part + (uint32_t)(kGemvWaves * 2 * kPartSlots * 4);
  l.total = l.res + (uint32_t)rows_wg * (uint32_t)m * 4u;
  return l;
}

// LDS layout (chunk c = 32 consecutive k of a row):
//   xs[c] : (4M + 1) slots of 16 bytes: slot 4m + j = for word j of chunk c the
//           fp16 pairs (x[8j], x[8j+4]), (x[8j+2], x[8j+6]), (x[8j+1], x[8j+5]),
//           (x[8j+3], x[8j+7]) of activation row m; slot 4M = -8 * 2^-20 * (sum of
//           the chunk's 32 activations) for each row.  The chunk stride (an odd
//           number of 16-byte slots) keeps the 16-byte reads of 16 consecutive
//           chunks on distinct banks, and one address serves all slots;
//   sc : a 16-byte-aligned copy of the scales of the workgroup's rows (plus slack);
//   part[wave][2][4] : partial sums of the first / last row of each wave;
//   res[row][m] : finished fp32 sums of the workgroup's rows, written to y at the end.
template <int M, bool GATED>
__global__ void __launch_bounds__(kGemvThreads)
gemv_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
            const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
            int n, int k, int gshift, int rows_base, int rows_extra, uint32_t sc_shift) {
  // rows_base / rows_extra count row units: single rows, or gate/up row pairs.
  constexpr int kUnit = GATED ? 2 : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int XS = XSumSlots<M>::value;
  constexpr int U = kLoadsInFlight;              // items in flight
  constexpr uint32_t kChunkBytes = (4 * M + 1) * 16;
  constexpr uint32_t kSumSlot = 4 * M * 16;
  // LDS operands of the next item are read ahead while they fit in registers.
  constexpr bool kReadAhead = M <= 2;
  const int C = k >> 5;                          // 32-weight chunks per row
  const int spr = C >> gshift;                   // scales per row

  const int lane = threadIdx.x & 63;
  // wave index, made explicitly wave-uniform so the bookkeeping lives in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // timeline stamps (profiling build only; the M = 1 decode kernel)
  constexpr bool kStamped = M == 1 && !GATED;
  W4A16_STAMP_DECL;
  if (kStamped) W4A16_STAMP(0);
  const int blk = blockIdx.x;
  const int nr = kUnit * (rows_base + (blk < rows_extra ? 1 : 0));       // rows of this workgroup
  const int wg_r0 = kUnit * (blk * rows_base + (blk < rows_extra ? blk : rows_extra));
  const int chunks = nr * C;                                             // chunks of the block
  const int items = (chunks + 63) >> 6;                                  // 1 KiB items
  // Waves 0..W/2-1 are the older wave of their SIMD and are issued first, so
  // they get a larger share (1 + skew) of the items than the younger half.
  auto bound = [&](int w) {
    constexpr int kHalf = kGemvWaves / 2;
    const uint32_t cum = w <= kHalf ? (uint32_t)w * (1024 + kGemvSkew)
                                    : (uint32_t)kHalf * (1024 + kGemvSkew) + (uint32_t)(w - kHalf) * (1024 - kGemvSkew);
    return (int)((cum * (uint32_t)items) / (uint32_t)(kGemvWaves * 1024));
  };
  const int t0 = bound(wave), t1 = bound(wave + 1);                      // this wave's items
  const GemvLayout L = gemv_layout(M, C, spr, kUnit * (rows_base + (rows_extra ? 1 : 0)));

  // ---- staging loads (activations, scales), issued before the weight stream ----
  // `scales` is rounded down to 16 bytes by the launcher and sc_shift bytes
  // added back here, so the 16-byte staging loads are aligned in memory
  const uint32_t sc_begin = (uint32_t)wg_r0 * (uint32_t)spr * 2u + sc_shift;
  const uint32_t sc_a0 = sc_begin & ~15u;
  const uint32_t sc_chunks = (sc_begin - sc_a0 + (uint32_t)nr * (uint32_t)spr * 2u + kScaleSlack + 15u) >> 4;
  const uint32_t sc_bytes = (uint32_t)n * (uint32_t)spr * 2u + sc_shift;
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(scales, sc_bytes);
  const int pairs = C * M;                        // (chunk, activation row) pairs
  u32x4 a[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = threadIdx.x + h * kGemvThreads;
    if (idx < pairs) {
      const int c = idx / M, m = idx - (idx / M) * M;
      const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)m * k + (size_t)c * 32);
#pragma unroll
      for (int w = 0; w < 4; ++w) a[h][w] = src[w];
    }
  }
  const u32x4 sv = load16_tail(sres, threadIdx.x < sc_chunks ? sc_a0 + threadIdx.x * 16u : kOutOfRange, sc_bytes);

  // ---- weight stream: items t0 .. t1-1 of this wave ----
  const uint32_t row_bytes = (uint32_t)k >> 1;
  // The descriptor covers exactly the workgroup's rows, so lanes past the block's
  // end in its last item read zero without a per-lane offset.
  const __amdgpu_buffer_rsrc_t wres =
      make_rsrc(reinterpret_cast<const uint8_t*>(packed) + (size_t)wg_r0 * row_bytes, (uint32_t)nr * row_bytes);
  const uint32_t voff = (uint32_t)lane * 16u;
  u32x4 wb[U];
  int iss = t0;
  uint32_t iss_off = (uint32_t)t0 << 10;
  auto issue = [&](int slot) {
    wb[slot] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
        wres, voff, iss < t1 ? iss_off : kOutOfRange, kStream));
    ++iss;
    iss_off += 1024u;
  };
#pragma unroll
  for (int u = 0; u < U; ++u) issue(u);

  // ---- cut-row bookkeeping, done while the first loads are in flight ----
  // Lane b (1 <= b < waves) of wave 0 adds, after the loop, the partial sums of
  // the row that the boundary between waves b - 1 and b cuts, if that row is cut
  // there first.  It records which waves hold a part of the row and which of them
  // left it in their last-row slot (their range starts before the row).
  int comb_row = -1;
  uint32_t comb_in = 0u, comb_last = 0u;
  if (threadIdx.x >= 1 && threadIdx.x < kGemvWaves) {
    const int b = threadIdx.x;
    const int cb = bound(b) << 6;
    const int start = (cb / C) * C, end = start + C;
    if (cb < chunks && cb != start && (b == 1 || (bound(b - 1) << 6) <= start)) {
      comb_row = start / C;
#pragma unroll
      for (int w2 = 0; w2 < kGemvWaves; ++w2) {
        const int a0 = bound(w2) << 6, a1 = bound(w2 + 1) << 6;
        if (a1 > a0 && a0 < end && a1 > start) comb_in |= 1u << w2;
        if (a0 < start) comb_last |= 1u << w2;
      }
    }
  }

  // ---- loop set-up that needs integer division, also done while the loads are in
  // flight (the empty asm statements keep the compiler from moving it past the
  // staging barrier) ----
  // Lane's chunk in the block: f = 64 t + lane; its chunk in the row, c = f mod C,
  // addresses the activations; f >> gshift indexes the block's scales.
  const int f_first = (t0 << 6) + lane;
  int c_first = f_first % C;
  int r_first = __builtin_amdgcn_readfirstlane((t0 << 6) / C);   // row of the wave's first chunk
  // the activation step per item: 64 chunks, or 64 mod C for rows shorter than 64 chunks
  int x_adv_chunks = __builtin_amdgcn_readfirstlane(C >= 64 ? 64 : 64 % C);
  // rows [whole_lo, whole_hi) lie wholly inside this wave's items (written to y by
  // the wave itself after its loop)
  int whole_lo = __builtin_amdgcn_readfirstlane(((t0 << 6) + C - 1) / C);
  int whole_hi = __builtin_amdgcn_readfirstlane(min((t1 << 6) / C, nr));
  asm volatile("" : "+v"(c_first));
  asm volatile("" : "+s"(r_first), "+s"(x_adv_chunks), "+s"(whole_lo), "+s"(whole_hi));

  // ---- staging: activations regrouped to the nibble pairing, chunk sums, scales ----
  const uint32_t one2 = 0x3C003C00u;  // fp16 pair (1, 1)
  auto stage_pair = [&](int idx, const u32x4 (&v4)[4]) {
    const int c = idx / M, m = idx - (idx / M) * M;
    uint8_t* cp = smem + L.xs + (uint32_t)c * kChunkBytes;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32x4 v = v4[w];          // x[32c+8w .. +7] as pairs (0,1),(2,3),(4,5),(6,7)
      s = dot2(v.x, one2, s);
      s = dot2(v.y, one2, s);
      s = dot2(v.z, one2, s);
      s = dot2(v.w, one2, s);
      u32x4 p;                        // regrouped to (0,4),(2,6),(1,5),(3,7)
      p.x = (v.x & 0xFFFFu) | (v.z << 16);
      p.y = (v.y & 0xFFFFu) | (v.w << 16);
      p.z = (v.x >> 16) | (v.z & 0xFFFF0000u);
      p.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
      *reinterpret_cast<u32x4*>(cp + (m * 4 + w) * 16) = p;
    }
    float* sum = reinterpret_cast<float*>(cp + kSumSlot);
    sum[m] = s * -0x1p-17f;   // -8 * 2^-20 * sum
    if (M == 3 && m == 0) sum[3] = 0.f;
  };
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = threadIdx.x + h * kGemvThreads;
    if (idx < pairs) stage_pair(idx, a[h]);
  }
  if (threadIdx.x < sc_chunks) *reinterpret_cast<u32x4*>(smem + L.sc + threadIdx.x * 16u) = sv;
  // Wide activations (more than two pairs per thread) and long scale windows.
  for (int idx = threadIdx.x + 2 * kGemvThreads; idx < pairs; idx += kGemvThreads) {
    const int c = idx / M, m = idx - (idx / M) * M;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)m * k + (size_t)c * 32);
    u32x4 v4[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) v4[w] = src[w];
    stage_pair(idx, v4);
  }
  for (uint32_t t = threadIdx.x + kGemvThreads; t < sc_chunks; t += kGemvThreads) {
    *reinterpret_cast<u32x4*>(smem + L.sc + t * 16u) = load16_tail(sres, sc_a0 + t * 16u, sc_bytes);
  }
  __syncthreads();
  if (kStamped) W4A16_STAMP(1);

  // ---- main loop over this wave's items ----
  float* parts = reinterpret_cast<float*>(smem + L.part);
  float* res = reinterpret_cast<float*>(smem + L.res);
  const uint32_t xs_end = L.xs + (uint32_t)C * kChunkBytes;
  const uint32_t xs_wrap = (uint32_t)C * kChunkBytes;
  // advance by 64 chunks (C >= 64: one wrap at most), or 64 mod C (whole rows skipped)
  const uint32_t x_adv = (uint32_t)x_adv_chunks * kChunkBytes;
  const uint32_t sc_base = L.sc + (sc_begin - sc_a0);
  const uint32_t s_step = (uint32_t)((64 >> gshift) * 2);
  struct Pos {
    uint32_t xa, sa;   // LDS addresses of the lane's activations and scale
  };
  auto advance = [&](Pos& p) {
    const uint32_t nx = p.xa + x_adv;
    p.xa = nx >= xs_end ? nx - xs_wrap : nx;
    p.sa += s_step;
  };
  struct Opnd {
    u32x4 xv[M][4];
    float xsv[XS];
    uint32_t s;
  };
  auto read_opnd = [&](const Pos& p, Opnd& o) {
    const uint8_t* xp = smem + p.xa;
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int w = 0; w < 4; ++w) o.xv[m][w] = *reinterpret_cast<const u32x4*>(xp + (m * 4 + w) * 16);
    const uint8_t* sp = xp + kSumSlot;
    if constexpr (XS == 1) {
      o.xsv[0] = *reinterpret_cast<const float*>(sp);
    } else if constexpr (XS == 2) {
      const float2 v = *reinterpret_cast<const float2*>(sp);
      o.xsv[0] = v.x; o.xsv[1] = v.y;
    } else {
      const f32x4 v = *reinterpret_cast<const f32x4*>(sp);
      o.xsv[0] = v.x; o.xsv[1] = v.y; o.xsv[2] = v.z; o.xsv[3] = v.w;
    }
    o.s = *reinterpret_cast<const uint16_t*>(smem + p.sa);
  };

  // One chunk: 2^-20 * sum x (u - 8) for each activation row (the scale is applied by the caller).
  auto chunk_dot = [&](const u32x4& q4, const Opnd& o, float (&v)[M]) {
    float lo[M], hi[M];
#pragma unroll
    for (int m = 0; m < M; ++m) { lo[m] = 0.f; hi[m] = o.xsv[m]; }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t q = w == 0 ? q4.x : (w == 1 ? q4.y : (w == 2 ? q4.z : q4.w));
      const uint32_t q8 = q >> 8;
      const uint32_t a0 = q & 0x000F000Fu, b0 = q8 & 0x000F000Fu;
      const uint32_t c0 = q & 0x00F000F0u, d0 = q8 & 0x00F000F0u;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        lo[m] = dot2(o.xv[m][w].x, a0, lo[m]);
        lo[m] = dot2(o.xv[m][w].y, b0, lo[m]);
        hi[m] = dot2(o.xv[m][w].z, c0, hi[m]);
        hi[m] = dot2(o.xv[m][w].w, d0, hi[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) v[m] = __builtin_fmaf(lo[m], 16.f, hi[m]);
  };

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;

  int row = r_first;                             // row of lane 0's chunk
  int row_end = (row + 1) * C;                   // block chunk where that row ends

  // Finished per-lane row sums wait in a queue of four values (rows in order,
  // M values each) and are reduced across lanes four at a time: a 32-lane and a
  // 16-lane swap put the four values in the four 16-lane rows, four DPP steps
  // finish the sums.  Rows the wave holds whole go to res; cut rows to the
  // wave's partial slots.
  float q0 = 0.f, q1 = 0.f, q2 = 0.f, q3 = 0.f;  // q3 oldest
  // The lane swaps are written as inline assembly because both registers are
  // outputs (the compiler's builtins for them lose one of the two results).
  // The s_nop before and after give the required wait states around them.
  auto swap32 = [](float& lo, float& hi) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(lo), "+v"(hi));
  };
  auto swap16 = [](float& lo, float& hi) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(lo), "+v"(hi));
  };
  int q_row = r_first;                           // row of the oldest queued value
  int q_n = 0;                                   // values queued
  const int v_idx = (lane >> 5) | ((lane >> 3) & 2);   // value a lane ends up holding
  auto flush = [&]() {
    float a2 = q3, b2 = q2, c2 = q1, d2 = q0;
    swap32(a2, b2);                              // a2 = a[0:32] | b[0:32], b2 = a[32:64] | b[32:64]
    swap32(c2, d2);
    float s1 = a2 + b2, s2 = c2 + d2;            // a | b and c | d, 32 lanes each
    swap16(s1, s2);                              // 16-lane rows: s1 = a b a b halves, s2 = c d c d
    float t = s1 + s2;                           // 16-lane rows hold a, c, b, d
    t = dpp_add<0xB1>(t);    // quad_perm [1,0,3,2]
    t = dpp_add<0x4E>(t);    // quad_perm [2,3,0,1]
    t = dpp_add<0x124>(t);   // row_ror:4
    t = dpp_add<0x128>(t);   // row_ror:8
    const int r = q_row + v_idx / M, m = v_idx - (v_idx / M) * M;
    // (rows past the block come from lanes past its end and are dropped)
    if ((lane & 15) == 0 && v_idx < q_n && r < nr) {
      const bool whole = r * C >= (t0 << 6) && (r + 1) * C <= (t1 << 6);
      const float tot = t * 0x1p20f;
      if (whole) {
        res[r * M + m] = tot;
      } else {
        parts[wave * (2 * kPartSlots) + (r == r_first ? 0 : kPartSlots) + m] = tot;
      }
    }
    q0 = q1 = q2 = q3 = 0.f;
    q_row += 4 / M;
    q_n = 0;
  };
  auto push_row = [&](const float (&val)[M]) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      q3 = q2; q2 = q1; q1 = q0; q0 = val[m];
    }
    q_n += M;
    if (q_n + M > 4) {
      // Line the queued values up as q3 = first (M = 3 leaves one empty slot).
      if (q_n == 3) { q3 = q2; q2 = q1; q1 = q0; q0 = 0.f; }
      flush();
    }
  };

  const int cnt_items = t1 - t0;
  Pos cur_pos;
  {
    cur_pos.xa = L.xs + (uint32_t)c_first * kChunkBytes;
    cur_pos.sa = sc_base + (uint32_t)(f_first >> gshift) * 2u;
  }
  Opnd cur;
  if (kReadAhead && cnt_items > 0) read_opnd(cur_pos, cur);

  // One item: u is its load slot, idx its index among this wave's items.
  auto consume = [&](int u, int idx) {
    Pos nxt = cur_pos;
    advance(nxt);
    Opnd on;
    if constexpr (kReadAhead) {
      if (idx + 1 < cnt_items) read_opnd(nxt, on);
    } else {
      read_opnd(cur_pos, cur);
    }
    float v[M];
    chunk_dot(wb[u], cur, v);
    const float sc = half_bits_to_float(cur.s);
    const int f0 = (t0 + idx) << 6;              // block chunk of lane 0
    if (row_end > f0 + 64) {
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = __builtin_fmaf(sc, v[m], acc[m]);
    } else {
      // One or more rows end inside this item: lanes before each end finish that row.
#pragma unroll
      for (int m = 0; m < M; ++m) v[m] *= sc;
      do {
        const int b = row_end - f0;              // lanes [0, b) belong to rows up to `row`
        float fin[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float mine = lane < b ? v[m] : 0.f;
          v[m] -= mine;
          fin[m] = acc[m] + mine;
          acc[m] = 0.f;
        }
        push_row(fin);
        ++row;
        row_end += C;
      } while (row_end <= f0 + 64);
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] += v[m];
    }
    cur_pos = nxt;
    if constexpr (kReadAhead) cur = on;
  };
  // The wave's last items run through the same loop (a wave-uniform test skips
  // the slots past the end; their loads are out of range and touch no memory),
  // so no separate straight-line tail is fetched cold while the stream drains.
  for (int base = 0; base < cnt_items; base += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u < cnt_items) consume(u, base + u);
      if (kStamped && base == 0 && u == 0) W4A16_STAMP(2);
      issue(u);
    }
  }
  // A row cut at the end of the wave's range, then whatever is still queued.
  if (cnt_items > 0 && row < nr && row * C < (t1 << 6)) push_row(acc);
  if (q_n > 0) {
    if (M == 1) {
      // Line the queued values up as q3 = first.
      for (int i = q_n; i < 4; ++i) { q3 = q2; q2 = q1; q1 = q0; q0 = 0.f; }
    } else if (M == 2 && q_n == 2) {
      q3 = q1; q2 = q0; q1 = 0.f; q0 = 0.f;
    }
    flush();
  }

  if (kStamped) W4A16_STAMP(3);
  // ---- the wave's whole rows go to y now (the loop left them in res; no
  // global store is issued inside the loop) ----
  if constexpr (!GATED) {
    for (int e = lane; e < (whole_hi - whole_lo) * M; e += 64) {
      const int rl = whole_lo + e / M, m = e - (e / M) * M;
      y[(size_t)m * n + wg_r0 + rl] = float_to_half_bits(res[rl * M + m]);
    }
  }
  // ---- rows cut between waves: after one workgroup barrier, the lanes chosen
  // above add the partials of their rows in wave order, all slots read at once
  // (a slot of a wave with no part of the row holds an unrelated value and is
  // not added), and store them ----
  __syncthreads();
  if (kStamped) W4A16_STAMP(4);
  if (comb_row >= 0) {
    float pv[kGemvWaves][M];
#pragma unroll
    for (int w2 = 0; w2 < kGemvWaves; ++w2) {
      const float* slot = parts + w2 * (2 * kPartSlots) + (((comb_last >> w2) & 1u) ? kPartSlots : 0);
#pragma unroll
      for (int m = 0; m < M; ++m) pv[w2][m] = slot[m];
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float sum = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kGemvWaves; ++w2) sum += ((comb_in >> w2) & 1u) ? pv[w2][m] : 0.f;
      if constexpr (GATED) {
        res[comb_row * M + m] = sum;
      } else {
        y[(size_t)m * n + wg_r0 + comb_row] = float_to_half_bits(sum);
      }
    }
  }

  if constexpr (GATED) {
    // a (gate, up) pair may have one row cut and the other whole: all rows in res first
    __syncthreads();
    const int pairs_wg = nr >> 1, n_out = n >> 1;
    for (int e = threadIdx.x; e < pairs_wg * M; e += kGemvThreads) {
      const int pr = e / M, m = e - (e / M) * M;
      const float g = res[(2 * pr) * M + m], u = res[(2 * pr + 1) * M + m];
      y[(size_t)m * n_out + (wg_r0 >> 1) + pr] = float_to_half_bits(g / (1.f + __expf(-g)) * u);
    }
  }
  if (kStamped) {
    W4A16_STAMP(5);
    W4A16_STAMP_FLUSH(wave);
  }
}

template <int M, bool GATED>
hipError_t launch_gemv_m(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y,
                         int n, int k, int group, const GemvPlan& plan, const DeviceInfo& dev,
                         hipStream_t stream) {
  static std::atomic<uint64_t> attr_set{0};   // one bit per device
  const uint64_t bit = 1ull << (dev.device & 63);
  if (!(attr_set.load(std::memory_order_acquire) & bit)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<M, GATED>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int gshift = group == 128 ? 2 : 0;   // log2(group / 32)
  const uint32_t sc_shift = (uint32_t)(reinterpret_cast<uintptr_t>(scales) & 15u);
  const uint16_t* sc_aligned = reinterpret_cast<const uint16_t*>(reinterpret_cast<uintptr_t>(scales) - sc_shift);
  return launch_kernel(gemv_kernel<M, GATED>, dim3(plan.blocks), dim3(kGemvThreads), plan.lds, stream, x, packed,
                       sc_aligned, y, n, k, gshift, plan.rows_base, plan.rows_extra, sc_shift);
}

size_t plan_lds(int m, int units, int k, int group, int blocks, int unit) {
  const int C = k / 32;
  const int spr = C / (group / 32);
  const int base = units / blocks, extra = units % blocks;
  return gemv_layout(m, C, spr, unit * (base + (extra ? 1 : 0))).total;
}

}  // namespace

GemvPlan gemv_plan(int m, int n, int k, int group, const DeviceInfo& dev, bool gated) {
  GemvPlan p;
  // Rows are handed out in units: single rows, or gate/up row pairs (n even).
  const int unit = gated ? 2 : 1;
  const int units = n / unit;
  p.gated = gated;
  if (units <= 0 || units * unit != n) return p;
  // One workgroup per CU; more (fewer rows, so fewer staged scales, each) until the LDS fits.
  int blocks = units < dev.num_cu ? units : dev.num_cu;
  while (blocks < units && plan_lds(m, units, k, group, blocks, unit) > dev.max_lds) {
    blocks = blocks * 2 < units ? blocks * 2 : units;
  }
  p.blocks = blocks;
  p.rows_base = units / blocks;
  p.rows_extra = units % blocks;
  p.lds = plan_lds(m, units, k, group, blocks, unit);
  p.ok = p.lds <= dev.max_lds;
  return p;
}

int64_t gemv_max_k(int m, int group, const DeviceInfo& dev) {
  // Fewest rows a workgroup can be given: one.
  int64_t best = 0;
  for (int64_t k = group; k <= (int64_t)1 << 22; k += group) {
    const int C = (int)(k / 32);
    if (gemv_layout(m, C, C / (group / 32), 1).total > dev.max_lds) break;
    best = k;
  }
  return best;
}

hipError_t launch_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int m,
                       int n, int k, int group, const GemvPlan& plan, const DeviceInfo& dev, hipStream_t stream) {
  if (plan.gated) {
    switch (m) {
      case 1: return launch_gemv_m<1, true>(x, packed, scales, y, n, k, group, plan, dev, stream);
      case 2: return launch_gemv_m<2, true>(x, packed, scales, y, n, k, group, plan, dev, stream);
      case 3: return launch_gemv_m<3, true>(x, packed, scales, y, n, k, group, plan, dev, stream);
      case 4: return launch_gemv_m<4, true>(x, packed, scales, y, n, k, group, plan, dev, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (m) {
    case 1: return launch_gemv_m<1, false>(x, packed, scales, y, n, k, group, plan, dev, stream);
    case 2: return launch_gemv_m<2, false>(x, packed, scales, y, n, k, group, plan, dev, stream);
    case 3: return launch_gemv_m<3, false>(x, packed, scales, y, n, k, group, plan, dev, stream);
    case 4: return launch_gemv_m<4, false>(x, packed, scales, y, n, k, group, plan, dev, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a16
