// gemv_mfma.hip -- batched decode GEMV (2 <= M <= 4) of the W4A16 int4 layer on fp16 MFMA.
//
// y[m, n] = sum_k x[m, k] * s[n, k / g] * q[n, k] for a few activation rows:
// the np4 column of the LLM170 CUDA/W4A16 page's benchmark tables, where the
// rows of a decode batch share one pass over the weights.  The product is a
// weight stream like the M = 1 decode step (gemv.hip), but reading M rows of
// activations for every weight from LDS would cost M times the LDS traffic, so
// the contraction runs on the matrix cores.
//
// * The instruction is v_mfma_f32_4x4x4_16b_f16: sixteen independent 4 x 4 x 4
//   products per wave, block b in lanes 4b .. 4b + 3.  The activations are the
//   A operand (row i of a block: activation row i, of which the first M are
//   real) and the weights the B operand (column j of a block: one weight row).
//   Its operand layout is what lets a weight load cover whole 128-byte lines:
//   the four lanes of a block need four different weight rows at the same k,
//   so one 16-byte-per-lane load gives lane l row (l & 3) + 4 (l >> 5) and
//   32-k chunk (l >> 2) & 7 of a 256-k line -- 8 rows x 128 contiguous bytes.
//   (With a 16 x 16 product the sixteen columns of one load would be sixteen
//   rows, 64 bytes each: half lines, which this part reads markedly slower.)
// * Each lane's 16 bytes (32 k) feed 8 MFMAs of 4 k.  Since 32 divides the
//   group size, a lane's 32 k lie in one quantisation group.  The codes enter
//   the MFMA without conversion instructions: one AND-OR per pair of codes
//   keeps two nibbles and sets an fp16 exponent above them.  The nibbles of
//   even k sit at mantissa bits 0-3 and take exponent 2^-10, giving
//   2^-10 + u 2^-20; those of odd k sit at bits 4-7 and take 2^-14, giving
//   2^-14 + 16 u 2^-24 = 2^-14 + u 2^-20: the same weight for u, exact, five
//   instructions per packed word.  The 8 MFMAs give t over the chunk; the
//   activations' biased sum b = sum x_even (2^-10 + 8 2^-20) + sum x_odd
//   (2^-14 + 8 2^-20) is staged per chunk, so t - b = 2^-20 sum x (u - 8),
//   and the scale is applied once per chunk on the four accumulators:
//   acc += s (t - b); the 2^20 is restored when a row is finished.  This is
//   exact for integer data and the same for every group size.
// * Work split: each workgroup (one per CU) owns a contiguous range of weight
//   rows (sizes differ by at most one row), covered by 8-row blocks.  Its units
//   (block, line) are dealt to the waves as contiguous runs in block-major
//   order, so every wave streams along its rows with several loads in flight,
//   like the M = 1 kernel's flat streams.  The older wave of each SIMD, whose
//   loads are issued first, takes a slightly larger run.
// * The activations are staged in LDS once per workgroup, each group of 8 k in
//   the order the dequantisation produces (k = 0, 4, 2, 6, 1, 5, 3, 7), with
//   the biased sum b of every 32-k chunk per row; the workgroup's scales are staged
//   beside them.  Lanes whose A row is not a real activation row read row
//   i mod M, whose results are never stored.
// * When a wave leaves a block, the eight lanes holding the chunks of one row
//   are added (DPP and one swizzle) and the row's partial sums go to LDS; at
//   the end the waves' partials are added in wave order (deterministic),
//   rounded once to fp16 and stored.
// * Gated variant (the SwiGLU gate/up pair of an FFN): the weight rows
//   interleave gate and up rows, workgroups own whole pairs, and the final
//   step writes SiLU(gate) * up for each pair.
//
// For integer activations, codes and power-of-two scales every product and
// partial sum is exact, so such inputs give bit-exact results.
#include <atomic>

#include "device.hpp"
#include "kernels.hpp"
#include "launch.hpp"
#include "mfma_operands.hpp"
#include "wave_stamps.hpp"

W4A16_STAMP_STORAGE(w4a16_wave_stamps_gemv_mfma)

namespace w4a16 {
namespace {

#ifndef W4A16_NP4_THREADS
#define W4A16_NP4_THREADS 512
#endif
#ifndef W4A16_NP4_LOADS_IN_FLIGHT
#define W4A16_NP4_LOADS_IN_FLIGHT 4
#endif
#ifndef W4A16_NP4_SHALLOW_LOADS
#define W4A16_NP4_SHALLOW_LOADS 3
#endif
#ifndef W4A16_NP4_SHALLOW_UNITS
#define W4A16_NP4_SHALLOW_UNITS 10
#endif
#ifndef W4A16_NP4_WG_PER_CU
#define W4A16_NP4_WG_PER_CU 1
#endif
#ifndef W4A16_NP4_SKEW
#define W4A16_NP4_SKEW 100
#endif
constexpr int kThreads = W4A16_NP4_THREADS;
constexpr int kWaves = kThreads / 64;
// Loads in flight per wave: a wave with few units (a small launch) does better
// with a shallower ring, a long stream with a deeper one (measured).
constexpr int kDepth = W4A16_NP4_LOADS_IN_FLIGHT;
constexpr int kShallowDepth = W4A16_NP4_SHALLOW_LOADS;
constexpr int kShallowUnits = W4A16_NP4_SHALLOW_UNITS;   // units per wave at or below which it is used
constexpr int kSkew = W4A16_NP4_SKEW;           // in 1/1024: extra share of the older wave of each SIMD
constexpr int KL = 256;                         // k per line: 128 bytes of a weight row
constexpr int kRows = 8;                        // weight rows per block (one load)
constexpr int kMaxBlocks = 32;                  // blocks per workgroup
constexpr uint32_t kScaleSlack = 256;           // staged past the workgroup's last scale

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Staged activation rows hold whole lines (zeros past K) plus 16 bytes, so
// consecutive rows start on different banks.
__host__ __device__ inline uint32_t x_pitch(int k) { return (uint32_t)((k + KL - 1) / KL) * KL * 2u + 16u; }

struct Layout {
  uint32_t xs, xsum, sc, red, total;            // byte offsets of the LDS regions, and the size
};
// m activation rows of k, a workgroup of `rows` weight rows with spr scales each.
__host__ __device__ inline Layout lds_layout(int m, int k, int spr, int rows) {
  Layout l;
  const int lines = (k + KL - 1) / KL;
  const int nb = (rows + kRows - 1) / kRows;
  l.xs = 0;
  l.xsum = (uint32_t)m * x_pitch(k);
  l.sc = l.xsum + (uint32_t)lines * 8u * 16u;   // [32-k chunk][4 rows] fp32
  l.red = l.sc + (((uint32_t)rows * (uint32_t)spr * 2u + 15u) & ~15u) + 32u + kScaleSlack;
  l.total = l.red + (uint32_t)(kWaves * nb * kRows) * 16u;
  return l;
}

__device__ inline f16x4 as_h4(uint32_t a, uint32_t b) { return __builtin_bit_cast(f16x4, u32x2{a, b}); }

// rows_base / rows_extra count row units: single rows, or (gate, up) row pairs
// (GATED).  `scales` is rounded down to 16 bytes by the launcher and sc_shift
// bytes added back here, so the 16-byte staging loads are aligned in memory.
template <int M, int G, bool GATED, int D>
__global__ void __launch_bounds__(kThreads)
gemv_mfma_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
                 const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
                 int N, int K, int rows_base, int rows_extra, uint32_t sc_shift) {
  constexpr int kUnit = GATED ? 2 : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // timeline stamps (profiling build only; the four-row, non-gated kernel)
  constexpr bool kStamped = M == 4 && !GATED;
  W4A16_STAMP_DECL;
  if (kStamped) W4A16_STAMP(0);
  const int lr = (lane & 3) + 4 * (lane >> 5);    // weight row of the block (B column)
  const int lc = (lane >> 2) & 7;                 // 32-k chunk of the line
  const int li = lane & 3;                        // A row of the 4 x 4 block

  const int blk = blockIdx.x;
  const int nr = kUnit * (rows_base + (blk < rows_extra ? 1 : 0));
  const int r0 = kUnit * (blk * rows_base + (blk < rows_extra ? blk : rows_extra));
  const int nb = (nr + kRows - 1) / kRows;        // blocks (<= kMaxBlocks, checked on the host)
  const int lines = (K + KL - 1) / KL;
  const int units = nb * lines;
  const int spr = K / G;
  const Layout L = lds_layout(M, K, spr, kUnit * (rows_base + (rows_extra ? 1 : 0)));
  const uint32_t xp = x_pitch(K);

  // ---- this wave's units [u0, u1) and its first loads ----
  // Waves 0 .. kWaves/2 - 1 are the older wave of their SIMD and issue first:
  // they take a share 1 + skew of the units, the younger half 1 - skew.
  auto bound = [&](int w) {
    constexpr int kHalf = kWaves / 2;
    const int64_t cum = w <= kHalf ? (int64_t)w * (1024 + kSkew)
                                   : (int64_t)kHalf * (1024 + kSkew) + (int64_t)(w - kHalf) * (1024 - kSkew);
    return (int)(cum * units / (kWaves * 1024));
  };
  const int u0 = bound(wave), u1 = bound(wave + 1);
  const uint32_t row_w = (uint32_t)K >> 1;
  // the descriptor covers exactly the workgroup's rows: rows past its range read zero
  const __amdgpu_buffer_rsrc_t wres =
      make_rsrc(reinterpret_cast<const uint8_t*>(packed) + (size_t)r0 * row_w, (uint32_t)nr * row_w);
  const uint32_t w_v = (uint32_t)lr * row_w + 16u * (uint32_t)lc;
  // on the last line, chunks that start at or past K load nothing (zeros)
  const bool tail_ok = KL * (lines - 1) + 32 * lc < K;
  const uint32_t w_v_tail = tail_ok ? w_v : kOutOfRange;
  // cursors (wave-uniform): the next unit to load is (ib, is), line-minor
  const int b_first = u0 / lines, s_first = u0 - b_first * lines;
  int iu = u0, ib = b_first, is = s_first;
  u32x4 ring[D];
  // Every slot is loaded unconditionally, in a fixed order, so the compiler can
  // wait for each load alone (vmcnt); a load past the wave's units has an
  // out-of-range offset and a zero scalar offset: it touches no memory.
  auto issue = [&](int slot) __attribute__((always_inline)) {
    const bool live = iu < u1;
    const uint32_t voff = !live ? kOutOfRange : (is == lines - 1 ? w_v_tail : w_v);
    ring[slot] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
        wres, voff, live ? (uint32_t)(kRows * ib) * row_w + 128u * (uint32_t)is : 0u, kStream));
    ++iu;
    if (++is == lines) {
      is = 0;
      ++ib;
    }
  };
  // ---- stage the activations (and their 32-k sums), the scales, zero partials ----
  // chunk c of row m: 8 k, stored permuted; 4 consecutive chunks (lanes) are one 32-k sum
  const int chunks = lines * (KL / 8);
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  // scales of the workgroup's rows, 16-byte chunks from an aligned start
  const uint32_t sc_begin = (uint32_t)r0 * (uint32_t)spr * 2u + sc_shift;
  const uint32_t sc_a0 = sc_begin & ~15u;
  const uint32_t sc_bytes = (uint32_t)N * (uint32_t)spr * 2u + sc_shift;
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(scales, sc_bytes);
  const uint32_t sc_chunks = (sc_begin - sc_a0 + (uint32_t)nr * (uint32_t)spr * 2u + 15u) >> 4;
  // thread tid takes chunks c0 + tid and c0 + tid + kThreads of every row: 2 M
  // loads in flight, no index division
  u32x4 sv[2][M];
  auto load_stage = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = c0 + h * kThreads + tid;
      const bool ok = c < chunks && 8 * c < K;
#pragma unroll
      for (int m = 0; m < M; ++m)
        sv[h][m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
            xres, ok ? ((uint32_t)m * (uint32_t)K + 8u * (uint32_t)c) * 2u : kOutOfRange, 0, 0));
    }
  };
  auto store_stage = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = c0 + h * kThreads + tid;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (c < chunks)
          *reinterpret_cast<u32x4*>(smem + L.xs + (uint32_t)m * xp + 16u * (uint32_t)c) = permute_a(sv[h][m]);
        // the 32-k sum over 4 chunks, which are 4 consecutive lanes (one DPP quad;
        // chunks per row are a multiple of 4 and so is the thread count)
        float sum = dot2(sv[h][m].x, kBiasPair, 0.f);
        sum = dot2(sv[h][m].y, kBiasPair, sum);
        sum = dot2(sv[h][m].z, kBiasPair, sum);
        sum = dot2(sv[h][m].w, kBiasPair, sum);
        sum = dpp_add<0xB1>(sum);    // quad_perm [1,0,3,2]
        sum = dpp_add<0x4E>(sum);    // quad_perm [2,3,0,1]
        if (c < chunks && (c & 3) == 0) reinterpret_cast<float*>(smem + L.xsum)[(c >> 2) * 4 + m] = sum;
      }
    }
  };
  // The first activation and scale loads go out before the first weight loads, so
  // the staging does not wait behind them (measured faster for short and long
  // streams alike).
  u32x4 sc_first = u32x4{};
  if ((uint32_t)tid < sc_chunks) sc_first = load16_tail(sres, sc_a0 + (uint32_t)tid * 16u, sc_bytes);
  load_stage(0);
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d);
  store_stage(0);
  for (int c0 = 2 * kThreads; c0 < chunks; c0 += 2 * kThreads) {
    load_stage(c0);
    store_stage(c0);
  }
  if ((uint32_t)tid < sc_chunks) *reinterpret_cast<u32x4*>(smem + L.sc + (uint32_t)tid * 16u) = sc_first;
  for (uint32_t t = tid + kThreads; t < sc_chunks; t += kThreads)
    *reinterpret_cast<u32x4*>(smem + L.sc + t * 16u) = load16_tail(sres, sc_a0 + t * 16u, sc_bytes);
  for (uint32_t t = tid; t < (uint32_t)(kWaves * nb * kRows); t += kThreads)
    reinterpret_cast<f32x4*>(smem + L.red)[t] = f32x4{};
  __syncthreads();
  if (kStamped) W4A16_STAMP(1);

  // ---- main loop over this wave's units ----
  // A operand: activation row li mod M, the lane's chunk (lanes of other rows read the same addresses)
  const uint8_t* xa = smem + L.xs + (uint32_t)(li % M) * xp + 64u * (uint32_t)lc;
  const uint8_t* xsa = smem + L.xsum + 16u * (uint32_t)lc;
  // the workgroup's scales (row-major, spr per row)
  const uint8_t* scb = smem + L.sc + (((uint32_t)r0 * (uint32_t)spr * 2u + sc_shift) & 15u);
  f32x4 acc = f32x4{};
  // consume cursor (b, s); a block's partial sums go to LDS after its last
  // line, or at the end if the wave stops inside the block
  int b = b_first, s = s_first;
  auto flush = [&]() __attribute__((always_inline)) {
    // add the eight chunk lanes of each row: lane bits 2, 3 (DPP), then bit 4
    f32x4 v = acc;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      float t = dpp_add<0x124>(v[i]);   // row_ror:4
      t = dpp_add<0x128>(t);            // row_ror:8
      t += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, t), 0x401F));   // lane ^ 16
      v[i] = t * 0x1p20f;
    }
    if (lc == 0) reinterpret_cast<f32x4*>(smem + L.red)[(wave * nb + b) * kRows + lr] = v;
    acc = f32x4{};
  };
  // Masks and exponents in registers, so each pair of codes is one v_and_or_b32.
  const uint32_t m_lo = __builtin_amdgcn_readfirstlane(0x000F000Fu), m_hi = __builtin_amdgcn_readfirstlane(0x00F000F0u);
  uint32_t e_even = 0x14001400u, e_odd = 0x04000400u;   // fp16 exponent fields 5 and 1, both halves
  asm volatile("" : "+v"(e_even), "+v"(e_odd));
  // The LDS operands of a unit: the lane's activations and chunk sums, and its
  // scale -- 0 for rows past the workgroup's range and chunks past K (zero
  // weights), read from a clamped, valid address so the read is unconditional.
  struct Opnd {
    u32x4 xf[4];
    f32x4 xsum;
    float sc;
  };
  auto read_opnd = [&](int bb, int ss, Opnd& o) __attribute__((always_inline)) {
    const uint8_t* xs = xa + 512u * (uint32_t)ss;
#pragma unroll
    for (int w = 0; w < 4; ++w) o.xf[w] = *reinterpret_cast<const u32x4*>(xs + 16 * w);
    o.xsum = *reinterpret_cast<const f32x4*>(xsa + 128u * (uint32_t)ss);
    const int row = kRows * bb + lr;
    const uint32_t kc = (uint32_t)(KL * ss + 32 * lc);
    const bool ok = row < nr && kc < (uint32_t)K;
    const uint32_t idx = ok ? (uint32_t)row * (uint32_t)spr + kc / G : 0u;
    const float v = half_bits_to_float(*reinterpret_cast<const uint16_t*>(scb + 2u * idx));
    o.sc = ok ? v : 0.f;
  };
  Opnd cur;
  read_opnd(b, s, cur);
  // One unit: the next unit's LDS operands are read before this one's arithmetic.
  auto consume = [&](const u32x4& wv) __attribute__((always_inline)) {
    const bool last_line = s + 1 == lines;
    Opnd nxt;
    read_opnd(last_line ? b + 1 : b, last_line ? 0 : s + 1, nxt);
    f32x4 t = f32x4{};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t q = w == 0 ? wv.x : (w == 1 ? wv.y : (w == 2 ? wv.z : wv.w));
      const uint32_t q8 = q >> 8;
      // even k (0, 4), (2, 6) with x pairs (0, 4), (2, 6); odd k (1, 5), (3, 7) likewise
      t = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(cur.xf[w].x, cur.xf[w].y),
                                             as_h4((q & m_lo) | e_even, (q8 & m_lo) | e_even), t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(cur.xf[w].z, cur.xf[w].w),
                                             as_h4((q & m_hi) | e_odd, (q8 & m_hi) | e_odd), t, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < M; ++i) acc[i] = __builtin_fmaf(cur.sc, t[i] - cur.xsum[i], acc[i]);
    if (last_line) flush();
    b += last_line ? 1 : 0;
    s = last_line ? 0 : s + 1;
    cur = nxt;
  };
  // Whole rounds of D units, then the wave's last units (fewer than D) after the
  // loop (for this kernel measured faster than skipping slots inside the loop).
  int u = u0;
  for (; u + D <= u1; u += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      consume(ring[d]);
      if (kStamped && d == 0 && u == u0) W4A16_STAMP(2);
      issue(d);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (u + d < u1) consume(ring[d]);
  if (s != 0) flush();
  if (kStamped) W4A16_STAMP(3);

  // ---- add the waves' partials in wave order, round once, store ----
  __syncthreads();
  if (kStamped) W4A16_STAMP(4);
  const f32x4* red = reinterpret_cast<const f32x4*>(smem + L.red);
  if constexpr (GATED) {
    // rows (2i, 2i + 1) of a block are one (gate, up) pair
    for (int t = tid; t < nb * (kRows / 2); t += kThreads) {
      const int bb = t / (kRows / 2), c = 2 * (t % (kRows / 2));
      f32x4 g = red[bb * kRows + c], v = red[bb * kRows + c + 1];
      for (int w = 1; w < kWaves; ++w) {
        g += red[(w * nb + bb) * kRows + c];
        v += red[(w * nb + bb) * kRows + c + 1];
      }
      const int row = kRows * bb + c;
      if (row < nr) {
#pragma unroll
        for (int m = 0; m < M; ++m)
          y[(size_t)m * (N >> 1) + ((r0 + row) >> 1)] = float_to_half_bits(g[m] / (1.f + __expf(-g[m])) * v[m]);
      }
    }
  } else {
    for (int t = tid; t < nb * kRows; t += kThreads) {
      const int bb = t / kRows, c = t % kRows;
      f32x4 v = red[bb * kRows + c];
      for (int w = 1; w < kWaves; ++w) v += red[(w * nb + bb) * kRows + c];
      const int row = kRows * bb + c;
      if (row < nr) {
#pragma unroll
        for (int m = 0; m < M; ++m) y[(size_t)m * N + r0 + row] = float_to_half_bits(v[m]);
      }
    }
  }
  if (kStamped) {
    W4A16_STAMP(5);
    W4A16_STAMP_FLUSH(wave);
  }
}

template <int M, int G, bool GATED, int D>
hipError_t launch_d(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int n, int k,
                    int blocks, size_t lds, const DeviceInfo& dev, hipStream_t stream) {
  static std::atomic<uint64_t> attr_set{0};   // one bit per device
  const uint64_t bit = 1ull << (dev.device & 63);
  auto kern = gemv_mfma_kernel<M, G, GATED, D>;
  if (!(attr_set.load(std::memory_order_acquire) & bit)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int units = GATED ? n / 2 : n;
  const uint32_t sc_shift = (uint32_t)(reinterpret_cast<uintptr_t>(scales) & 15u);
  const uint16_t* sc_aligned = reinterpret_cast<const uint16_t*>(reinterpret_cast<uintptr_t>(scales) - sc_shift);
  return launch_kernel(kern, dim3(blocks), dim3(kThreads), lds, stream, x, packed, sc_aligned, y, n, k,
                       units / blocks, units % blocks, sc_shift);
}

template <int M, int G, bool GATED>
hipError_t launch_m(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int n, int k,
                    int blocks, size_t lds, const DeviceInfo& dev, hipStream_t stream) {
  // units per wave of the largest workgroup: 8-row blocks x 256-k lines over the waves
  const int unit = GATED ? 2 : 1;
  const int per = n / unit;
  const int rows = unit * (per / blocks + (per % blocks ? 1 : 0));
  const int upw = ((rows + kRows - 1) / kRows) * ((k + KL - 1) / KL) / kWaves;
  return upw <= kShallowUnits ? launch_d<M, G, GATED, kShallowDepth>(x, packed, scales, y, n, k, blocks, lds, dev, stream)
                              : launch_d<M, G, GATED, kDepth>(x, packed, scales, y, n, k, blocks, lds, dev, stream);
}

template <int M, bool GATED>
hipError_t launch_g(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int n, int k,
                    int group, int blocks, size_t lds, const DeviceInfo& dev, hipStream_t stream) {
  return group == 32 ? launch_m<M, 32, GATED>(x, packed, scales, y, n, k, blocks, lds, dev, stream)
                     : launch_m<M, 128, GATED>(x, packed, scales, y, n, k, blocks, lds, dev, stream);
}

}  // namespace

bool gemv_mfma_plan(int m, int n, int k, int group, const DeviceInfo& dev, int* blocks, size_t* lds, bool gated) {
  if (m < 2 || m > 4 || n <= 0 || k <= 0 || (group != 32 && group != 128)) return false;
  // Rows are handed out in units: single rows, or (gate, up) row pairs.
  const int unit = gated ? 2 : 1;
  if (n % unit) return false;
  const int units = n / unit;
  // W4A16_NP4_WG_PER_CU workgroups per CU, more if a workgroup would exceed
  // kMaxBlocks row blocks.
  int g = dev.num_cu * W4A16_NP4_WG_PER_CU;
  const int per = kRows * kMaxBlocks / unit;
  if ((int64_t)g * per < units) g = (units + per - 1) / per;
  if (g > units) g = units;
  const int rows_max = unit * (units / g + (units % g ? 1 : 0));
  const size_t bytes = lds_layout(m, k, k / group, rows_max).total;
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
