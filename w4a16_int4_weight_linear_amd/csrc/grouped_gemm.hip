// grouped_gemm.hip -- MoE grouped GEMM of the W4A16 int4 weight-only layer on gfx950.
//
// The routed-expert layers of the 35B-A3B MoE model on the LLM170 CUDA/W4A16
// page (g32): x holds one row per (token, expert) pair, sorted by expert, and
// the rows offsets[e] .. offsets[e+1]-1 are multiplied by expert e's packed
// weights.  With a few rows per expert (16 on average for 512 tokens routed
// top-8 over 256 experts) the work is bound by streaming the experts' weights
// from HBM, not by the matrix cores, so the kernel is organised around that
// stream:
//
// * Work items are (expert, block of up to 32 of its rows), found on the device
//   from the offsets: expert e contributes ceil(rows_e / 32) items, so an
//   expert that received no rows reads nothing and a heavily routed expert is
//   spread over many workgroups (which then share its weights through L2/MALL)
//   instead of looping over its rows in one.
// * One 512-thread workgroup per (item, band of 256 output columns); each of
//   its eight waves owns 32 columns (two 16-column MFMA blocks).  The two bands
//   of an item are placed on the same XCD, so their activation rows meet in one
//   L2.
// * Weights are read in K steps of 256 k (one 128-byte line per weight row):
//   each load instruction covers 8 rows x 128 bytes, since loads of the MFMA
//   operand shape (16 rows x 64 bytes) make the memory system fetch some lines
//   twice (FETCH_SIZE 186-203 MB against 172 MB per launch).  The lines go
//   through a per-wave LDS tile into operand layout and are dequantised in
//   registers; one step is in flight ahead of use (deeper rings measured
//   slower).  The group scales arrive by one vector load per step and block.
// * The item's activation rows are staged in LDS one step at a time, double
//   buffered, with one workgroup barrier per step; the next step's rows are
//   loaded into registers a full step before they are written.
// * The weights are the MFMA's A operand (v_mfma_f32_16x16x32_f16, 16 columns
//   x 32 k) and the activations its B operand, so a lane ends with four
//   consecutive output columns of one row: 8-byte stores.
// * Gather variant (launch_grouped_gemm_gather): row r's activations are read
//   from token pair_token[r] of the unsorted token rows, so the expert-sorted
//   copy of the activations is never written.
// * SwiGLU variant (launch_grouped_gemm_swiglu, the experts' fused gate/up
//   projection): each expert's weight rows interleave gate (even) and up (odd)
//   rows, so a lane's four consecutive output columns are two whole (gate, up)
//   pairs, and the epilogue writes SiLU(gate) * up for both (fp32, rounded
//   once): the 2 x rows x n intermediate never reaches memory.
#include "device.hpp"
#include "kernels.hpp"
#include "launch.hpp"
#include "mfma_operands.hpp"

#include <type_traits>

namespace w4a16 {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kWaveN = 32;                 // columns per wave
constexpr int BN = kWaves * kWaveN;        // output columns per workgroup
constexpr int kNB = kWaveN / 16;           // 16-column MFMA blocks per wave
constexpr int RB = 32;                     // rows per work item
constexpr int KC = 128;                    // k per chunk: 16 bytes per lane and block in operand layout
constexpr int KS = 2 * KC;                 // k per K step: one 128-byte line per weight row
constexpr int kDepth = 1;                  // K steps of weights in flight (a deeper ring measured slower)
constexpr int kAPitch = KS * 2 + 16;       // bytes per staged activation row: rows shift by 4 banks
constexpr int kABuf = RB * kAPitch;        // one staged activation block
constexpr int kRowThreads = kThreads / RB;        // threads staging one activation row
constexpr int kXPieces = KS / 8 / kRowThreads;     // 16-byte activation pieces per thread and step
constexpr int kTileWave = kNB * 16 * 128;  // per-wave weight transpose tile
constexpr int kTileBase = 2 * kABuf;
constexpr int kLds = kTileBase + kWaves * kTileWave;

static_assert(kXPieces >= 1 && kXPieces * kRowThreads * 8 == KS, "activation staging covers a step");
static_assert(kLds <= 80 * 1024, "two workgroups per CU");

struct Item {
  int row_begin;   // first row of x / y
  int rows;        // rows of this item, 1..RB
  int expert;
};

// Work item `item` in expert order (expert e owns ceil(r_e / RB) consecutive
// items).  Every lane gets the same answer; false when `item` is past the
// last one.  Lane l inspects experts e0 + 4l .. e0 + 4l + 3 per round of 256.
__device__ inline bool find_item(const int32_t* __restrict__ offsets, int experts, int item, Item& out) {
  const int lane = lane_id();
  int base = 0;
  for (int e0 = 0; e0 < experts; e0 += 256) {
    const int eb = e0 + 4 * lane;
    int o[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) o[j] = offsets[min(eb + j, experts)];
    int cnt[4];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = eb + j < experts ? max(o[j + 1] - o[j], 0) : 0;
      cnt[j] = (r + RB - 1) / RB;
      sum += cnt[j];
    }
    int incl = sum;   // inclusive prefix sum over lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (item < base + total) {
      const uint64_t hit = __ballot(base + incl > item);
      const int L = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
      int before = base + __builtin_amdgcn_readlane(incl - sum, L);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = __builtin_amdgcn_readlane(cnt[j], L);
        if (item < before + c) {
          const int rb = item - before;
          const int first = __builtin_amdgcn_readlane(o[j], L) + rb * RB;
          const int last = __builtin_amdgcn_readlane(o[j + 1], L);
          out.row_begin = first;
          out.rows = min(RB, last - first);
          out.expert = e0 + 4 * L + j;
          return true;
        }
        before += c;
      }
      return false;   // unreachable with consistent counts
    }
    base += total;
  }
  return false;
}

// One item of MB 16-row blocks (rows <= 16 * MB).  G is the group size; ALIGNED:
// each scale row starts on a 16-byte (G = 32) or 4-byte (G = 128) boundary, so
// one vector load brings a K step's scales.
//
// Weight loads cover whole 128-byte lines: a load instruction reads 8 rows x
// 128 bytes (8 lanes per row), which is what the memory system serves without
// refetching (a load of 16 rows x 64 bytes, the MFMA operand shape, fetches
// some lines twice).  Each lane's 16 bytes are written to a per-wave LDS tile
// [16 rows][128 B] and read back in operand layout (lane = row li, 32 k of
// slice lq).  Inside a row the 16-byte slots are XOR-swizzled by (row / 2) so
// the operand reads hit distinct banks; the swizzle is applied to which piece
// a lane loads, so the LDS write stays one contiguous 1 KB per instruction.
template <int G, bool ALIGNED, int MB, bool SWIGLU>
__device__ __forceinline__ void item_body(const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed_e,
                                          const uint16_t* __restrict__ scales_e, uint16_t* __restrict__ y,
                                          int N, int K, int rows_total, const Item& it, int band, uint8_t* lds,
                                          const int32_t* __restrict__ pair_token, int x_rows) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane >> 4;   // which 32 k of a chunk (and which 4 columns of an output block)
  const int li = lane & 15;   // column within a block (and row within an output block)
  const int nw = band * BN + wave * kWaveN;

  const uint32_t row_w = (uint32_t)K >> 1;                 // packed bytes per weight row
  const uint32_t spr = (uint32_t)(K / G);                  // scales per weight row
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(packed_e, (uint32_t)N * row_w);
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(scales_e, (uint32_t)N * spr * 2u);
  const uint32_t kbytes = (uint32_t)K * 2u;
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(x, (uint32_t)x_rows * kbytes);
  const int steps = (K + KS - 1) / KS;

  // ---- whole-line weight loads: instruction i of block b reads rows 8 i .. 8 i + 7 ----
  uint32_t woff[kNB][2];   // per-lane byte offset of the first step (out of range: invalid row)
  int klim[2];             // step s is inside K for this lane while KS * s < klim
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * i + (lane >> 3);                     // row of the block tile
    const int q = (lane & 7) ^ ((r >> 1) & 7);             // 16-byte piece of the 128-byte line
    klim[i] = K - 32 * q;
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const int n = nw + b * 16 + r;
      woff[b][i] = n < N ? (uint32_t)n * row_w + 16u * (uint32_t)q : kOutOfRange;
    }
  }
  auto load_raw = [&](int s, int b, int i) -> u32x4 {
    const uint32_t off = KS * s < klim[i] ? woff[b][i] : kOutOfRange;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, off, 128 * s, kStream));
  };
  // per-wave transpose tile: [block][16 rows][128 B]
  uint8_t* tile = lds + kTileBase + wave * kTileWave;
  uint8_t* tile_w = tile + 16 * lane;
  const uint32_t swz = (uint32_t)((li >> 1) & 7);
  const uint8_t* tile_r0 = tile + li * 128 + 16 * ((uint32_t)lq ^ swz);         // chunk 0 of the step
  const uint8_t* tile_r1 = tile + li * 128 + 16 * ((uint32_t)(4 + lq) ^ swz);   // chunk 1

  // ---- scales, in operand layout (column nw + 16 b + li) ----
  uint32_t sbase[kNB];
  bool colok[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int n = nw + b * 16 + li;
    colok[b] = n < N;
    sbase[b] = (uint32_t)n * spr * 2u;
  }
  // G = 32, aligned, four steps per load: lane lq of row li loads the 16 bytes
  // (8 groups) of step 4 S + lq, so one instruction reads 64 contiguous bytes of
  // each scale row (loading each step's 16 bytes separately made the memory
  // system fetch every scale line several times).  A lane takes its scale from
  // the lane that loaded its step (a cross-lane read).
  auto load_s32x4 = [&](int S, int b) -> u32x4 {
    const int st = 4 * S + lq;
    const uint32_t off = (colok[b] && 8 * st < (int)spr) ? sbase[b] + 16u * (uint32_t)st : kOutOfRange;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sres, off, 0, 0));
  };
  // G = 128, aligned: groups 2 s, 2 s + 1
  auto load_s128 = [&](int s, int b) -> uint32_t {
    const uint32_t off = (colok[b] && 2 * s < (int)spr) ? sbase[b] + 4u * (uint32_t)s : kOutOfRange;
    return __builtin_amdgcn_raw_buffer_load_b32(sres, off, 0, 0);
  };
  // any alignment: the group of k = 128 c + 32 lq, chunk c = 2 s + h
  auto load_s16 = [&](int s, int h, int b) -> uint32_t {
    const int k = KC * (2 * s + h) + 32 * lq;
    const uint32_t off = (colok[b] && k < K) ? sbase[b] + 2u * (uint32_t)(k / G) : kOutOfRange;
    return __builtin_amdgcn_raw_buffer_load_b16(sres, off, 0, 0);
  };

  // ---- activation staging: thread -> row tid / 16, pieces (tid % 16) + 16 p of a step ----
  const int xr = tid / kRowThreads;
  const int xp = tid % kRowThreads;
  const bool xrow_ok = xr < it.rows;
  // gather: row r of the grouped product is token pair_token[r] of x (a token
  // outside x reads zero through the descriptor's range check)
  const int grow = it.row_begin + xr;
  const uint32_t xsrc = (pair_token && xrow_ok && grow < rows_total) ? (uint32_t)pair_token[grow] : (uint32_t)grow;
  const uint32_t xrow_off = xsrc < (uint32_t)x_rows ? xsrc * kbytes : kOutOfRange;
  auto load_x = [&](int s, u32x4 (&v)[kXPieces]) {
#pragma unroll
    for (int p = 0; p < kXPieces; ++p) {
      const int k = KS * s + 8 * (xp + kRowThreads * p);
      const uint32_t off = (xrow_ok && k < K) ? xrow_off + 2u * (uint32_t)k : kOutOfRange;
      v[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0));
    }
  };
  auto store_x = [&](int s, const u32x4 (&v)[kXPieces]) {
    uint8_t* dst = lds + (s & 1) * kABuf + xr * kAPitch + xp * 16;
#pragma unroll
    for (int p = 0; p < kXPieces; ++p) *reinterpret_cast<u32x4*>(dst + 16 * kRowThreads * p) = permute_a(v[p]);
  };

  // ---- prologue: kDepth steps of weights and scales, first activation block ----
  u32x4 raw[kDepth][kNB][2];
  uint32_t s128[kDepth][kNB];
  uint32_t s16[kDepth][kNB][2];
  auto issue_step = [&](int s, int slot) {
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      raw[slot][b][0] = load_raw(s, b, 0);
      raw[slot][b][1] = load_raw(s, b, 1);
      if constexpr (ALIGNED && G == 128) s128[slot][b] = load_s128(s, b);
      if constexpr (!ALIGNED) { s16[slot][b][0] = load_s16(s, 0, b); s16[slot][b][1] = load_s16(s, 1, b); }
    }
  };
#pragma unroll
  for (int d = 0; d < kDepth; ++d) issue_step(d, d);
  u32x4 sq_cur[kNB], sq_nxt[kNB];                   // G = 32 aligned: scales of steps 4 S .. 4 S + 3, 4 S + 4 ..
  if constexpr (ALIGNED && G == 32) {
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      sq_cur[b] = load_s32x4(0, b);
      sq_nxt[b] = load_s32x4(1, b);
    }
  }
  u32x4 xv[kXPieces];
  load_x(0, xv);
  store_x(0, xv);
  if (steps > 1) load_x(1, xv);
  __syncthreads();

  f32x4 acc[MB][kNB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int b = 0; b < kNB; ++b) acc[i][b] = f32x4{};

  // B-operand rows: this lane reads row li (+16 i), k 32 lq + 8 w of chunk h
  const uint8_t* xfrag = lds + li * kAPitch + 64 * lq;

  auto step = [&](int s, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    // transpose this step's weight lines into operand layout
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      *reinterpret_cast<u32x4*>(tile_w + b * 2048) = raw[slot][b][0];
      *reinterpret_cast<u32x4*>(tile_w + b * 2048 + 1024) = raw[slot][b][1];
    }
    u32x4 wq[2][kNB];
    f16x2 sv[2][kNB];
    if constexpr (ALIGNED && G == 32) {
      if ((s & 3) == 0 && s > 0) {
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
          sq_cur[b] = sq_nxt[b];
          sq_nxt[b] = load_s32x4((s >> 2) + 1, b);
        }
      }
    }
    // lane (li, lq) needs group 8 s + 4 h + lq: dword 2 h + lq / 2, half lq & 1 of
    // the 16 bytes that lane (li, s & 3) loaded
    const int src_lane = 16 * (s & 3) + li;
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      wq[0][b] = *reinterpret_cast<const u32x4*>(tile_r0 + b * 2048);
      wq[1][b] = *reinterpret_cast<const u32x4*>(tile_r1 + b * 2048);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (!ALIGNED) {
          const _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)s16[slot][b][h]);
          sv[h][b] = f16x2{v, v};
        } else if constexpr (G == 32) {
          const u32x4 v = sq_cur[b];
          const int lo = __shfl((int)(h ? v.z : v.x), src_lane);
          const int hi = __shfl((int)(h ? v.w : v.y), src_lane);
          const uint32_t d = (uint32_t)((lq >> 1) ? hi : lo);
          sv[h][b] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(d, d, (lq & 1) ? 0x03020302u : 0x01000100u));
        } else {
          const uint32_t v = s128[slot][b];
          sv[h][b] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(v, v, h ? 0x03020302u : 0x01000100u));
        }
      }
    }
    // refill the ring slot kDepth steps ahead (past the end: no memory access)
    issue_step(s + kDepth, slot);

    const uint8_t* xb = xfrag + (s & 1) * kABuf;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        f16x8 xf[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
          xf[i] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(xb + i * 16 * kAPitch + 256 * h + 16 * w));
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
          const u32x4 wv = wq[h][b];
          const uint32_t q = w == 0 ? wv.x : (w == 1 ? wv.y : (w == 2 ? wv.z : wv.w));
          const f16x8 wf = dequant_word(q, sv[h][b]);
#pragma unroll
          for (int i = 0; i < MB; ++i) acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, xf[i], acc[i][b], 0, 0, 0);
        }
      }
    }
    if (s + 1 < steps) {
      store_x(s + 1, xv);
      if (s + 2 < steps) load_x(s + 2, xv);
      __syncthreads();
    }
  };
  static_assert(kDepth == 1 || kDepth == 2, "the step loop cycles through the ring slots");
  for (int s = 0; s < steps; s += kDepth) {
    step(s, std::integral_constant<int, 0>{});
    if constexpr (kDepth == 2) {
      if (s + 1 < steps) step(s + 1, std::integral_constant<int, kDepth - 1>{});
    }
  }

  // ---- epilogue: lane holds columns 4 lq .. 4 lq + 3 of block b for row li (+16 i) ----
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r = i * 16 + li;
    const int row = it.row_begin + r;
    if (r >= it.rows || row < 0 || row >= rows_total) continue;
    if constexpr (SWIGLU) {
      // columns n0, n0 + 1 and n0 + 2, n0 + 3 are (gate, up) pairs: outputs n0 / 2, n0 / 2 + 1
      const int no = N >> 1;
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        const int c0 = (nw + b * 16 + 4 * lq) >> 1;
        const float g0 = acc[i][b][0], g1 = acc[i][b][2];
        const uint16_t h0 = float_to_half_bits(g0 / (1.0f + __expf(-g0)) * acc[i][b][1]);
        const uint16_t h1 = float_to_half_bits(g1 / (1.0f + __expf(-g1)) * acc[i][b][3]);
        uint16_t* dst = y + (size_t)row * no + c0;
        if ((no & 1) == 0 && c0 + 1 < no) {
          *reinterpret_cast<uint32_t*>(dst) = h0 | ((uint32_t)h1 << 16);
        } else {
          if (c0 < no) dst[0] = h0;
          if (c0 + 1 < no) dst[1] = h1;
        }
      }
      continue;
    }
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const int n0 = nw + b * 16 + 4 * lq;
      uint16_t h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = float_to_half_bits(acc[i][b][j]);
      uint16_t* dst = y + (size_t)row * N + n0;
      if ((N & 3) == 0 && n0 + 3 < N) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (n0 + j < N) dst[j] = h[j];
      }
    }
  }
}

template <int G, bool ALIGNED, bool SWIGLU>
__global__ void __launch_bounds__(kThreads)
grouped_gemm_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
                    const uint16_t* __restrict__ scales, const int32_t* __restrict__ offsets,
                    uint16_t* __restrict__ y, int experts, int N, int K, int rows_total, int bands,
                    const int32_t* __restrict__ pair_token, int x_rows) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];

  // Consecutive workgroup ids go to different XCDs (round robin over 8): the
  // bands of one item take ids 8 apart, so they run on the same XCD.
  const int bid = blockIdx.x;
  const int item = (bid / (8 * bands)) * 8 + (bid & 7);
  const int band = (bid >> 3) % bands;

  Item it;
  if (!find_item(offsets, experts, item, it) || it.rows <= 0) return;

  const size_t e = (size_t)it.expert;
  const uint32_t* pe = packed + e * (size_t)N * (size_t)(K >> 3);
  const uint16_t* se = scales + e * (size_t)N * (size_t)(K / G);
  if (it.rows > 16)
    item_body<G, ALIGNED, 2, SWIGLU>(x, pe, se, y, N, K, rows_total, it, band, lds, pair_token, x_rows);
  else
    item_body<G, ALIGNED, 1, SWIGLU>(x, pe, se, y, N, K, rows_total, it, band, lds, pair_token, x_rows);
}

}  // namespace

namespace {

// n: weight rows per expert (2 x the outputs for SWIGLU)
template <bool SWIGLU>
hipError_t launch_grouped(const uint16_t* x, const int32_t* pair_token, int x_rows, const uint32_t* packed,
                          const uint16_t* scales, const int32_t* offsets, uint16_t* y, int experts, int rows, int n,
                          int k, int group, hipStream_t stream) {
  const int bands = (n + BN - 1) / BN;
  // sum over experts of ceil(r_e / RB) <= experts + ceil(rows / RB); rounded up to whole XCD rounds
  const int64_t items = ((int64_t)experts + (rows + RB - 1) / RB + 7) / 8 * 8;
  const int64_t blocks = items * bands;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int spr = k / group;
  const dim3 grid((unsigned)blocks), block(kThreads);
  // one vector load per row brings a step's scales when every scale row is
  // 16-byte (g32) or 4-byte (g128) aligned in memory
  const uintptr_t sp = reinterpret_cast<uintptr_t>(scales);
  auto kern = group == 32
                  ? (spr % 8 == 0 && (sp & 15) == 0 ? grouped_gemm_kernel<32, true, SWIGLU>
                                                    : grouped_gemm_kernel<32, false, SWIGLU>)
                  : (spr % 2 == 0 && (sp & 3) == 0 ? grouped_gemm_kernel<128, true, SWIGLU>
                                                   : grouped_gemm_kernel<128, false, SWIGLU>);
  return launch_kernel(kern, grid, block, 0, stream, x, packed, scales, offsets, y, experts, n, k, rows, bands,
                       pair_token, x_rows);
}

}  // namespace

hipError_t launch_grouped_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                               const int32_t* offsets, uint16_t* y, int experts, int rows, int n, int k,
                               int group, const DeviceInfo&, hipStream_t stream) {
  return launch_grouped<false>(x, nullptr, rows, packed, scales, offsets, y, experts, rows, n, k, group, stream);
}

hipError_t launch_grouped_gemm_gather(const uint16_t* x, const int32_t* pair_token, int tokens,
                                      const uint32_t* packed, const uint16_t* scales, const int32_t* offsets,
                                      uint16_t* y, int experts, int rows, int n, int k, int group,
                                      const DeviceInfo&, hipStream_t stream) {
  return launch_grouped<false>(x, pair_token, tokens, packed, scales, offsets, y, experts, rows, n, k, group, stream);
}

hipError_t launch_grouped_gemm_swiglu(const uint16_t* x, const int32_t* pair_token, int x_rows,
                                      const uint32_t* packed, const uint16_t* scales, const int32_t* offsets,
                                      uint16_t* y, int experts, int rows, int n_out, int k, int group,
                                      const DeviceInfo&, hipStream_t stream) {
  return launch_grouped<true>(x, pair_token, x_rows, packed, scales, offsets, y, experts, rows, 2 * n_out, k, group,
                              stream);
}

}  // namespace w4a16
