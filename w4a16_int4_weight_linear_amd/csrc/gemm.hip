// gemm.hip -- prefill GEMM of the W4A16 int4 weight-only layer on gfx950 (fp16 MFMA).
//
// y[m, n] = sum_k x[m, k] * s[n, k / g] * q[n, k] for any M: the prompt
// (prefill) phase of the W4A16 models on the LLM170 CUDA/W4A16 page (pp512,
// pp1024, pp4096 columns).  Here the layer is a dense contraction, so it runs
// on the matrix cores: v_mfma_f32_32x32x16_f16, fp16 inputs, fp32 accumulation.
//
// * Tiles: 128 x 256 outputs, K steps of 128.  One persistent 512-thread
//   workgroup per CU; each of its eight wavefronts (two per SIMD, so one can
//   issue while the other waits on LDS or its dequantisation) owns a 128 x 32
//   slab (4 MFMA blocks of 32 x 32, 64 fp32 accumulators per lane).
// * The activation tile (128 x 128 fp16) and the packed weight tile (256 rows
//   x 64 bytes) of a K step go through a three-stage LDS ring (144 KB): they
//   are loaded straight from global memory into LDS (buffer loads with the
//   LDS bit: no registers, no LDS write instructions), 16 lanes per
//   activation row and 4 per weight row, so every 64-byte L2 request is used
//   whole.  Step r + 2 is loaded while step r computes.  The LDS layouts are
//   XOR-swizzled, so every operand read is free of bank conflicts.
// * Scales come in windows of 8 consecutive groups per weight row: one
//   16-byte global-to-LDS load per row per window into a double-buffered
//   LDS area (8 KB), issued in the first step of the previous window.
//   Loading the one 2-byte scale of a row per step instead would cost one
//   L2 request per row and step, about a third of all requests.  The load
//   is issued in every step, so the step code has no branch: in the steps
//   that need none it goes to a dummy LDS area with an out-of-range global
//   offset (no memory access).  When the rows' scales are not 16-byte
//   aligned (K / g not a multiple of 8), each stage carries its step's
//   scales instead (2-byte loads, stored zero-extended to 4 bytes).
// * Within a step a wavefront runs 8 MFMA sub-steps of 16 k.  The activation
//   operands of sub-step s + 2 are read from LDS and the weights of sub-step
//   s + 1 are dequantised in registers (mfma_operands.hpp) while the MFMAs of
//   sub-step s run; both run across the end of a step, so after the one
//   barrier per step the matrix cores restart at once.  Scheduling groups
//   interleave each MFMA with a few VALU instructions and LDS or global
//   accesses, and a scheduling fence after every sub-step keeps that
//   pipeline order.
// * Work split: whole tiles in data-parallel rounds, the 32 workgroups of an
//   XCD on a 4 x 8 block of neighbouring tiles (shared operands stay in the
//   XCD's L2); the tiles left over after the last full round are split
//   along K (stream-K) over the XCD's workgroups, computed first, and reduced
//   at the end by their contributors in a fixed order (deterministic).  The
//   details are at gemm_plan.
//
// For integer activations, codes and power-of-two scales every product and
// partial sum is exact, so such inputs give bit-exact results.
#include <mutex>

#include "device.hpp"
#include "kernels.hpp"
#include "launch.hpp"
#include "mfma_operands.hpp"

namespace w4a16 {
namespace {

constexpr int kThreads = 512;
constexpr int kWGPerCU = 1;
constexpr int BM = 128, BN = 256, BK = 128;
constexpr int kWaveN = 32;                  // output columns per wave
constexpr int kMB = BM / 32, kNB = kWaveN / 32;
constexpr int kWaves = kThreads / 64;
constexpr int kSub = BK / 16;               // MFMA sub-steps per K step
constexpr int kABytes = BM * BK * 2;        // activation tile: 128 rows of 256 bytes
constexpr int kBBytes = BN * BK / 2;        // packed weight tile: 256 rows of 64 bytes
constexpr int kStageBytes = kABytes + kBBytes;
constexpr int kWinBytes = BN * 16;            // one scale window: 256 rows x 8 groups x 2 bytes
constexpr int kXCD = 8;
constexpr size_t kPartialBytes = (size_t)BM * BN * 4;
constexpr uint32_t kSpinLimit = 1u << 24;   // flag polls before the fix-up gives up
static_assert(3 * kStageBytes + 2 * kWinBytes + 1024 <= 160 * 1024, "LDS use exceeds 160 KB");
static_assert(3 * (kStageBytes + BN * 4 * 4) <= 160 * 1024, "LDS use exceeds 160 KB");

// Work split.  T output tiles of BM x BN, I K steps each, W persistent
// workgroups (a multiple of the 8 XCDs; workgroup g runs on XCD g % 8).
// * Data-parallel rounds: the first D = floor(T / W) * W tiles (in the
//   grouped order of tile_coords) are computed whole, W at a time; in each
//   round the 32 workgroups of an XCD take 32 consecutive tiles, a block of
//   4 tile rows by 8 tile columns, so they share activation rows and weight
//   columns in the XCD's L2 while they move through K in step.
// * Stream-K remainder: the R = T - D leftover tiles are dealt to the XCDs in
//   contiguous ranges, and an XCD's (tile, K step) iterations are split
//   evenly over nsk of its workgroups (at least kMinSKSteps each), which
//   compute them first and store fp32 partial tiles.  A workgroup's range is
//   no longer than one tile, so it touches at most two tiles.
// * Fix-up, last: the contributors of a stream-K tile each reduce one slice
//   of it (all partials of the slice, in contributor order: deterministic)
//   and write fp16.  By then every partial was published long before.
struct GemmPlan {
  int tiles_m, tiles_n, tiles, iters;       // iters: K steps per tile
  int wgs, rounds, sk_tiles, nsk;           // nsk: stream-K workgroups per XCD
};

#ifndef W4A16_GEMM_MIN_SK_STEPS
#define W4A16_GEMM_MIN_SK_STEPS 5
#endif
// K steps per stream-K workgroup, at least: fewer, longer segments write fewer
// fp32 partials (measured best at 5 on the 512-row up projection; M = 384,
// 128 and 4096 unchanged)
constexpr int kMinSKSteps = W4A16_GEMM_MIN_SK_STEPS;
constexpr int kGroupM = 4;                  // tile rows per group of the tile order

GemmPlan gemm_plan(int m, int n, int k, const DeviceInfo& dev) {
  GemmPlan p;
  p.tiles_m = (m + BM - 1) / BM;
  p.tiles_n = (n + BN - 1) / BN;
  p.tiles = p.tiles_m * p.tiles_n;
  p.iters = (k + BK - 1) / BK;
  int per_xcd = (dev.num_cu * kWGPerCU) / kXCD;
  if (per_xcd < 1) per_xcd = 1;
  if (per_xcd > 64) per_xcd = 64;           // the fix-up polls one contributor per lane
  p.wgs = per_xcd * kXCD;
  p.rounds = p.tiles / p.wgs;
  p.sk_tiles = p.tiles - p.rounds * p.wgs;
  // stream-K workgroups per XCD, from the busiest XCD's ceil(R / 8) tiles;
  // at least one per tile, so no range is longer than a tile
  const int cnt_max = (p.sk_tiles + kXCD - 1) / kXCD;
  long long nsk = (long long)cnt_max * p.iters / kMinSKSteps;
  if (nsk < cnt_max) nsk = cnt_max;
  if (nsk > per_xcd) nsk = per_xcd;
  p.nsk = p.sk_tiles ? (int)nsk : 0;
  return p;
}

__device__ inline int xcd_begin(int xcd, int count) {
  const int q = count / kXCD, r = count % kXCD;
  return xcd * q + (xcd < r ? xcd : r);
}

// Tile order: groups of kGroupM tile rows; inside a group, column by column.
__device__ inline void tile_coords(int tau, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupM * tiles_n;
  const int grp = tau / per_group;
  const int first_m = grp * kGroupM;
  const int gsize = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int r = tau - grp * per_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

#define W4A16_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Barrier that publishes LDS: this thread's LDS reads and global-to-LDS
// loads are complete before it, and no LDS access moves across it.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Order of one MFMA sub-step's instructions: each of its 4 MFMAs is
// followed by up to five VALU instructions (the dequantisation of the next
// sub-step) and by one LDS read (operands two sub-steps ahead) and one global
// load.  A scheduling fence after every sub-step keeps
// the reads two sub-steps ahead of their use.
__device__ inline void schedule_substep() {
#pragma unroll
  for (int mi = 0; mi < kMB * kNB; ++mi) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // MFMA
    if (mi < 4) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);           // LDS read
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);           // global load
    }
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);             // VALU
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Empty uses that make a value live at this point: the work that produces a
// value carried into the next K step stays in the step that computes it
// (the exit branch between steps would otherwise let the compiler sink it
// into the next step, in front of that step's first MFMAs).
__device__ inline void keep(const u32x4& v) { asm volatile("" ::"v"(v)); }
__device__ inline void keep(const f16x8& v) { asm volatile("" ::"v"(v)); }
__device__ inline void keep(uint32_t v) { asm volatile("" ::"v"(v)); }

// One work item of a workgroup: a stream-K segment [a, b) of the tile at
// (m0, n0), or the whole tile (dp).
struct Item {
  int a, b, m0, n0;
  bool dp;
};

// SALIGN: every row's scales start on a 16-byte boundary (K / G a multiple
// of 8 and a 16-byte aligned scale array), so they come in LDS windows;
// otherwise with the stages.
template <int G, bool KTAIL, bool SALIGN>
__global__ void __launch_bounds__(kThreads)
gemm_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
            const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
            int M, int N, int K, int tiles_m, int tiles_n, int iters, int rounds, int sk_tiles, int nsk,
            float* __restrict__ partials, uint32_t* __restrict__ flags, uint32_t* __restrict__ counters,
            uint32_t* __restrict__ status) {
  constexpr int kGroups = BK / G;            // scale groups per K step (1 or 4)
  constexpr int kSBytes = SALIGN ? 0 : BN * kGroups * 4;       // per-stage scales (unaligned case)
  constexpr int kStage = kStageBytes + kSBytes;
  // one array per stage, so the compiler tracks loads into one stage apart
  // from reads of another
  __shared__ __attribute__((aligned(16))) uint8_t stage0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t stage2[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t swin[SALIGN ? 2 * kWinBytes : 16];   // scale windows
  __shared__ __attribute__((aligned(16))) uint8_t sdummy[SALIGN ? 1024 : 16];          // idle window loads
  __shared__ int give_up;
  auto stage = [&](int st) -> uint8_t* { return st == 0 ? stage0 : (st == 1 ? stage1 : stage2); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;            // K half of the MFMA operands
  const int li = lane & 31;

  // Workgroups are dealt to XCDs round robin: XCD x runs ids x, x+8, ...
  const int wg = blockIdx.x;
  const int wgs = gridDim.x;
  const int xcd = wg % kXCD;
  const int lwg = wg / kXCD;          // index among the XCD's workgroups
  const int per_xcd = wgs / kXCD;

  // This XCD's stream-K tiles and this workgroup's iteration range in them.
  const int d_tiles = rounds * wgs;
  const int sk_lo = xcd_begin(xcd, sk_tiles);
  const int sk_cnt = xcd_begin(xcd + 1, sk_tiles) - sk_lo;
  const long long sk_iters = (long long)sk_cnt * iters;
  auto sk_start = [&](int l) -> long long { return sk_iters * l / nsk; };
  const bool in_sk = lwg < nsk && sk_cnt > 0;
  const long long my_s = in_sk ? sk_start(lwg) : 0, my_e = in_sk ? sk_start(lwg + 1) : 0;
  const int n_seg = my_e > my_s ? (int)((my_e - 1) / iters - my_s / iters) + 1 : 0;   // 0, 1 or 2
  const int j_first = (int)(my_s / iters);

  const uint32_t kbytes = (uint32_t)K * 2u;
  const uint32_t wrow = (uint32_t)K >> 1;                      // packed bytes per weight row
  const uint32_t spr = (uint32_t)K / (uint32_t)G;              // scales per weight row
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(x, (uint32_t)M * kbytes);
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(packed, (uint32_t)N * wrow);
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(scales, (uint32_t)N * spr * 2u);
  // fp32 partial tiles: slot p at p * kPartialBytes; inside a slot, 16-byte
  // quad q of accumulator block blk of thread t at ((blk * 4 + q) * kThreads + t) * 16,
  // so every store or load instruction covers 1 KB contiguously
  const __amdgpu_buffer_rsrc_t pres = make_rsrc(partials, partials ? 2u * (uint32_t)wgs * (uint32_t)kPartialBytes : 0u);

  // ---- LDS layouts and per-lane offsets (the same for every tile)
  // Activations: row r of 256 bytes, 16-byte chunk c stored at c ^ (r % 16).
  // Load j of wave w fills rows 32 j + 4 w .. + 3 (lane i: row + i / 16,
  // stored chunk i % 16, so it fetches chunk (i % 16) ^ (row % 16)).
  const int a_row = tid >> 4;                                   // + 16 j
  const int a_chunk = (tid & 15) ^ (a_row & 15);
  // Operand reads: sub-step s takes k = 64 h + 8 s .. + 8 of row 32 i + li.
  uint32_t a_r[kSub];
#pragma unroll
  for (int s = 0; s < kSub; ++s) a_r[s] = (uint32_t)li * 256u + (uint32_t)(((8 * h + s) ^ (li & 15)) << 4);
  // Scale rows are loaded 64 per wave, so the first BN / 64 waves load them.
  const bool scale_wave = wave < BN / 64;
  // Weights: row n of 64 bytes, chunk c stored at c ^ ((n / 4) % 4).  Load j
  // of wave w fills rows 128 j + 16 w .. + 15 (lane i: row + i / 4).
  const int b_row = tid >> 2;                                   // + 64 j
  const int b_chunk = (tid & 3) ^ ((b_row >> 2) & 3);
  // Operand reads: lane (li, h) of column block nb takes k = 64 h .. + 64 of
  // column kWaveN wave + 32 nb + li, as two chunks (half hf: sub-steps 4 hf ..).
  uint32_t b_r[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
    b_r[hf] = (uint32_t)(wave * kWaveN + li) * 64u + (uint32_t)(((2 * h + hf) ^ ((li >> 2) & 3)) << 4);

  const int ktail = KTAIL ? iters - 1 : -1;
  const int krem = K - (iters - 1) * BK;                     // k in the last step
  const bool a_tail_ok = a_chunk * 8 < krem, b_tail_ok = b_chunk * 32 < krem;

  // Global offsets: the per-lane part (row within the tile, chunk) is the
  // same for every tile; the tile's first row and the K step go into the
  // scalar offset.  The range check covers the sum, so rows past M or N read
  // zeros (or, where the 32-bit offset wraps, other data of the same buffer:
  // such rows only feed outputs that are never stored).
  const uint32_t a_v = (uint32_t)a_row * kbytes + (uint32_t)a_chunk * 16u;
  const uint32_t b_v = (uint32_t)b_row * wrow + (uint32_t)b_chunk * 16u;
  const uint32_t s_v = (uint32_t)(64 * wave + lane) * spr * 2u;
  auto setup = [&](int item) {
    Item it;
    it.dp = item >= n_seg;
    int tau;
    if (!it.dp) {
      const long long lo = (long long)(j_first + item) * iters;
      it.a = (int)((my_s > lo ? my_s : lo) - lo);
      it.b = (int)((my_e < lo + iters ? my_e : lo + iters) - lo);
      tau = d_tiles + sk_lo + j_first + item;
    } else {
      tau = (item - n_seg) * wgs + xcd * per_xcd + lwg;
      it.a = 0;
      it.b = iters;
    }
    int tm, tn;
    tile_coords(tau, tiles_m, tiles_n, tm, tn);
    it.m0 = tm * BM;
    it.n0 = tn * BN;
    return it;
  };

  // Part p of step kt into LDS stage st: activations (p < 4: load p),
  // weights (p = 4, 5: load p - 4), and without SALIGN the step's scales
  // (p = 6).  In the last step of a K that is not a multiple of
  // 128, chunks and groups past K are sent outside the buffer.
  auto load_part = [&](const Item& it, int kt, int st, int p) {
    const bool tail = KTAIL && kt == ktail;
    uint8_t* base = stage(st);
    if (p < 4) {
      const int j = p;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, W4A16_LDS(base + (32 * j + 4 * wave) * 256), 16,
                                               (tail && !a_tail_ok) ? kOutOfRange : a_v,
                                               (uint32_t)(it.m0 + 32 * j) * kbytes + (uint32_t)kt * (BK * 2), 0, 0);
    } else if (p < 6) {
      const int j = p - 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, W4A16_LDS(base + kABytes + (128 * j + 16 * wave) * 64), 16,
                                               (tail && !b_tail_ok) ? kOutOfRange : b_v,
                                               (uint32_t)(it.n0 + 128 * j) * wrow + (uint32_t)kt * (BK / 2), 0, 0);
    } else if (p == 6 && !SALIGN && scale_wave) {
      // row n's kGroups scales at n * kGroups * 4; load q of wave v covers
      // rows 64 v + 16 q .. (g 32, lane i: row + i / 4, group i % 4) or
      // rows 64 v .. + 63 (g 128, lane i: row + i)
#pragma unroll
      for (int q = 0; q < kGroups; ++q) {
        const int row = kGroups == 1 ? 64 * wave + lane : 64 * wave + 16 * q + (lane >> 2);
        const uint32_t grp = (uint32_t)(kt * kGroups + (kGroups == 1 ? 0 : (lane & 3)));
        const uint32_t off = it.n0 + row < N && grp < spr ? ((uint32_t)(it.n0 + row) * spr + grp) * 2u : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sres, W4A16_LDS(base + kStageBytes + (64 * wave + 16 * q) * kGroups * 4),
                                                 2, off, 0, 0, 0);
      }
    }
  };
  auto load_stage = [&](const Item& it, int kt, int st) {
#pragma unroll
    for (int p = 0; p < 7; ++p) load_part(it, kt, st, p);
  };
  // Scale windows (SALIGN): groups [8 w, 8 w + 8) of all 256 rows of the
  // tile, [row][8 x 2 bytes] in buffer w % 2; wave v < 4 loads rows 64 v .. + 63
  // (lane i: row 64 v + i, 16 bytes), the other waves' loads go to the dummy area.
  auto load_window = [&](const Item& it, int w, bool live) {
    if constexpr (SALIGN)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sres, W4A16_LDS(live && scale_wave ? swin + (w & 1) * kWinBytes + 64 * wave * 16
                                                                                   : sdummy),
                                               16, live && scale_wave ? s_v : kOutOfRange, (uint32_t)it.n0 * spr * 2u + (uint32_t)w * 16u,
                                               0, 0);
  };
  auto window_of = [&](int kt) { return (kt * kGroups) >> 3; };
  auto clamp_of = [&](const Item& it, int r) { return it.a + (r < it.b - it.a ? r : it.b - it.a - 1); };
  // The loads an item needs before its first step: its first scale windows
  // and steps 0 and 1 (stages 0 and 1).
  auto prologue_loads = [&](const Item& it) {
    load_window(it, window_of(it.a), true);
    load_window(it, window_of(it.a) + 1, true);
    load_stage(it, clamp_of(it, 0), 0);
    load_stage(it, clamp_of(it, 1), 1);
  };
  auto read_a = [&](int st, int s, u32x4 (&dst)[kMB]) {
    const uint8_t* base = stage(st);
#pragma unroll
    for (int i = 0; i < kMB; ++i) dst[i] = *reinterpret_cast<const u32x4*>(base + i * 8192 + a_r[s]);
  };
  auto read_b = [&](int st, int hf, u32x4 (&dst)[kNB]) {
    const uint8_t* base = stage(st) + kABytes;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) dst[nb] = *reinterpret_cast<const u32x4*>(base + nb * 2048 + b_r[hf]);
  };
  // the scales of half hf of step kt, held in stage st (group kt for g 128;
  // 4 kt + 2 h + hf for g 32)
  auto read_scale = [&](int kt, int st, int hf, uint32_t (&dst)[kNB]) {
    const int w = window_of(kt);
    const int e = kt * kGroups - 8 * w + (kGroups == 1 ? 0 : 2 * h + hf);
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int row = wave * kWaveN + nb * 32 + li;
      const uint8_t* p = SALIGN ? swin + (w & 1) * kWinBytes + row * 16 + e * 2
                                : stage(st) + kStageBytes + row * (kGroups * 4) + (kGroups == 1 ? 0 : (2 * h + hf) * 4);
      dst[nb] = *reinterpret_cast<const uint16_t*>(p);
    }
  };
  auto dequant = [&](const u32x4 (&w)[kNB], const uint32_t (&sc)[kNB], int word, f16x8 (&dst)[kNB]) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const uint32_t q = word == 0 ? w[nb].x : (word == 1 ? w[nb].y : (word == 2 ? w[nb].z : w[nb].w));
      const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)sc[nb]);
      dst[nb] = dequant_word_natural(q, f16x2{sv, sv});
    }
  };

  // Stream-K segments first (their partials are then ready long before the
  // fix-up), then the data-parallel tiles.  The next item's first loads are
  // issued before this item's results are written, so their latency
  // overlaps the output work.
  const int n_items = n_seg + rounds;
  Item cur = setup(0);
  if (n_items > 0) prologue_loads(cur);
  for (int item = 0; item < n_items; ++item) {
    const bool dp = cur.dp;
    const int a = cur.a, b = cur.b, m0 = cur.m0, n0 = cur.n0;
    const int nw = n0 + wave * kWaveN;

    f32x16 acc[kMB][kNB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[i][nb] = f32x16{};

    // Registers carried across sub-steps: activation operands three deep
    // (sub-step g uses slot g % 3), the step's packed words and scales in two
    // halves (sub-steps 0-3 and 4-7), and the dequantised weights of the
    // current and the next sub-step.
    u32x4 aop[3][kMB];
    u32x4 bw[2][kNB];
    uint32_t sc[2][kNB];
    f16x8 bop[2][kNB];

    const int nsteps = b - a;
    auto clamp = [&](int r) { return a + (r < nsteps ? r : nsteps - 1); };
    // Prologue: the loads of the first windows and steps 0 and 1 were issued
    // before the previous item's results were written.
    lds_barrier();
    read_a(0, 0, aop[0]);
    read_a(0, 1, aop[1]);
    read_b(0, 0, bw[0]);
    read_scale(a, 0, 0, sc[0]);
    dequant(bw[0], sc[0], 0, bop[0]);

    // One K step r (stage r % 3 == U).  Runs the 8 sub-steps and, spread over
    // the first six, loads step r + 2 into the stage that step r - 1 used;
    // the barrier at its end publishes step r + 2 (read from the next step on).
    auto step = [&](auto u_tag, int r) {
      constexpr int U = decltype(u_tag)::value;
      constexpr int st_cur = U, st_nxt = (U + 1) % 3, st_ld = (U + 2) % 3;
      const int kt = a + r;
      // The first step of a window (other than the tile's first) loads the
      // next window; the buffer it fills was last read in the step before.
      const bool win_load = r > 0 && window_of(kt) != window_of(kt - 1);
      load_window(cur, window_of(kt) + 1, win_load);
#pragma unroll
      for (int s = 0; s < kSub; ++s) {
        const int g = 2 * U + s;            // sub-step index mod 3 (8 = 2 mod 3)
        load_part(cur, clamp(r + 2), st_ld, s);
        if (s + 2 < kSub) read_a(st_cur, s + 2, aop[(g + 2) % 3]);
        else read_a(st_nxt, s + 2 - kSub, aop[(g + 2) % 3]);
        if (s == 1) {
          read_b(st_cur, 1, bw[1]);
          read_scale(kt, st_cur, 1, sc[1]);
        }
        if (s == 4) {
          read_b(st_nxt, 0, bw[0]);
          read_scale(kt + 1, st_nxt, 0, sc[0]);
        }
        if (s + 1 < kSub) dequant(bw[(s + 1) >> 2], sc[(s + 1) >> 2], (s + 1) & 3, bop[(s + 1) & 1]);
        else dequant(bw[0], sc[0], 0, bop[0]);
#pragma unroll
        for (int i = 0; i < kMB; ++i) {
          const f16x8 av = __builtin_bit_cast(f16x8, aop[g % 3][i]);
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb)
            acc[i][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bop[s & 1][nb], acc[i][nb], 0, 0, 0);
        }
        schedule_substep();
      }
      // operands of the next step's first two sub-steps
      constexpr int g0 = (2 * (U + 1)) % 3;
#pragma unroll
      for (int i = 0; i < kMB; ++i) {
        keep(aop[g0][i]);
        keep(aop[(g0 + 1) % 3][i]);
      }
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        keep(bw[0][nb]);
        keep(sc[0][nb]);
        keep(bop[0][nb]);
      }
      lds_barrier();
    };

    for (int r = 0;;) {
      step(std::integral_constant<int, 0>{}, r);
      if (++r == nsteps) break;
      step(std::integral_constant<int, 1>{}, r);
      if (++r == nsteps) break;
      step(std::integral_constant<int, 2>{}, r);
      if (++r == nsteps) break;
    }

    // the next item's first loads (stages 0 and 1 and the windows are free
    // once the last step's barrier has passed)
    if (item + 1 < n_items) {
      const Item nxt = setup(item + 1);
      prologue_loads(nxt);
      cur = nxt;
    }

    if (dp) {
      // Output through LDS (stage 2, free once the last step's barrier has
      // passed; the next item's first load into it follows that item's first
      // barrier): each wave writes its 128 x 32 fp16 slab in two passes of 64
      // rows into its own 5 KB, [row][32 columns] with an 80-byte row pitch
      // (every write offset a constant), then stores whole 16-byte chunks,
      // 4 lanes per 64-byte row.  The accumulator of lane (li, h) holds
      // column li of each block, rows 8 * (r / 4) + 4 * h + r % 4.
      constexpr int kPitch = kWaveN * 2 + 16;
      constexpr int kRowLanes = kWaveN / 8;      // lanes per output row, 16 bytes each
      static_assert(kWaves * 64 * kPitch <= kStageBytes, "epilogue slabs exceed stage 2");
      uint8_t* ep = stage2 + wave * 64 * kPitch;
      uint8_t* ew = ep + 4 * h * kPitch + li * 2;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              *reinterpret_cast<uint16_t*>(ew + (ii * 32 + 8 * (r >> 2) + (r & 3)) * kPitch + nb * 64) =
                  float_to_half_bits(acc[2 * pass + ii][nb][r]);
        // a wave's LDS accesses complete in order: its own writes are visible
#pragma unroll
        for (int j = 0; j < kRowLanes; ++j) {
          const int row = (64 / kRowLanes) * j + lane / kRowLanes, c = lane % kRowLanes;
          const u32x4 v = *reinterpret_cast<const u32x4*>(ep + row * kPitch + c * 16);
          const int m = m0 + 64 * pass + row, n = nw + 8 * c;
          if (m < M) {
            uint16_t* dst = y + (size_t)m * N + n;
            if (n + 8 <= N && (N & 7) == 0) {
              *reinterpret_cast<u32x4*>(dst) = v;
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (n + e < N) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
            }
          }
        }
      }
    } else {
      // Publish the partial (slot 2 wg + item) for the fix-up: device-scope
      // stores, all complete (s_waitcnt) before the flag is raised.
      const uint32_t slot_off = (uint32_t)(2 * wg + item) * (uint32_t)kPartialBytes;
#pragma unroll
      for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 v = {acc[i][nb][4 * q], acc[i][nb][4 * q + 1], acc[i][nb][4 * q + 2], acc[i][nb][4 * q + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), pres,
                                                   (uint32_t)((((i * kNB + nb) * 4 + q) * kThreads + tid) * 16),
                                                   slot_off, kDeviceScope);
          }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) __hip_atomic_store(flags + 2 * wg + item, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- fix-up: each contributor of a stream-K tile reduces one slice of it.
  if (n_seg == 0) return;
  // Wave 0 builds the table of this workgroup's one or two stream-K tiles:
  // lane l describes the XCD's workgroup l (nsk <= 64) and polls its flag.
  __shared__ uint32_t fix_slot[2][64];       // partial slot of each contributor
  __shared__ int fix_c0[2], fix_c1[2];
  if (wave == 0) {
    const long long s0 = lane < nsk ? sk_start(lane) : 0, s1 = lane < nsk ? sk_start(lane + 1) : 0;
    bool pending = false;
    for (int e = 0; e < n_seg; ++e) {
      const long long lo = (long long)(j_first + e) * iters, hi = lo + iters;
      const bool mine = lane < nsk && s1 > s0 && s0 < hi && s1 > lo;
      const uint64_t m = __builtin_amdgcn_ballot_w64(mine);
      // second segment of its range if the range began before this tile
      const uint32_t slot = 2u * (uint32_t)(lane * kXCD + xcd) + (s0 < lo ? 1u : 0u);
      if (mine) fix_slot[e][lane] = slot;
      if (lane == 0) {
        fix_c0[e] = (int)__builtin_ctzll(m);
        fix_c1[e] = 63 - (int)__builtin_clzll(m);
      }
      pending = pending || mine;
    }
    // wait until every contributor of both tiles has raised its flag
    uint32_t spins = 0;
    bool failed_poll = false;
    for (;;) {
      bool missing = false;
      for (int e = 0; e < n_seg; ++e) {
        const long long lo = (long long)(j_first + e) * iters, hi = lo + iters;
        const bool mine = lane < nsk && s1 > s0 && s0 < hi && s1 > lo;
        if (mine) {
          const uint32_t slot = 2u * (uint32_t)(lane * kXCD + xcd) + (s0 < lo ? 1u : 0u);
          missing = missing || __hip_atomic_load(flags + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u;
        }
      }
      if (__builtin_amdgcn_ballot_w64(missing) == 0) break;
      __builtin_amdgcn_s_sleep(2);
      if (++spins == kSpinLimit) { failed_poll = true; break; }
    }
    (void)pending;
    if (lane == 0) {
      give_up = failed_poll ? 1 : 0;
      // recorded for the caller (w4a16_gemm_workspace_status)
      if (failed_poll) __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  const bool failed = give_up != 0;
  for (int e = 0; e < n_seg; ++e) {
    const int j = j_first + e;
    const int c0 = fix_c0[e], c1 = fix_c1[e];
    const int parts = c1 - c0 + 1;
    int tm, tn;
    tile_coords(d_tiles + sk_lo + j, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    // slice: 16-byte quads [ch0, ch1) of the partial layout (blk, q, thread);
    // the contributors' quads are summed in contributor order, 8 loads in flight
    constexpr int kChunks = kMB * kNB * 4 * kThreads;
    const int qs = lwg - c0;
    const int ch0 = kChunks * qs / parts, ch1 = kChunks * (qs + 1) / parts;
    for (int c = ch0 + tid; c < ch1; c += kThreads) {
      auto quad = [&](int l) {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             pres, (uint32_t)c * 16u, fix_slot[e][l] * (uint32_t)kPartialBytes,
                                             kDeviceScope));
      };
      f32x4 v = quad(c0);
      for (int l0 = c0 + 1; l0 <= c1; l0 += 8) {
        f32x4 pq[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) pq[u] = quad(l0 + u <= c1 ? l0 + u : c0);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (l0 + u <= c1) v += pq[u];
      }
      const int t = c % kThreads, bq = c / kThreads;
      const int blk = bq >> 2, q = bq & 3;
      const int i = blk / kNB, nb = blk % kNB;
      const int cl = t & 63, ch = cl >> 5;
      const int n = n0 + (t >> 6) * kWaveN + nb * 32 + (cl & 31);
      if (n < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + i * 32 + 8 * q + 4 * ch + r;
          if (m < M) y[(size_t)m * N + n] = failed ? (uint16_t)0x7E00u : float_to_half_bits(v[r]);
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
      // the last contributor to finish reading clears the tile's flags
      const uint32_t done = __hip_atomic_fetch_add(counters + xcd * per_xcd + j, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      if (done == (uint32_t)parts - 1u) {
        for (int l = c0; l <= c1; ++l)
          __hip_atomic_store(flags + fix_slot[e][l], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(counters + xcd * per_xcd + j, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ---- scratch of the allocation-free entry point (w4a16_gemm_noalloc) ----
// The split-K workspace of up to kScratchWGs persistent workgroups (256: one per
// CU of an MI355X) lives in this file-scope device array, which every GPU the
// library runs on holds until the process ends.  Host code never uses the
// array's name as an address: each device's copy is looked up once, with that
// device current, and kept in g_scratch.  Zero-initialised at load; the caller
// clears the flags and counters before every use.
constexpr int kScratchWGs = 256;
constexpr size_t kScratchBytes =
    kWorkspaceHeader + 2 * (size_t)kScratchWGs * kPartialBytes + 3 * (size_t)kScratchWGs * sizeof(uint32_t);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];

}  // namespace

hipError_t gemm_scratch(const DeviceInfo& dev, void** ptr, size_t* bytes) {
  const int d = dev.device;
  if (d < 0 || d >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[d], [d] {
    // dev.device is the current device (current_device_info read it)
    void* p = nullptr;
    g_scratch_err[d] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[d] = g_scratch_err[d] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[d] != hipSuccess) return g_scratch_err[d];
  *ptr = g_scratch[d];
  *bytes = kScratchBytes;
  return hipSuccess;
}

size_t gemm_workspace_flags_offset(int64_t m, int64_t n, int64_t k, const DeviceInfo& dev) {
  const GemmPlan p = gemm_plan((int)m, (int)n, (int)k, dev);
  return kWorkspaceHeader + 2 * (size_t)p.wgs * kPartialBytes;
}

size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int, const DeviceInfo& dev) {
  const GemmPlan p = gemm_plan((int)m, (int)n, (int)k, dev);
  if (p.sk_tiles == 0) return 0;
  // the status word (kWorkspaceHeader bytes), two partial slots and two flags per
  // workgroup, one counter per stream-K tile slot
  return kWorkspaceHeader + 2 * (size_t)p.wgs * kPartialBytes + 3 * (size_t)p.wgs * sizeof(uint32_t);
}

hipError_t launch_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int m,
                       int n, int k, int group, void* workspace, const DeviceInfo& dev, hipStream_t stream) {
  const GemmPlan p = gemm_plan(m, n, k, dev);
  float* partials = nullptr;
  uint32_t* flags = nullptr;
  uint32_t* counters = nullptr;
  uint32_t* status = nullptr;
  if (workspace) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    status = reinterpret_cast<uint32_t*>(ws);
    partials = reinterpret_cast<float*>(ws + kWorkspaceHeader);
    flags = reinterpret_cast<uint32_t*>(ws + kWorkspaceHeader + 2 * (size_t)p.wgs * kPartialBytes);
    counters = flags + 2 * (size_t)p.wgs;
  }
  const bool tail = k % BK != 0;
  const bool salign = (k / group) % 8 == 0 && (reinterpret_cast<uintptr_t>(scales) & 15) == 0;
  auto kern = group == 128 ? (salign ? gemm_kernel<128, false, true> : gemm_kernel<128, false, false>)
              : tail       ? gemm_kernel<32, true, false>
              : salign     ? gemm_kernel<32, false, true>
                           : gemm_kernel<32, false, false>;
  return launch_kernel(kern, dim3(p.wgs), dim3(kThreads), 0, stream, x, packed, scales, y, m, n, k, p.tiles_m,
                       p.tiles_n, p.iters, p.rounds, p.sk_tiles, p.nsk, partials, flags, counters, status);
}

}  // namespace w4a16
