// gemm.hip -- prefill GEMM of the W4A16 int4 weight-only layer on gfx950 (fp16 MFMA).
//
// y[m, n] = sum_k x[m, k] * s[n, k / g] * q[n, k] for any M: the prompt
// (prefill) phase of the W4A16 models on the LLM170 CUDA/W4A16 page (pp512,
// pp1024, pp4096 columns).  Here the layer is a dense contraction, so it runs
// on the matrix cores: v_mfma_f32_32x32x16_f16, fp16 inputs, fp32 accumulation.
//
// * Tiles: 128 x 256 output tiles, K steps of 64.  A 256-thread workgroup
//   runs four wavefronts of 128 x 64 (4 x 2 MFMA blocks of 32 x 32, 128 fp32
//   accumulators per lane, held in the accumulation registers); one
//   persistent workgroup per CU.
// * A software pipeline hides memory latency: the loads of K step k + 3 are
//   in flight while step k computes.  Activations (the MFMA A operand) come
//   into a ring of registers, are written to a double-buffered LDS tile
//   (128 x 64 per step) one step before use, with an XOR swizzle of the
//   16-byte chunks so the MFMA operand reads are free of bank conflicts.
//   Weights (the B operand) never touch LDS: each lane loads one 16-byte
//   packed chunk per 32-column block and K step into a ring of registers and
//   dequantises it in natural k order (mfma_operands.hpp).
// * Work split (stream-K, per XCD): the tiles are dealt to the 8 XCDs in
//   contiguous, column-band-major ranges (each packed weight is read from HBM
//   by one XCD only); inside an XCD the (tile, K step) iterations are split
//   evenly over its persistent workgroups, so a tile may be shared by two or
//   more workgroups.  Every workgroup walks its range from the end, and the
//   workgroup holding a tile's last K step finishes it: the others store fp32
//   partial tiles in the workspace and raise a flag; the finisher waits for
//   the flags of lower-numbered workgroups only (dispatched earlier), adds the
//   partials in a fixed order (deterministic) and writes fp16.  It clears the
//   flags it consumed, so the workspace stays ready for the next call.
//
// For integer activations, codes and power-of-two scales every product and
// partial sum is exact, so such inputs give bit-exact results.
#include "device.hpp"
#include "kernels.hpp"
#include "mfma_operands.hpp"

namespace w4a16 {
namespace {

constexpr int kThreads = 256;
constexpr int kWGPerCU = 1;
constexpr int BM = 128, BN = 256, BK = 64;
constexpr int kWaveN = 64;                  // output columns per wave
constexpr int kMB = BM / 32, kNB = kWaveN / 32;
constexpr int kAhead = 3;                   // K steps between a load and its use
constexpr int kUnroll = 6;                  // lcm(register ring 3, LDS double buffer 2)
constexpr int kATile = BM * BK * 2;         // bytes per LDS A buffer (128 rows of 128 bytes, swizzled)
constexpr int kXCD = 8;
constexpr int kMinItersPerWG = 8;           // keep stream-K segments from getting tiny
constexpr size_t kPartialBytes = (size_t)BM * BN * 4;
constexpr uint32_t kSpinLimit = 1u << 24;   // flag polls before a finisher gives up

struct GemmPlan {
  int tiles_m, tiles_n, tiles, iters;       // iters: K steps per tile
  int wg_per_xcd, wgs;
};

GemmPlan gemm_plan(int m, int n, int k, const DeviceInfo& dev) {
  GemmPlan p;
  p.tiles_m = (m + BM - 1) / BM;
  p.tiles_n = (n + BN - 1) / BN;
  p.tiles = p.tiles_m * p.tiles_n;
  p.iters = (k + BK - 1) / BK;
  const long long total = (long long)p.tiles * p.iters;
  int per_xcd = (dev.num_cu * kWGPerCU) / kXCD;
  const long long useful = (total / kXCD + kMinItersPerWG - 1) / kMinItersPerWG;
  if (useful < per_xcd) per_xcd = (int)(useful < 1 ? 1 : useful);
  p.wg_per_xcd = per_xcd < 1 ? 1 : per_xcd;
  p.wgs = p.wg_per_xcd * kXCD;
  return p;
}

// XOR swizzle of the 16-byte chunks of an LDS A row (128 bytes).  An operand
// read has 16 lanes at a time reading one logical chunk of 16 consecutive
// rows; with 64 four-byte banks two rows share a bank line, so the chunk is
// moved by (row / 2) % 8: the 16 lanes land on 16 distinct bank quads.
__device__ inline int swz(int row) { return (row >> 1) & 7; }

__device__ inline int xcd_tile_begin(int xcd, int tiles) {
  const int q = tiles / kXCD, r = tiles % kXCD;
  return xcd * q + (xcd < r ? xcd : r);
}

__global__ void __launch_bounds__(kThreads)
gemm_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
            const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
            int M, int N, int K, int gshift, int tiles_m, int tiles, int iters, int wg_per_xcd,
            float* __restrict__ partials, uint32_t* __restrict__ flags) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2 * kATile];
  __shared__ int give_up;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;            // K half of the MFMA operands
  const int li = lane & 31;

  // Workgroups are dealt to XCDs round robin: XCD x runs ids x, x+8, ...
  const int wg = blockIdx.x;
  const int xcd = wg % kXCD;
  const int lwg = wg / kXCD;          // index among the XCD's workgroups
  const int t_begin = xcd_tile_begin(xcd, tiles);
  const int t_count = xcd_tile_begin(xcd + 1, tiles) - t_begin;
  const long long xiters = (long long)t_count * iters;
  const long long s_w = xiters * lwg / wg_per_xcd;
  const long long e_w = xiters * (lwg + 1) / wg_per_xcd;
  auto owner_start = [&](int l) { return xiters * l / wg_per_xcd; };

  const uint32_t kbytes = (uint32_t)K * 2u;
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(x, (uint32_t)M * kbytes);
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(packed, (uint32_t)N * ((uint32_t)K >> 1));
  const uint32_t spr = (uint32_t)K >> (5 + gshift);   // scales per row
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(scales, (uint32_t)N * spr * 2u);

  long long it = e_w;
  while (it > s_w) {
    // ---- the segment [a, b) of tile t that ends at `it`
    const int tl = (int)((it - 1) / iters);                  // tile index within the XCD's range
    const long long tile_lo = (long long)tl * iters;
    const int a = (int)((s_w > tile_lo ? s_w : tile_lo) - tile_lo);
    const int b = (int)(it - tile_lo);
    const int t = t_begin + tl;
    const int tm = t % tiles_m, tn = t / tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int nw = n0 + wave * kWaveN;

    // Per-lane parts of the load offsets are fixed for the whole segment; the
    // K step only moves the scalar offset.  A step past b gets a scalar
    // offset outside every buffer (zeros, no memory access), and in a last
    // step that covers only 32 of its 64 k the lanes beyond K get a
    // per-lane offset outside the buffer -- selects, not branches, so the
    // load counts stay fixed.
    const int ktail = (K % BK) ? iters - 1 : iters;   // step whose upper half lies past K
    // Per-lane parts of the load offsets are fixed for the whole segment; the
    // K step only moves the scalar offset.  A step past b gets a scalar
    // offset outside every buffer (zeros, no memory access), and in a last
    // step that covers only 32 of its 64 k the lanes beyond K get a per-lane
    // offset outside the buffer -- selects, not branches, so every step
    // issues the same loads and the wait counts stay exact.
    //
    // A: thread t loads 4 chunks of 16 bytes per step: slot t + 256 j holds
    // row r = slot / 8 at physical column c' = slot % 8 and is fetched from
    // the row's logical chunk c = c' ^ swz(r).
    uint32_t avoff[4], avoff_tail[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int slot = tid + j * kThreads;
      const int row = slot >> 3, c = (slot & 7) ^ swz(row);
      avoff[j] = (m0 + row < M) ? (uint32_t)(m0 + row) * kbytes + (uint32_t)c * 16u : kOutOfRange;
      avoff_tail[j] = c < 4 ? avoff[j] : kOutOfRange;
    }
    auto load_a = [&](int kt, u32x4 (&ra)[4]) {
      const uint32_t soff = kt < b ? (uint32_t)kt * (BK * 2) : kOutOfRange;
      const bool tail = kt == ktail;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ra[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              xres, tail ? avoff_tail[j] : avoff[j], soff, 0));
    };
    auto store_a = [&](int buf, const u32x4 (&ra)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u32x4*>(As + buf * kATile + (tid + j * kThreads) * 16) = ra[j];
    };
    uint32_t bvoff[kNB], bvoff_tail[kNB], svoff[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int n = nw + nb * 32 + li;
      bvoff[nb] = n < N ? (uint32_t)n * ((uint32_t)K >> 1) + (uint32_t)h * 16u : kOutOfRange;
      bvoff_tail[nb] = h == 0 ? bvoff[nb] : kOutOfRange;
      svoff[nb] = n < N ? ((uint32_t)n * spr + (gshift == 0 ? (uint32_t)h : 0u)) * 2u : kOutOfRange;
    }
    auto load_b = [&](int kt, u32x4 (&rb)[kNB], uint32_t (&rs)[kNB]) {
      const bool live = kt < b;
      const uint32_t wsoff = live ? (uint32_t)kt * (BK / 2) : kOutOfRange;
      const uint32_t ssoff = live ? (((uint32_t)kt * BK) >> (5 + gshift)) * 2u : kOutOfRange;
      const bool tail = kt == ktail;
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        rb[nb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               wres, tail ? bvoff_tail[nb] : bvoff[nb], wsoff, kStream));
        rs[nb] = __builtin_amdgcn_raw_buffer_load_b16(sres, svoff[nb], ssoff, 0);
      }
    };

    f32x16 acc[kMB][kNB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[i][nb] = f32x16{};

    u32x4 ra[kAhead][4];
    u32x4 rb[kAhead][kNB];
    uint32_t rs[kAhead][kNB];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      load_a(a + u, ra[u]);
      load_b(a + u, rb[u], rs[u]);
    }
    store_a(0, ra[0]);
    __syncthreads();

    // The step count is padded to a multiple of the unroll: a padding step
    // reads only zeros, so it adds exactly nothing, and the unrolled body has
    // no branches.
    for (int base = a; base < b; base += kUnroll) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int kt = base + u;
        const int slot = u % kAhead;          // register ring slot of step kt
        const uint8_t* at = As + (u & 1) * kATile;
        // All 16 operand reads of the step first, so their LDS latencies
        // overlap; the MFMAs then wait only for the reads they use.
        u32x4 av[BK / 16][kMB];
#pragma unroll
        for (int s = 0; s < BK / 16; ++s)
#pragma unroll
          for (int i = 0; i < kMB; ++i) {
            const int row = i * 32 + li;
            const int c = 4 * h + s;              // logical 16-byte chunk of the row
            av[s][i] = *reinterpret_cast<const u32x4*>(at + row * (BK * 2) + ((c ^ swz(row)) << 4));
          }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
          f16x8 bop[kNB];
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            const u32x4 w = rb[slot][nb];
            const uint32_t q = s == 0 ? w.x : (s == 1 ? w.y : (s == 2 ? w.z : w.w));
            const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)rs[slot][nb]);
            bop[nb] = dequant_word_natural(q, f16x2{sv, sv});
          }
#pragma unroll
          for (int i = 0; i < kMB; ++i) {
            const f16x8 aop = __builtin_bit_cast(f16x8, av[s][i]);
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb)
              acc[i][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, bop[nb], acc[i][nb], 0, 0, 0);
          }
        }
        store_a((u + 1) & 1, ra[(u + 1) % kAhead]);      // step kt + 1's activations into the other buffer
        load_a(kt + kAhead, ra[slot]);                    // refill the ring
        load_b(kt + kAhead, rb[slot], rs[slot]);
        __syncthreads();
      }
    }
    __builtin_amdgcn_s_waitcnt(0);            // drain the loads past the segment (zeros, no memory access)

    // ---- partial or finished tile
    // slot wg: the partial this workgroup publishes (at most one per call);
    // slot wgs + wg: where a finisher parks its own accumulators while it sums
    float* my_part = partials + (size_t)(b < iters ? wg : (int)gridDim.x + wg) * (kPartialBytes / 4);
    auto store_partial = [&]() {
#pragma unroll
      for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          *reinterpret_cast<f32x16*>(my_part + ((size_t)((i * kNB + nb) * kThreads + tid) * 16)) = acc[i][nb];
    };
    if (b < iters) {
      // not the tile's last K step: publish the partial for the finisher
      store_partial();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      if (tid == 0) __hip_atomic_store(flags + wg, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else if (a == 0) {
      // the whole tile is ours: convert straight from the accumulators.
      // lane holds column li of each block, rows 8*(r/4) + 4*h + r%4
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const int n = nw + nb * 32 + li;
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < kMB; ++i) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (m < M) y[(size_t)m * N + n] = float_to_half_bits(acc[i][nb][r]);
          }
        }
      }
    } else {
      // Lower-numbered workgroups of this XCD hold the K steps [0, a), each
      // as the first segment it computed (one that needs no waiting).  Park
      // our own partial, wait for theirs, then sum: ours first, then theirs
      // nearest first (a fixed order, so the result is deterministic).
      store_partial();
      if (tid == 0) give_up = 0;
      __syncthreads();
      if (tid == 0) {
        for (int l = lwg - 1; l >= 0 && owner_start(l + 1) > tile_lo; --l) {
          if (owner_start(l) == owner_start(l + 1)) continue;   // empty range: no partial
          uint32_t spins = 0;
          while (__hip_atomic_load(flags + l * kXCD + xcd, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins == kSpinLimit) { give_up = 1; break; }
          }
        }
      }
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const bool failed = give_up != 0;
#pragma unroll
      for (int i = 0; i < kMB; ++i) {
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const size_t off = (size_t)((i * kNB + nb) * kThreads + tid) * 16;
          f32x16 v = *reinterpret_cast<const f32x16*>(my_part + off);
          for (int l = lwg - 1; l >= 0 && owner_start(l + 1) > tile_lo; --l) {
            if (owner_start(l) == owner_start(l + 1)) continue;
            v += *reinterpret_cast<const f32x16*>(partials + (size_t)(l * kXCD + xcd) * (kPartialBytes / 4) + off);
          }
          const int n = nw + nb * 32 + li;
          if (n < N) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int m = m0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
              if (m < M) y[(size_t)m * N + n] = failed ? (uint16_t)0x7E00u : float_to_half_bits(v[r]);
            }
          }
        }
      }
      __syncthreads();
      if (tid == 0) {
        for (int l = lwg - 1; l >= 0 && owner_start(l + 1) > tile_lo; --l)
          if (owner_start(l) != owner_start(l + 1))
            __hip_atomic_store(flags + l * kXCD + xcd, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    it = tile_lo + a;
  }
}

}  // namespace

size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int, const DeviceInfo& dev) {
  const GemmPlan p = gemm_plan((int)m, (int)n, (int)k, dev);
  return 2 * (size_t)p.wgs * kPartialBytes + (size_t)p.wgs * sizeof(uint32_t);
}

hipError_t launch_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, uint16_t* y, int m,
                       int n, int k, int group, void* workspace, const DeviceInfo& dev, hipStream_t stream) {
  const GemmPlan p = gemm_plan(m, n, k, dev);
  const int gshift = group == 128 ? 2 : 0;
  float* partials = static_cast<float*>(workspace);
  uint32_t* flags = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + 2 * (size_t)p.wgs * kPartialBytes);
  hipLaunchKernelGGL(gemm_kernel, dim3(p.wgs), dim3(kThreads), 0, stream, x, packed, scales, y, m, n, k, gshift,
                     p.tiles_m, p.tiles, p.iters, p.wg_per_xcd, partials, flags);
  return hipGetLastError();
}

}  // namespace w4a16
