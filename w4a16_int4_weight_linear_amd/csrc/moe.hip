// moe.hip -- the routed-expert (MoE) steps either side of the grouped product.
//
// The 35B-A3B MoE layers of the LLM170 / infr pages route every token to its
// top-k experts, run each expert's rows through its weights (grouped_gemm.hip,
// whose gather variant reads the token rows directly), and combine the k
// expert outputs of a token with the router weights.  These two kernels are the
// routing permute and the combine.
//
// * Routing: one workgroup counts the (token, slot) pairs per expert with LDS
//   atomics, turns the counts into the row offsets (exclusive prefix sum: lane
//   shifts within a wave, one LDS exchange across waves), and gives every pair
//   a row inside its expert's range with an LDS cursor.  Each thread keeps the
//   expert ids it read for the count in registers for the scatter.  The
//   order of rows inside one expert is whatever the atomics give: it changes
//   nothing downstream (each row's product is computed on its own, and the
//   combine reads a token's pairs in slot order through pair_row).  Expert ids
//   outside [0, E) get no row (pair_row = -1) and are not counted.
// * Combine: one thread per (token, 8 output columns): the k expert rows of the
//   token are fetched eight slots at a time (all requests in flight together),
//   accumulated in slot order in fp32 with the router weights, then rounded once
//   to fp16.
#include "device.hpp"
#include "kernels.hpp"
#include "launch.hpp"

namespace w4a16 {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kHeld = 8;                     // expert ids each routing thread keeps in registers
constexpr int kCombineSlots = 8;             // slots whose rows the combine fetches together

__global__ void __launch_bounds__(kRouteThreads)
moe_route_kernel(const int32_t* __restrict__ ids, int pairs, int topk, int experts, int32_t* __restrict__ offsets,
                 int32_t* __restrict__ pair_token, int32_t* __restrict__ pair_row) {
  extern __shared__ int32_t smem_i[];
  int32_t* cnt = smem_i;                    // [experts]: counts, then the next free row of each expert
  int32_t* wsum = smem_i + experts;         // [kRouteWaves]: per-wave totals of the segment sums
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < experts; e += kRouteThreads) cnt[e] = 0;
  // The first kHeld pairs of each thread are read once and kept for the scatter.
  int held[kHeld];
#pragma unroll
  for (int i = 0; i < kHeld; ++i) {
    const int p = tid + i * kRouteThreads;
    held[i] = p < pairs ? ids[p] : -1;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kHeld; ++i) {
    const int e = held[i];
    if (e >= 0 && e < experts) atomicAdd(&cnt[e], 1);
  }
  for (int p = tid + kHeld * kRouteThreads; p < pairs; p += kRouteThreads) {
    const int e = ids[p];
    if (e >= 0 && e < experts) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // Exclusive prefix sum of the counts: each thread sums one contiguous segment,
  // a wave scans its 64 segment sums with lane shifts, and the wave totals
  // (one exchange through LDS) give each wave its start.
  const int seg = (experts + kRouteThreads - 1) / kRouteThreads;
  const int e0 = tid * seg;
  int s = 0;
  for (int e = e0; e < e0 + seg && e < experts; ++e) s += cnt[e];
  int inc = s;                                      // inclusive scan within the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(inc, d, 64);
    if (lane >= d) inc += v;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int before = 0;                                   // totals of the earlier waves
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int run = before + inc - s;                       // exclusive start of this segment
  for (int e = e0; e < e0 + seg && e < experts; ++e) {
    const int c = cnt[e];
    offsets[e] = run;
    cnt[e] = run;                                   // cursor: next free row of expert e
    run += c;
  }
  if (tid == kRouteThreads - 1) offsets[experts] = before + inc;
  __syncthreads();
  auto place = [&](int p, int e) {
    if (e >= 0 && e < experts) {
      const int r = atomicAdd(&cnt[e], 1);
      pair_token[r] = p / topk;
      pair_row[p] = r;
    } else {
      pair_row[p] = -1;
    }
  };
#pragma unroll
  for (int i = 0; i < kHeld; ++i) {
    const int p = tid + i * kRouteThreads;
    if (p < pairs) place(p, held[i]);
  }
  for (int p = tid + kHeld * kRouteThreads; p < pairs; p += kRouteThreads) place(p, ids[p]);
}

__global__ void __launch_bounds__(256)
moe_combine_kernel(const uint16_t* __restrict__ yp, const int32_t* __restrict__ pair_row,
                   const float* __restrict__ w, uint16_t* __restrict__ out, int tokens, int topk, int n, int rows) {
  const int chunks = (n + 7) >> 3;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (int64_t)tokens * chunks) return;
  const int t = (int)(g / chunks);
  const int c0 = (int)(g - (int64_t)t * chunks) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const bool vec = (n & 7) == 0;
  // Slots are taken kCombineSlots at a time: their row indices and weights,
  // then their rows, are all requested before the first is used, and the
  // rows are accumulated in slot order.
  for (int j0 = 0; j0 < topk; j0 += kCombineSlots) {
    int r[kCombineSlots];
    float wj[kCombineSlots];
#pragma unroll
    for (int q = 0; q < kCombineSlots; ++q) {
      const int j = j0 + q;
      r[q] = j < topk ? pair_row[(int64_t)t * topk + j] : -1;
      wj[q] = j < topk ? w[(int64_t)t * topk + j] : 0.f;
    }
    if (vec) {
      u32x4 v[kCombineSlots];
#pragma unroll
      for (int q = 0; q < kCombineSlots; ++q)
        v[q] = (r[q] >= 0 && r[q] < rows) ? *reinterpret_cast<const u32x4*>(yp + (int64_t)r[q] * n + c0)
                                          : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int q = 0; q < kCombineSlots; ++q) {
        if (r[q] < 0 || r[q] >= rows) continue;    // a pair without a row contributes nothing
        const uint32_t wd[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = __builtin_fmaf(wj[q], half_bits_to_float(wd[i] & 0xFFFFu), acc[2 * i]);
          acc[2 * i + 1] = __builtin_fmaf(wj[q], half_bits_to_float(wd[i] >> 16), acc[2 * i + 1]);
        }
      }
    } else {
      for (int q = 0; q < kCombineSlots; ++q) {
        if (r[q] < 0 || r[q] >= rows) continue;
        const uint16_t* src = yp + (int64_t)r[q] * n + c0;
        for (int i = 0; i < 8 && c0 + i < n; ++i) acc[i] = __builtin_fmaf(wj[q], half_bits_to_float(src[i]), acc[i]);
      }
    }
  }
  uint16_t* dst = out + (int64_t)t * n + c0;
  if (vec) {
    u32x4 v;
    v.x = float_to_half_bits(acc[0]) | ((uint32_t)float_to_half_bits(acc[1]) << 16);
    v.y = float_to_half_bits(acc[2]) | ((uint32_t)float_to_half_bits(acc[3]) << 16);
    v.z = float_to_half_bits(acc[4]) | ((uint32_t)float_to_half_bits(acc[5]) << 16);
    v.w = float_to_half_bits(acc[6]) | ((uint32_t)float_to_half_bits(acc[7]) << 16);
    *reinterpret_cast<u32x4*>(dst) = v;
  } else {
    for (int i = 0; i < 8 && c0 + i < n; ++i) dst[i] = float_to_half_bits(acc[i]);
  }
}

}  // namespace

size_t moe_route_lds(int experts) { return (size_t)(experts + kRouteWaves) * sizeof(int32_t); }

hipError_t launch_moe_route(const int32_t* ids, int pairs, int topk, int experts, int32_t* offsets,
                            int32_t* pair_token, int32_t* pair_row, const DeviceInfo& dev, hipStream_t stream) {
  const size_t lds = moe_route_lds(experts);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_route_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
    if (e != hipSuccess) return e;
  }
  return launch_kernel(moe_route_kernel, dim3(1), dim3(kRouteThreads), lds, stream, ids, pairs, topk, experts, offsets,
                       pair_token, pair_row);
}

hipError_t launch_moe_combine(const uint16_t* y_pairs, const int32_t* pair_row, const float* weights, uint16_t* out,
                              int tokens, int topk, int n, int rows, hipStream_t stream) {
  const int64_t threads = (int64_t)tokens * ((n + 7) / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  return launch_kernel(moe_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, y_pairs, pair_row, weights,
                       out, tokens, topk, n, rows);
}

}  // namespace w4a16
