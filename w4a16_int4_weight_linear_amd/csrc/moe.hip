// moe.hip -- the routed-expert (MoE) steps either side of the grouped product.
//
// The 35B-A3B MoE layers of the LLM170 / infr pages route every token to its
// top-k experts, run each expert's rows through its weights (grouped_gemm.hip,
// whose gather variant reads the token rows directly), and combine the k
// expert outputs of a token with the router weights.  These two kernels are the
// routing permute and the combine.
//
// * Routing: one workgroup counts the (token, slot) pairs per expert with LDS
//   atomics, turns the counts into the row offsets (exclusive prefix sum), and
//   gives every pair a row inside its expert's range with an LDS cursor.  The
//   order of rows inside one expert is whatever the atomics give: it changes
//   nothing downstream (each row's product is computed on its own, and the
//   combine reads a token's pairs in slot order through pair_row).  Expert ids
//   outside [0, E) get no row (pair_row = -1) and are not counted.
// * Combine: one thread per (token, 8 output columns): the k expert rows of the
//   token are read in slot order and accumulated in fp32 with the router
//   weights, then rounded once to fp16.
#include "device.hpp"
#include "kernels.hpp"

namespace w4a16 {
namespace {

constexpr int kRouteThreads = 1024;

__global__ void __launch_bounds__(kRouteThreads)
moe_route_kernel(const int32_t* __restrict__ ids, int pairs, int topk, int experts, int32_t* __restrict__ offsets,
                 int32_t* __restrict__ pair_token, int32_t* __restrict__ pair_row) {
  extern __shared__ int32_t smem_i[];
  int32_t* cnt = smem_i;                    // [experts]: counts, then the next free row of each expert
  int32_t* part = smem_i + experts;         // [kRouteThreads]: per-thread segment sums
  const int tid = threadIdx.x;
  for (int e = tid; e < experts; e += kRouteThreads) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < pairs; p += kRouteThreads) {
    const int e = ids[p];
    if (e >= 0 && e < experts) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // exclusive prefix sum of the counts: each thread sums one contiguous segment,
  // the segment sums are scanned across the workgroup, then each segment is walked
  const int seg = (experts + kRouteThreads - 1) / kRouteThreads;
  const int e0 = tid * seg;
  int s = 0;
  for (int e = e0; e < e0 + seg && e < experts; ++e) s += cnt[e];
  part[tid] = s;
  __syncthreads();
  for (int d = 1; d < kRouteThreads; d <<= 1) {     // inclusive scan (Hillis-Steele)
    const int v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;                          // exclusive start of this segment
  for (int e = e0; e < e0 + seg && e < experts; ++e) {
    const int c = cnt[e];
    offsets[e] = run;
    cnt[e] = run;                                   // cursor: next free row of expert e
    run += c;
  }
  if (tid == kRouteThreads - 1) offsets[experts] = part[tid];
  __syncthreads();
  for (int p = tid; p < pairs; p += kRouteThreads) {
    const int e = ids[p];
    if (e >= 0 && e < experts) {
      const int r = atomicAdd(&cnt[e], 1);
      pair_token[r] = p / topk;
      pair_row[p] = r;
    } else {
      pair_row[p] = -1;
    }
  }
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
  for (int j = 0; j < topk; ++j) {
    const int r = pair_row[(int64_t)t * topk + j];
    if (r < 0 || r >= rows) continue;               // a pair without a row contributes nothing
    const float wj = w[(int64_t)t * topk + j];
    const uint16_t* src = yp + (int64_t)r * n + c0;
    if (vec) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src);
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(wj, half_bits_to_float(wd[i] & 0xFFFFu), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(wj, half_bits_to_float(wd[i] >> 16), acc[2 * i + 1]);
      }
    } else {
      for (int i = 0; i < 8 && c0 + i < n; ++i) acc[i] = __builtin_fmaf(wj, half_bits_to_float(src[i]), acc[i]);
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

size_t moe_route_lds(int experts) { return (size_t)(experts + kRouteThreads) * sizeof(int32_t); }

hipError_t launch_moe_route(const int32_t* ids, int pairs, int topk, int experts, int32_t* offsets,
                            int32_t* pair_token, int32_t* pair_row, const DeviceInfo& dev, hipStream_t stream) {
  const size_t lds = moe_route_lds(experts);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_route_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
    if (e != hipSuccess) return e;
  }
  (void)hipGetLastError();   // drop an error left by an earlier HIP call of the process
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), lds, stream, ids, pairs, topk, experts, offsets,
                     pair_token, pair_row);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t* y_pairs, const int32_t* pair_row, const float* weights, uint16_t* out,
                              int tokens, int topk, int n, int rows, hipStream_t stream) {
  const int64_t threads = (int64_t)tokens * ((n + 7) / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  (void)hipGetLastError();
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, y_pairs, pair_row, weights,
                     out, tokens, topk, n, rows);
  return hipGetLastError();
}

}  // namespace w4a16
