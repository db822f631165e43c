// device.hpp -- small gfx950 device helpers shared by the W4A16 kernels.
//
// Nothing here is specific to one kernel: buffer-resource loads (out-of-range
// offsets return zero and touch no memory, which is how tails and padding are
// masked without branches), the fp16 pair dot product, and DPP reductions
// across a 64-wide wavefront.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Word 3 of a raw buffer descriptor on gfx9-family parts (32-bit data format).
constexpr int kRawBufferFlags = 0x00020000;
// Cache policy bit for data streamed exactly once (non-temporal).
constexpr int kStream = 2;

// Cache policy for data handed between workgroups on different CUs (and so,
// on this multi-XCD part, possibly different L2s): device scope (sc1), so a
// store reaches and a load reads the device coherence point, and no L2
// write-back or invalidation is needed around the exchange.
constexpr int kDeviceScope = 16;

// An offset that lies outside every buffer: loads from it return 0.
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferFlags);
}

// 16 bytes at byte offset `off` of a buffer of `bytes` bytes.  A load that
// reaches past the end is out of range as a whole and would return zero, so the
// partial last chunk of a buffer is assembled from 2-byte loads (each either
// fully inside or fully outside); bytes past the end read as zero.
__device__ inline u32x4 load16_tail(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t bytes) {
  if (off >= bytes || off + 16u <= bytes) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, off + 4u * i, 0, 0);
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, off + 4u * i + 2u, 0, 0);
    w[i] = (lo & 0xFFFFu) | (hi << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// acc + a.lo * b.lo + a.hi * b.hi, products of fp16 pairs accumulated in fp32.
__device__ inline float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
}

__device__ inline float half_bits_to_float(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__device__ inline uint16_t float_to_half_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);  // round to nearest even
}

template <int CTRL>
__device__ inline float dpp_add(float v) {
  int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false);
  return v + __builtin_bit_cast(float, moved);
}

// Sum over all 64 lanes; every lane receives the total.  Within each 16-lane
// DPP row: swap neighbours, swap pairs, then rotate by 4 and by 8; the four
// row sums are then combined through scalar reads of lanes 0, 16, 32, 48.
__device__ inline float wave_sum(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x124>(v);  // row_ror:4
  v = dpp_add<0x128>(v);  // row_ror:8
  int b = __builtin_bit_cast(int, v);
  float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ inline int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

}  // namespace w4a16
