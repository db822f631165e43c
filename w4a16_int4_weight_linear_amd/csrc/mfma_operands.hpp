// mfma_operands.hpp -- building fp16 MFMA operands from packed int4 weights
// and fp16 activations (shared by the dense and the grouped GEMM).
//
// An MFMA sums over the eight k of a lane's operand slice in any order, so A
// and B only have to agree on it.  Both use the order k = 0,4,1,5,2,6,3,7 of
// each 8-element slice (one packed word): it is the order in which two
// instructions per pair turn nibbles into fp16.
#pragma once

#include "device.hpp"

namespace w4a16 {

// fp16 pairs (u_j, u_j+4) of packed word q as exact codes times the scale.
__device__ inline f16x8 dequant_word(uint32_t q, f16x2 s2) {
  const f16x2 bias = {(_Float16)-1032.f, (_Float16)-1032.f};
  f16x2 r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t t = ((q >> (4 * j)) & 0x000F000Fu) | 0x64006400u;   // (1024 + u_j, 1024 + u_j+4)
    r[j] = (__builtin_bit_cast(f16x2, t) + bias) * s2;
  }
  f16x8 out;
  out[0] = r[0][0]; out[1] = r[0][1]; out[2] = r[1][0]; out[3] = r[1][1];
  out[4] = r[2][0]; out[5] = r[2][1]; out[6] = r[3][0]; out[7] = r[3][1];
  return out;
}

// (x0..x7 as pairs (0,1),(2,3),(4,5),(6,7)) -> pairs (0,4),(1,5),(2,6),(3,7).
__device__ inline u32x4 permute_a(u32x4 v) {
  u32x4 p;
  p.x = (v.x & 0xFFFFu) | (v.z << 16);
  p.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
  p.z = (v.y & 0xFFFFu) | (v.w << 16);
  p.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
  return p;
}

}  // namespace w4a16
