// mfma_operands.hpp -- building fp16 MFMA operands from packed int4 weights
// and fp16 activations (shared by the dense and the grouped GEMM).
//
// An MFMA sums over the eight k of a lane's operand slice in any order, so A
// and B only have to agree on it.  Both use the order k = 0,4,2,6,1,5,3,7 of
// each 8-element slice (one packed word): the order in which a byte permute
// turns pairs of nibbles into fp16.
#pragma once

#include "device.hpp"

namespace w4a16 {

// The eight codes of packed word q as fp16 operand values q_k * s, in the
// slice order (0,4), (2,6), (1,5), (3,7).  Masking by 0x0F0F0F0F leaves the
// even nibbles u0, u2, u4, u6 one per byte (the odd ones after a shift by 4);
// a byte permute pairs two of them with the byte 0x64 above each, giving the
// fp16 values 1024 + u exactly; subtracting 1032 gives the code q = u - 8
// exactly, and one multiply by the group scale rounds once.
__device__ inline f16x8 dequant_word(uint32_t q, f16x2 s2) {
  const uint32_t magic = 0x64646464u;
  const uint32_t qa = q & 0x0F0F0F0Fu;            // bytes u0 u2 u4 u6
  const uint32_t qb = (q >> 4) & 0x0F0F0F0Fu;     // bytes u1 u3 u5 u7
  const f16x2 bias = {(_Float16)-1032.f, (_Float16)-1032.f};
  const uint32_t t[4] = {__builtin_amdgcn_perm(magic, qa, 0x04020400u),    // (u0, u4)
                         __builtin_amdgcn_perm(magic, qa, 0x04030401u),    // (u2, u6)
                         __builtin_amdgcn_perm(magic, qb, 0x04020400u),    // (u1, u5)
                         __builtin_amdgcn_perm(magic, qb, 0x04030401u)};   // (u3, u7)
  f16x2 r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = (__builtin_bit_cast(f16x2, t[j]) + bias) * s2;
  f16x8 out;
  out[0] = r[0][0]; out[1] = r[0][1]; out[2] = r[1][0]; out[3] = r[1][1];
  out[4] = r[2][0]; out[5] = r[2][1]; out[6] = r[3][0]; out[7] = r[3][1];
  return out;
}

// The eight codes of packed word q as fp16 operand values q_k * s in natural
// k order (used where the activations reach the MFMA untouched, e.g. loaded
// straight into LDS): the two nibble bytes are interleaved by one more byte
// permute each before the pairs are formed.
__device__ inline f16x8 dequant_word_natural(uint32_t q, f16x2 s2) {
  const uint32_t magic = 0x64646464u;
  const uint32_t qa = q & 0x0F0F0F0Fu;            // bytes u0 u2 u4 u6
  const uint32_t qb = (q >> 4) & 0x0F0F0F0Fu;     // bytes u1 u3 u5 u7
  const uint32_t i0 = __builtin_amdgcn_perm(qb, qa, 0x05010400u);   // bytes u0 u1 u2 u3
  const uint32_t i1 = __builtin_amdgcn_perm(qb, qa, 0x07030602u);   // bytes u4 u5 u6 u7
  const f16x2 bias = {(_Float16)-1032.f, (_Float16)-1032.f};
  const uint32_t t[4] = {__builtin_amdgcn_perm(magic, i0, 0x04010400u),    // (u0, u1)
                         __builtin_amdgcn_perm(magic, i0, 0x04030402u),    // (u2, u3)
                         __builtin_amdgcn_perm(magic, i1, 0x04010400u),    // (u4, u5)
                         __builtin_amdgcn_perm(magic, i1, 0x04030402u)};   // (u6, u7)
  f16x2 r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = (__builtin_bit_cast(f16x2, t[j]) + bias) * s2;
  f16x8 out;
  out[0] = r[0][0]; out[1] = r[0][1]; out[2] = r[1][0]; out[3] = r[1][1];
  out[4] = r[2][0]; out[5] = r[2][1]; out[6] = r[3][0]; out[7] = r[3][1];
  return out;
}

// Codes without conversion instructions (the batched decode kernels): one AND-OR
// per pair keeps two nibbles of a packed word and sets an fp16 exponent above
// them.  The nibbles of even k (mantissa bits 0-3, exponent field 5) read
// 2^-10 + u 2^-20; those of odd k (bits 4-7, exponent field 1) read
// 2^-14 + 16 u 2^-24 = 2^-14 + u 2^-20, so each code is u 2^-20 above a per-k
// bias, exact.  Subtracting the activations' biased sum b = sum x_even (2^-10 +
// 8 2^-20) + sum x_odd (2^-14 + 8 2^-20) from the product leaves
// 2^-20 sum x (u - 8).  kBiasPair is that (even k, odd k) fp16 pair.
constexpr uint32_t kBiasPair = 0x04801408u;

// Eight activations (pairs (0,1),(2,3),(4,5),(6,7)) rearranged into the same
// slice order: pairs (0,4), (2,6), (1,5), (3,7).
__device__ inline u32x4 permute_a(u32x4 v) {
  u32x4 p;
  p.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);   // (x0, x4)
  p.y = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);   // (x2, x6)
  p.z = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);   // (x1, x5)
  p.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);   // (x3, x7)
  return p;
}

}  // namespace w4a16
