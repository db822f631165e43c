// host_pack.cpp -- host-side quantiser and nibble packing of the W4A16 format.
//
// Scheme (LLM170, CUDA/W4A16 page, opening description): int4 symmetric
// weights, one fp16 scale per group of 128 (32 for MoE) input features.  The
// storage rules (offset-binary nibbles, eight per uint32 along K, low nibble
// first) and the quantiser's rounding are documented in include/w4a16.h.
//
// Plain C++ with no HIP dependency, so it is built and tested on any host.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/w4a16.h"

namespace {

// fp32 -> fp16 bits, round to nearest even (IEEE 754 binary16), including
// subnormals, overflow to infinity and NaN.
uint16_t f32_to_f16_bits(float f) {
  uint32_t b;
  std::memcpy(&b, &f, 4);
  const uint32_t sign = (b >> 16) & 0x8000u;
  const uint32_t absb = b & 0x7FFFFFFFu;
  if (absb >= 0x7F800000u) {                       // inf or nan
    return (uint16_t)(sign | 0x7C00u | (absb > 0x7F800000u ? 0x200u : 0u));
  }
  const int exp = (int)(absb >> 23) - 127;         // unbiased exponent
  if (exp > 15) return (uint16_t)(sign | 0x7C00u); // too large: inf (rounding cannot save it)
  uint32_t mant = absb & 0x7FFFFFu;
  if (exp >= -14) {                                // normal fp16 range
    uint32_t h = ((uint32_t)(exp + 15) << 10) | (mant >> 13);
    const uint32_t rest = mant & 0x1FFFu;
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) ++h;   // may carry into exponent / inf
    return (uint16_t)(sign | h);
  }
  if (exp < -25) return (uint16_t)sign;            // below half the smallest subnormal
  // subnormal: value = m * 2^-24 with m = round(1.mant * 2^(exp + 24))
  mant |= 0x800000u;                               // implicit 1, value = mant * 2^(exp - 23)
  const int shift = -exp - 1;                      // 13 + (-14 - exp)
  uint32_t h = mant >> shift;
  const uint32_t rest = mant & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rest > half || (rest == half && (h & 1u))) ++h;
  return (uint16_t)(sign | h);
}

float f16_bits_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu;
  const uint32_t m = h & 0x3FFu;
  float v;
  if (e == 0) {
    v = std::ldexp((float)m, -24);
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = std::ldexp((float)(m | 0x400u), (int)e - 25);
  }
  return sign ? -v : v;
}

bool valid_group(int32_t g) { return g == 32 || g == 128; }

}  // namespace

extern "C" {

w4a16_status w4a16_quantize(const float* w, int64_t n, int64_t k, int32_t group, uint32_t* packed,
                   uint16_t* scales) {
  if (!valid_group(group)) return W4A16_ERR_GROUP;
  if (n < 0 || k < 0 || k % group) return W4A16_ERR_SHAPE;
  if (n == 0 || k == 0) return W4A16_OK;
  if (!w || !packed || !scales) return W4A16_ERR_NULL;
  const int64_t groups = k / group;
  // First pass: validate everything so that nothing is written on error.
  for (int64_t i = 0; i < n * k; ++i) {
    if (!std::isfinite(w[i])) return W4A16_ERR_RANGE;
  }
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t g = 0; g < groups; ++g) {
      const float* blk = w + r * k + g * group;
      float a = 0.f;
      for (int i = 0; i < group; ++i) a = std::fmax(a, std::fabs(blk[i]));
      const uint16_t sb = f32_to_f16_bits(a / 7.0f);
      if ((sb & 0x7C00u) == 0x7C00u) return W4A16_ERR_RANGE;
    }
  }
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t g = 0; g < groups; ++g) {
      const float* blk = w + r * k + g * group;
      float a = 0.f;
      for (int i = 0; i < group; ++i) a = std::fmax(a, std::fabs(blk[i]));
      const uint16_t sb = f32_to_f16_bits(a / 7.0f);       // fp32 divide, RNE to fp16
      scales[r * groups + g] = sb;
      const float s = f16_bits_to_f32(sb);
      uint32_t* out = packed + (r * k + g * group) / 8;
      for (int j = 0; j < group / 8; ++j) {
        uint32_t word = 0;
        for (int i = 0; i < 8; ++i) {
          int q = 0;
          if (s != 0.f) {
            const float t = std::nearbyint(blk[8 * j + i] / s);   // fp32 divide, ties to even
            q = t < -8.f ? -8 : (t > 7.f ? 7 : (int)t);
          }
          word |= (uint32_t)(q + 8) << (4 * i);
        }
        out[j] = word;
      }
    }
  }
  return W4A16_OK;
}

w4a16_status w4a16_pack(const int8_t* q, int64_t n, int64_t k, uint32_t* packed) {
  if (n < 0 || k < 0 || k % 8) return W4A16_ERR_SHAPE;
  if (n == 0 || k == 0) return W4A16_OK;
  if (!q || !packed) return W4A16_ERR_NULL;
  for (int64_t i = 0; i < n * k; ++i) {
    if (q[i] < -8 || q[i] > 7) return W4A16_ERR_RANGE;
  }
  for (int64_t i = 0; i < n * k / 8; ++i) {
    uint32_t word = 0;
    for (int j = 0; j < 8; ++j) word |= (uint32_t)(q[8 * i + j] + 8) << (4 * j);
    packed[i] = word;
  }
  return W4A16_OK;
}

w4a16_status w4a16_unpack(const uint32_t* packed, int64_t n, int64_t k, int8_t* q) {
  if (n < 0 || k < 0 || k % 8) return W4A16_ERR_SHAPE;
  if (n == 0 || k == 0) return W4A16_OK;
  if (!q || !packed) return W4A16_ERR_NULL;
  for (int64_t i = 0; i < n * k / 8; ++i) {
    const uint32_t word = packed[i];
    for (int j = 0; j < 8; ++j) q[8 * i + j] = (int8_t)((int)((word >> (4 * j)) & 0xFu) - 8);
  }
  return W4A16_OK;
}

}  // extern "C"
