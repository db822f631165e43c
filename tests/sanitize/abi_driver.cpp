// abi_driver.cpp -- drives the C ABI's host code under AddressSanitizer and
// UndefinedBehaviorSanitizer: the quantiser, pack/unpack round trips over
// ragged shapes and edge values, and every validation path of every device
// entry point (with stand-in launchers: no GPU is touched).  Exit status 0
// and "sanitize driver: ok" when every expectation holds; any sanitizer report
// aborts the process.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "../../include/w4a16.h"

static int g_checks = 0, g_fail = 0;
static void expect(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok) {
    ++g_fail;
    std::fprintf(stderr, "FAILED line %d: %s\n", line, what);
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// A 16-byte aligned address that is never dereferenced (device pointers).
static void* fake(uintptr_t extra = 0) { return reinterpret_cast<void*>((uintptr_t)0x10000 + extra); }
template <typename T> static T* F(uintptr_t extra = 0) { return static_cast<T*>(fake(extra)); }

static void host_routines() {
  std::mt19937 rng(7);
  std::normal_distribution<float> nd(0.f, 0.02f);
  for (int group : {32, 128}) {
    for (int n : {1, 3, 17}) {
      for (int kg : {1, 2, 5}) {
        const int k = kg * group;
        // exact-size heap buffers, so any overrun is reported
        std::vector<float> w((size_t)n * k);
        for (auto& v : w) v = nd(rng);
        w[0] = 0.f;
        if (n > 1) for (int i = 0; i < group; ++i) w[(size_t)k + i] = 0.f;   // an all-zero group
        std::vector<uint32_t> packed((size_t)n * k / 8);
        std::vector<uint16_t> scales((size_t)n * kg);
        EXPECT(w4a16_quantize(w.data(), n, k, group, packed.data(), scales.data()) == W4A16_OK);
        std::vector<int8_t> q((size_t)n * k);
        EXPECT(w4a16_unpack(packed.data(), n, k, q.data()) == W4A16_OK);
        bool in_range = true;
        for (int8_t c : q) in_range = in_range && c >= -8 && c <= 7;
        EXPECT(in_range);
        std::vector<uint32_t> again((size_t)n * k / 8);
        EXPECT(w4a16_pack(q.data(), n, k, again.data()) == W4A16_OK);
        EXPECT(std::memcmp(again.data(), packed.data(), again.size() * 4) == 0);
      }
    }
  }
  // errors
  std::vector<float> w(128, 1.f);
  std::vector<uint32_t> packed(16);
  std::vector<uint16_t> scales(1);
  w[5] = std::numeric_limits<float>::quiet_NaN();
  EXPECT(w4a16_quantize(w.data(), 1, 128, 128, packed.data(), scales.data()) == W4A16_ERR_RANGE);
  w[5] = 1e30f;                                                   // scale overflows fp16
  EXPECT(w4a16_quantize(w.data(), 1, 128, 128, packed.data(), scales.data()) == W4A16_ERR_RANGE);
  EXPECT(w4a16_quantize(w.data(), 1, 96, 128, packed.data(), scales.data()) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_quantize(w.data(), 1, 128, 64, packed.data(), scales.data()) == W4A16_ERR_GROUP);
  EXPECT(w4a16_quantize(nullptr, 1, 128, 128, packed.data(), scales.data()) == W4A16_ERR_NULL);
  EXPECT(w4a16_quantize(w.data(), 0, 128, 128, nullptr, nullptr) == W4A16_OK);
  std::vector<int8_t> q(8, 0);
  q[3] = 8;
  EXPECT(w4a16_pack(q.data(), 1, 8, packed.data()) == W4A16_ERR_RANGE);
  EXPECT(w4a16_pack(q.data(), 1, 12, packed.data()) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_unpack(nullptr, 1, 8, q.data()) == W4A16_ERR_NULL);
  EXPECT(w4a16_unpack(packed.data(), -1, 8, q.data()) == W4A16_ERR_SHAPE);
  for (int s = 0; s <= 9; ++s) EXPECT(w4a16_status_str(s) != nullptr);
  EXPECT(w4a16_abi_version() == W4A16_ABI_VERSION);
}

static void device_validation() {
  const uint16_t* x = F<const uint16_t>();
  const uint32_t* p = F<const uint32_t>();
  const uint16_t* s = F<const uint16_t>();
  uint16_t* y = F<uint16_t>();
  // every error is found before a device is touched; a valid call reaches the
  // (absent) device and reports W4A16_ERR_HIP
  EXPECT(w4a16_gemv(x, p, s, y, 1, 64, 128, 64, nullptr) == W4A16_ERR_GROUP);
  EXPECT(w4a16_gemv(x, p, s, y, 1, 64, 100, 32, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemv(x, p, s, y, 5, 64, 128, 128, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemv(x, p, s, nullptr, 1, 64, 128, 128, nullptr) == W4A16_ERR_NULL);
  EXPECT(w4a16_gemv(F<const uint16_t>(8), p, s, y, 1, 64, 128, 128, nullptr) == W4A16_ERR_ALIGN);
  EXPECT(w4a16_gemv(x, p, s, y, 1, (int64_t)1 << 40, 128, 128, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemv(x, p, s, y, INT64_MIN, 64, 128, 128, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemv(nullptr, nullptr, nullptr, nullptr, 0, 64, 128, 128, nullptr) == W4A16_OK);
  EXPECT(w4a16_gemv(x, p, s, y, 1, 64, 128, 128, nullptr) == W4A16_ERR_HIP);
  EXPECT(w4a16_gemv_max_k(2, 128) == 0);
  EXPECT(w4a16_gemm(x, p, s, y, 8, 64, 128, 16, nullptr, 0, nullptr) == W4A16_ERR_GROUP);
  EXPECT(w4a16_gemm(x, p, s, y, 8, 64, 128, 128, fake(4), 0, nullptr) == W4A16_ERR_ALIGN);
  EXPECT(w4a16_gemm(x, p, s, y, INT64_MAX, INT64_MAX, INT64_MAX, 128, nullptr, 0, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemm(x, p, s, y, 600, 64, 128, 128, nullptr, 0, nullptr) == W4A16_ERR_HIP);
  EXPECT(w4a16_gemm_workspace_bytes(INT64_MAX, 64, 128, 128) == 0);
  EXPECT(w4a16_gemm_noalloc(x, p, s, y, 8, 64, 128, 16, nullptr) == W4A16_ERR_GROUP);
  EXPECT(w4a16_gemm_noalloc(x, p, s, nullptr, 8, 64, 128, 128, nullptr) == W4A16_ERR_NULL);
  EXPECT(w4a16_gemm_noalloc(x, p, s, F<uint16_t>(2), 8, 64, 128, 128, nullptr) == W4A16_ERR_ALIGN);
  EXPECT(w4a16_gemm_noalloc(nullptr, nullptr, nullptr, nullptr, 0, 64, 128, 128, nullptr) == W4A16_OK);
  EXPECT(w4a16_gemm_noalloc(x, p, s, y, 600, 64, 128, 128, nullptr) == W4A16_ERR_HIP);
  EXPECT(w4a16_gemm_workspace_status(nullptr, 4096, nullptr) == W4A16_ERR_NULL);
  EXPECT(w4a16_gemm_workspace_status(fake(4), 4096, nullptr) == W4A16_ERR_ALIGN);
  EXPECT(w4a16_gemm_workspace_status(fake(), 16, nullptr) == W4A16_ERR_WORKSPACE);
  EXPECT(w4a16_gemv_swiglu(x, p, s, y, 17, 64, 128, 128, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemv_swiglu(x, p, s, y, 1, (int64_t)1 << 40, 128, 128, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemv_swiglu(x, p, s, y, 1, 64, 128, 128, nullptr) == W4A16_ERR_HIP);
  const int32_t* off = F<const int32_t>();
  EXPECT(w4a16_grouped_gemm(x, p, s, off, y, 4, 16, 64, 128, 48, nullptr) == W4A16_ERR_GROUP);
  EXPECT(w4a16_grouped_gemm(x, p, s, off, y, 0, 16, 64, 128, 32, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_grouped_gemm(x, p, s, F<const int32_t>(2), y, 4, 16, 64, 128, 32, nullptr) == W4A16_ERR_ALIGN);
  EXPECT(w4a16_grouped_gemm(x, p, s, off, y, INT32_MAX, 16, 1 << 20, 1 << 20, 32, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_grouped_gemm(x, p, s, off, y, 4, 16, 64, 128, 32, nullptr) == W4A16_ERR_HIP);
  const int32_t* tok = F<const int32_t>();
  EXPECT(w4a16_grouped_gemm_gather(x, nullptr, p, s, off, y, 4, 16, 8, 64, 128, 32, nullptr) == W4A16_ERR_NULL);
  EXPECT(w4a16_grouped_gemm_gather(x, tok, p, s, off, y, 4, 16, 8, 64, 128, 32, nullptr) == W4A16_ERR_HIP);
  EXPECT(w4a16_grouped_gemm_swiglu(x, nullptr, p, s, off, y, 4, 16, 0, 64, 128, 48, nullptr) == W4A16_ERR_GROUP);
  EXPECT(w4a16_grouped_gemm_swiglu(x, nullptr, p, s, off, y, 4, 16, 0, (int64_t)1 << 30, 128, 32, nullptr) ==
         W4A16_ERR_SHAPE);
  EXPECT(w4a16_grouped_gemm_swiglu(x, F<const int32_t>(2), p, s, off, y, 4, 16, 8, 64, 128, 32, nullptr) ==
         W4A16_ERR_ALIGN);
  EXPECT(w4a16_grouped_gemm_swiglu(x, nullptr, p, s, off, y, 4, 16, 0, 64, 128, 32, nullptr) == W4A16_ERR_HIP);
  EXPECT(w4a16_grouped_gemm_swiglu(x, tok, p, s, off, y, 4, 16, 8, 64, 128, 32, nullptr) == W4A16_ERR_HIP);
  int32_t* o = F<int32_t>();
  EXPECT(w4a16_moe_route(off, 4, 0, 8, o, o, o, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_moe_route(off, INT64_MAX, 8, 8, o, o, o, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_moe_route(off, 4, 2, 8, o, o, o, nullptr) == W4A16_ERR_HIP);
  EXPECT(w4a16_moe_combine(x, off, F<const float>(), y, 4, 0, 32, 64, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_moe_combine(x, off, F<const float>(), y, INT64_MAX, 2, 32, 64, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_moe_combine(x, off, F<const float>(), y, 4, 2, 32, 64, nullptr) == W4A16_ERR_HIP);
  EXPECT(w4a16_hbm_read_probe(fake(), 1000, F<uint32_t>(), 4096, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_hbm_read_probe(nullptr, 1024, F<uint32_t>(), 4096, nullptr) == W4A16_ERR_NULL);
  EXPECT(w4a16_hbm_read_probe(fake(8), 1024, F<uint32_t>(), 4096, nullptr) == W4A16_ERR_ALIGN);
  EXPECT(w4a16_hbm_read_probe(fake(), 0, nullptr, 0, nullptr) == W4A16_OK);
  EXPECT(w4a16_hbm_read_probe(fake(), 1024, F<uint32_t>(), 4096, nullptr) == W4A16_ERR_HIP);
  EXPECT(w4a16_hbm_read_probe_sink_words() == 0);
}

int main() {
  host_routines();
  device_validation();
  if (g_fail) {
    std::fprintf(stderr, "sanitize driver: %d of %d checks failed\n", g_fail, g_checks);
    return 1;
  }
  std::printf("sanitize driver: ok (%d checks)\n", g_checks);
  return 0;
}
