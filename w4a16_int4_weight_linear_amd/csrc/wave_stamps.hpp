// wave_stamps.hpp -- per-wave timeline stamps for a profiling build.
//
// Built with -DW4A16_WAVE_STAMPS (build.py --wave-stamps, a separate library),
// the weight-streaming kernels read the 100 MHz real-time counter at a few
// points of each wave's life (start, activations staged, first unit done, loop
// end, ...), keep the values in registers and store them once, at the end, to a
// per-file device array that the host reads back through an extern "C"
// accessor.  Only the first 256 workgroups of 8 waves are recorded, one launch
// at a time (each launch overwrites the array).  Without the macro every stamp
// compiles to nothing and the kernels are exactly the product kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {
constexpr int kStampSlots = 8;                  // stamps per wave
constexpr int kStampWaves = 256 * 8;            // workgroups x waves recorded
}  // namespace w4a16

#ifdef W4A16_WAVE_STAMPS

// One array per source file; NAME is the host accessor's symbol.
#define W4A16_STAMP_STORAGE(NAME)                                                                   \
  namespace w4a16 {                                                                                \
  __device__ uint64_t g_wave_stamps[kStampWaves * kStampSlots];                                    \
  }                                                                                                \
  extern "C" int NAME(void* host, size_t bytes) {                                                  \
    const size_t n = sizeof(w4a16::g_wave_stamps);                                                 \
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(w4a16::g_wave_stamps), bytes < n ? bytes : n, \
                                    0, hipMemcpyDeviceToHost);                                     \
  }
#define W4A16_STAMP_DECL uint64_t stamp_[w4a16::kStampSlots] = {}
#define W4A16_STAMP(i) (stamp_[(i)] = __builtin_amdgcn_s_memrealtime())
// Lane 0 of each recorded wave stores its stamps (call once, at the very end).
#define W4A16_STAMP_FLUSH(wave)                                                                    \
  do {                                                                                             \
    if (blockIdx.x < 256 && (threadIdx.x & 63) == 0) {                                             \
      for (int i_ = 0; i_ < w4a16::kStampSlots; ++i_)                                              \
        w4a16::g_wave_stamps[(blockIdx.x * 8 + (wave)) * w4a16::kStampSlots + i_] = stamp_[i_];    \
    }                                                                                              \
  } while (0)

#else

#define W4A16_STAMP_STORAGE(NAME)
#define W4A16_STAMP_DECL ((void)0)
#define W4A16_STAMP(i) ((void)0)
#define W4A16_STAMP_FLUSH(wave) ((void)0)

#endif
