// misc.hip -- y = 0 for the empty sum (k == 0).
#include "device.hpp"
#include "kernels.hpp"
#include "launch.hpp"

namespace w4a16 {
namespace {
__global__ void zero_fill_kernel(uint16_t* __restrict__ y, size_t count) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) y[i] = 0;
}
}  // namespace

hipError_t launch_zero_fill(uint16_t* y, size_t count, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  size_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  return launch_kernel(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, y, count);
}
}  // namespace w4a16
