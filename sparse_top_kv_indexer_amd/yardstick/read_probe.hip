// Streaming-read yardstick: reads a buffer once with 16-byte loads, four in
// flight per thread, and folds the words into one value per workgroup so the
// loads are not dead.  Not part of the decode step or its library: it
// measures what a plain read reaches on the device, the second yardstick
// beside the HBM peak (built as libskv_yardstick.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/skv_yardstick.h"

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4_t* p, int64_t n16,
                                                         uint32_t* sink) {
  uint32_t x = 0u;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^
         d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t a = p[i];
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
  __shared__ uint32_t w[4];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = w[0] ^ w[1] ^ w[2] ^ w[3];
}

}  // namespace

extern "C" {

int32_t skv_read_probe(const void* buf, size_t bytes, int32_t n_wg, uint32_t* sink,
                       hipStream_t stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 || n_wg < 1) return 1;
  read_probe_kernel<<<n_wg, 256, 0, stream>>>((const u32x4_t*)buf, (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
