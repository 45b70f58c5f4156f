// Streaming-read yardsticks: what plain reads reach on the device, the
// second yardstick beside the HBM peak (built as libskv_yardstick.so; not
// part of the decode step or its library).
//  * read_probe_kernel: the buffer once, in grid-stride order, with 16-byte
//    loads, four in flight per thread (optionally marked non-temporal);
//  * read_pieces_kernel: the buffer once as 4 KB pieces visited in a given
//    order (a permutation), one piece per wave at a time (1 KB per load
//    instruction), four pieces in flight per wave -- the access pattern of a
//    scan over a pool of 4 KB (block, head) runs in permuted block order.
// Both fold the words into one value per workgroup so no load is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/skv_yardstick.h"

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

template <bool NT>
__device__ __forceinline__ u32x4_t load16(const u32x4_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

__device__ __forceinline__ void fold_out(uint32_t x, uint32_t* sink) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
  __shared__ uint32_t w[4];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = w[0] ^ w[1] ^ w[2] ^ w[3];
}

template <bool NT>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4_t* p, int64_t n16,
                                                         uint32_t* sink) {
  uint32_t x = 0u;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = load16<NT>(p + i), b = load16<NT>(p + i + stride),
                  c = load16<NT>(p + i + 2 * stride), d = load16<NT>(p + i + 3 * stride);
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^
         d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t a = load16<NT>(p + i);
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  fold_out(x, sink);
}

__global__ __launch_bounds__(256) void read_pieces_kernel(const u32x4_t* p, const int32_t* order,
                                                          int64_t n_pieces, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int64_t n_waves = ((int64_t)gridDim.x * 256) >> 6;
  uint32_t x = 0u;
  for (int64_t i = wave; i < n_pieces; i += 4 * n_waves) {
    u32x4_t a[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t pi = i + u * n_waves;
      const int32_t o = pi < n_pieces ? order[pi] : -1;
      const u32x4_t* b = (o >= 0 && o < n_pieces) ? p + (int64_t)o * 256 : nullptr;
#pragma unroll
      for (int c = 0; c < 4; ++c) a[u][c] = b ? b[c * 64 + lane] : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) x ^= a[u][c][0] ^ a[u][c][1] ^ a[u][c][2] ^ a[u][c][3];
  }
  fold_out(x, sink);
}

}  // namespace

extern "C" {

int32_t skv_read_probe(const void* buf, size_t bytes, int32_t n_wg, uint32_t* sink,
                       hipStream_t stream) {
  return skv_read_probe_ex(buf, bytes, n_wg, 0, sink, stream);
}

int32_t skv_read_probe_ex(const void* buf, size_t bytes, int32_t n_wg, int32_t nontemporal,
                          uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 || n_wg < 1) return 1;
  if (nontemporal)
    read_probe_kernel<true><<<n_wg, 256, 0, stream>>>((const u32x4_t*)buf, (int64_t)(bytes / 16),
                                                       sink);
  else
    read_probe_kernel<false><<<n_wg, 256, 0, stream>>>((const u32x4_t*)buf, (int64_t)(bytes / 16),
                                                        sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int32_t skv_read_pieces(const void* buf, const int32_t* order, int64_t n_pieces, int32_t n_wg,
                        uint32_t* sink, hipStream_t stream) {
  if (!buf || !order || !sink || n_pieces < 1 || n_wg < 1) return 1;
  read_pieces_kernel<<<n_wg, 256, 0, stream>>>((const u32x4_t*)buf, order, n_pieces, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
