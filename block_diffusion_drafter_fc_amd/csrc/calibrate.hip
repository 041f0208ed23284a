// calibrate.hip -- a pure streaming read of known size, for calibrating the
// HBM byte counters against the LM head's own load pattern: each workgroup
// reads one contiguous run with 16-byte non-temporal loads (a wave reads 1 KB
// of contiguous memory per load instruction, as the LM head does over its
// packed weights) and writes one 16-byte checksum.
#include "common.h"
#include "kernels.h"

namespace {

__global__ __launch_bounds__(256, 2) void k_read_calibration(const u32x4* __restrict__ src,
                                                             size_t n16, u32x4* __restrict__ out) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b = (size_t)blockIdx.x * per, e = b + per < n16 ? b + per : n16;
  u32x4 acc[4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  size_t i = b + threadIdx.x;
  // four independent loads in flight per lane per iteration
  for (; i + 3 * 256 < e; i += 4 * 256) {
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] ^= __builtin_nontemporal_load(src + i + u * 256);
  }
  for (; i < e; i += 256) acc[0] ^= __builtin_nontemporal_load(src + i);
  u32x4 x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    x[0] ^= (uint32_t)__shfl_xor((int)x[0], m, 64);
    x[1] ^= (uint32_t)__shfl_xor((int)x[1], m, 64);
    x[2] ^= (uint32_t)__shfl_xor((int)x[2], m, 64);
    x[3] ^= (uint32_t)__shfl_xor((int)x[3], m, 64);
  }
  __shared__ u32x4 red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

hipError_t launch_read_calibration(const void* src, size_t bytes, void* out, int workgroups,
                                   hipStream_t st) {
  if (bytes % 16 != 0 || workgroups < 1 || workgroups > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read_calibration, dim3(workgroups), dim3(256), 0, st, (const u32x4*)src,
                     bytes / 16, (u32x4*)out);
  return hipGetLastError();
}
