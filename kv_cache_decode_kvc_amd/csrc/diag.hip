// Bandwidth diagnostics: a plain streaming read (the achievable read rate on
// this device, measured beside the attention kernels) and a plain copy of
// known size (to scale hardware byte counters).

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

constexpr int kDiagBlocks = 8192;

size_t stream_read_blocks(size_t bytes) {
  const size_t vecs = bytes / 16;
  size_t blocks = (vecs + 255) / 256;
  return blocks < kDiagBlocks ? (blocks ? blocks : 1) : kDiagBlocks;
}

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* src, size_t nvec,
                                                          float* sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride],
                d = src[i + 3 * stride];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^
           c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < nvec; i += stride) {
    const u32x4 a = src[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  // keep the loads live: one word per workgroup
  __shared__ uint32_t red[4];
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0)
    sink[blockIdx.x] = __uint_as_float((red[0] ^ red[1] ^ red[2] ^ red[3]) & 0x007FFFFFu);
}

__global__ __launch_bounds__(256) void copy_kernel(u32x4* dst, const u32x4* src, size_t nvec) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride)
    dst[i] = src[i];
}

hipError_t launch_stream_read(const void* src, size_t bytes, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)stream_read_blocks(bytes)), dim3(256), 0, s,
                     reinterpret_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)stream_read_blocks(bytes)), dim3(256), 0, s,
                     reinterpret_cast<u32x4*>(dst), reinterpret_cast<const u32x4*>(src), bytes / 16);
  return hipGetLastError();
}

}  // namespace kvc
