// Bandwidth diagnostics: a plain streaming read (the achievable read rate on
// this device for the decode kernels' load pattern, measured beside them)
// and a plain copy of known size (to scale hardware byte counters).

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

constexpr int kDiagBlocks = 8192;

// Streaming read: each workgroup reads one contiguous slab (as a decode
// workgroup reads one split of a sequence's rows) with the decode kernels'
// loads: 16-byte buffer loads with the non-temporal policy, four in flight
// per lane.  Slabs are whole multiples of 64 KiB (the last one shorter).
constexpr size_t kSlabGran = 64 * 1024;

static size_t stream_slab(size_t bytes) {
  size_t slab = (bytes + kDiagBlocks - 1) / kDiagBlocks;
  slab = (slab + kSlabGran - 1) / kSlabGran * kSlabGran;
  return slab ? slab : kSlabGran;
}

size_t stream_read_blocks(size_t bytes) {
  const size_t blocks = (bytes + stream_slab(bytes) - 1) / stream_slab(bytes);
  return blocks ? blocks : 1;
}

__global__ __launch_bounds__(256) void stream_read_kernel(const char* src, size_t bytes,
                                                          size_t slab, float* sink) {
  const size_t begin = (size_t)blockIdx.x * slab;
  const size_t len = bytes - begin < slab ? bytes - begin : slab;   // < 2^31 (slab <= 512 KiB
                                                                    // per 4 GiB)
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src + begin, (uint32_t)len);
  uint32_t acc = 0;
  // offsets past len read zeros (buffer range check)
  for (uint32_t off = threadIdx.x * 16u; off < (uint32_t)len; off += 4u * 256u * 16u) {
    const u32x4 a = buf_load16_stream(r, off), b = buf_load16_stream(r, off + 4096u),
                c = buf_load16_stream(r, off + 8192u), d = buf_load16_stream(r, off + 12288u);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^
           c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
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
                     static_cast<const char*>(src), bytes, stream_slab(bytes), sink);
  return hipGetLastError();
}

// (the copy keeps a grid of at most kDiagBlocks workgroups striding over the
// whole buffer)
static size_t copy_blocks(size_t bytes) {
  const size_t blocks = (bytes / 16 + 255) / 256;
  return blocks < kDiagBlocks ? (blocks ? blocks : 1) : kDiagBlocks;
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)copy_blocks(bytes)), dim3(256), 0, s,
                     reinterpret_cast<u32x4*>(dst), reinterpret_cast<const u32x4*>(src), bytes / 16);
  return hipGetLastError();
}

}  // namespace kvc
