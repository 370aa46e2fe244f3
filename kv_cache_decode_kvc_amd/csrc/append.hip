// Cache append: the new token's key and value go to slot seq_lens[b], then
// the length grows by one ("KV cache" guide, "Two tensors per layer"; the
// podcast's decode walk-through: the cache grows by one entry per layer per
// token).  A bit copy; one workgroup per sequence so that the length is read
// once, every element is written, and only then the length is bumped.

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

template <typename U>
__device__ inline void copy_rows(const AppendParams& p, int b, int n,
                                 const void* src_v, void* dst_v, int units) {
  const U* src = reinterpret_cast<const U*>(src_v);
  U* dst = reinterpret_cast<U*>(dst_v);
  const int total = p.n_kv * units;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int jj = e / units, c = e - jj * units;
    dst[(((size_t)b * p.n_kv + jj) * p.L_max + n) * units + c] =
        src[((size_t)b * p.n_kv + jj) * units + c];
  }
}

__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  __shared__ int s_n;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) s_n = p.seq_lens[b];
  __syncthreads();
  const int n = s_n;
  if (n < 0 || n >= p.L_max) {
    if (threadIdx.x == 0 && p.flag) atomicOr(p.flag, 1);
    return;
  }
  const size_t row_bytes = (size_t)p.d * p.elem_bytes;
  if (row_bytes % 16 == 0) {
    const int units = (int)(row_bytes / 16);
    copy_rows<u32x4>(p, b, n, p.k_new, p.k_cache, units);
    if (p.v_cache) copy_rows<u32x4>(p, b, n, p.v_new, p.v_cache, units);
  } else if (row_bytes % 4 == 0) {
    const int units = (int)(row_bytes / 4);
    copy_rows<uint32_t>(p, b, n, p.k_new, p.k_cache, units);
    if (p.v_cache) copy_rows<uint32_t>(p, b, n, p.v_new, p.v_cache, units);
  } else {
    const int units = (int)(row_bytes / 2);
    copy_rows<uint16_t>(p, b, n, p.k_new, p.k_cache, units);
    if (p.v_cache) copy_rows<uint16_t>(p, b, n, p.v_new, p.v_cache, units);
  }
  __syncthreads();
  if (threadIdx.x == 0) p.seq_lens[b] = n + 1;
}

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  hipLaunchKernelGGL(append_kernel, dim3(p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvc
