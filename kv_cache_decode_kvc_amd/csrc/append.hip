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

// FP8 E4M3 append: each new number x (bf16) is stored as the E4M3 code of
// x * (1 / scale) computed in float32, clamped to +-448 and rounded to
// nearest even by the hardware conversion (the storage reading of the
// guide's "Fewer bits per number": one byte per number, one scale per
// tensor).  Four numbers per thread.
// A NaN input gives code 0x7F (the conversion itself returns 0xFF for it).
__device__ inline uint32_t quant4_fp8(uint2 x, float inv) {
  float f[4] = {bf16_lo(x.x) * inv, bf16_hi(x.x) * inv, bf16_lo(x.y) * inv, bf16_hi(x.y) * inv};
  uint32_t nan_bytes = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    nan_bytes |= (f[i] != f[i] ? 0xFFu : 0u) << (8 * i);
    f[i] = fminf(fmaxf(f[i], -kFp8Max), kFp8Max);
  }
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0u, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w, true);
  return (w & ~nan_bytes) | (0x7F7F7F7Fu & nan_bytes);
}

__device__ inline void quant_rows(const AppendParams& p, int b, int n, const void* src_v,
                                  void* dst_v, float inv) {
  const uint2* src = reinterpret_cast<const uint2*>(src_v);
  uint32_t* dst = reinterpret_cast<uint32_t*>(dst_v);
  const int units = p.d / 4;
  const int total = p.n_kv * units;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int jj = e / units, c = e - jj * units;
    dst[(((size_t)b * p.n_kv + jj) * p.L_max + n) * units + c] =
        quant4_fp8(src[((size_t)b * p.n_kv + jj) * units + c], inv);
  }
}

__global__ __launch_bounds__(256) void append_fp8_kernel(AppendParams p) {
  __shared__ int s_n;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) s_n = p.seq_lens[b];
  __syncthreads();
  const int n = s_n;
  if (n < 0 || n >= p.L_max) {
    if (threadIdx.x == 0 && p.flag) atomicOr(p.flag, 1);
    return;
  }
  quant_rows(p, b, n, p.k_new, p.k_cache, p.k_inv);
  quant_rows(p, b, n, p.v_new, p.v_cache, p.v_inv);
  __syncthreads();
  if (threadIdx.x == 0) p.seq_lens[b] = n + 1;
}

hipError_t launch_append_fp8(const AppendParams& p, hipStream_t s) {
  hipLaunchKernelGGL(append_fp8_kernel, dim3(p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Paged append: slot n of sequence b is offset n % beta of block
// block_table[b][n / beta] in pools [num_blocks, n_kv, beta, d].  A full
// table sets flag bit 0, an invalid block bit 1; then nothing is written and
// the length stays.
__global__ __launch_bounds__(256) void append_paged_kernel(AppendParams p) {
  __shared__ int s_n, s_blk;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) {
    const int n = p.seq_lens[b];
    int blk = -1;
    if (n >= 0 && n < (p.max_blocks << p.page_shift))
      blk = p.block_table[(size_t)b * p.max_blocks + (n >> p.page_shift)];
    s_n = n;
    s_blk = blk;
  }
  __syncthreads();
  const int n = s_n, blk = s_blk;
  if (n < 0 || n >= (p.max_blocks << p.page_shift)) {
    if (threadIdx.x == 0 && p.flag) atomicOr(p.flag, 1);
    return;
  }
  if (blk < 0 || blk >= p.num_blocks) {
    if (threadIdx.x == 0 && p.flag) atomicOr(p.flag, 2);
    return;
  }
  const int beta = 1 << p.page_shift;
  const int units = p.d * p.elem_bytes / 16;
  const int total = p.n_kv * units;
  const u32x4* ks = reinterpret_cast<const u32x4*>(p.k_new);
  const u32x4* vs = reinterpret_cast<const u32x4*>(p.v_new);
  u32x4* kd = reinterpret_cast<u32x4*>(p.k_cache);
  u32x4* vd = reinterpret_cast<u32x4*>(p.v_cache);
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int jj = e / units, c = e - jj * units;
    const size_t dst = (((size_t)blk * p.n_kv + jj) * beta + (n & (beta - 1))) * units + c;
    const size_t src = ((size_t)b * p.n_kv + jj) * units + c;
    kd[dst] = ks[src];
    vd[dst] = vs[src];
  }
  __syncthreads();
  if (threadIdx.x == 0) p.seq_lens[b] = n + 1;
}

hipError_t launch_append_paged(const AppendParams& p, hipStream_t s) {
  hipLaunchKernelGGL(append_paged_kernel, dim3(p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  hipLaunchKernelGGL(append_kernel, dim3(p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvc
