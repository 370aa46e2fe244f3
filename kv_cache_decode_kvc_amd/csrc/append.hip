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

// FP4 append (E2M1 numbers, one E4M3 scale per 16 channels): one thread per
// 16-channel block of a new row.  scale = E4M3(float32(amax / 6)) (nearest
// even, saturating at 448); each number becomes the E2M1 code nearest
// float32(x / scale), ties to the even code, saturating at 6, sign bit from
// the quotient's sign; a zero scale stores zero codes.  Codes are packed two
// per byte, the even channel in the low nibble.
__device__ inline uint32_t e2m1_code(float q) {
  const float a = fabsf(q);
  const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
                     (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return c | (signbit(q) ? 8u : 0u);
}

__device__ inline void quant_block_fp4(const uint16_t* src, uint8_t* codes, uint8_t* scale) {
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
  const u32x4 w0 = s4[0], w1 = s4[1];
  float x[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w0[i]);
    x[2 * i + 1] = bf16_hi(w0[i]);
    x[8 + 2 * i] = bf16_lo(w1[i]);
    x[8 + 2 * i + 1] = bf16_hi(w1[i]);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float s_raw = fminf(__fdiv_rn(amax, 6.0f), kFp8Max);
  const uint32_t sc = __builtin_amdgcn_cvt_pk_fp8_f32(s_raw, 0.f, 0u, false) & 0xFFu;
  const float s = __builtin_amdgcn_cvt_f32_fp8(sc, 0);
  uint32_t lo = 0, hi = 0;
  if (s > 0.f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo |= e2m1_code(__fdiv_rn(x[i], s)) << (4 * i);
      hi |= e2m1_code(__fdiv_rn(x[8 + i], s)) << (4 * i);
    }
  }
  *reinterpret_cast<u32x2*>(codes) = u32x2{lo, hi};
  *scale = (uint8_t)sc;
}

__global__ __launch_bounds__(256) void append_fp4_kernel(AppendParams p) {
  __shared__ int s_n;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) s_n = p.seq_lens[b];
  __syncthreads();
  const int n = s_n;
  if (n < 0 || n >= p.L_max) {
    if (threadIdx.x == 0 && p.flag) atomicOr(p.flag, 1);
    return;
  }
  const int nb = p.d / 16;                 // blocks per row
  const int per = p.n_kv * nb;
  for (int e = threadIdx.x; e < 2 * per; e += blockDim.x) {
    const int t = e / per, rem = e - t * per;
    const int jj = rem / nb, blk = rem - jj * nb;
    const size_t unit = (size_t)b * p.n_kv + jj;
    const size_t slot = unit * p.L_max + n;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(t ? p.v_new : p.k_new) +
                          unit * p.d + blk * 16;
    uint8_t* codes = reinterpret_cast<uint8_t*>(t ? p.v_cache : p.k_cache) + slot * (p.d / 2) + blk * 8;
    uint8_t* scale = reinterpret_cast<uint8_t*>(t ? p.v_scales : p.k_scales) + slot * nb + blk;
    quant_block_fp4(src, codes, scale);
  }
  __syncthreads();
  if (threadIdx.x == 0) p.seq_lens[b] = n + 1;
}

hipError_t launch_append_fp4(const AppendParams& p, hipStream_t s) {
  hipLaunchKernelGGL(append_fp4_kernel, dim3(p.B), dim3(256), 0, s, p);
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
