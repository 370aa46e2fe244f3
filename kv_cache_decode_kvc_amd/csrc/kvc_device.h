// Device helpers for gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Buffer resource word 3 for gfx9-family raw buffers: 32-bit data format,
// no swizzle.  Accesses at offsets >= num_records return zero, which is how
// the kernels keep reads inside one sequence's valid rows.
constexpr int kBufWord3 = 0x00020000;
constexpr uint32_t kOobOffset = 0x80000000u;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                   uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, kBufWord3);
}

__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Cache policy for data read exactly once per step (the K/V rows): the
// non-temporal hint streams it past the caches; measured on MI355X it
// sustains 6.7-7.1 TB/s against about 6.0 TB/s for default-policy loads.
constexpr int kStream = 2;

__device__ inline u32x4 buf_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStream));
}

__device__ inline u32x2 buf_load8_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2,
                            __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kStream));
}

__device__ inline bf16x8 as_bf16x8(u32x4 x) {
  return __builtin_bit_cast(bf16x8, x);
}

// float -> bf16 round to nearest even (hardware conversion on gfx950).
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ inline f16x8 as_f16x8(u32x4 x) { return __builtin_bit_cast(f16x8, x); }

// Eight E2M1 codes (byte i holds channels 2i (low nibble) and 2i + 1) times
// the block scale s (an E4M3 value, here as f16), as eight f16.  Exact: the
// conversion (scale operand 1.0) gives the code values 0 .. 6, E4M3 values
// are f16 numbers, and their product has at most 6 significant bits and
// lies in 2^-10 .. 2688 (f16 normal numbers hold 11 bits from 2^-14 to
// 65504).  One conversion and one packed f16 multiply per two numbers.
// (m: the multipliers of the low and the high code of each byte)
__device__ inline u32x4 fp4x8_to_f16x8(uint32_t w, f16x2 m) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * m);
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * m);
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * m);
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * m);
  return r;
}
__device__ inline u32x4 fp4x8_to_f16x8(uint32_t w, _Float16 s) {
  return fp4x8_to_f16x8(w, f16x2{s, s});
}

// Two E4M3 codes (bits 0-7 and 8-15 of w) as two f16, exactly.
__device__ inline f16x2 e4m3x2_to_f16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

__device__ inline uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ inline float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(uint32_t u) {
  return __uint_as_float(u & 0xFFFF0000u);
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Device-scope coherent buffer accesses (cache policy SC1): a store is
// written through to the point of coherence that all XCDs share, and a load
// misses in the per-XCD caches.  Workgroups exchange split results this way,
// so no L2 writeback or invalidate is needed (a device-scope fence would
// write back and invalidate the whole L2 of the XCD).
constexpr int kCoherent = 16;
constexpr int kWsRecords = 0x7FFFFFF0;   // offsets are checked on the host

__device__ inline void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCoherent);
}
__device__ inline void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, kCoherent);
}
__device__ inline f32x4 load_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
}
__device__ inline float load_coherent1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCoherent));
}

// Wait until every vector memory access this wave issued has completed
// (s_waitcnt vmcnt(0)); the empty asm keeps the compiler from moving memory
// accesses across it.
__device__ inline void wait_vm_all() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kFp8Max = 448.0f;   // largest finite E4M3 value

// Eight E4M3 codes (bytes 0..7 of x) -> eight bf16 in the same order.  Every
// E4M3 value is exact in bf16; the conversion's scale is 1.
__device__ inline u32x4 fp8x8_to_bf16x8(u32x2 x) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, true));
  return r;
}
constexpr float kLn2 = 0.693147180559945309f;

// exp2 of (x - m) where m may be -inf (then every x is -inf too): 0.
__device__ inline float exp2_rel(float x, float m_use) {
  return __builtin_amdgcn_exp2f(x - m_use);
}

}  // namespace kvc
