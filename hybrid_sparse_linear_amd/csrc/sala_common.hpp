// Device-side helpers shared by the libsala HIP kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sala {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two fp32 -> one dword of two bf16 (round to nearest even, hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r.x = (__bf16)lo;
  r.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu);
}

// ---------------------------------------------------------------- MFMA
// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l holds A[row l%16][k = 8*(l/16) .. +7], B[k = 8*(l/16) .. +7][col l%16],
// and D[row 4*(l/16) + i][col l%16] in element i (i = 0..3).  Only the
// pairing of A's and B's k slots matters for the product, so any fixed
// permutation of k applied to both operands gives the same result.
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- LDS access
template <typename T>
__device__ __forceinline__ T lds_load(const void *base, uint32_t byte_off) {
  return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + byte_off);
}
template <typename T>
__device__ __forceinline__ void lds_store(void *base, uint32_t byte_off, const T &v) {
  *reinterpret_cast<T *>(reinterpret_cast<char *>(base) + byte_off) = v;
}

// ---------------------------------------------------------------- global access
__device__ __forceinline__ u32x4 gload16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void gstore16(void *p, const u32x4 &v) { *reinterpret_cast<u32x4 *>(p) = v; }

// ---------------------------------------------------------------- wave reductions (wave64)
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Order-preserving map fp32 -> uint32 (larger float => larger key); -0 maps as +0.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace sala
