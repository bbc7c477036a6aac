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

// gfx950 transposed LDS read (ds_read_b64_tr_b16).  In each group of 16 lanes,
// lane i receives element i%4 of the 8-byte pieces read by lanes 4r + i/4,
// r = 0..3, as its elements r.  So if lane 4r + c of group g reads the 4
// columns m0+4c .. m0+4c+3 of row k0 + 8g + 4h + r of a k-major bf16 matrix,
// lane i of group g receives column m0 + i at rows k0 + 8g + 4h + 0..3: half
// (h) of the 16x32 MFMA operand fragment with m = i.  Two reads (h = 0, 1)
// give the whole fragment.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr(const void *lds, uint32_t byte_off) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(reinterpret_cast<const char *>(lds) + byte_off));
  return __builtin_bit_cast(u32x2, v);
}

// Row swizzle of 16-byte chunks for row-major bf16 tiles of 256-byte rows in
// LDS that are read both as plain 16-byte operand rows (16 rows of a 32-key
// pair, see pair_key) and with lds_read_tr (rows k0 + 8g + 4h + r): row bits
// 0, 1, 3 go to chunk bits 1, 2, 3.  Chunk bit 0 stays: candidate swizzles
// measured with the bank-conflict counter on gfx950 show that XOR-ing it
// costs extra cycles on 16-byte reads, and this map is conflict-free for both
// access patterns.  For the transposed reads it depends on g and r only.
__device__ __forceinline__ uint32_t fkv(uint32_t row) {
  return ((row & 1u) << 1) | (((row >> 1) & 1u) << 2) | (((row >> 3) & 1u) << 3);
}
// Per-lane constants of a transposed fragment read (lane l = 16g + 4r + c):
// byte offset of its row and 8-byte half, and the XOR applied to the tile's
// chunk index.
// Chunk swizzle for tiles read as 16 consecutive rows at one 16-byte chunk
// (plain reads): row bits 0..2 go to chunk bits 1..3 (conflict-free by the
// same measurement as fkv).
__device__ __forceinline__ uint32_t fst(uint32_t row) { return (row & 7u) << 1; }
__device__ __forceinline__ uint32_t tr_lane_off(int l, int rowb) {
  return (8 * (l >> 4) + ((l & 15) >> 2)) * rowb + (l & 1) * 8;
}
__device__ __forceinline__ uint32_t tr_lane_xor(int l) {
  return (((l & 3) >> 1) ^ fkv(8 * (l >> 4) + ((l & 15) >> 2)));
}
// 16x32 operand fragment (m = 16 columns of tile `tile`, k = 32 rows from the
// row whose byte offset is base_k0) of a k-major, fkv-swizzled LDS matrix with
// nch 16-byte chunks per row.
__device__ __forceinline__ u32x4 tr_frag(const void *lds, uint32_t base_k0, uint32_t lane_off, uint32_t lane_xor,
                                         int tile, int nch, int rowb) {
  const uint32_t off = base_k0 + lane_off + (((uint32_t)(2 * tile) ^ lane_xor) & (uint32_t)(nch - 1)) * 16u;
  const u32x2 a = lds_read_tr(lds, off), b = lds_read_tr(lds, off + 4 * rowb);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// Key permutation inside a 32-key pair of 16-key tiles: MFMA row r of tile t
// (t = 0, 1) holds key 8*(r/4) + 4*t + r%4, so that after K Q^T each lane's
// 4+4 accumulator rows of the two tiles are 8 consecutive keys -- exactly the
// k slots of the B operand of a following V^T P^T product.  Both tiles of a
// pair therefore hold keys from the whole 32-key range.
__device__ __forceinline__ int pair_key(int t, int r) { return ((r >> 2) << 3) + (t << 2) + (r & 3); }

// ---------------------------------------------------------------- global access
__device__ __forceinline__ u32x4 gload16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void gstore16(void *p, const u32x4 &v) { *reinterpret_cast<u32x4 *>(p) = v; }

// Buffer loads: a resource over [p, p + bytes) (bytes < 2^31) held in SGPRs
// and a 32-bit byte offset per lane, so per-lane addresses cost one VGPR
// instead of two; loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// 16 bytes per lane from buffer offset off straight into LDS: lane l's bytes
// land at lds + 16 l (lds wave-uniform).
__device__ __forceinline__ void bload16_lds(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3))) *)lds, 16, off, 0, 0, 0);
}

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

// Sum over aligned groups of G consecutive lanes (G = 4 or 8), every lane of
// a group receiving the group's sum: DPP quad permutations [1,0,3,2] and
// [2,3,0,1], then (G = 8) the half-row mirror, which pairs each lane with one
// of the other quad.
template <int G>
__device__ __forceinline__ float lane_group_sum(float x) {
  static_assert(G == 4 || G == 8, "group of 4 or 8 lanes");
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  if constexpr (G == 8) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  return x;
}

// Max / sum over the four 16-lane rows of a wave, at each position within a
// row, every lane receiving the result: v_permlane16_swap pairs rows 0-1 and
// 2-3, v_permlane32_swap the two halves (VALU lane exchanges, no LDS round
// trip).  With both operands the same register each swap returns the pair's
// two rows, so combining its two results reduces over the pair.
__device__ __forceinline__ float row4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// acc + lo + hi of a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float dot2_bf16_ones(uint32_t pair, float acc) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pair), __builtin_bit_cast(bf16x2v, 0x3F803F80u),
                                         acc, false);
}

// 1 / (1 + e^-x) with the hardware exp2 and reciprocal (about 1 ulp each).
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// Order-preserving map fp32 -> uint32 (larger float => larger key); -0 maps as +0.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace sala
