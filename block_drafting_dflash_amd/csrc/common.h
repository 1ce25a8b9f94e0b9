// Device-side helpers shared by the DFlash kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;


// ---- bf16 <-> f32 (bf16 stored as raw 16-bit words) -----------------------------------
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// nearest bf16, ties to even; NaN stays NaN, overflow rounds to inf (gfx950 converts in
// hardware, v_cvt_pk_bf16_f32, two values per instruction)
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// activation load/store in either f32 or bf16 storage
template <bool BF16> __device__ __forceinline__ float act_ld(const void* p, int64_t i) {
  if constexpr (BF16) return bf2f(((const uint16_t*)p)[i]);
  else return ((const float*)p)[i];
}
template <bool BF16> __device__ __forceinline__ void act_st(void* p, int64_t i, float v) {
  if constexpr (BF16) ((uint16_t*)p)[i] = f2bf(v);
  else ((float*)p)[i] = v;
}

// ---- f32 operands for bf16 MFMA ---------------------------------------------------------
// An f32 value v travels as the bf16 pair hi = bf16(v), lo = bf16(v - hi): v - hi is exact
// in f32, so hi + lo carries about 16 significant bits (relative error <= 2^-17) and a
// product with a bf16 weight costs two exact MFMA products instead of one rounded operand.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = f2bf(v);
  lo = f2bf(v - bf2f(hi));
}
// the same for two values at once: packed hi pair and packed lo pair (a in the low halves)
__device__ __forceinline__ void split2_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = f2bf2(a, b);
  lo = f2bf2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}
// Store of an activation operand: two bf16 planes (SPLIT) or f32.
template <bool SPLIT> __device__ __forceinline__ void op_st(void* hi, void* lo, int64_t i, float v) {
  if constexpr (SPLIT) {
    uint16_t h, l;
    split_bf16(v, h, l);
    ((uint16_t*)hi)[i] = h;
    ((uint16_t*)lo)[i] = l;
  } else {
    ((float*)hi)[i] = v;
  }
}

// ---- MFMA (A = activations [16 rows x k], B = weights [k x 16 cols]) ---------------------
// 16x16x32 bf16: lane l supplies A[l%16][8*(l/16)+j] and B[8*(l/16)+j][l%16], j = 0..7;
// result element q of lane l is D[4*(l/16)+q][l%16]. Products are exact, sums in f32.
__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// 16x16x4 f32: lane l supplies A[l%16][l/16] and B[l/16][l%16]; same result layout.
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- wave reductions --------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum over each 16-lane row of the wave (DPP, no LDS): quad xor 1, quad xor 2, then the
// two quads of each half-row (mirror) and the two halves (rotate by 8). Every lane of a row
// ends with the same bits: each step adds two values that all lanes of a group share.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x128>(v);  // row_ror 8
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int o) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, o, 64);
  hi = __shfl_xor(hi, o, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// (value, index) key whose unsigned order is: larger value first, then lower index.
__device__ __forceinline__ unsigned long long argmax_key(float v, int32_t idx) {
  uint32_t u = (v == 0.0f) ? 0u : __float_as_uint(v);  // +0 and -0 compare equal
  uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (uint32_t)(~(uint32_t)idx);
}
__device__ __forceinline__ int32_t argmax_key_index(unsigned long long key) {
  return (int32_t)(~(uint32_t)(key & 0xffffffffull));
}
