// device_common.h -- small device helpers shared by the gfx950 scan kernels:
// bf16 packing, the ReLU feature map on packed bf16, hi/lo splitting of fp32
// values into two bf16 terms, and the MFMA operand types.
//
// MFMA conventions used throughout (wave64, gfx950):
//   v_mfma_f32_32x32x16_bf16  A: lane l holds row (l & 31), 8 k-slots of group (l >> 5)
//                             B: lane l holds col (l & 31), the same 8 k-slots
//                             C: lane l, reg r holds C[8*(r>>2) + 4*(l>>5) + (r&3)][l & 31]
//   v_mfma_f32_16x16x4_f32    A: lane l holds A[l & 15][l >> 4]
//                             B: lane l holds B[l >> 4][l & 15]
//                             C: lane l, reg r holds C[4*(l>>4) + r][l & 15]
// Only the C layouts matter for correctness of a contraction: A and B share
// their k-slot assignment, so any consistent placement of the contracted index
// (tokens or dimensions) into the slots sums over all of it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linscan {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN of the same sign.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ReLU on two packed bf16 values: a value whose sign bit is set becomes +0.
// As 16-bit integers, exactly those values are negative, so a signed max
// with zero implements it (v_pk_max_i16).
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t w) {
  shortx2 s = __builtin_bit_cast(shortx2, w);
  shortx2 zero = {0, 0};
  s = __builtin_elementwise_max(s, zero);
  return __builtin_bit_cast(uint32_t, s);
}
__device__ __forceinline__ float relu_f32(float x) { return signbit(x) ? 0.0f : x; }

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi): 16 significant bits.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

__device__ __forceinline__ floatx16 mfma32x32x16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16x16x4f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16-byte global load / store through 32-bit words.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Token-tensor element types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {  // bf16 bits
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16(x); }
};

}  // namespace linscan
