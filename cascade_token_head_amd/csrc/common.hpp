// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "layout.hpp"

namespace spatten {

using bf16_t = uint16_t;

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 <-> fp32. bf16 is the top half of an fp32 bit pattern; the rounding
// to bf16 is to nearest, ties to even, with NaN kept quiet.
__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(uint32_t(v) << 16);
}

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// gfx950 converts pairs with v_cvt_pk_bf16_f32 (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return bf16_t(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// Loads/stores of T-typed element e of an untyped tensor.
template <typename T>
__device__ __forceinline__ float load_elem(const void* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float load_elem<bf16_t>(const void* p, int64_t i) {
  return bf16_to_f32(static_cast<const bf16_t*>(p)[i]);
}

template <typename T>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_elem<float>(void* p, int64_t i, float v) {
  static_cast<float*>(p)[i] = v;
}
template <>
__device__ __forceinline__ void store_elem<bf16_t>(void* p, int64_t i, float v) {
  static_cast<bf16_t*>(p)[i] = f32_to_bf16(v);
}

// 2^x with the hardware v_exp_f32 (about 1 ulp; results below 2^-126 flush
// to zero, exp2(-inf) = 0), without the library's subnormal range handling.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-wide reductions (64 lanes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// MFMA 32x32x16 bf16 -> fp32 (gfx950). Operand lane layout:
//   A: lane l holds A[row l%32][k 8*(l/32) .. +8]
//   B: lane l holds B[k 8*(l/32) .. +8][col l%32]
//   C: lane l, register r holds C[row 8*(r/4) + 4*(l/32) + r%4][col l%32]
__device__ __forceinline__ floatx16 mfma32x32x16(const bf16x8& a, const bf16x8& b,
                                                  const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// MFMA 16x16x32 bf16 -> fp32 (gfx950).
//   A: lane l holds A[row l%16][k 8*(l/16) .. +8]
//   B: lane l holds B[k 8*(l/16) .. +8][col l%16]
//   C: lane l, register r holds C[row 4*(l/16) + r][col l%16]
__device__ __forceinline__ floatx4 mfma16x16x32(const bf16x8& a, const bf16x8& b,
                                                 const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace spatten

#define SPATTEN_LAUNCH_CHECK()                                   \
  do {                                                           \
    if (hipGetLastError() != hipSuccess) return SPATTEN_EHIP;    \
  } while (0)
