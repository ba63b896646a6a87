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

// Combine each lane's value with that of lane ^ 32 (v_permlane32_swap on
// gfx950 exchanges the two 32-lane halves without a trip through LDS; the
// two returned registers hold each half's value for every lane pair).
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// Per-token symmetric int8 code of x under row scale s (s = max|x| / 127),
// fp32 with IEEE division and round-half-to-even; a zero row codes to 0.
__device__ __forceinline__ int quant_code(float x, float s) {
  if (s == 0.0f) return 0;
  float q = __builtin_rintf(x / s);
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return int(q);
}

// Eight contiguous values from a 16-byte aligned address, as fp32.
__device__ __forceinline__ void load8_f32(const bf16_t* x, float* v) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(x);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8_f32(const float* x, float* v) {
  const float4 a = reinterpret_cast<const float4*>(x)[0];
  const float4 b = reinterpret_cast<const float4*>(x)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// One full wave quantizes a row of `dim` values (dim even) into its MSB and
// LSB nibble planes (byte p: element 2p in the low nibble, 2p+1 in the high
// one) and its scale. Rows of up to 2048 values in 8-value groups are held
// in registers, so every load is issued before the first use.
// The row's dim/2 plane bytes go out in segments of seg bytes, segment i
// at byte i * seg_stride of mrow / lrow (seg = dim/2: one contiguous row;
// seg = head_dim/2 with seg_stride = one head's slab: head-major planes).
template <typename T>
__device__ __forceinline__ void quantize_row_wave(const T* x, int dim, uint8_t* mrow,
                                                  uint8_t* lrow, float* scale, int seg,
                                                  int64_t seg_stride) {
  const int lane = threadIdx.x & 63;
  const int nch = dim >> 3;
  const bool grouped = (dim & 7) == 0 && nch <= 4 * 64 && (seg & 3) == 0 &&
                       (seg_stride & 3) == 0 &&
                       (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(mrow) & 3) == 0 &&
                       (reinterpret_cast<uintptr_t>(lrow) & 3) == 0;
  auto at = [&](int p) { return int64_t(p / seg) * seg_stride + p % seg; };
  if (grouped) {
    float v[4][8];
    float amax = 0.0f;
    // every lane loads all four groups (past the row: its last group again,
    // then zeroed), with no branch between the loads, so the four requests
    // are in flight together
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = lane + 64 * i;
      load8_f32(x + 8 * (ch < nch ? ch : nch - 1), v[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = lane + 64 * i < nch;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[i][e] = in ? v[i][e] : 0.0f;
        amax = fmaxf(amax, fabsf(v[i][e]));
      }
    }
    amax = wave_max(amax);
    const float s = amax / 127.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = lane + 64 * i;
      if (ch < nch) {
        uint32_t mw = 0, lw = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int qc = quant_code(v[i][e], s);
          mw |= uint32_t((qc >> 4) & 15) << (4 * e);
          lw |= uint32_t(qc & 15) << (4 * e);
        }
        *reinterpret_cast<uint32_t*>(mrow + at(4 * ch)) = mw;
        *reinterpret_cast<uint32_t*>(lrow + at(4 * ch)) = lw;
      }
    }
    if (lane == 0) *scale = s;
    return;
  }
  const int half = dim >> 1;
  float amax = 0.0f;
  for (int p = lane; p < half; p += 64) {
    amax = fmaxf(amax, fabsf(load_elem<T>(x, 2 * p)));
    amax = fmaxf(amax, fabsf(load_elem<T>(x, 2 * p + 1)));
  }
  amax = wave_max(amax);
  const float s = amax / 127.0f;
  for (int p = lane; p < half; p += 64) {
    const int q0 = quant_code(load_elem<T>(x, 2 * p), s);
    const int q1 = quant_code(load_elem<T>(x, 2 * p + 1), s);
    mrow[at(p)] = uint8_t(((q0 >> 4) & 15) | (((q1 >> 4) & 15) << 4));
    lrow[at(p)] = uint8_t((q0 & 15) | ((q1 & 15) << 4));
  }
  if (lane == 0) *scale = s;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace spatten

#define SPATTEN_LAUNCH_CHECK()                                   \
  do {                                                           \
    if (hipGetLastError() != hipSuccess) return SPATTEN_EHIP;    \
  } while (0)
