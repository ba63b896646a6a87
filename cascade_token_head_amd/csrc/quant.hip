// Per-token symmetric int8 quantization of K/V rows, split into
// separately fetchable 4-bit MSB and LSB planes (SpAtten, section III
// "Progressive Quantization"; IV "Quantization Support": the bitwidth
// converter splits fetched bits and joins MSBs with LSBs).
//
// One wave per row. Arithmetic is fp32 with IEEE division and
// round-half-to-even, so codes are reproducible bit for bit:
//   s = max|x| / 127, q = clamp(rint(x / s), -127, 127), msb = q >> 4,
//   lsb = q & 15; byte j of a plane holds element 2j (low nibble) and
//   element 2j+1 (high nibble).
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace spatten {
namespace {

__device__ __forceinline__ int quant_code(float x, float s) {
  if (s == 0.0f) return 0;
  float q = __builtin_rintf(x / s);
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return int(q);
}

template <typename T>
__global__ void __launch_bounds__(256)
quantize_kernel(const T* __restrict__ kv, int batch, int n, int dim, int64_t kv_bs,
                uint8_t* __restrict__ msb, uint8_t* __restrict__ lsb, float* __restrict__ scale,
                int64_t pbs) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= int64_t(batch) * n) return;
  const int64_t b = row / n, r = row - b * n;
  const T* x = kv + b * kv_bs + r * dim;
  const int half = dim >> 1;
  float amax = 0.0f;
  for (int p = lane; p < half; p += 64) {
    amax = fmaxf(amax, fabsf(load_elem<T>(x, 2 * p)));
    amax = fmaxf(amax, fabsf(load_elem<T>(x, 2 * p + 1)));
  }
  amax = wave_max(amax);
  const float s = amax / 127.0f;
  uint8_t* mrow = msb + (b * pbs + r) * half;
  uint8_t* lrow = lsb + (b * pbs + r) * half;
  for (int p = lane; p < half; p += 64) {
    const int q0 = quant_code(load_elem<T>(x, 2 * p), s);
    const int q1 = quant_code(load_elem<T>(x, 2 * p + 1), s);
    mrow[p] = uint8_t(((q0 >> 4) & 15) | (((q1 >> 4) & 15) << 4));
    lrow[p] = uint8_t((q0 & 15) | ((q1 & 15) << 4));
  }
  if (lane == 0) scale[b * pbs + r] = s;
}

}  // namespace

int launch_quantize(const void* kv, int dtype, int batch, int n, int dim, int64_t kv_bs,
                    uint8_t* msb, uint8_t* lsb, float* scale, int64_t pbs, hipStream_t stream) {
  const int64_t rows = int64_t(batch) * n;
  if (rows == 0) return SPATTEN_OK;
  const unsigned blocks = unsigned(ceil_div(rows, 4));
  if (dtype == SPATTEN_BF16)
    SPATTEN_TIMED("quantize", stream,
                  quantize_kernel<bf16_t><<<blocks, 256, 0, stream>>>(
                      static_cast<const bf16_t*>(kv), batch, n, dim, kv_bs, msb, lsb, scale, pbs));
  else
    SPATTEN_TIMED("quantize", stream,
                  quantize_kernel<float><<<blocks, 256, 0, stream>>>(
                      static_cast<const float*>(kv), batch, n, dim, kv_bs, msb, lsb, scale, pbs));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

}  // namespace spatten
