// Per-token symmetric int8 quantization of K/V rows, split into
// separately fetchable 4-bit MSB and LSB planes (SpAtten, "A. Cascade
// Token Pruning", bullet "Progressive Quantization"; section IV, bullet
// "Quantization Support": the bitwidth
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

// Planes token-major (head_dim 0: row r of sequence b at (b*pbs + r) rows
// of dim/2 bytes) or head-major (head h's slab of pbs rows of head_dim/2
// bytes at slab b*H + h, so one head's rows are contiguous).
template <typename T>
__global__ void __launch_bounds__(256)
quantize_kernel(const T* __restrict__ kv, int batch, int n, int dim, int head_dim,
                int64_t kv_bs, uint8_t* __restrict__ msb, uint8_t* __restrict__ lsb,
                float* __restrict__ scale, int64_t pbs) {
  const int64_t row = int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= int64_t(batch) * n) return;
  const int64_t b = row / n, r = row - b * n;
  const int half = dim >> 1;
  int64_t off;
  int seg;
  int64_t seg_stride;
  if (head_dim > 0) {
    seg = head_dim >> 1;
    seg_stride = pbs * seg;
    off = (b * (dim / head_dim) * pbs + r) * seg;
  } else {
    seg = half;
    seg_stride = 0;
    off = (b * pbs + r) * half;
  }
  quantize_row_wave<T>(kv + b * kv_bs + r * dim, dim, msb + off, lsb + off, scale + b * pbs + r,
                       seg, seg_stride);
}

}  // namespace

int launch_quantize(const void* kv, int dtype, int batch, int n, int dim, int head_dim,
                    int64_t kv_bs, uint8_t* msb, uint8_t* lsb, float* scale, int64_t pbs,
                    hipStream_t stream) {
  const int64_t rows = int64_t(batch) * n;
  if (rows == 0) return SPATTEN_OK;
  const unsigned blocks = unsigned(ceil_div(rows, 4));
  if (dtype == SPATTEN_BF16)
    SPATTEN_TIMED("quantize", stream,
                  quantize_kernel<bf16_t><<<blocks, 256, 0, stream>>>(
                      static_cast<const bf16_t*>(kv), batch, n, dim, head_dim, kv_bs, msb, lsb,
                      scale, pbs));
  else
    SPATTEN_TIMED("quantize", stream,
                  quantize_kernel<float><<<blocks, 256, 0, stream>>>(
                      static_cast<const float*>(kv), batch, n, dim, head_dim, kv_bs, msb, lsb,
                      scale, pbs));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

}  // namespace spatten
