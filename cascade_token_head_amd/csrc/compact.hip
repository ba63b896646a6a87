// Multi-tensor row gather: pruned tokens leave x, their importance scores,
// positions and (for decode) every layer's K/V cache rows in one launch
// (SpAtten, "A. Cascade Token Pruning": a pruned token's Q, K and V are
// gone from every later head and layer).
//
// The pages route pruning's random row addresses through an on-chip
// crossbar; here each destination row is a contiguous copy, split into
// 16-byte units when the addresses allow, so consecutive lanes touch
// consecutive bytes of the same row and HBM access stays coalesced.
//
// In-place form (decode caches, whose row order carries no meaning): of the
// k selected rows, those already below k stay; the i-th selected row at or
// above k moves into the i-th unselected row below k. A cut that drops one
// entry from k + 1 moves at most one row per tensor instead of all k.
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace spatten {
namespace {

struct CompactTensor {
  const char* src;
  char* dst;
  int64_t row_bytes, sbs, dbs;
  int32_t vec_shift;
};

constexpr int kCompactMax = 48;

struct CompactParams {
  CompactTensor t[kCompactMax];
};

template <int V>
struct VecT;
template <> struct VecT<16> { using T = u32x4; };
template <> struct VecT<8> { using T = uint64_t; };
template <> struct VecT<4> { using T = uint32_t; };
template <> struct VecT<2> { using T = uint16_t; };
template <> struct VecT<1> { using T = uint8_t; };

// Unit u of the tensor's batch * k rows: row u / upr, sequence row / k.
// I is the index type: 32-bit unsigned when every unit index of the launch
// fits (its divisions are a few instructions), 64-bit otherwise.
template <int V, typename I>
__device__ __forceinline__ void copy_units(const CompactTensor& t, const int32_t* __restrict__ idx,
                                           int k, int64_t total, int64_t start, int64_t step) {
  using T = typename VecT<V>::T;
  const I upr = I(t.row_bytes / V), kk = I(k);
  for (int64_t u64 = start; u64 < total; u64 += step) {
    const I u = I(u64);
    const I row = u / upr, part = u - row * upr;
    const I b = row / kk, r = row - b * kk;
    const int64_t sr = idx[int64_t(row)];
    const T* s = reinterpret_cast<const T*>(t.src + int64_t(b) * t.sbs + sr * t.row_bytes) + part;
    T* d = reinterpret_cast<T*>(t.dst + int64_t(b) * t.dbs + int64_t(r) * t.row_bytes) + part;
    *d = *s;
  }
}

template <typename I>
__global__ void __launch_bounds__(256)
compact_kernel(CompactParams p, const int32_t* __restrict__ idx, int batch, int k) {
  const CompactTensor& t = p.t[blockIdx.y];
  const int64_t total = int64_t(batch) * k * (t.row_bytes >> t.vec_shift);
  const int64_t start = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t step = int64_t(gridDim.x) * blockDim.x;
  switch (t.vec_shift) {
    case 4: copy_units<16, I>(t, idx, k, total, start, step); break;
    case 3: copy_units<8, I>(t, idx, k, total, start, step); break;
    case 2: copy_units<4, I>(t, idx, k, total, start, step); break;
    case 1: copy_units<2, I>(t, idx, k, total, start, step); break;
    default: copy_units<1, I>(t, idx, k, total, start, step); break;
  }
}

int vec_shift_for(const void* s, const void* d, int64_t rb, int64_t sbs, int64_t dbs) {
  const uint64_t all = uint64_t(reinterpret_cast<uintptr_t>(s)) |
                       uint64_t(reinterpret_cast<uintptr_t>(d)) | uint64_t(rb) |
                       uint64_t(sbs) | uint64_t(dbs);
  for (int sh = 4; sh > 0; --sh)
    if ((all & ((uint64_t(1) << sh) - 1)) == 0) return sh;
  return 0;
}

// moves per workgroup of the in-place form
constexpr int kMovesPerBlock = 16;

struct InplaceTensor {
  char* base;
  int64_t row_bytes, pitch, bs;
  int32_t vec_shift;
};

struct InplaceParams {
  InplaceTensor t[kCompactMax];
};

template <int V>
__device__ __forceinline__ void move_units(const InplaceTensor& t, char* bbase, const int* src,
                                           const int* dst, int nmoves) {
  using T = typename VecT<V>::T;
  constexpr int U = 8;  // loads in flight per thread before their stores
  const int upr = int(t.row_bytes / V);
  const int total = nmoves * upr;
  for (int u0 = threadIdx.x; u0 < total; u0 += U * blockDim.x) {
    T buf[U];
#pragma unroll
    for (int w = 0; w < U; ++w) {
      const int u = u0 + w * blockDim.x;
      if (u < total) {
        const int m = u / upr, part = u - m * upr;
        buf[w] = reinterpret_cast<const T*>(bbase + int64_t(src[m]) * t.pitch)[part];
      }
    }
    // sources sit at or above k, destinations below it: no overlap
#pragma unroll
    for (int w = 0; w < U; ++w) {
      const int u = u0 + w * blockDim.x;
      if (u < total) {
        const int m = u / upr, part = u - m * upr;
        reinterpret_cast<T*>(bbase + int64_t(dst[m]) * t.pitch)[part] = buf[w];
      }
    }
  }
}

// grid (ceil(max moves / kMovesPerBlock), batch, tensors): each workgroup
// moves its share of one tensor's rows of one sequence. Sequence b's
// selection idx[b, 0:k] is ascending and staged in LDS (k ints); c = number
// of selected rows below k, and the k - c selected rows at or above k are
// idx[c..k-1]. With d_j = idx[j] - j (non-decreasing for j < c), the i-th
// unselected row below k is i + #{j < c : d_j <= i}.
__global__ void __launch_bounds__(128)
compact_inplace_kernel(InplaceParams p, const int32_t* __restrict__ idx, int k) {
  extern __shared__ int sel[];
  __shared__ int src[kMovesPerBlock], dst[kMovesPerBlock];
  __shared__ int nbelow;
  const int b = blockIdx.y;
  const int32_t* ib = idx + int64_t(b) * k;
  for (int j = threadIdx.x; j < k; j += blockDim.x) sel[j] = ib[j];
  __syncthreads();
  if (threadIdx.x == 0) {
    int lo = 0, hi = k;  // first j with idx[j] >= k
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sel[mid] < k) lo = mid + 1; else hi = mid;
    }
    nbelow = lo;
  }
  __syncthreads();
  const int c = nbelow, moves = k - c;
  const int m0 = blockIdx.x * kMovesPerBlock;
  if (m0 >= moves) return;
  const int nm = moves - m0 < kMovesPerBlock ? moves - m0 : kMovesPerBlock;
  if (threadIdx.x < nm) {
    const int i = m0 + threadIdx.x;
    int lo = 0, hi = c;  // first j in [0, c) with idx[j] - j > i
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sel[mid] - mid <= i) lo = mid + 1; else hi = mid;
    }
    dst[threadIdx.x] = i + lo;
    src[threadIdx.x] = sel[c + i];
  }
  __syncthreads();
  const InplaceTensor& t = p.t[blockIdx.z];
  char* bbase = t.base + int64_t(b) * t.bs;
  switch (t.vec_shift) {
    case 4: move_units<16>(t, bbase, src, dst, nm); break;
    case 3: move_units<8>(t, bbase, src, dst, nm); break;
    case 2: move_units<4>(t, bbase, src, dst, nm); break;
    case 1: move_units<2>(t, bbase, src, dst, nm); break;
    default: move_units<1>(t, bbase, src, dst, nm); break;
  }
}

}  // namespace

int launch_compact_inplace(int n_tensors, void* const* base, const int64_t* row_bytes,
                           const int64_t* row_pitch, const int64_t* bs, const int32_t* idx,
                           int batch, int n, int k, hipStream_t stream) {
  if (n_tensors == 0 || batch == 0 || k == n) return SPATTEN_OK;
  const int max_moves = k < n - k ? k : n - k;
  const unsigned blocks = unsigned(ceil_div(max_moves, kMovesPerBlock));
  for (int t0 = 0; t0 < n_tensors; t0 += kCompactMax) {
    InplaceParams p{};
    const int cnt = n_tensors - t0 < kCompactMax ? n_tensors - t0 : kCompactMax;
    for (int i = 0; i < cnt; ++i) {
      const int t = t0 + i;
      p.t[i].base = static_cast<char*>(base[t]);
      p.t[i].row_bytes = row_bytes[t];
      p.t[i].pitch = row_pitch ? row_pitch[t] : row_bytes[t];
      p.t[i].bs = bs[t];
      p.t[i].vec_shift = vec_shift_for(base[t], base[t], row_bytes[t], p.t[i].pitch, bs[t]);
    }
    SPATTEN_TIMED("compact_inplace", stream,
                  compact_inplace_kernel<<<dim3(blocks, unsigned(batch), unsigned(cnt)),
                                           dim3(128), size_t(k) * sizeof(int), stream>>>(p, idx,
                                                                                        k));
    SPATTEN_LAUNCH_CHECK();
  }
  return SPATTEN_OK;
}

int launch_compact(int n_tensors, const void* const* src, void* const* dst,
                   const int64_t* row_bytes, const int64_t* sbs, const int64_t* dbs,
                   const int32_t* idx, int batch, int k, hipStream_t stream) {
  if (n_tensors == 0 || batch == 0 || k == 0) return SPATTEN_OK;
  for (int t0 = 0; t0 < n_tensors; t0 += kCompactMax) {
    const int cnt = n_tensors - t0 < kCompactMax ? n_tensors - t0 : kCompactMax;
    CompactParams p{};
    int64_t max_units = 0;
    for (int i = 0; i < cnt; ++i) {
      const int t = t0 + i;
      CompactTensor& c = p.t[i];
      c.src = static_cast<const char*>(src[t]);
      c.dst = static_cast<char*>(dst[t]);
      c.row_bytes = row_bytes[t];
      c.sbs = sbs[t];
      c.dbs = dbs[t];
      c.vec_shift = vec_shift_for(src[t], dst[t], row_bytes[t], sbs[t], dbs[t]);
      const int64_t units = int64_t(batch) * k * (row_bytes[t] >> c.vec_shift);
      if (units > max_units) max_units = units;
    }
    int64_t blocks = ceil_div(max_units, 256);
    if (blocks > 8192) blocks = 8192;
    // 32-bit unit indices while the largest, plus one grid stride, stay below 2^31
    if (max_units + blocks * 256 < (int64_t(1) << 31))
      SPATTEN_TIMED("compact", stream,
                    compact_kernel<uint32_t><<<dim3(unsigned(blocks), cnt), dim3(256), 0, stream>>>(
                        p, idx, batch, k));
    else
      SPATTEN_TIMED("compact", stream,
                    compact_kernel<int64_t><<<dim3(unsigned(blocks), cnt), dim3(256), 0, stream>>>(
                        p, idx, batch, k));
    SPATTEN_LAUNCH_CHECK();
  }
  return SPATTEN_OK;
}

}  // namespace spatten
