// On-the-fly top-k by radix select (SpAtten, "B. Top-k Engine": find the
// k-th largest as a threshold, filter, then eliminate the dropped entries
// while keeping input order).
//
// One workgroup per row; rows of up to 32 keys per thread are read once into
// registers. Scores map to order-preserving uint32 keys (larger
// value -> larger key; -0.0 below +0.0). Four MSD passes of 8 bits find the
// exact key T of the k-th ranked element with LDS histograms; wave ballots
// fold lanes that share a digit into one LDS atomic. A final pass in index
// order keeps every key > T plus the first (k - #above) keys == T, and
// writes each survivor at its prefix-count position, computed with wave
// ballots and a cross-wave scan - the GPU form of the order-preserving zero
// eliminator.
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace spatten {
namespace {

constexpr int kMaxWaves = 16;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u ^ 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (uint64_t(1) << lane) - 1; }

// Block-wide exclusive scan of one count per wave; returns this wave's
// offset and writes the block total to *total. Uses LDS `buf` of kMaxWaves.
__device__ __forceinline__ int wave_offsets(int wave_count, int wave, int nwaves, int lane,
                                            int* buf, int* total) {
  if (lane == 0) buf[wave] = wave_count;
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < nwaves; ++w) {
    const int c = buf[w];
    off += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off;
}

// PT > 0: the row is read once into registers (PT keys per thread, n <=
// PT * blockDim); PT == 0: every pass re-reads the row.
template <int PT>
__global__ void __launch_bounds__(1024)
topk_radix_kernel(const float* __restrict__ scores, int n, int64_t row_stride, int k,
                  int32_t* __restrict__ out_idx, float* __restrict__ kth_out) {
  __shared__ uint32_t hist[256];
  __shared__ int scan_buf[kMaxWaves];
  // per (j, wave) counts of > T and == T keys, then their exclusive prefixes
  __shared__ int pre_gt[PT > 0 ? PT * kMaxWaves : 1], pre_eq[PT > 0 ? PT * kMaxWaves : 1];
  __shared__ uint32_t sh_digit;
  __shared__ int sh_krem;

  const int b = blockIdx.x;
  const float* s = scores + int64_t(b) * row_stride;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthreads = blockDim.x, nwaves = nthreads >> 6;
  const int iters = (n + nthreads - 1) / nthreads;

  uint32_t keys[PT > 0 ? PT : 1];
  if constexpr (PT > 0) {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int i = tid + j * nthreads;
      keys[j] = i < n ? order_key(s[i]) : 0u;
    }
  }
  auto key_at = [&](int j, int i) -> uint32_t {
    if constexpr (PT > 0)
      return keys[j];
    else
      return order_key(s[i]);
  };

  uint32_t prefix = 0, mask = 0;
  int krem = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += nthreads) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < (PT > 0 ? PT : 1 << 20); ++j) {
      if (j >= iters) break;  // uniform
      const int i = tid + j * nthreads;
      bool cand = false;
      uint32_t dig = 0;
      if (i < n) {
        const uint32_t key = key_at(j, i);
        cand = (key & mask) == prefix;
        dig = (key >> shift) & 255u;
      }
      // fold lanes that share a digit: up to four digit groups per wave
      // become one atomic each, the rest add one by one
      uint64_t rem = __ballot(cand);
      for (int it = 0; it < 4 && rem; ++it) {
        const int leader = __ffsll((long long)rem) - 1;
        const uint32_t d0 = __shfl(dig, leader, 64);
        const uint64_t grp = __ballot(cand && dig == d0) & rem;
        if (lane == leader) atomicAdd(&hist[d0], uint32_t(__popcll(grp)));
        rem &= ~grp;
      }
      if ((rem >> lane) & 1) atomicAdd(&hist[dig], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 255-4l .. 252-4l (descending digit order)
      uint32_t c[4], tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * lane - j];
        tot += c[j];
      }
      uint32_t incl = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      const uint64_t hit = __ballot(incl >= uint32_t(krem));
      const int first = __ffsll((long long)hit) - 1;
      if (lane == first) {
        uint32_t cum = incl - tot;
        for (int j = 0; j < 4; ++j) {
          if (cum + c[j] >= uint32_t(krem)) {
            sh_digit = uint32_t(255 - 4 * lane - j);
            sh_krem = krem - int(cum);
            break;
          }
          cum += c[j];
        }
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    krem = sh_krem;
    __syncthreads();
  }
  const uint32_t T = prefix;  // key of the k-th ranked element
  if (tid == 0 && kth_out) kth_out[b] = key_value(T);

  // ordered selection: key > T, or key == T among the first krem ties
  int32_t* out = out_idx + int64_t(b) * k;
  if constexpr (PT > 0) {
    // Element i = j * nthreads + 64 * wave + lane, so index order is (j,
    // wave, lane). Count the > T and == T keys of every (j, wave), turn the
    // counts into exclusive prefixes in that order (one wave scans them),
    // and each key's output position is then the number of > T keys before
    // it plus the number of selected ties before it, min(== T before, krem).
    const int E = iters * nwaves;  // (j, wave) pairs, at most PT * kMaxWaves
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      if (j >= iters) break;  // uniform
      const int i = tid + j * nthreads;
      const uint32_t key = keys[j];
      const uint64_t gtm = __ballot(i < n && key > T);
      const uint64_t eqm = __ballot(i < n && key == T);
      if (lane == 0) {
        pre_gt[j * nwaves + wave] = __popcll(gtm);
        pre_eq[j * nwaves + wave] = __popcll(eqm);
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int per = (E + 63) / 64, e0 = lane * per;
      int sg = 0, se = 0;
      for (int e = e0; e < e0 + per && e < E; ++e) {
        sg += pre_gt[e];
        se += pre_eq[e];
      }
      int ig = sg, ie = se;  // inclusive scans over the lanes
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int yg = __shfl_up(ig, o, 64), ye = __shfl_up(ie, o, 64);
        if (lane >= o) {
          ig += yg;
          ie += ye;
        }
      }
      int rg = ig - sg, re = ie - se;  // this lane's exclusive starts
      for (int e = e0; e < e0 + per && e < E; ++e) {
        const int cg = pre_gt[e], ce = pre_eq[e];
        pre_gt[e] = rg;
        pre_eq[e] = re;
        rg += cg;
        re += ce;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      if (j >= iters) break;  // uniform
      const int i = tid + j * nthreads;
      const uint32_t key = keys[j];
      const bool gt = i < n && key > T;
      const bool eq = i < n && key == T;
      const uint64_t lt = lanemask_lt(lane);
      const int gt_before = pre_gt[j * nwaves + wave] + __popcll(__ballot(gt) & lt);
      const int eq_before = pre_eq[j * nwaves + wave] + __popcll(__ballot(eq) & lt);
      const bool sel = gt || (eq && eq_before < krem);
      const int pos = gt_before + (eq_before < krem ? eq_before : krem);
      if (sel && pos < k) out[pos] = i;
    }
  } else {
    int run_sel = 0, run_eq = 0;
    for (int j = 0;; ++j) {
      if (j >= iters || run_sel >= k) break;  // uniform
      const int i = tid + j * nthreads;
      uint32_t key = 0;
      if (i < n) key = key_at(j, i);
      const bool gt = i < n && key > T;
      const bool eq = i < n && key == T;
      const uint64_t eqm = __ballot(eq);
      int eq_tot;
      const int eq_off = wave_offsets(__popcll(eqm), wave, nwaves, lane, scan_buf, &eq_tot);
      const int eq_rank = run_eq + eq_off + __popcll(eqm & lanemask_lt(lane));
      const bool sel = gt || (eq && eq_rank < krem);
      const uint64_t selm = __ballot(sel);
      int sel_tot;
      const int sel_off = wave_offsets(__popcll(selm), wave, nwaves, lane, scan_buf, &sel_tot);
      const int pos = run_sel + sel_off + __popcll(selm & lanemask_lt(lane));
      if (sel && pos < k) out[pos] = i;
      run_sel += sel_tot;
      run_eq += eq_tot;
    }
  }
}

}  // namespace

int launch_topk(const float* scores, int batch, int n, int64_t row_stride, int k,
                int32_t* out_idx, float* kth, hipStream_t stream) {
  if (batch == 0) return SPATTEN_OK;
  int threads = 256;
  if (n > 2048) threads = 512;
  if (n > 8192) threads = 1024;
  const dim3 grid(batch), block(threads);
  if (n <= 8 * threads)
    SPATTEN_TIMED("topk", stream, topk_radix_kernel<8><<<grid, block, 0, stream>>>(
                                      scores, n, row_stride, k, out_idx, kth));
  else if (n <= 32 * threads)
    SPATTEN_TIMED("topk", stream, topk_radix_kernel<32><<<grid, block, 0, stream>>>(
                                      scores, n, row_stride, k, out_idx, kth));
  else
    SPATTEN_TIMED("topk", stream, topk_radix_kernel<0><<<grid, block, 0, stream>>>(
                                      scores, n, row_stride, k, out_idx, kth));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

}  // namespace spatten
