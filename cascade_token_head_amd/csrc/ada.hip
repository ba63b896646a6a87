// Representative-token selection with a Gram threshold, and its cascade
// across layers ("Cascade Token Selection for Transformer Attention
// Acceleration": a token is representative when its largest cosine with
// every preceding token is below 1 - tau^2; the cascade inherits the
// previous layer's set and validates it with an r x r product among the
// members and a (T - r) x r product between the other tokens and the
// members that stayed).
//
// Every product is one kernel, ada_gram_max: for each token a of an
// ascending token list A, the largest cosine with the tokens b of an
// ascending list B that precede it (b < a). Since B is ascending, the
// tokens before a are a prefix of B, so a 64-row tile of A stops at the
// first B tile past its last token - the causal structure of the full Gram
// product, and of the cross product, costs only the pairs it needs. The
// dot products run on fp32 MFMA (32x32x2) from LDS-staged row chunks of
// the raw activations; the cosine is the dot scaled by both rows' inverse
// norms.
//
// The range of B tiles a row tile needs is split over workgroups, which
// combine their row maxima with an integer atomicMax on order-preserving
// keys of the fp32 cosines (a maximum does not depend on the order).
//
// Lists and decisions: ada_lists turns the inherited flags into the
// ascending member list R and the list N of the other tokens (an ordered
// compaction: per-thread counts, a block scan, then writes), ada_valid
// keeps the members whose removal cosine is below the threshold, and
// ada_finish writes the layer's flags, the cosine each decision was taken
// on and the counts.
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace spatten {
namespace {

constexpr int kAdaThreads = 1024;  // list and decision kernels: one workgroup per sequence
constexpr int kGT = 64;            // Gram tile: 64 A tokens x 64 B tokens
constexpr int kGK = 32;            // feature chunk staged in LDS

// 1 / |x_t| per row (0 for a zero row); one wave per row.
__global__ void __launch_bounds__(256)
ada_invnorm(const float* __restrict__ x, int64_t rows, int d, float* __restrict__ inv) {
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* p = x + row * d;
  float s = 0.0f;
  for (int c = lane * 4; c < d; c += 256) {
    const float4 v = *reinterpret_cast<const float4*>(p + c);
    s = fmaf(v.x, v.x, s);
    s = fmaf(v.y, v.y, s);
    s = fmaf(v.z, v.z, s);
    s = fmaf(v.w, v.w, s);
  }
  s = wave_sum(s);
  if (lane == 0) inv[row] = s > 0.0f ? 1.0f / sqrtf(s) : 0.0f;
}

// Order-preserving map of fp32 to uint32 (larger value -> larger key), so
// that workgroups can combine maxima with an integer atomicMax.
__device__ __forceinline__ uint32_t max_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
constexpr uint32_t kKeyNegInf = 0x007fffffu;  // max_key(-inf)

// Every entry of a [B, T] key array to kKeyNegInf.
__device__ __forceinline__ void clear_keys(uint32_t* keys, int T, int b) {
  for (int t = threadIdx.x; t < T; t += blockDim.x) keys[int64_t(b) * T + t] = kKeyNegInf;
}

// Exclusive block scan of one count per thread (kAdaThreads threads).
__device__ __forceinline__ int block_scan(int v, int* total) {
  __shared__ int wsum[kAdaThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kAdaThreads / 64; ++w) {
    off += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return off + incl - v;
}

// Per sequence: R = tokens with prev[t] != 0 (every token when prev is
// null), N = the others, both ascending; cnt[b*4 + 0] = |R|, [1] = |N|.
__global__ void __launch_bounds__(kAdaThreads)
ada_lists(const int32_t* __restrict__ prev, int T, int32_t* __restrict__ listR,
          int32_t* __restrict__ listN, int32_t* __restrict__ cnt, uint32_t* __restrict__ rkeys) {
  const int b = blockIdx.x, tid = threadIdx.x;
  clear_keys(rkeys, T, b);
  const int per = (T + kAdaThreads - 1) / kAdaThreads;
  const int t0 = tid * per, t1 = t0 + per < T ? t0 + per : T;
  const int32_t* pf = prev ? prev + int64_t(b) * T : nullptr;
  int nr = 0;
  for (int t = t0; t < t1; ++t) nr += (!pf || pf[t] != 0) ? 1 : 0;
  int totr;
  const int offr = block_scan(nr, &totr);
  int offn = t0 - offr;  // tokens before t0 that are not members
  int r = offr;
  int32_t* lr = listR + int64_t(b) * T;
  int32_t* ln = listN + int64_t(b) * T;
  for (int t = t0; t < t1; ++t) {
    if (!pf || pf[t] != 0)
      lr[r++] = t;
    else
      ln[offn++] = t;
  }
  if (tid == 0) {
    cnt[b * 4 + 0] = totr;
    cnt[b * 4 + 1] = T - totr;
  }
}

// B tiles per workgroup (measured: 1 made the cascade's products at
// T = 512 slower, 63 instead of 48 us per launch, though the full product
// gained from the extra workgroups)
constexpr int kGJ = 4;

// For i < nA[b]: keys[b*T + i] = max(keys[b*T + i], key of the largest
// cos(A[i], B[j]) over j < nB[b] with B[j] < A[i]). grid (T / 64 tiles of
// A, T / (64 kGJ) ranges of B, batch): each workgroup takes one 64-row A
// tile and up to kGJ 64-row B tiles of its range that precede the tile's
// last token, four waves each computing a 32 x 32 block per B tile. The
// feature chunks stream through LDS with the next chunk's rows requested
// before the current chunk's MFMAs. keys must hold kKeyNegInf (or an
// earlier maximum) on entry.
__global__ void __launch_bounds__(256)
ada_gram_max(const float* __restrict__ x, const float* __restrict__ inv, int T, int d,
             const int32_t* __restrict__ listA, const int32_t* __restrict__ cntA, int ia,
             const int32_t* __restrict__ listB, const int32_t* __restrict__ cntB, int ib,
             uint32_t* __restrict__ keys) {
  constexpr int LDK = kGK + 4;  // padded row: 16-byte stores, spread banks
  __shared__ __attribute__((aligned(16))) float As[kGT][LDK];
  __shared__ __attribute__((aligned(16))) float Bs[kGT][LDK];
  __shared__ int posA[kGT], posB[kGT];
  __shared__ float invA[kGT], invB[kGT];
  __shared__ float rmax[2][kGT];
  __shared__ int cnt_s[4];
  const int b = blockIdx.z;
  const int nA = cntA[b * 4 + ia], nB = cntB[b * 4 + ib];
  const int i0 = blockIdx.x * kGT;
  const int jr0 = blockIdx.y * (kGJ * kGT);
  if (i0 >= nA || jr0 >= nB) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* A = listA + int64_t(b) * T;
  const int32_t* B = listB + int64_t(b) * T;
  const float* xb = x + int64_t(b) * T * d;
  const float* ivb_ = inv + int64_t(b) * T;
  const int last = (i0 + kGT < nA ? i0 + kGT : nA) - 1;
  // B is ascending, so the entries of this workgroup's range (at most
  // kGJ * 64 = 256, one per thread) that precede the tile's last token are
  // a prefix of the range: counted with one load per thread and ballots
  static_assert(kGJ * kGT <= 256, "one range entry per thread");
  const int amax = A[last];
  const int W = kGJ * kGT < nB - jr0 ? kGJ * kGT : nB - jr0;
  const bool before = tid < W && B[jr0 + tid] < amax;
  const uint64_t bal = __ballot(before);
  if (lane == 0) cnt_s[wave] = __popcll(bal);
  if (tid < kGT) {
    const int i = i0 + tid <= last ? i0 + tid : last;  // rows past the list repeat the last
    posA[tid] = A[i];
    invA[tid] = ivb_[A[i]];
  }
  __syncthreads();
  const int jend = jr0 + cnt_s[0] + cnt_s[1] + cnt_s[2] + cnt_s[3];
  if (jr0 >= jend) return;  // uniform
  const int mt = wave >> 1, nt = wave & 1;  // this wave's 32 x 32 block
  const int l32 = lane & 31, hi = lane >> 5;
  // staging: 64 rows x 32 features per operand, two float4 per thread each
  const int sr = tid >> 2, sc = (tid & 3) * 8;
  float best[4][4];  // running max of this lane's rows (C layout)
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int q = 0; q < 4; ++q) best[g][q] = -INFINITY;
  const float* arow = xb + int64_t(posA[sr]) * d + sc;
  for (int j0 = jr0; j0 < jend; j0 += kGT) {
    __syncthreads();  // the previous tile's posB / invB readers are done
    if (tid < kGT) {
      const int j = j0 + tid < jend ? j0 + tid : jend - 1;
      posB[tid] = j0 + tid < jend ? B[j] : 0x7fffffff;  // past the range: never precedes
      invB[tid] = ivb_[B[j]];
    }
    __syncthreads();
    const int jr = j0 + sr < jend ? j0 + sr : jend - 1;
    const float* brow = xb + int64_t(B[jr]) * d + sc;
    float4 a0 = *reinterpret_cast<const float4*>(arow);
    float4 a1 = *reinterpret_cast<const float4*>(arow + 4);
    float4 b0 = *reinterpret_cast<const float4*>(brow);
    float4 b1 = *reinterpret_cast<const float4*>(brow + 4);
    floatx16 acc = {};
    for (int k0 = 0; k0 < d; k0 += kGK) {
      __syncthreads();  // the previous chunk's MFMA reads are done
      *reinterpret_cast<float4*>(&As[sr][sc]) = a0;
      *reinterpret_cast<float4*>(&As[sr][sc + 4]) = a1;
      *reinterpret_cast<float4*>(&Bs[sr][sc]) = b0;
      *reinterpret_cast<float4*>(&Bs[sr][sc + 4]) = b1;
      __syncthreads();
      if (k0 + kGK < d) {  // next chunk in flight during this one's MFMAs
        a0 = *reinterpret_cast<const float4*>(arow + k0 + kGK);
        a1 = *reinterpret_cast<const float4*>(arow + k0 + kGK + 4);
        b0 = *reinterpret_cast<const float4*>(brow + k0 + kGK);
        b1 = *reinterpret_cast<const float4*>(brow + k0 + kGK + 4);
      }
#pragma unroll
      for (int kk = 0; kk < kGK; kk += 2) {
        // A operand: row l32 of the wave's A block, feature kk + hi; B
        // operand: feature kk + hi of B row l32 (G = A B^T)
        const float av = As[mt * 32 + l32][kk + hi];
        const float bv = Bs[nt * 32 + l32][kk + hi];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
      }
    }
    // C layout: register r holds row 8*(r/4) + 4*hi + r%4, column l32
    const int pb = posB[nt * 32 + l32];
    const float ivb = invB[nt * 32 + l32];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = mt * 32 + 8 * g + 4 * hi + q;
        float c = acc[4 * g + q] * invA[row] * ivb;
        c = pb < posA[row] ? c : -INFINITY;
        best[g][q] = fmaxf(best[g][q], c);
      }
    }
  }
  // each row over the 32 columns of the half-wave, then over the two waves
  // that share the rows, then across workgroups
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v = best[g][q];
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
      best[g][q] = v;
    }
  __syncthreads();
  if (l32 == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int q = 0; q < 4; ++q) rmax[nt][mt * 32 + 8 * g + 4 * hi + q] = best[g][q];
  }
  __syncthreads();
  if (tid < kGT && i0 + tid <= last) {
    const float m = fmaxf(rmax[0][tid], rmax[1][tid]);
    if (m > -INFINITY) atomicMax(keys + int64_t(b) * T + i0 + tid, max_key(m));
  }
}

// Members of R whose removal cosine is below the threshold, in order:
// listV and cnt[b*4 + 2].
__global__ void __launch_bounds__(kAdaThreads)
ada_valid(const int32_t* __restrict__ listR, const uint32_t* __restrict__ rkeys, int T,
          float theta, int32_t* __restrict__ listV, int32_t* __restrict__ cnt,
          uint32_t* __restrict__ akeys) {
  const int b = blockIdx.x, tid = threadIdx.x;
  clear_keys(akeys, T, b);
  const int nR = cnt[b * 4 + 0];
  const int per = (nR + kAdaThreads - 1) / kAdaThreads;
  const int i0 = tid * per, i1 = i0 + per < nR ? i0 + per : nR;
  const uint32_t* ck = rkeys + int64_t(b) * T;
  int nv = 0;
  for (int i = i0; i < i1; ++i) nv += key_value(ck[i]) < theta ? 1 : 0;
  int tot;
  int o = block_scan(nv, &tot);
  const int32_t* R = listR + int64_t(b) * T;
  int32_t* V = listV + int64_t(b) * T;
  for (int i = i0; i < i1; ++i)
    if (key_value(ck[i]) < theta) V[o++] = R[i];
  if (tid == 0) cnt[b * 4 + 2] = tot;
}

// The layer's flags and decision cosines. Full selection (cascade = 0):
// every token is in R and flag = cosine < theta. Cascade: members of V
// keep their flag, tokens of N with addition cosine < theta join.
// counts[b*4 + 0..3] = set size, removed, added, Gram pairs evaluated.
__global__ void __launch_bounds__(kAdaThreads)
ada_finish(const int32_t* __restrict__ listR, const int32_t* __restrict__ listN,
           const int32_t* __restrict__ listV, const uint32_t* __restrict__ rkeys,
           const uint32_t* __restrict__ akeys, const int32_t* __restrict__ cnt, int T, float theta,
           int cascade, int32_t* __restrict__ flags, float* __restrict__ maxcos,
           int32_t* __restrict__ counts) {
  __shared__ int red[2];
  __shared__ unsigned long long psum;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int nR = cnt[b * 4 + 0], nN = cnt[b * 4 + 1], nV = cascade ? cnt[b * 4 + 2] : 0;
  const int64_t base = int64_t(b) * T;
  const int32_t* R = listR + base;
  const int32_t* N = listN + base;
  const int32_t* V = listV + base;
  int32_t* f = flags + base;
  if (tid < 2) red[tid] = 0;
  if (tid == 0) psum = 0;
  for (int t = tid; t < T; t += kAdaThreads) f[t] = 0;
  __syncthreads();
  int nsel = 0, nadd = 0;
  unsigned long long pairs = 0;
  for (int i = tid; i < nR; i += kAdaThreads) {
    const float c = key_value(rkeys[base + i]);
    if (maxcos) maxcos[base + R[i]] = c;
    if (!cascade && c < theta) {
      f[R[i]] = 1;
      ++nsel;
    }
  }
  if (cascade) {
    for (int i = tid; i < nV; i += kAdaThreads) f[V[i]] = 1;
    for (int i = tid; i < nN; i += kAdaThreads) {
      const float c = key_value(akeys[base + i]);
      if (maxcos) maxcos[base + N[i]] = c;
      if (c < theta) {
        f[N[i]] = 1;
        ++nadd;
      }
      // valid members before N[i]: a lower bound in V
      int lo = 0, hi = nV;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (V[mid] < N[i]) lo = mid + 1; else hi = mid;
      }
      pairs += lo;
    }
  }
  if (nsel + nadd) atomicAdd(&red[0], nsel + nadd);
  if (nadd) atomicAdd(&red[1], nadd);
  if (pairs) atomicAdd(&psum, pairs);
  __syncthreads();
  if (tid == 0 && counts) {
    const int64_t rr = int64_t(nR) * (nR - 1) / 2;  // pairs s < t among R
    counts[b * 4 + 0] = cascade ? nV + red[1] : red[0];
    counts[b * 4 + 1] = cascade ? nR - nV : 0;
    counts[b * 4 + 2] = cascade ? red[1] : 0;
    const int64_t p = rr + int64_t(psum);
    counts[b * 4 + 3] = int32_t(p < 0x7fffffff ? p : 0x7fffffff);
  }
}

}  // namespace

int launch_ada_select(const AdaArgs& a, hipStream_t stream) {
  if (a.batch == 0) return SPATTEN_OK;
  const int64_t rows = int64_t(a.batch) * a.T;
  SPATTEN_TIMED("ada_invnorm", stream,
                ada_invnorm<<<unsigned(ceil_div(rows, 4)), 256, 0, stream>>>(a.x, rows, a.d,
                                                                            a.inv));
  SPATTEN_LAUNCH_CHECK();
  SPATTEN_TIMED("ada_lists", stream,
                ada_lists<<<a.batch, kAdaThreads, 0, stream>>>(a.prev, a.T, a.listR, a.listN,
                                                              a.cnt, a.rc));
  SPATTEN_LAUNCH_CHECK();
  const dim3 gg(unsigned(ceil_div(a.T, kGT)), unsigned(ceil_div(a.T, kGT * kGJ)),
                unsigned(a.batch));
  // r x r (every token against every preceding one for the full selection)
  SPATTEN_TIMED("ada_gram", stream,
                ada_gram_max<<<gg, 256, 0, stream>>>(a.x, a.inv, a.T, a.d, a.listR, a.cnt, 0,
                                                    a.listR, a.cnt, 0, a.rc));
  SPATTEN_LAUNCH_CHECK();
  const float theta = 1.0f - a.tau * a.tau;
  const int cascade = a.prev != nullptr;
  if (cascade) {
    SPATTEN_TIMED("ada_valid", stream,
                  ada_valid<<<a.batch, kAdaThreads, 0, stream>>>(a.listR, a.rc, a.T, theta,
                                                                a.listV, a.cnt, a.ac));
    SPATTEN_LAUNCH_CHECK();
    // (T - r) x r: the other tokens against the members that stayed
    SPATTEN_TIMED("ada_gram", stream,
                  ada_gram_max<<<gg, 256, 0, stream>>>(a.x, a.inv, a.T, a.d, a.listN, a.cnt, 1,
                                                      a.listV, a.cnt, 2, a.ac));
    SPATTEN_LAUNCH_CHECK();
  }
  SPATTEN_TIMED("ada_finish", stream,
                ada_finish<<<a.batch, kAdaThreads, 0, stream>>>(
                    a.listR, a.listN, a.listV, a.rc, a.ac, a.cnt, a.T, theta, cascade, a.flags,
                    a.maxcos, a.counts));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

}  // namespace spatten
