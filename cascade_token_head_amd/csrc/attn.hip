// Prefill attention over the kept tokens and heads with token and head
// importance fused in (SpAtten: section II "Attention mechanism",
// "Cascade pruning"; "B. Motivation" - token importance is the column sum
// of the attention probabilities; head importance is the magnitude of the
// head's output).
//
// Token importance needs the normalised probabilities P[i, j] summed over
// queries i, so every row's log-sum-exp must be known first. Two passes:
//   forward   (query-major, one workgroup per 128 queries of one head):
//             online softmax over 64-key LDS tiles, O = P V, the row LSE
//             and a partial sum of |O|;
//   col-sum   (key-major, one workgroup per 256 keys of one head): loops
//             over every query tile, rebuilds P = exp(S - LSE) and sums it
//             down each column in registers - deterministic, no atomics,
//             and the n x n matrix never exists.
// bf16 path on gfx950 MFMA 32x32x16. In the forward pass S is computed
// transposed (keys as rows) so that each lane holds one query's scores:
// row statistics stay in-lane, and the key rows fed to the MFMA are
// permuted so each lane's 16 scores are 16 consecutive keys, which is
// exactly the k-slot order the P V MFMA wants - P never leaves registers.
// fp32 path: plain VALU kernels for the fp32 workload.
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace spatten {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ bf16 forward

template <int DH, bool CAUSAL>
__global__ void __launch_bounds__(256)
attn_fwd_bf16(AttnArgs a) {
  constexpr int KT = 64;        // keys per iteration
  constexpr int KS = DH + 8;    // LDS row stride of the K tile
  constexpr int VS = KT + 8;    // LDS row stride of the V^T tile
  constexpr int NKC = KT * DH / 8 / 256;  // 16-byte K chunks per thread
  constexpr int NVC = DH * KT / 8 / 256;  // 16-byte V^T chunks per thread
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][KT * KS];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][DH * VS];
  __shared__ float red[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = lane >> 5, col = lane & 31;
  const int b = blockIdx.z, s = blockIdx.y;
  const int qb = CAUSAL ? int(gridDim.x) - 1 - int(blockIdx.x) : int(blockIdx.x);
  const int q0 = qb * 128;
  const int n = a.n, n_pad = a.n_pad;
  const int64_t bs = int64_t(b) * a.h_kept + s;
  const bf16_t* Q = static_cast<const bf16_t*>(a.q) + bs * n_pad * DH;
  const bf16_t* K = static_cast<const bf16_t*>(a.k) + bs * n_pad * DH;
  const bf16_t* VT = static_cast<const bf16_t*>(a.vt) + bs * DH * n_pad;
  const int my_q = q0 + 32 * wave + col;

  bf16x8 qf[DH / 16];
#pragma unroll
  for (int kk = 0; kk < DH / 16; ++kk)
    qf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(Q + int64_t(my_q) * DH + 16 * kk + 8 * G));

  const float sc = kLog2e / sqrtf(float(DH));
  float m = -INFINITY, lsum = 0.0f;
  floatx16 o[DH / 32];
#pragma unroll
  for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;

  const int kend = CAUSAL ? min(n, q0 + 128) : n;
  const int ntiles = int(ceil_div(kend, KT));

  u32x4 rk[NKC], rv[NVC];
  auto gload = [&](int it) {
    const int k0 = it * KT;
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int c = tid + 256 * i;
      rk[i] = *reinterpret_cast<const u32x4*>(K + int64_t(k0) * DH + c * 8);
    }
#pragma unroll
    for (int i = 0; i < NVC; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, k8 = (c & 7) * 8;
      rv[i] = *reinterpret_cast<const u32x4*>(VT + int64_t(row) * n_pad + k0 + k8);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (DH / 8), c8 = (c % (DH / 8)) * 8;
      *reinterpret_cast<u32x4*>(&Ks[buf][row * KS + c8]) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < NVC; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, k8 = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(&Vs[buf][row * VS + k8]) = rv[i];
    }
  };

  // MFMA row r of a 32-key score tile is fed key 16*((r>>2)&1) + 4*(r>>3) + (r&3);
  // the C layout then gives lane group G the keys 16G .. 16G+15 in order.
  const int kperm = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);

  gload(0);
  sstore(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1, k0 = it * KT;
    if (it + 1 < ntiles) gload(it + 1);
    floatx16 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[t][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk) {
        const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(
            &Ks[buf][(32 * t + kperm) * KS + 16 * kk + 8 * G]));
        st[t] = mfma32x32x16(kf, qf[kk], st[t]);
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 32 * t + 16 * G + i;
        float v = st[t][i] * sc;
        const bool masked = key >= n || (CAUSAL && key > my_q);
        v = masked ? -INFINITY : v;
        st[t][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m, tmax);
    const float alpha = exp2f(m - m_new);
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    bf16x8 pb[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = exp2f(st[t][8 * u + 2 * j] - m);
          const float p1 = exp2f(st[t][8 * u + 2 * j + 1] - m);
          lsum += p0 + p1;
          w[j] = pack_bf16x2(p0, p1);
        }
        pb[t][u] = as_bf16x8(w);
      }
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 vf = as_bf16x8(*reinterpret_cast<const u32x4*>(
              &Vs[buf][(32 * dt + col) * VS + 32 * t + 16 * G + 8 * u]));
          o[dt] = mfma32x32x16(vf, pb[t][u], o[dt]);
        }
    if (it + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }

  lsum += __shfl_xor(lsum, 32, 64);
  const float inv = 1.0f / lsum;
  float gsum = 0.0f;
  if (my_q < n) {
    bf16_t* orow = static_cast<bf16_t*>(a.o) + (int64_t(b) * n + my_q) * (a.h_kept * DH) + s * DH;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * dt + 8 * q4 + 4 * G;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = o[dt][4 * q4 + e] * inv;
          gsum += fabsf(v[e]);
        }
        uint64_t pk = uint64_t(pack_bf16x2(v[0], v[1])) | (uint64_t(pack_bf16x2(v[2], v[3])) << 32);
        *reinterpret_cast<uint64_t*>(orow + d0) = pk;
      }
  }
  if (G == 0) a.lse[bs * n_pad + my_q] = m + log2f(lsum);
  gsum = wave_sum(gsum);
  if (lane == 0) red[wave] = gsum;
  __syncthreads();
  if (tid == 0) a.gpart[bs * a.nqb + qb] = red[0] + red[1] + red[2] + red[3];
}

// ------------------------------------------------------------------ bf16 column sums

template <int DH, bool CAUSAL>
__global__ void __launch_bounds__(256)
attn_colsum_bf16(AttnArgs a) {
  constexpr int QT = 128;      // queries per iteration
  constexpr int QS = DH + 8;
  constexpr int NQC = QT * DH / 8 / 256;
  __shared__ __attribute__((aligned(16))) bf16_t Qs[2][QT * QS];
  __shared__ float Ls[2][QT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = lane >> 5, col = lane & 31;
  const int b = blockIdx.z, s = blockIdx.y;
  const int k0 = blockIdx.x * kAttnKBlock;
  const int n = a.n, n_pad = a.n_pad;
  const int64_t bs = int64_t(b) * a.h_kept + s;
  const bf16_t* Q = static_cast<const bf16_t*>(a.q) + bs * n_pad * DH;
  const bf16_t* K = static_cast<const bf16_t*>(a.k) + bs * n_pad * DH;
  const float* L = a.lse + bs * n_pad;
  const int kw = k0 + 64 * wave;

  // K^T operand: lane holds K[key kw + 32t + col][16kk + 8G .. +8]
  bf16x8 kf[2][DH / 16];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = min(kw + 32 * t + col, n_pad - 1);
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk)
      kf[t][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(K + int64_t(key) * DH + 16 * kk + 8 * G));
  }
  const float sc = kLog2e / sqrtf(float(DH));
  float acc[2] = {0.0f, 0.0f};

  const int qstart = CAUSAL ? k0 : 0;
  const int ntiles = qstart < n ? int(ceil_div(n - qstart, QT)) : 0;

  u32x4 rq[NQC];
  float rl = 0.0f;
  auto gload = [&](int it) {
    const int qt0 = qstart + it * QT;
#pragma unroll
    for (int i = 0; i < NQC; ++i) {
      const int c = tid + 256 * i;
      rq[i] = *reinterpret_cast<const u32x4*>(Q + int64_t(qt0) * DH + c * 8);
    }
    if (tid < QT) rl = L[qt0 + tid];
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NQC; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (DH / 8), c8 = (c % (DH / 8)) * 8;
      *reinterpret_cast<u32x4*>(&Qs[buf][row * QS + c8]) = rq[i];
    }
    if (tid < QT) Ls[buf][tid] = rl;
  };

  if (ntiles > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1, qt0 = qstart + it * QT;
    if (it + 1 < ntiles) gload(it + 1);
#pragma unroll
    for (int u = 0; u < QT / 32; ++u) {
      floatx16 st[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[t][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk) {
        const bf16x8 qa = as_bf16x8(*reinterpret_cast<const u32x4*>(
            &Qs[buf][(32 * u + col) * QS + 16 * kk + 8 * G]));
#pragma unroll
        for (int t = 0; t < 2; ++t) st[t] = mfma32x32x16(qa, kf[t][kk], st[t]);
      }
      // st[t][r]: query qt0 + 32u + 8(r/4) + 4G + r%4, key kw + 32t + col
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = 32 * u + 8 * (r >> 2) + 4 * G + (r & 3);
        const int qi = qt0 + ql;
        const float l2 = Ls[buf][ql];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int key = kw + 32 * t + col;
          const float p = exp2f(st[t][r] * sc - l2);
          const bool keep = qi < n && (!CAUSAL || key <= qi);
          acc[t] += keep ? p : 0.0f;
        }
      }
    }
    if (it + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float v = acc[t] + __shfl_xor(acc[t], 32, 64);
    const int key = kw + 32 * t + col;
    if (G == 0 && key < n) a.colsum[bs * n_pad + key] = v;
  }
}

// ------------------------------------------------------------------ fp32 path

// One workgroup per kAttnF32Rows query rows of one head; score rows live in
// dynamic LDS (rows x n_pad floats).
template <bool CAUSAL>
__global__ void __launch_bounds__(256)
attn_fwd_f32(AttnArgs a) {
  extern __shared__ float S[];
  constexpr int R = kAttnF32Rows;
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.z, s = blockIdx.y, rb = blockIdx.x, r0 = rb * R;
  const int n = a.n, n_pad = a.n_pad, dh = a.dh;
  const int64_t bs = int64_t(b) * a.h_kept + s;
  const float* Q = static_cast<const float*>(a.q) + bs * n_pad * dh;
  const float* K = static_cast<const float*>(a.k) + bs * n_pad * dh;
  const float* VT = static_cast<const float*>(a.vt) + bs * dh * n_pad;
  const float scale = 1.0f / sqrtf(float(dh));
  for (int e = tid; e < R * n; e += 256) {
    const int r = e / n, j = e - r * n, qi = r0 + r;
    float v = -INFINITY;
    if (qi < n && !(CAUSAL && j > qi)) {
      float d = 0.0f;
      for (int c = 0; c < dh; ++c) d = fmaf(Q[int64_t(qi) * dh + c], K[int64_t(j) * dh + c], d);
      v = d * scale;
    }
    S[r * n_pad + j] = v;
  }
  __syncthreads();
  // each wave normalises R/4 rows
  for (int r = wave; r < R; r += 4) {
    const int qi = r0 + r;
    float mx = -INFINITY;
    for (int j = lane; j < n; j += 64) mx = fmaxf(mx, S[r * n_pad + j]);
    mx = wave_max(mx);
    float sum = 0.0f;
    for (int j = lane; j < n; j += 64) {
      const float e = qi < n ? expf(S[r * n_pad + j] - mx) : 0.0f;
      S[r * n_pad + j] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    const float inv = qi < n ? 1.0f / sum : 0.0f;
    for (int j = lane; j < n; j += 64) S[r * n_pad + j] *= inv;
    if (lane == 0 && qi < n) a.lse[bs * n_pad + qi] = (mx + logf(sum)) * kLog2e;
  }
  __syncthreads();
  float gsum = 0.0f;
  for (int e = tid; e < R * dh; e += 256) {
    const int r = e / dh, c = e - r * dh, qi = r0 + r;
    if (qi >= n) continue;
    float acc = 0.0f;
    for (int j = 0; j < n; ++j) acc = fmaf(S[r * n_pad + j], VT[int64_t(c) * n_pad + j], acc);
    static_cast<float*>(a.o)[(int64_t(b) * n + qi) * (a.h_kept * dh) + s * dh + c] = acc;
    gsum += fabsf(acc);
  }
  gsum = wave_sum(gsum);
  if (lane == 0) red[wave] = gsum;
  __syncthreads();
  if (tid == 0) a.gpart[bs * a.nqb + rb] = red[0] + red[1] + red[2] + red[3];
}

// Column sums: thread per key, loop over queries, P = exp2(S*log2e - lse2).
template <bool CAUSAL>
__global__ void __launch_bounds__(256)
attn_colsum_f32(AttnArgs a) {
  const int b = blockIdx.z, s = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int n = a.n, n_pad = a.n_pad, dh = a.dh;
  if (j >= n) return;
  const int64_t bs = int64_t(b) * a.h_kept + s;
  const float* Q = static_cast<const float*>(a.q) + bs * n_pad * dh;
  const float* K = static_cast<const float*>(a.k) + bs * n_pad * dh;
  const float* L = a.lse + bs * n_pad;
  const float scale = kLog2e / sqrtf(float(dh));
  float acc = 0.0f;
  for (int i = CAUSAL ? j : 0; i < n; ++i) {
    float d = 0.0f;
    for (int c = 0; c < dh; ++c) d = fmaf(Q[int64_t(i) * dh + c], K[int64_t(j) * dh + c], d);
    acc += exp2f(d * scale - L[i]);
  }
  a.colsum[bs * n_pad + j] = acc;
}

// ------------------------------------------------------------------ helpers

// V^T columns n .. n_pad-1 must hold zeros: masked probabilities are exactly
// 0 and multiply them in the P V product.
template <typename T>
__global__ void pad_zero_kernel(T* vt, int rows, int n, int n_pad) {
  const int w = n_pad - n;
  const int64_t total = int64_t(rows) * w;
  for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = e / w;
    vt[r * n_pad + n + (e - r * w)] = T(0);
  }
}

__global__ void __launch_bounds__(256)
importance_kernel(const float* __restrict__ colsum, const float* __restrict__ gpart,
                  const float* __restrict__ lse, const int32_t* __restrict__ head_idx,
                  int h_kept, int H, int n, int n_pad, int nqb, float* __restrict__ a,
                  float* __restrict__ g, float* __restrict__ lse_out) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j < n) {
    float acc = 0.0f;
    for (int s = 0; s < h_kept; ++s) acc += colsum[(int64_t(b) * h_kept + s) * n_pad + j];
    a[int64_t(b) * n + j] += acc;
    if (lse_out)
      for (int s = 0; s < h_kept; ++s)
        lse_out[(int64_t(b) * h_kept + s) * n + j] = lse[(int64_t(b) * h_kept + s) * n_pad + j] * kLn2;
  }
  if (blockIdx.x == 0 && threadIdx.x < h_kept) {
    const int s = threadIdx.x;
    float acc = 0.0f;
    for (int q = 0; q < nqb; ++q) acc += gpart[(int64_t(b) * h_kept + s) * nqb + q];
    g[int64_t(b) * H + head_idx[b * h_kept + s]] += acc;
  }
}

template <int DH, bool CAUSAL>
int run_bf16(const AttnArgs& a, hipStream_t stream) {
  const dim3 g1(unsigned(ceil_div(a.n, kAttnQBlock)), a.h_kept, a.batch);
  SPATTEN_TIMED("attn_fwd", stream, attn_fwd_bf16<DH, CAUSAL><<<g1, 256, 0, stream>>>(a));
  SPATTEN_LAUNCH_CHECK();
  const dim3 g2(unsigned(ceil_div(a.n, kAttnKBlock)), a.h_kept, a.batch);
  SPATTEN_TIMED("attn_colsum", stream, attn_colsum_bf16<DH, CAUSAL><<<g2, 256, 0, stream>>>(a));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

template <bool CAUSAL>
int run_f32(const AttnArgs& a, hipStream_t stream) {
  const dim3 g1(unsigned(ceil_div(a.n, kAttnF32Rows)), a.h_kept, a.batch);
  const size_t lds = size_t(kAttnF32Rows) * a.n_pad * sizeof(float);
  SPATTEN_TIMED("attn_fwd", stream, attn_fwd_f32<CAUSAL><<<g1, 256, lds, stream>>>(a));
  SPATTEN_LAUNCH_CHECK();
  const dim3 g2(unsigned(ceil_div(a.n, 256)), a.h_kept, a.batch);
  SPATTEN_TIMED("attn_colsum", stream, attn_colsum_f32<CAUSAL><<<g2, 256, 0, stream>>>(a));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

}  // namespace

int launch_pad_zero(const AttnArgs& a, hipStream_t stream) {
  if (a.n_pad == a.n) return SPATTEN_OK;
  const int rows = a.batch * a.h_kept * a.dh;
  const int64_t total = int64_t(rows) * (a.n_pad - a.n);
  const int64_t nb = ceil_div(total, 256);
  const unsigned blocks = unsigned(nb < 4096 ? nb : 4096);
  if (a.dtype == SPATTEN_BF16)
    SPATTEN_TIMED("pad_zero", stream,
                  pad_zero_kernel<bf16_t><<<blocks, 256, 0, stream>>>(
                      static_cast<bf16_t*>(const_cast<void*>(a.vt)), rows, a.n, a.n_pad));
  else
    SPATTEN_TIMED("pad_zero", stream,
                  pad_zero_kernel<float><<<blocks, 256, 0, stream>>>(
                      static_cast<float*>(const_cast<void*>(a.vt)), rows, a.n, a.n_pad));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

int launch_attention(const AttnArgs& a, hipStream_t stream) {
  if (a.dtype == SPATTEN_F32) return a.causal ? run_f32<true>(a, stream) : run_f32<false>(a, stream);
  if (a.dh == 64) return a.causal ? run_bf16<64, true>(a, stream) : run_bf16<64, false>(a, stream);
  if (a.dh == 128) return a.causal ? run_bf16<128, true>(a, stream) : run_bf16<128, false>(a, stream);
  return SPATTEN_EUNSUPPORTED;
}

int launch_importance(const float* colsum, const float* gpart, const float* lse,
                      const int32_t* head_idx, int batch, int h_kept, int H, int n, int n_pad,
                      int nqb, float* a, float* g, float* lse_out, hipStream_t stream) {
  const dim3 grid(unsigned(ceil_div(n, 256)), batch);
  SPATTEN_TIMED("importance", stream,
                importance_kernel<<<grid, 256, 0, stream>>>(colsum, gpart, lse, head_idx, h_kept,
                                                            H, n, n_pad, nqb, a, g, lse_out));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

}  // namespace spatten
