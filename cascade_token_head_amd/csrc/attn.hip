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
// Local value pruning (a threshold on each exact probability before P V)
// adds a second forward pass that reads the first pass's LSE (bf16), or is
// applied to the normalised scores in LDS (fp32). Per-head token pruning
// (bf16, bidirectional): each head's kept tokens are gathered into its own
// K / V^T slabs and serve as the keys of that head, every token as a query;
// the column sums are added at each kept token's position of the head
// slot's own importance row.
#include <type_traits>

#include "common.hpp"
#include "importance.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace spatten {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Workgroup i runs on XCD i % 8. Attention grids are 1-D over (block,
// head, sequence) with the block index fastest; each XCD takes a contiguous
// run of that order, so the blocks of one head run on one XCD together and
// re-read that head's K/V (forward) or Q (column sums) from its own L2.
// Block 0 is the longest one (causal). When an XCD holds whole (head,
// sequence) groups but only a few blocks per CU, its groups are dispatched
// interleaved by block (every group's longest block first) instead of one
// group after another, which would leave the last group's long blocks to
// start late and run alone.
struct XcdItem {
  bool valid;
  int blk, s, b;
};
__device__ __forceinline__ XcdItem xcd_item(int nblk, int h, int batch) {
  const int total = nblk * h * batch;
  const int per = (total + 7) / 8;
  const int x = int(blockIdx.x) & 7, u = int(blockIdx.x) >> 3;
  int t = x * per + u;
  if ((h * batch) % 8 == 0 && per <= 128) {
    const int groups = per / nblk;  // whole groups per XCD
    t = x * per + (u % groups) * nblk + u / groups;
  }
  XcdItem it;
  it.valid = t < total;
  it.blk = t % nblk;
  it.s = (t / nblk) % h;
  it.b = t / (nblk * h);
  return it;
}

inline unsigned xcd_grid(int64_t total) { return unsigned(8 * ((total + 7) / 8)); }

// ------------------------------------------------------------------ bf16 forward

// NU 32-query groups per wave; a workgroup covers QB queries with
// QB / (32 NU) waves sharing each K/V tile. MINW: waves per SIMD the
// register budget is sized for. VP: local value pruning ("A. Cascade Token
// Pruning", bullet "Local Value Pruning"), a second pass once the first
// has written every row's log2-sum-exp: the exp2 reference is that LSE, so
// each probability is exact when formed, those below a.v_threshold are
// zeroed before the P V MFMA, and O needs no normalisation. It rewrites O
// and the |O| partials and leaves the LSE as it was.
template <int DH, bool CAUSAL, int NU, int MINW, bool VP = false>
__global__ void __launch_bounds__(2 * attn_qblock(DH) / NU, MINW)
attn_fwd_bf16(AttnArgs a) {
  // dh 128: K/V loads run two tiles ahead (the register budget allows a
  // second staging set); dh 64 keeps one set to stay at three waves/SIMD
  constexpr bool DEEP = DH == 128;
  constexpr int QB = attn_qblock(DH);
  constexpr int NT = 2 * QB / NU;  // threads per workgroup
  constexpr int WAVES = NT / 64;
  constexpr int KT = 64;        // keys per iteration
  constexpr int KS = DH + 8;    // LDS row stride of the K tile
  constexpr int VS = KT + 8;    // LDS row stride of the V^T tile
  constexpr int NKC = KT * DH / 8 / NT;  // 16-byte K chunks per thread
  constexpr int NVC = DH * KT / 8 / NT;  // 16-byte V^T chunks per thread
  constexpr int QW = 32 * NU;             // queries per wave
  constexpr float kRescale = 8.0f;        // log2 headroom before O is rescaled
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][KT * KS];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][DH * VS];
  __shared__ float red[WAVES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = lane >> 5, col = lane & 31;
  const int nqb_grid = int(ceil_div(a.n, QB));
  const XcdItem item = xcd_item(nqb_grid, a.h_kept, a.batch);
  if (!item.valid) return;
  const int b = item.b, s = item.s;
  // causal: the longest rows (last query blocks) first
  const int qb = CAUSAL ? nqb_grid - 1 - item.blk : item.blk;
  const int q0 = qb * QB;
  const int wq0 = q0 + QW * wave;        // first query of this wave
  const int n = a.n, n_pad = a.n_pad;
  // keys: the layer's tokens, or (per-head pruning) the head's own kept
  // tokens gathered into their own K / V^T slabs
  const int nk = a.nk, nk_pad = a.nk_pad;
  const int64_t bs = int64_t(b) * a.h_kept + s;
  const bf16_t* Q = static_cast<const bf16_t*>(a.q) + bs * n_pad * DH;
  const bf16_t* K = static_cast<const bf16_t*>(a.kk) + bs * nk_pad * DH;
  const bf16_t* VT = static_cast<const bf16_t*>(a.vtk) + bs * DH * nk_pad;
  const bool wave_live = wq0 < n;

  // Q operand (B of S^T = K Q^T): lane holds Q[query][16kk + 8G .. +8]
  bf16x8 qf[NU][DH / 16];
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk)
      qf[u][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(
          Q + int64_t(wq0 + 32 * u + col) * DH + 16 * kk + 8 * G));

  const float sc = kLog2e / sqrtf(float(DH));
  float mref[NU];  // max used as the exp2 reference (raw score units)
  float lsum[NU];
  float lse2[NU];  // VP: the row's log2-sum-exp from the first pass
  floatx16 o[DH / 32][NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    mref[u] = -INFINITY;
    lsum[u] = 0.0f;
    const int my_q = wq0 + 32 * u + col;
    lse2[u] = VP && my_q < a.n ? a.lse[bs * a.n_pad + my_q] : 0.0f;
  }
#pragma unroll
  for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][u][r] = 0.0f;

  const int kend = CAUSAL ? min(n, q0 + QB) : nk;
  const int ntiles = int(ceil_div(kend, KT));
  const int wave_kend = CAUSAL ? min(n, wq0 + QW) : nk;   // keys this wave can see

  // register staging: one set, or two when loads run two tiles ahead
  constexpr int NSET = DEEP ? 2 : 1;
  u32x4 rk[NSET][NKC], rv[NSET][NVC];
  auto gload = [&](int set, int it) {
    const int k0 = it * KT;
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int c = tid + NT * i;
      rk[set][i] = *reinterpret_cast<const u32x4*>(K + int64_t(k0) * DH + c * 8);
    }
#pragma unroll
    for (int i = 0; i < NVC; ++i) {
      const int c = tid + NT * i;
      const int row = c >> 3, k8 = (c & 7) * 8;
      rv[set][i] = *reinterpret_cast<const u32x4*>(VT + int64_t(row) * nk_pad + k0 + k8);
      // keys past the end get exact zeros (their probabilities are 0, and
      // the padding itself is never written)
      if (k0 + KT > nk) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = k0 + k8 + 2 * e;
          const uint32_t lo = key < nk ? 0xffffu : 0u, hi = key + 1 < nk ? 0xffff0000u : 0u;
          rv[set][i][e] &= lo | hi;
        }
      }
    }
  };
  auto sstore = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int c = tid + NT * i;
      const int row = c / (DH / 8), c8 = (c % (DH / 8)) * 8;
      *reinterpret_cast<u32x4*>(&Ks[buf][row * KS + c8]) = rk[set][i];
    }
#pragma unroll
    for (int i = 0; i < NVC; ++i) {
      const int c = tid + NT * i;
      const int row = c >> 3, k8 = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(&Vs[buf][row * VS + k8]) = rv[set][i];
    }
  };

  // MFMA row r of a 32-key score tile is fed key 16*((r>>2)&1) + 4*(r>>3) + (r&3);
  // the C layout then gives lane group G the keys 16G .. 16G+15 in order.
  const int kperm = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);

  // A 32-key sub-tile (keys k0 + 32t ..) runs in two parts: S^T by MFMA
  // (qk), then online softmax in registers and O^T += V^T P^T (soft_pv).
  // The tile loop issues both sub-tiles' qk before the first soft_pv, so
  // the second sub-tile's MFMAs execute under the first one's softmax VALU
  // work, and the first one's P V MFMAs under the second one's softmax.
  // Masking is applied only to sub-tiles that cross the sequence end or the
  // causal diagonal, so interior sub-tiles carry no masking code.
  // K fragments go through a ring of RING registers: RING reads in flight,
  // one new read issued per MFMA, so LDS latency hides under the MFMAs
  constexpr int NKK = DH / 16, RING = NKK < 4 ? NKK : 4;
  auto qk = [&](int buf, int t, floatx16* st) {
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[u][r] = 0.0f;
    bf16x8 kf[RING];
    auto kread = [&](int kk) {
      return as_bf16x8(*reinterpret_cast<const u32x4*>(
          &Ks[buf][(32 * t + kperm) * KS + 16 * kk + 8 * G]));
    };
#pragma unroll
    for (int p = 0; p < RING; ++p) kf[p] = kread(p);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int u = 0; u < NU; ++u) st[u] = mfma32x32x16(kf[kk % RING], qf[u][kk], st[u]);
      if (kk + RING < NKK) kf[kk % RING] = kread(kk + RING);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, RING, 0);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, NU, 0);
      if (kk + RING < NKK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  auto mask = [&](floatx16* st, int k0, int t) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int my_q = wq0 + 32 * u + col;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 32 * t + 16 * G + i;
        const bool m = key >= nk || (CAUSAL && key > my_q);
        st[u][i] = m ? -INFINITY : st[u][i];
      }
    }
  };
  auto soft_pv = [&](floatx16* st, int buf, int t) {
    bf16x8 pb[2][NU];  // [s2][u]
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if constexpr (VP) {
        // exact probabilities against the known LSE; below the threshold
        // a V row does not enter this query's output
        const float tau = a.v_threshold;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          u32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float p0 = fast_exp2(fmaf(st[u][8 * s2 + 2 * j], sc, -lse2[u]));
            float p1 = fast_exp2(fmaf(st[u][8 * s2 + 2 * j + 1], sc, -lse2[u]));
            p0 = p0 >= tau ? p0 : 0.0f;
            p1 = p1 >= tau ? p1 : 0.0f;
            w[j] = pack_bf16x2(p0, p1);
          }
          pb[s2][u] = as_bf16x8(w);
        }
        continue;
      }
      float m4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        m4[i] = fmaxf(fmaxf(st[u][4 * i], st[u][4 * i + 1]), fmaxf(st[u][4 * i + 2], st[u][4 * i + 3]));
      const float tmax = xor32_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
      // move the reference only when a score would exceed it by 2^kRescale
      const bool grow = tmax * sc > mref[u] * sc + kRescale || mref[u] == -INFINITY;
      if (__ballot(grow)) {
        const float m_new = grow ? fmaxf(mref[u], tmax) : mref[u];
        const float alpha = mref[u] == -INFINITY ? 0.0f : fast_exp2((mref[u] - m_new) * sc);
        mref[u] = m_new;
        lsum[u] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt) o[dt][u] = o[dt][u] * alpha;
      }
      const float msc = (mref[u] == -INFINITY ? 0.0f : mref[u]) * sc;
      float ps[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 w;
        float pp[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(fmaf(st[u][8 * s2 + 2 * j], sc, -msc));
          const float p1 = fast_exp2(fmaf(st[u][8 * s2 + 2 * j + 1], sc, -msc));
          pp[j] = p0 + p1;
          w[j] = pack_bf16x2(p0, p1);
        }
        ps[s2] = (pp[0] + pp[1]) + (pp[2] + pp[3]);
        pb[s2][u] = as_bf16x8(w);
      }
      lsum[u] += ps[0] + ps[1];
    }
    // V fragments through the same kind of ring (DH / 16 of them)
    bf16x8 vf[RING];
    auto vread = [&](int i) {
      const int dt = i >> 1, s2 = i & 1;
      return as_bf16x8(*reinterpret_cast<const u32x4*>(
          &Vs[buf][(32 * dt + col) * VS + 32 * t + 16 * G + 8 * s2]));
    };
#pragma unroll
    for (int p = 0; p < RING; ++p) vf[p] = vread(p);
#pragma unroll
    for (int i = 0; i < NKK; ++i) {
#pragma unroll
      for (int u = 0; u < NU; ++u) o[i >> 1][u] = mfma32x32x16(vf[i % RING], pb[i & 1][u], o[i >> 1][u]);
      if (i + RING < NKK) vf[i % RING] = vread(i + RING);
    }
  };

  auto tile = [&](int buf, int k0) {
    const bool live0 = wave_live && k0 < wave_kend;
    const bool live1 = wave_live && k0 + 32 < wave_kend;
    floatx16 st0[NU], st1[NU];
    if (live0) qk(buf, 0, st0);
    if (live1) qk(buf, 1, st1);
    if (live0) {
      if ((k0 + 32 > nk) || (CAUSAL && k0 + 31 > wq0)) mask(st0, k0, 0);
      soft_pv(st0, buf, 0);
    }
    if (live1) {
      if ((k0 + 64 > nk) || (CAUSAL && k0 + 63 > wq0)) mask(st1, k0, 1);
      soft_pv(st1, buf, 1);
    }
  };

  if constexpr (!DEEP) {
    // loads one tile ahead: fetched during tile it, stored after it
    gload(0, 0);
    sstore(0, 0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const int buf = it & 1;
      if (it + 1 < ntiles) gload(0, it + 1);
      tile(buf, it * KT);
      if (it + 1 < ntiles) sstore(0, buf ^ 1);
      __syncthreads();
    }
  } else {
    // loads two tiles ahead: register set s holds the tile stored at the
    // start of the step that computes from the other LDS buffer
    gload(0, 0);
    sstore(0, 0);
    if (ntiles > 1) gload(0, 1);
    if (ntiles > 2) gload(1, 2);
    __syncthreads();
    auto step = [&](int it, int set) {
      const int buf = it & 1;
      if (it + 1 < ntiles) sstore(set, buf ^ 1);
      if (it + 3 < ntiles) gload(set, it + 3);
      tile(buf, it * KT);
      __syncthreads();
    };
    int it = 0;
    for (; it + 1 < ntiles; it += 2) {
      step(it, 0);
      step(it + 1, 1);
    }
    if (it < ntiles) step(it, 0);
  }

  float gsum = 0.0f;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int my_q = wq0 + 32 * u + col;
    const float l = lsum[u] + __shfl_xor(lsum[u], 32, 64);
    const float inv = VP ? 1.0f : 1.0f / l;
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
            v[e] = o[dt][u][4 * q4 + e] * inv;
            gsum += fabsf(v[e]);
          }
          const uint64_t pk = uint64_t(pack_bf16x2(v[0], v[1])) |
                              (uint64_t(pack_bf16x2(v[2], v[3])) << 32);
          *reinterpret_cast<uint64_t*>(orow + d0) = pk;
        }
      if (!VP && G == 0) a.lse[bs * n_pad + my_q] = mref[u] * sc + log2f(l);
    }
  }
  gsum = wave_sum(gsum);
  if (lane == 0) red[wave] = gsum;
  __syncthreads();
  if (tid == 0) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) t += red[w];
    a.gpart[bs * a.nqb + qb] = t;
  }
}

// ------------------------------------------------------------------ bf16 column sums

template <int DH, bool CAUSAL>
__global__ void __launch_bounds__(256)
attn_colsum_bf16(AttnArgs a) {
  constexpr int QT = 128;      // queries per iteration
  constexpr int QS = DH + 8;
  constexpr int NQC = QT * DH / 8 / 256;
  __shared__ __attribute__((aligned(16))) bf16_t Qs[2][QT * QS];
  __shared__ __attribute__((aligned(16))) float Ls[2][QT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = lane >> 5, col = lane & 31;
  const XcdItem item = xcd_item(int(ceil_div(a.nk, kAttnKBlock)), a.h_kept, a.batch);
  if (!item.valid) return;
  const int b = item.b, s = item.s;
  const int k0 = item.blk * kAttnKBlock;
  const int n = a.n, n_pad = a.n_pad, nk = a.nk, nk_pad = a.nk_pad;
  const int64_t bs = int64_t(b) * a.h_kept + s;
  const bf16_t* Q = static_cast<const bf16_t*>(a.q) + bs * n_pad * DH;
  const bf16_t* K = static_cast<const bf16_t*>(a.kk) + bs * nk_pad * DH;
  const float* L = a.lse + bs * n_pad;
  const int kw = k0 + 64 * wave;

  // K^T operand: lane holds K[key kw + 32t + col][16kk + 8G .. +8]
  bf16x8 kf[2][DH / 16];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = min(kw + 32 * t + col, nk_pad - 1);
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk)
      kf[t][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(K + int64_t(key) * DH + 16 * kk + 8 * G));
  }
  const float sc = kLog2e / sqrtf(float(DH));
  float acc[2][4] = {};

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
      // st[t][r]: query qt0 + 32u + 8(r/4) + 4G + r%4, key kw + 32t + col;
      // register r adds into partial sum r%4 (four independent chains)
      const int qa = qt0 + 32 * u;
      const bool need_mask = (qa + 31 >= n) || (CAUSAL && qa < kw + 64);
      float4 l4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        l4[q] = *reinterpret_cast<const float4*>(&Ls[buf][32 * u + 8 * q + 4 * G]);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = 32 * u + 8 * (r >> 2) + 4 * G + (r & 3);
          const int qi = qt0 + ql;
          const float l2 = l4[r >> 2][r & 3];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int key = kw + 32 * t + col;
            const float p = fast_exp2(fmaf(st[t][r], sc, -l2));
            const bool keep = qi < n && (!CAUSAL || key <= qi);
            acc[t][r & 3] += keep ? p : 0.0f;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float l2 = l4[r >> 2][r & 3];
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[t][r & 3] += fast_exp2(fmaf(st[t][r], sc, -l2));
        }
      }
    }
    if (it + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float v = xor32_sum((acc[t][0] + acc[t][1]) + (acc[t][2] + acc[t][3]));
    const int key = kw + 32 * t + col;
    if (G == 0 && key < nk) a.colsum[bs * n_pad + key] = v;
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
    // local value pruning: probabilities below the threshold leave P V
    const float tau = a.v_threshold;
    for (int j = lane; j < n; j += 64) {
      const float p = S[r * n_pad + j] * inv;
      S[r * n_pad + j] = p >= tau ? p : 0.0f;
    }
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
  const int64_t bs = int64_t(b) * a.h_kept + s;
  const float* Q = static_cast<const float*>(a.q) + bs * n_pad * dh;
  const float* K = static_cast<const float*>(a.k) + bs * n_pad * dh;
  const float* L = a.lse + bs * n_pad;
  const float scale = kLog2e / sqrtf(float(dh));
  if (j < n) {
    float acc = 0.0f;
    for (int i = CAUSAL ? j : 0; i < n; ++i) {
      float d = 0.0f;
      for (int c = 0; c < dh; ++c) d = fmaf(Q[int64_t(i) * dh + c], K[int64_t(j) * dh + c], d);
      acc += fast_exp2(d * scale - L[i]);
    }
    a.colsum[bs * n_pad + j] = acc;
  }
}

// The importance reduction alone (when no tiled output projection follows
// to carry it): one workgroup per 256 entries of a sequence.
__global__ void __launch_bounds__(256)
importance_kernel(PrefillImp p) {
  prefill_importance_block(p, int(blockIdx.x));
}

PrefillImp prefill_imp(const AttnArgs& a) {
  PrefillImp p{};
  p.colsum = a.colsum;
  p.gpart = a.gpart;
  p.lse = a.lse;
  p.lse_out = a.lse_out;
  p.a = a.a;
  p.g = a.g;
  p.head_idx = a.head_idx;
  p.head_keys = a.head_keys;
  p.batch = a.batch;
  p.h_kept = a.h_kept;
  p.H = a.H;
  p.n = a.n;
  p.n_pad = a.n_pad;
  p.nk = a.nk;
  p.nqb = a.nqb;
  p.pieces = int(ceil_div(a.n, 256));
  p.pending = 1;
  return p;
}

// After the column sums: hand the importance pass to the caller, or run it.
int finish_importance(const AttnArgs& a, hipStream_t stream) {
  if (a.imp_out) {
    *a.imp_out = prefill_imp(a);
    return SPATTEN_OK;
  }
  return launch_prefill_importance(prefill_imp(a), stream);
}

// Per-head pruning: the kept tokens of slot s (head_keys[b, s, 0 .. nk-1])
// gathered from the layer's K [.., n_pad, DH] and V^T [.., DH, n_pad] into
// the slot's own K [.., nk_pad, DH] and V^T [.., DH, nk_pad] (columns past
// nk of a gathered 64-key tile are zero). grid (nk / 64, h_kept, batch).
template <int DH>
__global__ void __launch_bounds__(256)
gather_keys_bf16(AttnArgs a) {
  __shared__ int tok[64];
  const int j0 = blockIdx.x * 64, s = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t bs = int64_t(b) * a.h_kept + s;
  if (tid < 64) tok[tid] = j0 + tid < a.nk ? a.head_keys[bs * a.nk + j0 + tid] : -1;
  __syncthreads();
  const bf16_t* K = static_cast<const bf16_t*>(a.k) + bs * a.n_pad * DH;
  const bf16_t* VT = static_cast<const bf16_t*>(a.vt) + bs * DH * a.n_pad;
  bf16_t* Kc = static_cast<bf16_t*>(const_cast<void*>(a.kk)) + bs * a.nk_pad * DH;
  bf16_t* VTc = static_cast<bf16_t*>(const_cast<void*>(a.vtk)) + bs * DH * a.nk_pad;
  for (int c = tid; c < 64 * DH / 8; c += 256) {
    const int r = c / (DH / 8), c8 = (c % (DH / 8)) * 8;
    if (tok[r] >= 0)
      *reinterpret_cast<u32x4*>(Kc + int64_t(j0 + r) * DH + c8) =
          *reinterpret_cast<const u32x4*>(K + int64_t(tok[r]) * DH + c8);
  }
  for (int c = tid; c < DH * 8; c += 256) {
    const int d = c >> 3, j8 = (c & 7) * 8;
    bf16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = tok[j8 + e];
      v[e] = t >= 0 ? VT[int64_t(d) * a.n_pad + t] : bf16_t(0);
    }
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = uint32_t(v[2 * e]) | (uint32_t(v[2 * e + 1]) << 16);
    *reinterpret_cast<u32x4*>(VTc + int64_t(d) * a.nk_pad + j0 + j8) = w;
  }
}

template <int DH, bool CAUSAL>
int run_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.head_keys) {
    const dim3 gk(unsigned(ceil_div(a.nk, 64)), a.h_kept, a.batch);
    SPATTEN_TIMED("gather_keys", stream, gather_keys_bf16<DH><<<gk, 256, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
  }
  // 32 queries per wave: more resident waves hide the MFMA -> softmax ->
  // MFMA latency chain better than larger per-wave tiles
  constexpr int QB = attn_qblock(DH), NU = 1, MINW = DH == 64 ? 3 : 1;
  const dim3 g1(xcd_grid(ceil_div(a.n, QB) * a.h_kept * a.batch));
  SPATTEN_TIMED("attn_fwd", stream,
                attn_fwd_bf16<DH, CAUSAL, NU, MINW><<<g1, 2 * QB / NU, 0, stream>>>(a));
  SPATTEN_LAUNCH_CHECK();
  if (a.v_threshold > 0.0f) {
    SPATTEN_TIMED("attn_fwd_vprune", stream,
                  (attn_fwd_bf16<DH, CAUSAL, NU, MINW, true><<<g1, 2 * QB / NU, 0, stream>>>(a)));
    SPATTEN_LAUNCH_CHECK();
  }
  const dim3 g2(xcd_grid(ceil_div(a.nk, kAttnKBlock) * a.h_kept * a.batch));
  SPATTEN_TIMED("attn_colsum", stream, attn_colsum_bf16<DH, CAUSAL><<<g2, 256, 0, stream>>>(a));
  SPATTEN_LAUNCH_CHECK();
  return finish_importance(a, stream);
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
  return finish_importance(a, stream);
}

}  // namespace

int launch_prefill_importance(const PrefillImp& p, hipStream_t stream) {
  if (!p.pending || p.batch == 0 || p.pieces == 0) return SPATTEN_OK;
  SPATTEN_TIMED("importance", stream,
                importance_kernel<<<unsigned(p.pieces * p.batch), 256, 0, stream>>>(p));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

int launch_attention(const AttnArgs& a, hipStream_t stream) {
  if (a.dtype == SPATTEN_F32) return a.causal ? run_f32<true>(a, stream) : run_f32<false>(a, stream);
  if (a.dh == 64) return a.causal ? run_bf16<64, true>(a, stream) : run_bf16<64, false>(a, stream);
  if (a.dh == 128) return a.causal ? run_bf16<128, true>(a, stream) : run_bf16<128, false>(a, stream);
  return SPATTEN_EUNSUPPORTED;
}

}  // namespace spatten
