// Decode token importance (SpAtten, "B. Motivation": a token's importance
// is the probability mass it receives, summed over heads and queries, and
// cumulative over layers and steps), applied once every score and row
// log2-sum-exp of the layer is in the stash. It runs as extra workgroups of
// the output projection (or alone), so it costs no launch of its own.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace spatten {

// Workgroup `blk` of the pass: sequence blk / pieces, and its share of the
// sequence's entries (span entries; with per_head the H * lc (head, entry)
// pairs): a[b, j] += sum_h exp2(score[b, h, j] - lse2[b, h]), the heads
// added in order, or a[b, h, j] += exp2(score[b, h, j] - lse2[b, h]).
__device__ __forceinline__ void importance_block(const ImpArgs& p, int blk) {
  const int b = blk / p.pieces, piece = blk - b * p.pieces;
  const int nt = blockDim.x, t = threadIdx.x;
  const float* sp = p.scores + int64_t(b) * p.H * p.lc_pad;
  const float* lp = p.lse + int64_t(b) * p.H;
  const int e0 = piece * p.span;
  if (p.per_head) {
    const int total = p.H * p.lc;
    const int e1 = e0 + p.span < total ? e0 + p.span : total;
    float* ab = p.a + int64_t(b) * p.H * p.cap;
    for (int i0 = e0 + t; i0 < e1; i0 += 4 * nt) {
      float sv[4], av[4];
      int ai[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * nt;
        if (i < e1) {
          const int h = i / p.lc, j = i - h * p.lc;
          ai[u] = h * p.cap + j;
          sv[u] = sp[int64_t(h) * p.lc_pad + j] - lp[h];
          av[u] = ab[ai[u]];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + u * nt < e1) ab[ai[u]] = av[u] + fast_exp2(sv[u]);
    }
    return;
  }
  const int e1 = e0 + p.span < p.lc ? e0 + p.span : p.lc;
  float* ab = p.a + int64_t(b) * p.cap;
  for (int j = e0 + t; j < e1; j += nt) {
    const float old = ab[j];
    float acc = 0.0f;
    for (int h0 = 0; h0 < p.H; h0 += 8) {
      float sv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        sv[u] = h0 + u < p.H ? sp[int64_t(h0 + u) * p.lc_pad + j] : 0.0f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (h0 + u < p.H) acc += fast_exp2(sv[u] - lp[h0 + u]);
    }
    ab[j] = old + acc;
  }
}

}  // namespace spatten
