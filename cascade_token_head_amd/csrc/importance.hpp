// Token and head importance (SpAtten, "B. Motivation": a token's importance
// is the probability mass it receives, summed over heads and queries, and
// cumulative over layers and steps; a head's is the magnitude of its
// output). Decode applies it once every score and row log2-sum-exp of the
// layer is in the stash; prefill once the column sums and |O| partials are
// written. Both run as extra workgroups of the output projection's launch
// (or alone), so they cost no launch of their own.
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

// Prefill importance, workgroup blk (sequence blk / pieces, entries
// 256 * piece ..): the reduction the attention's column sums and |O|
// partials feed. Threads past 256 have nothing to do.
__device__ __forceinline__ void prefill_importance_block(const PrefillImp& p, int blk) {
  const int b = blk / p.pieces, piece = blk - b * p.pieces;
  const int t = threadIdx.x;
  if (t >= 256) return;
  const int j = piece * 256 + t;
  if (p.head_keys) {
    // per-head pruning: a[b, s, token] += column sum of key j of slot s
    if (j < p.nk)
      for (int s = 0; s < p.h_kept; ++s) {
        const int64_t bs = int64_t(b) * p.h_kept + s;
        p.a[bs * p.n + p.head_keys[bs * p.nk + j]] += p.colsum[bs * p.n_pad + j];
      }
  } else if (j < p.n) {
    float acc = 0.0f;
    for (int s = 0; s < p.h_kept; ++s) acc += p.colsum[(int64_t(b) * p.h_kept + s) * p.n_pad + j];
    p.a[int64_t(b) * p.n + j] += acc;
  }
  if (j < p.n && p.lse_out)
    for (int s = 0; s < p.h_kept; ++s)
      p.lse_out[(int64_t(b) * p.h_kept + s) * p.n + j] =
          p.lse[(int64_t(b) * p.h_kept + s) * p.n_pad + j] * 0.6931471805599453f;
  if (piece == 0 && t < p.h_kept) {
    float acc = 0.0f;
    for (int q = 0; q < p.nqb; ++q) acc += p.gpart[(int64_t(b) * p.h_kept + t) * p.nqb + q];
    p.g[int64_t(b) * p.H + p.head_idx[b * p.h_kept + t]] += acc;
  }
}

}  // namespace spatten
