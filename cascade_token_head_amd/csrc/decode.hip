// Decode attention: one new query per sequence against the kept K/V cache,
// with cumulative token importance (SpAtten, section II "Attention-based NLP
// models": generation handles one new token per step against cached K and
// V) and progressive quantization (section III "Progressive Quantization";
// "E. ... Progressive Quantization": MSBs first, LSBs fetched and the row
// recomputed when its largest probability is below a threshold).
//
// The cache is token-major [B, cap, D], so one cache row holds every head
// of one token. A workgroup owns (sequence, 64-entry chunk) and streams the
// chunk's rows once, coalesced: each thread owns one 8-dim column group
// (one head's slice), reduces its partial dot with the 7 neighbouring lanes
// of the same head, and accumulates p * v for its column group. Chunks are
// combined per (b, h) in a second kernel (split-K over the cache length, so
// a few hundred rows still fill 256 CUs). Scores stay in a small fp32 stash
// so the importance kernel can form exact normalised probabilities.
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace spatten {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int CH = kDecChunk;
constexpr int kMaxHeads = 32;

enum { kBf16 = 0, kMsb = 1, kFull = 2 };

// Eight cache values of column group c of row j before the row scale:
// bf16 values, 16*msb (MSB plane only, LSBs taken as zero) or the full
// code 16*msb + lsb.
template <int KIND>
__device__ __forceinline__ void load8(const DecodeArgs& a, bool is_v, int64_t row, int c, int D,
                                      float* out) {
  if (KIND == kBf16) {
    const bf16_t* base = static_cast<const bf16_t*>(is_v ? a.v_cache : a.k_cache);
    const u32x4 w = *reinterpret_cast<const u32x4*>(base + row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = __uint_as_float(w[e] << 16);
      out[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
    const uint8_t* mp = is_v ? a.v_msb : a.k_msb;
    const uint32_t m = *reinterpret_cast<const uint32_t*>(mp + row * (D / 2) + 4 * c);
    uint32_t l = 0;
    if (KIND == kFull) {
      const uint8_t* lp = is_v ? a.v_lsb : a.k_lsb;
      l = *reinterpret_cast<const uint32_t*>(lp + row * (D / 2) + 4 * c);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int mn = int((m >> (4 * e)) & 15u);
      const int ms = mn >= 8 ? mn - 16 : mn;
      const int code = 16 * ms + (KIND == kFull ? int((l >> (4 * e)) & 15u) : 0);
      out[e] = float(code);
    }
  }
}

template <int KIND>
__device__ __forceinline__ float row_scale(const DecodeArgs& a, bool is_v, int64_t row) {
  if (KIND == kBf16) return 1.0f;
  return (is_v ? a.v_scale : a.k_scale)[row];
}

// grid (nchunk, B); block = (D/8) * R threads
template <int KIND>
__global__ void __launch_bounds__(256)
decode_partial(DecodeArgs a) {
  __shared__ float S[kMaxHeads][CH];
  __shared__ int hflag[kMaxHeads];
  __shared__ float obuf[256 * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int H = a.H, dh = a.dh, D = H * dh;
  const int V = D / 8, R = blockDim.x / V;
  const int c = tid % V, r = tid / V;
  const int h = (8 * c) / dh;
  const int j0 = chunk * CH;
  const int nwaves = blockDim.x >> 6;

  if (KIND == kMsb && chunk == 0 && b == 0 && tid == 0) a.queue[0] = 0;
  if (KIND == kFull) {
    if (tid < H) hflag[tid] = a.flags[b * H + tid];
    __syncthreads();
    int any = 0;
    for (int i = 0; i < H; ++i) any |= hflag[i];
    if (!any) return;
  }
  const bool active = r < R && (KIND != kFull || hflag[h]);

  float q[8];
  if (active) {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + int64_t(b) * D + 8 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = bf16_to_f32(qp[e]);
  }
  const float sc = kLog2e / sqrtf(float(dh));
  for (int jl = r; jl < CH; jl += R) {
    const int j = j0 + jl;
    float part = 0.0f;
    float ks = 0.0f;
    if (active && j < a.lc) {
      float kv[8];
      const int64_t row = int64_t(b) * a.cap + j;
      load8<KIND>(a, false, row, c, D, kv);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf(q[e], kv[e], part);
      ks = row_scale<KIND>(a, false, row);
    }
    part += __shfl_xor(part, 1, 64);
    part += __shfl_xor(part, 2, 64);
    part += __shfl_xor(part, 4, 64);
    if (r < R && (c & 7) == 0 && (KIND != kFull || hflag[h])) {
      const float sv = j < a.lc ? part * ks * sc : -INFINITY;
      S[h][jl] = sv;
      if (j < a.lc) a.scores[(int64_t(b) * H + h) * a.lc_pad + j] = sv;
    }
  }
  __syncthreads();
  // per-head chunk statistics; S becomes exp2(S - m)
  for (int hh = wave; hh < H; hh += nwaves) {
    if (KIND == kFull && !hflag[hh]) continue;
    const float v = S[hh][lane];
    const float m = wave_max(v);
    const float e = fast_exp2(v - m);
    const float l = wave_sum(e);
    S[hh][lane] = e;
    if (lane == 0) {
      const int64_t i = (int64_t(b) * H + hh) * a.nchunk + chunk;
      a.mpart[i] = m;
      a.lpart[i] = l;
    }
  }
  __syncthreads();
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (active) {
    for (int jl = r; jl < CH; jl += R) {
      const int j = j0 + jl;
      if (j >= a.lc) break;
      float vv[8];
      const int64_t row = int64_t(b) * a.cap + j;
      load8<KIND>(a, true, row, c, D, vv);
      const float w = S[h][jl] * row_scale<KIND>(a, true, row);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, vv[e], acc[e]);
    }
  }
  // reduce the R key phases of each column group
  if (r > 0 && active) {
#pragma unroll
    for (int e = 0; e < 8; ++e) obuf[((r - 1) * V + c) * 8 + e] = acc[e];
  }
  __syncthreads();
  if (r == 0 && active) {
    for (int rr = 1; rr < R; ++rr)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += obuf[((rr - 1) * V + c) * 8 + e];
    const int d0 = 8 * c - h * dh;
    float* op = a.opart + ((int64_t(b) * H + h) * a.nchunk + chunk) * dh + d0;
#pragma unroll
    for (int e = 0; e < 8; ++e) op[e] = acc[e];
  }
}

// One wave per (b, h): combine chunk statistics into lse, max probability
// and the normalised output row.
//   phase 0: every row, write o.
//   phase 1: every row; rows with max p < threshold are flagged and queued
//            for recompute, the others write o.
//   phase 2: queued rows only (after the recompute pass), write o.
__global__ void __launch_bounds__(64)
decode_combine(DecodeArgs a, int phase) {
  const int lane = threadIdx.x;
  int b, h;
  if (phase == 2) {
    if (int(blockIdx.x) >= a.queue[0]) return;
    const int e = a.queue[1 + blockIdx.x];
    b = e / a.H;
    h = e - b * a.H;
  } else {
    b = blockIdx.x / a.H;
    h = blockIdx.x - b * a.H;
  }
  const int64_t bh = int64_t(b) * a.H + h;
  float M = -INFINITY;
  for (int ci = lane; ci < a.nchunk; ci += 64) M = fmaxf(M, a.mpart[bh * a.nchunk + ci]);
  M = wave_max(M);
  float L = 0.0f;
  for (int ci = lane; ci < a.nchunk; ci += 64)
    L += a.lpart[bh * a.nchunk + ci] * fast_exp2(a.mpart[bh * a.nchunk + ci] - M);
  L = wave_sum(L);
  const float lse2 = M + log2f(L);
  const float cmax = 1.0f / L;  // largest probability: exp2(M - lse2)
  bool write_o = true;
  if (lane == 0) {
    a.lse[bh] = lse2;
    if (phase != 2) a.cmax[bh] = cmax;
  }
  if (phase == 1) {
    const bool flag = cmax < a.threshold;
    write_o = !flag;
    if (lane == 0) {
      a.flags[bh] = flag ? 1 : 0;
      if (a.recompute) a.recompute[bh] = flag ? 1 : 0;
      if (flag) {
        const int slot = atomicAdd(a.queue, 1);
        a.queue[1 + slot] = int(bh);
      }
    }
  } else if (phase == 0 && a.recompute && lane == 0) {
    a.recompute[bh] = 0;
  }
  if (!write_o) return;
  const float inv = 1.0f / L;
  for (int d = lane; d < a.dh; d += 64) {
    float acc = 0.0f;
    for (int ci = 0; ci < a.nchunk; ++ci)
      acc += a.opart[(bh * a.nchunk + ci) * a.dh + d] * fast_exp2(a.mpart[bh * a.nchunk + ci] - M);
    static_cast<bf16_t*>(a.o)[int64_t(b) * a.H * a.dh + h * a.dh + d] = f32_to_bf16(acc * inv);
  }
}

// a[b, j] += sum_h exp2(score[b, h, j] - lse2[b, h]) for j < lc
__global__ void __launch_bounds__(256)
decode_importance(DecodeArgs a) {
  __shared__ float lse[kMaxHeads];
  const int b = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (threadIdx.x < a.H) lse[threadIdx.x] = a.lse[int64_t(b) * a.H + threadIdx.x];
  __syncthreads();
  if (j >= a.lc) return;
  float acc = 0.0f;
  for (int h = 0; h < a.H; ++h)
    acc += fast_exp2(a.scores[(int64_t(b) * a.H + h) * a.lc_pad + j] - lse[h]);
  a.a[int64_t(b) * a.cap + j] += acc;
}

}  // namespace

int launch_decode(const DecodeArgs& a, bool quantized, hipStream_t stream) {
  const int D = a.H * a.dh;
  const int V = D / 8;
  int R = 256 / V;
  if (R < 1) R = 1;
  const dim3 gp(a.nchunk, a.batch);
  const int threads = V * R;
  if (threads > 256 || a.H > kMaxHeads || (V * 8 != D)) return SPATTEN_EUNSUPPORTED;
  if (!quantized) {
    SPATTEN_TIMED("decode_attn", stream, decode_partial<kBf16><<<gp, threads, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
    SPATTEN_TIMED("decode_combine", stream, decode_combine<<<a.batch * a.H, 64, 0, stream>>>(a, 0));
    SPATTEN_LAUNCH_CHECK();
  } else {
    SPATTEN_TIMED("pq_attn_msb", stream, decode_partial<kMsb><<<gp, threads, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
    SPATTEN_TIMED("decode_combine", stream, decode_combine<<<a.batch * a.H, 64, 0, stream>>>(a, 1));
    SPATTEN_LAUNCH_CHECK();
    SPATTEN_TIMED("pq_attn_recompute", stream, decode_partial<kFull><<<gp, threads, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
    SPATTEN_TIMED("decode_combine", stream, decode_combine<<<a.batch * a.H, 64, 0, stream>>>(a, 2));
    SPATTEN_LAUNCH_CHECK();
  }
  const dim3 gi(unsigned(ceil_div(a.lc, 256)), a.batch);
  SPATTEN_TIMED("decode_importance", stream, decode_importance<<<gi, 256, 0, stream>>>(a));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

}  // namespace spatten
