// Decode attention: one new query per sequence against the kept K/V cache,
// with cumulative token importance (SpAtten, section II "Attention-based NLP
// models": generation handles one new token per step against cached K and
// V) and progressive quantization ("A. Cascade Token Pruning", bullet "Progressive Quantization";
// "E. ... Progressive Quantization": MSBs first, LSBs fetched and the row
// recomputed when its largest probability is below a threshold).
//
// The bf16 cache is token-major [B, cap, D], so one cache row holds every
// head of one token; the quantized planes are head-major [B, H, cap, dh/2],
// so one (sequence, head) slab is contiguous. Three families of kernels:
//
// decode_bh (dense and quantized): one workgroup per (sequence, head) row
// streams that head's slice of the whole cache with an online softmax per
// row group and writes the normalised output and the row's log2-sum-exp;
// no cross-workgroup combine. Quantized caches code this step's k and v
// rows into the planes first, score with 16 * msb, and recompute the whole
// row from both planes in the same workgroup when its largest MSB-pass
// probability is below the threshold.
//
// Local value pruning ("A. Cascade Token Pruning", bullet "Local Value
// Pruning": after the softmax a head drops its low-probability V vectors).
// A V row can only be skipped once the row's exact probabilities are known,
// i.e. after the softmax over the whole cache. decode_vrow gives each
// (sequence, head) row one workgroup that keeps all of the row's scores in
// LDS, so it reads K, forms the probabilities and then fetches only the V
// head slices (128 bytes of a cache row) that reach the threshold. Caches
// too long for LDS take a split path over 32-row chunks: decode_scores
// (K only, scores and per-chunk statistics), decode_vprune (exact
// probabilities per chunk, importance, kept V rows) and decode_vsum (sum of
// the chunk outputs).
//
// Token importance: every path leaves its fp32 scores in a stash; the
// importance pass (in the output projection's launch, or decode_importance)
// adds sum over heads of exp2(s - lse) to each kept token's score.
#include "common.hpp"
#include "importance.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace spatten {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int CH = kDecChunk;  // cache entries per chunk
// one 32-lane half-wave of decode_vprune holds a head's chunk statistics
static_assert(CH == 32, "decode kernels are written for 32-row chunks");
constexpr int KB = 16;         // rows per load batch
constexpr int kMaxHeads = 32;

enum { kBf16 = 0, kMsb = 1 };

template <int KIND>
__device__ __forceinline__ u32x4 load_row(const void* bf, int64_t row, int c, int D) {
  return *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(bf) + row * D + 8 * c);
}

// signed nibble e of an 8-nibble word
__device__ __forceinline__ float msb_val(uint32_t w, int e) {
  const int mn = int((w >> (4 * e)) & 15u);
  return float(mn >= 8 ? mn - 16 : mn);
}

// The 8 signed nibbles of a word, each offset by +8 (so 0..15): flipping a
// nibble's top bit maps two's-complement -8..7 to 0..15, and the even and
// odd nibbles then convert straight from bytes. u[e] = nibble e + 8.
__device__ __forceinline__ void nibbles_plus8(uint32_t w, float* u) {
  const uint32_t x = w ^ 0x88888888u;
  const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u[2 * k] = float((lo >> (8 * k)) & 0xffu);
    u[2 * k + 1] = float((hi >> (8 * k)) & 0xffu);
  }
}

// The 8 full int8 codes 16 * msb + lsb of a word pair, each offset by +128
// (so 0..255): the offset MSB nibble becomes the high half of a byte whose
// low half is the LSB nibble. u[e] = code e + 128.
__device__ __forceinline__ void codes_plus128(uint32_t wm, uint32_t wl, float* u) {
  const uint32_t x = wm ^ 0x88888888u;
  const uint32_t ev = ((x & 0x0F0F0F0Fu) << 4) | (wl & 0x0F0F0F0Fu);
  const uint32_t od = (x & 0xF0F0F0F0u) | ((wl >> 4) & 0x0F0F0F0Fu);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u[2 * k] = float((ev >> (8 * k)) & 0xffu);
    u[2 * k + 1] = float((od >> (8 * k)) & 0xffu);
  }
}

// Scores and per-chunk statistics only (the split value-pruning path, for
// caches whose scores do not fit one workgroup's LDS): grid (nchunk, B);
// block = (D/8) * R threads, R rows of the chunk at a time. A thread owns
// one 8-dim column group (one head's slice) of every R-th row of the chunk
// and issues all of its row loads before using them; partial dots reduce
// over the 8 lanes of a head.
__global__ void __launch_bounds__(256)
decode_scores(DecodeArgs a) {
  __shared__ float S[kMaxHeads][CH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int H = a.H, dh = a.dh, D = H * dh;
  const int V = D / 8, R = blockDim.x / V;
  const int c = tid % V, r = tid / V;
  const int h = (8 * c) / dh;
  const int j0 = chunk * CH;
  // a partial last wave (e.g. 160 threads for 5 heads) takes part in the
  // per-head statistics loop too, so it must count in the stride
  const int nwaves = (blockDim.x + 63) >> 6;
  const int kpt = CH / R;  // rows per thread
  const int64_t rowb = int64_t(b) * a.cap;
  float q[8];
  load8_f32(static_cast<const bf16_t*>(a.q) + int64_t(b) * D + 8 * c, q);
  const float sc = kLog2e / sqrtf(float(dh));
  // Rows past the cache end are read at row lc-1 (a valid address) and
  // masked with a -inf score.
  auto row_of = [&](int tt) {
    const int j = j0 + r + R * tt;
    return rowb + (j < a.lc ? j : a.lc - 1);
  };
  for (int t0 = 0; t0 < kpt; t0 += KB) {
    u32x4 raw[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) raw[u] = load_row<kBf16>(a.k_cache, row_of(t0 + u < kpt ? t0 + u : t0), c, D);
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d = fmaf(q[2 * e], __uint_as_float(raw[u][e] << 16), d);
        d = fmaf(q[2 * e + 1], __uint_as_float(raw[u][e] & 0xffff0000u), d);
      }
      d += __shfl_xor(d, 1, 64);
      d += __shfl_xor(d, 2, 64);
      d += __shfl_xor(d, 4, 64);
      const int jl = r + R * (t0 + u), j = j0 + jl;
      if (t0 + u < kpt && (c & 7) == 0) {
        const float sv = j < a.lc ? d * sc : -INFINITY;
        S[h][jl] = sv;
        if (j < a.lc) a.scores[(int64_t(b) * H + h) * a.lc_pad + j] = sv;
      }
    }
  }
  __syncthreads();
  // per-head chunk statistics, two heads per wave (32 lanes each)
  for (int hh = 2 * wave + (lane >> 5); hh < H; hh += 2 * nwaves) {
    const int l32 = lane & 31;
    const float v = S[hh][l32];
    float m = v;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float e = fast_exp2(v - m);
    float l = e;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    if (l32 == 0) {
      const int64_t i = (int64_t(b) * H + hh) * a.nchunk + chunk;
      a.mpart[i] = m;
      a.lpart[i] = l;
    }
  }
}


// Local value pruning, one workgroup per (sequence, head) row, grid B * H,
// 256 threads = 32 row groups x 8 lanes; lane c8 of row group g owns the
// 16-byte slice c8 (dims 8 c8 .. 8 c8 + 7) of rows g, g + 32, ... of the
// head. Needs lc_pad <= kVrowMaxRows and dh 64.
__global__ void __launch_bounds__(256)
decode_vrow(DecodeArgs a) {
  __shared__ float S[kVrowMaxRows];
  __shared__ float ob[32][65];
  __shared__ float red[8];
  __shared__ int kred[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = t >> 3, c8 = t & 7;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - b * a.H;
  const int D = a.H * 64;
  const int64_t rowb = int64_t(b) * a.cap;
  const int col = h * 64 + 8 * c8;
  const int lc = a.lc;
  const int nit = (lc + 31) >> 5;  // rows per row group
  const float tau = a.v_threshold;
  float q[8];
  {
    const u32x4 w =
        *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(a.q) + int64_t(b) * D + col);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q[2 * e] = __uint_as_float(w[e] << 16);
      q[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  const float sc = kLog2e / 8.0f;  // log2(e) / sqrt(64)
  const bf16_t* kc = static_cast<const bf16_t*>(a.k_cache) + col;
  const bf16_t* vc = static_cast<const bf16_t*>(a.v_cache) + col;
  // ---- scores of the whole row (rows past the end read row lc-1, unused)
  for (int i0 = 0; i0 < nit; i0 += KB) {
    u32x4 raw[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int j = g + 32 * (i0 + u);
      raw[u] = *reinterpret_cast<const u32x4*>(kc + (rowb + (j < lc ? j : lc - 1)) * D);
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d = fmaf(q[2 * e], __uint_as_float(raw[u][e] << 16), d);
        d = fmaf(q[2 * e + 1], __uint_as_float(raw[u][e] & 0xffff0000u), d);
      }
      d += __shfl_xor(d, 1, 64);
      d += __shfl_xor(d, 2, 64);
      d += __shfl_xor(d, 4, 64);
      const int j = g + 32 * (i0 + u);
      if (c8 == 0 && j < lc) {
        S[j] = d * sc;
        a.scores[int64_t(bh) * a.lc_pad + j] = d * sc;
      }
    }
  }
  __syncthreads();
  // ---- row log2-sum-exp
  float m = -INFINITY;
  for (int j = t; j < lc; j += 256) m = fmaxf(m, S[j]);
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float l = 0.0f;
  for (int j = t; j < lc; j += 256) l += fast_exp2(S[j] - M);
  l = wave_sum(l);
  if (lane == 0) red[4 + wave] = l;
  __syncthreads();
  const float L = (red[4] + red[5]) + (red[6] + red[7]);
  const float lse2 = M + log2f(L);
  // ---- P V over the rows that reach the threshold; the others are not read
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int kept = 0;
  for (int i0 = 0; i0 < nit; i0 += KB) {
    u32x4 vr[KB];
    float pw[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int j = g + 32 * (i0 + u);
      const float p = j < lc ? fast_exp2(S[j] - lse2) : 0.0f;
      if (j < lc && p >= tau) {
        vr[u] = *reinterpret_cast<const u32x4*>(vc + (rowb + j) * D);
        pw[u] = p;
        kept += c8 == 0 ? 1 : 0;
      } else {
        vr[u] = u32x4{0u, 0u, 0u, 0u};
        pw[u] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(pw[u], __uint_as_float(vr[u][e] << 16), acc[2 * e]);
        acc[2 * e + 1] = fmaf(pw[u], __uint_as_float(vr[u][e] & 0xffff0000u), acc[2 * e + 1]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) ob[g][8 * c8 + e] = acc[e];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) kept += __shfl_xor(kept, o, 64);
  if (lane == 0) kred[wave] = kept;
  __syncthreads();
  if (t < 64) {
    float o = 0.0f;
    for (int r = 0; r < 32; ++r) o += ob[r][t];
    static_cast<bf16_t*>(a.o)[int64_t(b) * D + h * 64 + t] = f32_to_bf16(o);
  }
  if (t == 0) {
    a.lse[bh] = lse2;
    a.cmax[bh] = 1.0f / L;
    if (a.v_kept) a.v_kept[bh] = (kred[0] + kred[1]) + (kred[2] + kred[3]);
    if (a.recompute) a.recompute[bh] = 0;
  }
}

// Local value pruning, after the K-only scores pass. grid (nchunk, B), the
// thread layout of decode_scores. Each half-wave combines one head's chunk
// statistics into its log2-sum-exp, forms the chunk's 32 probabilities and
// counts the kept rows; the workgroup then adds the chunk's importance
// (it owns those a entries) and accumulates p V over the kept rows only.
__global__ void __launch_bounds__(256)
decode_vprune(DecodeArgs a) {
  __shared__ float P[kMaxHeads][CH];
  __shared__ float obuf[256 * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int H = a.H, dh = a.dh, D = H * dh;
  const int V = D / 8, R = blockDim.x / V;
  const int c = tid % V, r = tid / V;
  const int h = (8 * c) / dh;
  const int j0 = chunk * CH;
  const int nwaves = (blockDim.x + 63) >> 6;
  const int kpt = CH / R;
  const int64_t rowb = int64_t(b) * a.cap;
  const float tau = a.v_threshold;

  for (int hh = 2 * wave + (lane >> 5); hh < H; hh += 2 * nwaves) {
    const int l32 = lane & 31;
    const int64_t bh = int64_t(b) * H + hh;
    const float* mp = a.mpart + bh * a.nchunk;
    const float* lp = a.lpart + bh * a.nchunk;
    float M = -INFINITY;
    for (int ci = l32; ci < a.nchunk; ci += 32) M = fmaxf(M, mp[ci]);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float L = 0.0f;
    for (int ci = l32; ci < a.nchunk; ci += 32) L += lp[ci] * fast_exp2(mp[ci] - M);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);
    const float lse2 = M + log2f(L);
    const int j = j0 + l32;
    const bool valid = j < a.lc;
    const float p = valid ? fast_exp2(a.scores[bh * a.lc_pad + j] - lse2) : 0.0f;
    P[hh][l32] = p;
    const uint64_t kept = __ballot(valid && p >= tau);
    if (l32 == 0) {
      a.kcount[bh * a.nchunk + chunk] = __popcll(kept >> (lane & 32) & 0xffffffffull);
      if (chunk == 0) {
        a.lse[bh] = lse2;
        a.cmax[bh] = 1.0f / L;
      }
    }
  }
  __syncthreads();
  if (tid < CH && j0 + tid < a.lc) {
    if (a.per_head) {
      for (int hh = 0; hh < H; ++hh) a.a[(int64_t(b) * H + hh) * a.cap + j0 + tid] += P[hh][tid];
    } else {
      float s = 0.0f;
      for (int hh = 0; hh < H; ++hh) s += P[hh][tid];
      a.a[rowb + j0 + tid] += s;
    }
  }
  // P V over this head's kept rows; a dropped row is not read
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int t0 = 0; t0 < kpt; t0 += KB) {
    u32x4 vraw[KB];
    float pw[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int jl = r + R * (t0 + u);
      const bool in = t0 + u < kpt;
      pw[u] = in ? P[h][jl] : 0.0f;
      if (in && j0 + jl < a.lc && pw[u] >= tau) {
        vraw[u] = load_row<kBf16>(a.v_cache, rowb + j0 + jl, c, D);
      } else {
        vraw[u] = u32x4{0u, 0u, 0u, 0u};
        pw[u] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(pw[u], __uint_as_float(vraw[u][e] << 16), acc[2 * e]);
        acc[2 * e + 1] = fmaf(pw[u], __uint_as_float(vraw[u][e] & 0xffff0000u), acc[2 * e + 1]);
      }
    }
  }
  if (r > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) obuf[((r - 1) * V + c) * 8 + e] = acc[e];
  }
  __syncthreads();
  if (r == 0) {
    for (int rr = 1; rr < R; ++rr)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += obuf[((rr - 1) * V + c) * 8 + e];
    const int d0 = 8 * c - h * dh;
    float* op = a.opart + ((int64_t(b) * H + h) * a.nchunk + chunk) * dh + d0;
#pragma unroll
    for (int e = 0; e < 8; ++e) op[e] = acc[e];
  }
}

// Value pruning, last step: one wave per (b, h), lane = output dim (dh 64).
// The chunk partials are already normalised, so O is their plain sum.
__global__ void __launch_bounds__(64)
decode_vsum(DecodeArgs a) {
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const float* op = a.opart + bh * a.nchunk * a.dh + lane;
  float acc = 0.0f;
  for (int k = 0; k < a.nchunk; k += 8) {
    float ov[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) ov[u] = k + u < a.nchunk ? op[int64_t(k + u) * a.dh] : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += ov[u];
  }
  static_cast<bf16_t*>(a.o)[bh * a.dh + lane] = f32_to_bf16(acc);
  int cnt = 0;
  for (int ci = lane; ci < a.nchunk; ci += 64) cnt += a.kcount[bh * a.nchunk + ci];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if (lane == 0) {
    if (a.v_kept) a.v_kept[bh] = cnt;
    if (a.recompute) a.recompute[bh] = 0;
  }
}

// ------------------------------------------------ one workgroup per (sequence, head)
//
// Dense and progressive-quantization decode: the workgroup streams its
// head's slice of every cache row (bf16: 128 bytes of K and of V;
// quantized: the 32-byte rows of its own slab of each plane it reads - the
// planes are head-major, so a workgroup's reads fill whole cache lines -
// plus the row scales), with K
// and V of a row requested together, and keeps an online softmax per row
// group: each load batch raises the group's reference maximum once and
// rescales its running sum and output. The groups then meet in LDS, so the
// workgroup ends with the row's exact log2-sum-exp and normalised output
// and no cross-workgroup combine is needed. Scores go to the stash for the
// importance pass (a = sum over heads of exp2(s - lse)). Workgroups are
// mapped so that the heads of one sequence, which read neighbouring slices
// of the same cache lines, run on one XCD and share its L2.
//
// Quantized caches: this step's k and v rows are coded into the planes by
// every head's workgroup for its own slice (each computes the same
// per-token scale from the whole row), kept in LDS and entered last. When
// the row's largest MSB-pass probability (1 / sum) is below the threshold,
// the workgroup recomputes the whole row at once with both planes of K and
// V. A quantized row has 512 threads (128 row groups of 4 lanes): the rows
// of a batch (B * H) are few, so each takes more of a CU.

template <int KIND>
struct BhCfg;
template <>
struct BhCfg<kBf16> {
  static constexpr int NT = 256;  // threads
  static constexpr int LPR = 8;   // lanes per cache row, 16 bytes (8 dims) of K and of V each
  static constexpr int DPL = 8;   // head dims per lane
  static constexpr int KB = 8;    // rows per lane per load batch
  static constexpr int WAVES = 4; // waves per SIMD it is built for
};
template <>
struct BhCfg<kMsb> {
  static constexpr int NT = 512;
  static constexpr int LPR = 4;   // lanes per cache row, 8 bytes (16 nibbles) of each plane
  static constexpr int DPL = 16;
  static constexpr int KB = 9;    // MSB pass; the recompute reads four planes, KBF rows a batch
  static constexpr int KBF = 4;
  static constexpr int WAVES = 2;
};

template <int DPL>
struct BhState {
  float m;      // reference maximum of the row group's scores (log2 units)
  float l;      // sum of exp2(s - m) over the group's rows
  float wsum;   // quantized: sum of the V weights, to remove the code offset
  float acc[DPL];
};

template <int DPL>
__device__ __forceinline__ void bh_reset(BhState<DPL>& st) {
  st.m = -INFINITY;
  st.l = 0.0f;
  st.wsum = 0.0f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) st.acc[e] = 0.0f;
}

// Raise the reference maximum to bm (if larger) and rescale what was summed.
template <int DPL>
__device__ __forceinline__ void bh_raise(BhState<DPL>& st, float bm) {
  if (bm > st.m) {
    const float r = fast_exp2(st.m - bm);  // 0 while nothing was summed
    st.l *= r;
    st.wsum *= r;
#pragma unroll
    for (int e = 0; e < DPL; ++e) st.acc[e] *= r;
    st.m = bm;
  }
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Keeps the loads requested before it in front of the code after it: the
// compiler would otherwise sink a pass's first batch of loads below the
// wait for the query (into the pass's loop), serialising two round trips.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }
// Returns w unchanged, from behind an empty asm statement: code using the
// result stays below an earlier issue_fence, and so does the wait for w.
__device__ __forceinline__ u32x4 after_fence(u32x4 w) {
  asm volatile("" : "+v"(w));
  return w;
}

// bf16 cache: rows r0..r1-1 of head h; row r0 + g + 32 i belongs to row group g.
// One load batch: this lane's 16-byte slices of K and V of KB rows.
struct BfRows {
  u32x4 k[BhCfg<kBf16>::KB], v[BhCfg<kBf16>::KB];
};

// Requests batch i0 (rows r0 + g + 32 (i0 + u)); past r1 a valid row is
// read and masked later.
__device__ __forceinline__ void bh_load_bf16(const DecodeArgs& a, int b, int h, int g, int cl,
                                             int r0, int r1, int i0, BfRows& t) {
  constexpr int NG = BhCfg<kBf16>::NT / BhCfg<kBf16>::LPR, KBb = BhCfg<kBf16>::KB;
  const int D = a.H * 64;
  const int64_t rowb = int64_t(b) * a.cap;
  const bf16_t* kc = static_cast<const bf16_t*>(a.k_cache) + h * 64 + 8 * cl;
  const bf16_t* vc = static_cast<const bf16_t*>(a.v_cache) + h * 64 + 8 * cl;
#pragma unroll
  for (int u = 0; u < KBb; ++u) {
    const int j = r0 + g + NG * (i0 + u);
    const int64_t row = rowb + (j < r1 ? j : r0);
    t.k[u] = *reinterpret_cast<const u32x4*>(kc + row * D);
    t.v[u] = *reinterpret_cast<const u32x4*>(vc + row * D);
  }
}

// The pass over the rows; t holds batch 0 on entry (requested by the caller
// before it waited for the query, so the two round trips overlap).
__device__ __forceinline__ void bh_pass_bf16(const DecodeArgs& a, int b, int h, int g, int cl,
                                             int r0, int r1, const float* q, BhState<8>& st,
                                             BfRows& t) {
  constexpr int NG = BhCfg<kBf16>::NT / BhCfg<kBf16>::LPR, KBb = BhCfg<kBf16>::KB;
  float* srow = a.scores + (int64_t(b) * a.H + h) * a.lc_pad;
  const float sc = kLog2e * 0.125f;  // log2(e) / sqrt(64)
  const int nit = (r1 - r0 + NG - 1) / NG;
  for (int i0 = 0; i0 < nit; i0 += KBb) {
    if (i0 > 0) bh_load_bf16(a, b, h, g, cl, r0, r1, i0, t);
    float s[KBb];
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < KBb; ++u) {
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d = fmaf(q[2 * e], __uint_as_float(t.k[u][e] << 16), d);
        d = fmaf(q[2 * e + 1], __uint_as_float(t.k[u][e] & 0xffff0000u), d);
      }
      d += __shfl_xor(d, 1, 64);
      d += __shfl_xor(d, 2, 64);
      d += __shfl_xor(d, 4, 64);
      const int j = r0 + g + NG * (i0 + u);
      s[u] = j < r1 ? d * sc : -INFINITY;
      if (cl == 0 && j < r1) srow[j] = s[u];
      bm = fmaxf(bm, s[u]);
    }
    bh_raise(st, bm);
#pragma unroll
    for (int u = 0; u < KBb; ++u) {
      const int j = r0 + g + NG * (i0 + u);
      const float p = j < r1 ? fast_exp2(s[u] - st.m) : 0.0f;
      st.l += p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st.acc[2 * e] = fmaf(p, __uint_as_float(t.v[u][e] << 16), st.acc[2 * e]);
        st.acc[2 * e + 1] = fmaf(p, __uint_as_float(t.v[u][e] & 0xffff0000u), st.acc[2 * e + 1]);
      }
    }
  }
}

// Offset codes of one lane's 16 dims of a row: MSB only (nibble + 8, the
// value being 16 * nibble) or both planes (code + 128).
template <bool FULL>
__device__ __forceinline__ void bh_codes(uint2 m, uint2 l, float* u) {
  if constexpr (FULL) {
    codes_plus128(m.x, l.x, u);
    codes_plus128(m.y, l.y, u + 8);
  } else {
    nibbles_plus8(m.x, u);
    nibbles_plus8(m.y, u + 8);
  }
}

// One row's score and its entry into the state: codes cu of K (offset),
// the K and V row scales, and the V codes cv.
template <bool FULL>
__device__ __forceinline__ float bh_q_dot(const float* q, float qsum, const float* cu, float ks) {
  const float kmul = FULL ? 1.0f : 16.0f;  // value = scale * kmul * code
  const float qoff = (FULL ? 128.0f : 8.0f) * qsum;
  float d = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) d = fmaf(q[e], cu[e], d);
  d = (d - qoff) * kmul;
  d += __shfl_xor(d, 1, 64);
  d += __shfl_xor(d, 2, 64);
  return d * ks * (kLog2e * 0.125f);
}

// Quantized cache: rows r0..r1-1 of head h read from the head-major planes
// (row r0 + g + 128 i belongs to row group g), MSB only or (FULL) both.
// VP (local value pruning): K only - the scores also go to sS, and V waits
// for the exact probabilities (bh_vpass_q).
template <bool FULL, bool VP = false>
__device__ __forceinline__ void bh_pass_q(const DecodeArgs& a, int b, int h, int g, int cl,
                                          int r0, int r1, const float* q, float qsum,
                                          BhState<16>& st, float* sS = nullptr) {
  constexpr int LPR = BhCfg<kMsb>::LPR, NG = BhCfg<kMsb>::NT / LPR;
  constexpr int KBq = FULL ? BhCfg<kMsb>::KBF : BhCfg<kMsb>::KB;
  // row scales: one per token [B, cap], or with per-head pruning one per
  // (head, slot) [B, H, cap], since each head's slot r holds its own entry
  const int64_t rowb = (a.per_head ? int64_t(b) * a.H + h : int64_t(b)) * a.cap;
  // head-major planes: this head's slab of 32-byte rows, this lane's 8 bytes
  const int64_t slab = (int64_t(b) * a.H + h) * a.cap * 32 + 8 * cl;
  float* srow = a.scores + (int64_t(b) * a.H + h) * a.lc_pad;
  const float kmul = FULL ? 1.0f : 16.0f;
  const int nit = (r1 - r0 + NG - 1) / NG;
  for (int i0 = 0; i0 < nit; i0 += KBq) {
    uint2 km[KBq], vm[KBq], kl[KBq], vl[KBq];
    float ks[KBq], vs[KBq];
#pragma unroll
    for (int u = 0; u < KBq; ++u) {
      const int j = r0 + g + NG * (i0 + u);
      const int jr = j < r1 ? j : r0;  // past the range: a valid row, masked
      const int64_t po = slab + int64_t(jr) * 32;
      km[u] = *reinterpret_cast<const uint2*>(a.k_msb + po);
      if constexpr (!VP) vm[u] = *reinterpret_cast<const uint2*>(a.v_msb + po);
      if constexpr (FULL) {
        kl[u] = *reinterpret_cast<const uint2*>(a.k_lsb + po);
        if constexpr (!VP) vl[u] = *reinterpret_cast<const uint2*>(a.v_lsb + po);
      } else {
        kl[u] = uint2{0u, 0u};
        if constexpr (!VP) vl[u] = uint2{0u, 0u};
      }
      ks[u] = a.k_scale[rowb + jr];
      if constexpr (!VP) vs[u] = a.v_scale[rowb + jr];
    }
    float s[KBq];
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < KBq; ++u) {
      float cu[16];
      bh_codes<FULL>(km[u], kl[u], cu);
      const float sv = bh_q_dot<FULL>(q, qsum, cu, ks[u]);
      const int j = r0 + g + NG * (i0 + u);
      s[u] = j < r1 ? sv : -INFINITY;
      if (cl == 0 && j < r1) {
        srow[j] = s[u];
        if constexpr (VP) sS[j] = s[u];
      }
      bm = fmaxf(bm, s[u]);
    }
    bh_raise(st, bm);
#pragma unroll
    for (int u = 0; u < KBq; ++u) {
      const int j = r0 + g + NG * (i0 + u);
      const float w = j < r1 ? fast_exp2(s[u] - st.m) : 0.0f;
      st.l += w;
      if constexpr (!VP) {
        const float wv = w * vs[u] * kmul;
        st.wsum += wv;
        float cu[16];
        bh_codes<FULL>(vm[u], vl[u], cu);
#pragma unroll
        for (int e = 0; e < 16; ++e) st.acc[e] = fmaf(wv, cu[e], st.acc[e]);
      }
    }
  }
}

// The new row (index lc-1) from its codes in LDS (MSB words, and LSB words
// for the recompute): enters the state of row group 0.
template <bool FULL, bool VP = false>
__device__ __forceinline__ void bh_new_row_q(const DecodeArgs& a, int b, int h, int g, int cl,
                                             const float* q, float qsum, BhState<16>& st,
                                             const uint32_t (*nw)[8], const uint32_t (*nlw)[8],
                                             const float* nscale, float* sS = nullptr) {
  if (g != 0) return;
  const int j = a.lc - 1;
  const float kmul = FULL ? 1.0f : 16.0f;
  const uint2 km = {nw[0][2 * cl], nw[0][2 * cl + 1]};
  const uint2 kl = {nlw[0][2 * cl], nlw[0][2 * cl + 1]};
  const uint2 vm = {nw[1][2 * cl], nw[1][2 * cl + 1]};
  const uint2 vl = {nlw[1][2 * cl], nlw[1][2 * cl + 1]};
  float cu[16];
  bh_codes<FULL>(km, kl, cu);
  const float s = bh_q_dot<FULL>(q, qsum, cu, nscale[0]);
  if (cl == 0) {
    a.scores[(int64_t(b) * a.H + h) * a.lc_pad + j] = s;
    if constexpr (VP) sS[j] = s;
  }
  bh_raise(st, s);
  const float w = fast_exp2(s - st.m);
  st.l += w;
  if constexpr (VP) return;
  const float wv = w * nscale[1] * kmul;
  st.wsum += wv;
  bh_codes<FULL>(vm, vl, cu);
#pragma unroll
  for (int e = 0; e < 16; ++e) st.acc[e] = fmaf(wv, cu[e], st.acc[e]);
}

// Local value pruning, quantized: the V rows of the exact probabilities
// p_j = exp2(sS[j] - lse2) >= tau only (rows 0..lc-2 from the planes, MSB
// only or FULL, the new row lc-1 from its codes in LDS), p_j V_j summed
// into st.acc with the code offset tracked in st.wsum; returns this lane's
// count of kept rows (counted once per row, by lane cl == 0).
template <bool FULL>
__device__ __forceinline__ int bh_vpass_q(const DecodeArgs& a, int b, int h, int g, int cl,
                                          float lse2, const float* sS, BhState<16>& st,
                                          const uint32_t (*nw)[8], const uint32_t (*nlw)[8],
                                          const float* nscale) {
  constexpr int LPR = BhCfg<kMsb>::LPR, NG = BhCfg<kMsb>::NT / LPR, KBV = 8;
  const float kmul = FULL ? 1.0f : 16.0f;
  const float tau = a.v_threshold;
  const int64_t rowb = (a.per_head ? int64_t(b) * a.H + h : int64_t(b)) * a.cap;
  const int64_t slab = (int64_t(b) * a.H + h) * a.cap * 32 + 8 * cl;
  int kept = 0;
  // batches of KBV rows per group: the kept rows' loads are all requested
  // before the first is used
  for (int i0 = 0; g + NG * i0 < a.lc; i0 += KBV) {
    uint2 vm[KBV], vl[KBV];
    float vs[KBV], pw[KBV];
#pragma unroll
    for (int u = 0; u < KBV; ++u) {
      const int j = g + NG * (i0 + u);
      const float p = j < a.lc ? fast_exp2(sS[j] - lse2) : 0.0f;
      const bool keep = j < a.lc && p >= tau;  // uniform over the row group's lanes
      pw[u] = keep ? p : 0.0f;
      kept += keep && cl == 0 ? 1 : 0;
      vm[u] = vl[u] = uint2{0u, 0u};
      vs[u] = 0.0f;
      if (keep && j == a.lc - 1) {  // the new row, from its codes in LDS
        vm[u] = uint2{nw[1][2 * cl], nw[1][2 * cl + 1]};
        vl[u] = uint2{nlw[1][2 * cl], nlw[1][2 * cl + 1]};
        vs[u] = nscale[1];
      } else if (keep) {
        const int64_t po = slab + int64_t(j) * 32;
        vm[u] = *reinterpret_cast<const uint2*>(a.v_msb + po);
        if (FULL) vl[u] = *reinterpret_cast<const uint2*>(a.v_lsb + po);
        vs[u] = a.v_scale[rowb + j];
      }
    }
#pragma unroll
    for (int u = 0; u < KBV; ++u) {
      const float wv = pw[u] * vs[u] * kmul;
      st.wsum += wv;
      float cu[16];
      bh_codes<FULL>(vm[u], vl[u], cu);
#pragma unroll
      for (int e = 0; e < 16; ++e) st.acc[e] = fmaf(wv, cu[e], st.acc[e]);
    }
  }
  return kept;
}

// The row groups of the workgroup meet: M = largest reference maximum, L =
// sum of every group's sum at M, and (threads 0..63) o = dim t of the
// unnormalised output at M.
template <int NT, int NG, int DPL>
__device__ __forceinline__ void bh_combine(const BhState<DPL>& st, int g, int cl,
                                           float (*red)[65], float* wred, float* M, float* L,
                                           float* o) {
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float wm = wave_max(st.m);
  __syncthreads();  // red and wred may still be read by an earlier combine
  if (lane == 0) wred[wave] = wm;
  __syncthreads();
  float Mb = wred[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) Mb = fmaxf(Mb, wred[w]);
  const float f = st.m > -INFINITY ? fast_exp2(st.m - Mb) : 0.0f;
  const float lw = wave_sum(cl == 0 ? st.l * f : 0.0f);
#pragma unroll
  for (int e = 0; e < DPL; ++e) red[g][DPL * cl + e] = st.acc[e] * f;
  if (lane == 0) wred[NW + wave] = lw;
  __syncthreads();
  *M = Mb;
  float Ls = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) Ls += wred[NW + w];
  *L = Ls;
  // every wave sums NG / NW of the row groups for all 64 dims, then wave 0
  // adds the NW partial rows (red rows 0..NW-1 are rewritten only after
  // every wave has read its own rows)
  constexpr int RPW = NG / NW;
  float part = 0.0f;
#pragma unroll
  for (int r = 0; r < RPW; ++r) part += red[wave * RPW + r][lane];
  __syncthreads();
  red[wave][lane] = part;
  __syncthreads();
  float acc = 0.0f;
  if (t < 64) {
#pragma unroll
    for (int w = 0; w < NW; ++w) acc += red[w][t];
  }
  *o = acc;
}

// grid B * H workgroups of BhCfg<KIND>::NT threads; head_dim 64, H <= 32.
// VP (quantized only): local value pruning, lc <= kVrowMaxRows.
template <int KIND, bool VP = false>
__global__ void __launch_bounds__(BhCfg<KIND>::NT, BhCfg<KIND>::WAVES)
decode_bh(DecodeArgs a) {
  constexpr int NT = BhCfg<KIND>::NT, LPR = BhCfg<KIND>::LPR, NG = NT / LPR;
  constexpr int DPL = BhCfg<KIND>::DPL, NW = NT / 64;
  static_assert(!VP || KIND == kMsb, "value pruning here is the quantized variant");
  __shared__ float red[NG][65];
  __shared__ float sS[VP ? kVrowMaxRows : 1];  // the row's scores (log2 units)
  __shared__ int kred[NW];
  __shared__ float wred[2 * NW];
  __shared__ uint32_t nw[2][8];   // new row of this head: [k, v] MSB words
  __shared__ uint32_t nlw[2][8];  // and LSB words
  __shared__ float nscale[2];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = t / LPR, cl = t - g * LPR;
  // Workgroups go to the 8 XCDs round-robin; map each XCD's share to a
  // contiguous range of (b, h) rows, so the heads of one sequence - which
  // read neighbouring slices of the same cache lines - share one L2.
  const int nb = int(gridDim.x);
  const int bh = (nb & 7) == 0 ? (int(blockIdx.x) & 7) * (nb >> 3) + (int(blockIdx.x) >> 3)
                               : int(blockIdx.x);
  const int b = bh / a.H, h = bh - b * a.H;
  const int D = a.H * 64;
  const bf16_t* qp = static_cast<const bf16_t*>(a.q) + int64_t(b) * D + h * 64 + DPL * cl;
  float q[DPL];
  float qsum = 0.0f;
  BhState<DPL> st;
  bh_reset(st);
  float M, L, o;
  float cm;
  bool flag = false;
  int vkept = a.lc;
  if constexpr (KIND == kBf16) {
    // the query's words are requested first and converted only after the
    // first batch of cache rows has been requested too
    const u32x4 qw = *reinterpret_cast<const u32x4*>(qp);
    BfRows rows;
    bh_load_bf16(a, b, h, g, cl, 0, a.lc, 0, rows);
    issue_fence();
    const u32x4 w = after_fence(qw);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q[2 * e] = __uint_as_float(w[e] << 16);
      q[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
    bh_pass_bf16(a, b, h, g, cl, 0, a.lc, q, st, rows);
    bh_combine<NT, NG, DPL>(st, g, cl, red, wred, &M, &L, &o);
    cm = 1.0f / L;
  } else {
    // the query first (requesting the first batch of plane rows before
    // its wait, as the bf16 path does, measured slower here)
    load8_f32(qp, q);
    load8_f32(qp + 8, q + 8);
#pragma unroll
    for (int e = 0; e < DPL; ++e) qsum += q[e];
    // this step's k and v rows: requested now, used after the old rows
    float xk[8], xv[8];
    const bool hasx = t < D / 8;
    if (hasx) {
      load8_f32(static_cast<const bf16_t*>(a.knew) + int64_t(b) * D + 8 * t, xk);
      load8_f32(static_cast<const bf16_t*>(a.vnew) + int64_t(b) * D + 8 * t, xv);
    }
    bh_pass_q<false, VP>(a, b, h, g, cl, 0, a.lc - 1, q, qsum, st, sS);
    // code the new row: per-token scale from the whole row, then this
    // head's 64 dims into the planes (the arithmetic of spatten_quantize_kv,
    // so every head's workgroup finds the same scale)
    float amk = 0.0f, amv = 0.0f;
    if (hasx) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        amk = fmaxf(amk, fabsf(xk[e]));
        amv = fmaxf(amv, fabsf(xv[e]));
      }
    }
    amk = wave_max(amk);
    amv = wave_max(amv);
    if (lane == 0) {
      wred[wave] = amk;
      wred[NW + wave] = amv;
    }
    __syncthreads();
    float mk = wred[0], mv = wred[NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      mk = fmaxf(mk, wred[w]);
      mv = fmaxf(mv, wred[NW + w]);
    }
    const float sk = mk / 127.0f, sv = mv / 127.0f;
    // the new row's scale slot: shared by the heads (written once), or per
    // head under per-head pruning (each head's workgroup writes its own)
    const int64_t nrow = (a.per_head ? int64_t(b) * a.H + h : int64_t(b)) * a.cap + a.lc - 1;
    if (wave < 2) {
      const bf16_t* src = static_cast<const bf16_t*>(wave == 0 ? a.knew : a.vnew) +
                          int64_t(b) * D + h * 64;
      const int qc = quant_code(bf16_to_f32(src[lane]), wave == 0 ? sk : sv);
      uint32_t mn = uint32_t((qc >> 4) & 15) << (4 * (lane & 7));
      uint32_t ln = uint32_t(qc & 15) << (4 * (lane & 7));
#pragma unroll
      for (int o2 = 1; o2 < 8; o2 <<= 1) {
        mn |= __shfl_xor(mn, o2, 64);
        ln |= __shfl_xor(ln, o2, 64);
      }
      if ((lane & 7) == 0) {
        const int w = lane >> 3;
        nw[wave][w] = mn;
        nlw[wave][w] = ln;
        const int64_t po = ((int64_t(b) * a.H + h) * a.cap + a.lc - 1) * 32 + 4 * w;
        uint8_t* mp = (wave == 0 ? a.k_msb : a.v_msb) + po;
        uint8_t* lp = (wave == 0 ? a.k_lsb : a.v_lsb) + po;
        *reinterpret_cast<uint32_t*>(mp) = mn;
        *reinterpret_cast<uint32_t*>(lp) = ln;
      }
    }
    if (t == 0) {
      nscale[0] = sk;
      nscale[1] = sv;
      if (h == 0 || a.per_head) {
        a.k_scale[nrow] = sk;
        a.v_scale[nrow] = sv;
      }
    }
    __syncthreads();
    bh_new_row_q<false, VP>(a, b, h, g, cl, q, qsum, st, nw, nlw, nscale, sS);
#pragma unroll
    for (int e = 0; e < 16; ++e) st.acc[e] = fmaf(-8.0f, st.wsum, st.acc[e]);
    bh_combine<NT, NG, DPL>(st, g, cl, red, wred, &M, &L, &o);
    cm = 1.0f / L;
    flag = cm < a.threshold;  // uniform: every thread read the same L
    if (flag) {
      // flat row: the old rows again with both planes, then the new row
      // from its codes in LDS (this workgroup wrote its planes; the scale
      // may come from another head's workgroup, so it is not read back)
      bh_reset(st);
      bh_pass_q<true, VP>(a, b, h, g, cl, 0, a.lc - 1, q, qsum, st, sS);
      bh_new_row_q<true, VP>(a, b, h, g, cl, q, qsum, st, nw, nlw, nscale, sS);
#pragma unroll
      for (int e = 0; e < 16; ++e) st.acc[e] = fmaf(-128.0f, st.wsum, st.acc[e]);
      bh_combine<NT, NG, DPL>(st, g, cl, red, wred, &M, &L, &o);
    }
    if constexpr (VP) {
      // exact probabilities against the final row log2-sum-exp; the V rows
      // below the threshold are not read. The groups' sums are already
      // normalised, so they meet at a common reference of 0 and L = 1.
      __syncthreads();  // sS complete
      const float lse2 = M + log2f(L);
      bh_reset(st);
      st.m = 0.0f;
      const int kc = flag ? bh_vpass_q<true>(a, b, h, g, cl, lse2, sS, st, nw, nlw, nscale)
                          : bh_vpass_q<false>(a, b, h, g, cl, lse2, sS, st, nw, nlw, nscale);
      const float off = flag ? -128.0f : -8.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) st.acc[e] = fmaf(off, st.wsum, st.acc[e]);
      const int kw = wave_sum_int(kc);
      if (lane == 0) kred[wave] = kw;
      float M2, L2;
      bh_combine<NT, NG, DPL>(st, g, cl, red, wred, &M2, &L2, &o);
      M = lse2;   // the row's statistics as the plain path reports them
      L = 1.0f;
      vkept = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) vkept += kred[w];
    }
  }
  if (t < 64) static_cast<bf16_t*>(a.o)[int64_t(b) * D + h * 64 + t] = f32_to_bf16(o / L);
  if (t == 0) {
    a.lse[bh] = M + log2f(L);
    a.cmax[bh] = cm;
    if (a.recompute) a.recompute[bh] = flag ? 1 : 0;
    if (a.v_kept) a.v_kept[bh] = vkept;
  }
}

// Importance of the entries a workgroup of the output projection (or of
// decode_importance) owns, after the attention has written every score
// and row log2-sum-exp.
__global__ void __launch_bounds__(256)
decode_importance(ImpArgs p) {
  importance_block(p, blockIdx.x);
}

}  // namespace

int launch_decode(const DecodeArgs& a, bool quantized, ImpArgs* imp, hipStream_t stream) {
  if (a.dh != 64 || a.H > kMaxHeads) return SPATTEN_EUNSUPPORTED;
  // the importance pass that follows reads the stash and the row LSE
  imp->scores = a.scores;
  imp->lse = a.lse;
  imp->a = a.a;
  imp->batch = a.batch;
  imp->H = a.H;
  imp->lc = a.lc;
  imp->lc_pad = a.lc_pad;
  imp->cap = a.cap;
  imp->per_head = a.per_head;
  imp->span = kImpSpan;
  imp->pieces = int(ceil_div(int64_t(a.per_head ? a.H : 1) * a.lc, kImpSpan));
  imp->pending = 1;
  if (!quantized && a.v_threshold > 0.0f && a.lc_pad <= kVrowMaxRows) {
    SPATTEN_TIMED("decode_vrow", stream, decode_vrow<<<a.batch * a.H, 256, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
    return SPATTEN_OK;
  }
  if (!quantized && a.v_threshold > 0.0f) {
    // split path: scores and chunk statistics, then exact probabilities per
    // chunk (importance included) with the kept V rows, then the sum
    const int D = a.H * a.dh;
    const int V = D / 8;
    int R = 256 / V;
    if (R < 1) R = 1;
    while (R > 1 && CH % R != 0) --R;
    const int threads = V * R;
    if (threads > 256 || threads < 128) return SPATTEN_EUNSUPPORTED;
    const dim3 gp(a.nchunk, a.batch);
    SPATTEN_TIMED("decode_scores", stream, (decode_scores<<<gp, threads, 0, stream>>>(a)));
    SPATTEN_LAUNCH_CHECK();
    SPATTEN_TIMED("decode_vprune", stream, decode_vprune<<<gp, threads, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
    SPATTEN_TIMED("decode_vsum", stream, decode_vsum<<<a.batch * a.H, 64, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
    imp->pending = 0;
    return SPATTEN_OK;
  }
  const int blocks = a.batch * a.H;
  if (!quantized) {
    SPATTEN_TIMED("decode_attn", stream,
                  decode_bh<kBf16><<<blocks, BhCfg<kBf16>::NT, 0, stream>>>(a));
  } else {
    if (a.v_threshold > 0.0f) {
      if (a.lc_pad > kVrowMaxRows) return SPATTEN_EUNSUPPORTED;
      SPATTEN_TIMED("pq_attn_vprune", stream,
                    (decode_bh<kMsb, true><<<blocks, BhCfg<kMsb>::NT, 0, stream>>>(a)));
    } else {
      SPATTEN_TIMED("pq_attn", stream,
                    decode_bh<kMsb><<<blocks, BhCfg<kMsb>::NT, 0, stream>>>(a));
    }
  }
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

int launch_importance(const ImpArgs& p, hipStream_t stream) {
  if (!p.pending || p.batch == 0) return SPATTEN_OK;
  SPATTEN_TIMED("decode_importance", stream,
                decode_importance<<<p.batch * p.pieces, 256, 0, stream>>>(p));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

}  // namespace spatten
