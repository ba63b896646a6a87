// Decode attention: one new query per sequence against the kept K/V cache,
// with cumulative token importance (SpAtten, section II "Attention-based NLP
// models": generation handles one new token per step against cached K and
// V) and progressive quantization ("A. Cascade Token Pruning", bullet "Progressive Quantization";
// "E. ... Progressive Quantization": MSBs first, LSBs fetched and the row
// recomputed when its largest probability is below a threshold).
//
// The cache is token-major [B, cap, D], so one cache row holds every head
// of one token. decode_partial: a workgroup owns (sequence, 32-entry chunk)
// and streams the chunk's K rows, then its V rows, once and coalesced. Each
// thread owns one 8-dim column group (one head's slice) of every R-th row of
// the chunk and issues all of its row loads before using any of them, so a
// thread keeps up to 16 loads in flight; partial dots are reduced with the 7
// neighbouring lanes of the same head. Chunks are combined per (sequence,
// head): split-K over the cache length, so a few hundred rows still fill 256
// CUs. Scores stay in a small fp32 stash so the importance pass can form the
// exact normalised probabilities.
//
// Quantized caches: the MSB pass first codes this step's k and v rows into
// the planes (in the workgroup that owns the new row), then scores and
// accumulates with 16 * msb; decode_flag marks each (sequence, head) row
// whose largest MSB-pass probability is below the threshold and appends it
// to the recompute queue; decode_recompute runs one workgroup per (queued
// row, chunk) over both planes of that head only. decode_finish combines
// what is left, writes O and adds the probabilities that produced O to the
// token importance.
//
// Local value pruning ("A. Cascade Token Pruning", bullet "Local Value Pruning": after the softmax
// a head drops its low-probability V vectors). A V row can only be skipped
// once the row's exact probabilities are known, i.e. after the softmax over
// the whole cache. decode_vrow gives each (sequence, head) row one
// workgroup that keeps all of the row's scores in LDS, so it reads K, forms
// the probabilities and then fetches only the V head slices (128 bytes of a
// cache row) that reach the threshold; decode_finish adds the importance.
// Caches too long for LDS take a split path: a K-only scores pass with
// per-chunk statistics, decode_vprune (exact probabilities per chunk,
// importance, kept V rows) and decode_vsum (sum of the chunk outputs).
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace spatten {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int CH = kDecChunk;  // cache entries per chunk
// one 32-lane half-wave holds a head's chunk statistics, and the recompute
// kernel maps its 64 threads to 32 rows x 2 halves of a head
static_assert(CH == 32, "decode kernels are written for 32-row chunks");
constexpr int KB = 16;         // rows per load batch
constexpr int kMaxHeads = 32;
constexpr int kRecomputeSlots = 128;

enum { kBf16 = 0, kMsb = 1 };

template <int KIND>
struct RawRow {
  using T = u32x4;  // 8 bf16 values
};
template <>
struct RawRow<kMsb> {
  using T = uint32_t;  // 8 MSB nibbles
};

template <int KIND>
__device__ __forceinline__ typename RawRow<KIND>::T load_row(const void* bf, const uint8_t* msb,
                                                             int64_t row, int c, int D) {
  if constexpr (KIND == kBf16)
    return *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(bf) + row * D + 8 * c);
  else
    return *reinterpret_cast<const uint32_t*>(msb + row * (D / 2) + 4 * c);
}

// signed MSB nibble e of an 8-nibble word
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

// grid (nchunk, B); block = (D/8) * R threads, R rows of the chunk at a time.
// WITH_V = false stops after the scores and chunk statistics.
template <int KIND, bool WITH_V = true>
__global__ void __launch_bounds__(256)
decode_partial(DecodeArgs a) {
  using Raw = typename RawRow<KIND>::T;
  __shared__ float S[kMaxHeads][CH];
  __shared__ float obuf[256 * 8];
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

  if constexpr (KIND == kMsb) {
    if (chunk == 0 && b == 0 && tid == 0) a.queue[0] = 0;
    if (a.knew && chunk == (a.lc - 1) / CH) {
      // this workgroup owns the new row: code it before reading it (waves 0
      // and 1 are always full, since the block has at least 128 threads)
      const int64_t nr = rowb + a.lc - 1;
      if (wave == 0)
        quantize_row_wave<bf16_t>(static_cast<const bf16_t*>(a.knew) + int64_t(b) * D, D,
                                  a.k_msb + nr * (D / 2), a.k_lsb + nr * (D / 2), a.k_scale + nr);
      else if (wave == 1)
        quantize_row_wave<bf16_t>(static_cast<const bf16_t*>(a.vnew) + int64_t(b) * D, D,
                                  a.v_msb + nr * (D / 2), a.v_lsb + nr * (D / 2), a.v_scale + nr);
      __threadfence_block();
      __syncthreads();
    }
  }

  float q[8];
  {
    const u32x4 w =
        *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(a.q) + int64_t(b) * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q[2 * e] = __uint_as_float(w[e] << 16);
      q[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  const float sc = kLog2e / sqrtf(float(dh));
  // MSB dots use nibble + 8: sum q (n + 8) - 8 sum q
  float qsum8 = 0.0f;
  if constexpr (KIND == kMsb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) qsum8 += q[e];
    qsum8 *= 8.0f;
  }

  // Rows past the cache end are read at row lc-1 (a valid address) and
  // masked: their score is -inf, so their weight in P V is exactly 0.
  auto row_of = [&](int tt) {
    const int j = j0 + r + R * tt;
    return rowb + (j < a.lc ? j : a.lc - 1);
  };

  // ---- scores
  for (int t0 = 0; t0 < kpt; t0 += KB) {
    Raw raw[KB];
    float ks[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int64_t row = row_of(t0 + u < kpt ? t0 + u : t0);
      raw[u] = load_row<KIND>(a.k_cache, a.k_msb, row, c, D);
      if constexpr (KIND == kMsb) ks[u] = a.k_scale[row];
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      float d = 0.0f;
      if constexpr (KIND == kBf16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          d = fmaf(q[2 * e], __uint_as_float(raw[u][e] << 16), d);
          d = fmaf(q[2 * e + 1], __uint_as_float(raw[u][e] & 0xffff0000u), d);
        }
      } else {
        float nv[8];
        nibbles_plus8(raw[u], nv);
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(q[e], nv[e], d);
        d = (d - qsum8) * 16.0f;
      }
      d += __shfl_xor(d, 1, 64);
      d += __shfl_xor(d, 2, 64);
      d += __shfl_xor(d, 4, 64);
      if constexpr (KIND == kMsb) d *= ks[u];
      const int jl = r + R * (t0 + u), j = j0 + jl;
      if (t0 + u < kpt && (c & 7) == 0) {
        const float sv = j < a.lc ? d * sc : -INFINITY;
        S[h][jl] = sv;
        if (j < a.lc) a.scores[(int64_t(b) * H + h) * a.lc_pad + j] = sv;
      }
    }
  }

  // V rows of the first batch are in flight across the softmax barrier
  Raw vraw[KB];
  float vs[KB];
  auto load_v = [&](int t0) {
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int64_t row = row_of(t0 + u < kpt ? t0 + u : t0);
      vraw[u] = load_row<KIND>(a.v_cache, a.v_msb, row, c, D);
      if constexpr (KIND == kMsb) vs[u] = a.v_scale[row];
    }
  };
  if constexpr (WITH_V) load_v(0);
  __syncthreads();
  // ---- per-head chunk statistics, two heads per wave (32 lanes each);
  // S becomes exp2(S - m)
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
    S[hh][l32] = e;
    if (l32 == 0) {
      const int64_t i = (int64_t(b) * H + hh) * a.nchunk + chunk;
      a.mpart[i] = m;
      a.lpart[i] = l;
    }
  }
  if constexpr (!WITH_V) return;
  __syncthreads();
  // ---- P V for this thread's column group
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float wsum = 0.0f;  // MSB path: sum of weights, to remove the +8 offset
  for (int t0 = 0; t0 < kpt; t0 += KB) {
    if (t0 > 0) load_v(t0);
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (t0 + u >= kpt) break;
      const float p = S[h][r + R * (t0 + u)];
      if constexpr (KIND == kBf16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(p, __uint_as_float(vraw[u][e] << 16), acc[2 * e]);
          acc[2 * e + 1] = fmaf(p, __uint_as_float(vraw[u][e] & 0xffff0000u), acc[2 * e + 1]);
        }
      } else {
        const float w = 16.0f * p * vs[u];
        float nv[8];
        nibbles_plus8(vraw[u], nv);
        wsum += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, nv[e], acc[e]);
      }
    }
  }
  if constexpr (KIND == kMsb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(-8.0f, wsum, acc[e]);
  }
  // reduce the R row phases of each column group
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

// Cache rows one decode_vrow workgroup keeps scores for in LDS.
constexpr int kVrowMaxRows = 4096;

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
// thread layout of decode_partial. Each half-wave combines one head's chunk
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
        vraw[u] = load_row<kBf16>(a.v_cache, nullptr, rowb + j0 + jl, c, D);
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

// One wave combines the chunk statistics of row (b, h) into its log2-sum-exp
// (returned) and 1 / sum (the largest probability, exp2(M - lse2)); with
// write_o it also writes the normalised bf16 output row (lane = dim, dh 64).
// The loads are issued up front as one round: lane i's chunk statistics
// (chunks i, i + 64, ...) and, for the output, the first kPre chunks'
// partials of dim `lane`. Lane i's first chunk weight is broadcast with
// readlane; chunks past kPre follow in batches of eight loads.
constexpr int kPre = 16;
__device__ float combine_row(const DecodeArgs& a, int b, int h, bool write_o, float* cmax) {
  const int lane = threadIdx.x & 63;
  const int64_t bh = int64_t(b) * a.H + h;
  const float* mp = a.mpart + bh * a.nchunk;
  const float* lp = a.lpart + bh * a.nchunk;
  const float* op = a.opart + bh * a.nchunk * a.dh + lane;
  float ov[kPre];
  if (write_o) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) ov[u] = u < a.nchunk ? op[int64_t(u) * a.dh] : 0.0f;
  }
  const bool has = lane < a.nchunk;
  const float m0 = has ? mp[lane] : -INFINITY;
  const float l0 = has ? lp[lane] : 0.0f;
  // this lane's running (max, sum) over its chunks
  float M = m0, Ls = l0;
  for (int ci = lane + 64; ci < a.nchunk; ci += 64) {
    const float m = mp[ci], l = lp[ci];
    const float mn = fmaxf(M, m);
    Ls = Ls * fast_exp2(M - mn) + l * fast_exp2(m - mn);
    M = mn;
  }
  const float Mw = wave_max(M);
  const float L = wave_sum(M == -INFINITY ? 0.0f : Ls * fast_exp2(M - Mw));
  const float inv = 1.0f / L;
  if (cmax) *cmax = inv;
  if (write_o) {
    const float w0 = has ? fast_exp2(m0 - Mw) : 0.0f;
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < kPre; ++u)
      acc += ov[u] * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w0), u));
    for (int g0 = 0; g0 < a.nchunk; g0 += 64) {
      const int cnt = a.nchunk - g0 < 64 ? a.nchunk - g0 : 64;
      const float wl = g0 == 0 ? w0 : (lane < cnt ? fast_exp2(mp[g0 + lane] - Mw) : 0.0f);
      for (int k = g0 == 0 ? kPre : 0; k < cnt; k += 8) {
        float ovb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) ovb[u] = k + u < cnt ? op[int64_t(g0 + k + u) * a.dh] : 0.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          acc += ovb[u] * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), k + u));
      }
    }
    static_cast<bf16_t*>(a.o)[int64_t(b) * a.H * a.dh + h * a.dh + lane] = f32_to_bf16(acc * inv);
  }
  return Mw + log2f(L);
}

// Quantized caches, after the MSB pass: one wave per (b, h). A row whose
// largest MSB-pass probability is below the threshold is flagged and queued
// for recompute; the others write O now.
__global__ void __launch_bounds__(64)
decode_flag(DecodeArgs a) {
  const int b = blockIdx.x / a.H, h = blockIdx.x - b * a.H;
  const int64_t bh = int64_t(b) * a.H + h;
  float cmax;
  const float lse2 = combine_row(a, b, h, false, &cmax);
  const bool flag = cmax < a.threshold;
  if (!flag) combine_row(a, b, h, true, nullptr);
  if (threadIdx.x == 0) {
    a.lse[bh] = lse2;
    a.cmax[bh] = cmax;
    a.flags[bh] = flag ? 1 : 0;
    if (a.recompute) a.recompute[bh] = flag ? 1 : 0;
    if (flag) a.queue[1 + atomicAdd(a.queue, 1)] = int(bh);
  }
}

// Recompute queued (b, h) rows with both planes of K and V (code = 16 *
// msb + lsb). grid (nchunk, slots); workgroup (chunk, s) takes queue
// entries s, s + slots, ... ; thread t = (row t/2 of the chunk, 32-dim half
// t%2 of the head). Rewrites the row's scores and chunk partials.
__global__ void __launch_bounds__(64)
decode_recompute(DecodeArgs a) {
  __shared__ float ob[CH][65];
  const int count = a.queue[0];
  const int t = threadIdx.x, jl = t >> 1, half = t & 1;
  const int D = a.H * a.dh;
  const int chunk = blockIdx.x;
  const int j = chunk * CH + jl;
  const bool valid = j < a.lc;
  const float sc = kLog2e / sqrtf(float(a.dh));
  for (int slot = blockIdx.y; slot < count; slot += gridDim.y) {
    const int e = a.queue[1 + slot];
    const int b = e / a.H, h = e - b * a.H;
    const int64_t bh = int64_t(b) * a.H + h;
    const int64_t row = int64_t(b) * a.cap + (valid ? j : a.lc - 1);
    const int64_t off = row * (D / 2) + (h * a.dh + 32 * half) / 2;
    const u32x4 km = *reinterpret_cast<const u32x4*>(a.k_msb + off);
    const u32x4 kl = *reinterpret_cast<const u32x4*>(a.k_lsb + off);
    const u32x4 vm = *reinterpret_cast<const u32x4*>(a.v_msb + off);
    const u32x4 vl = *reinterpret_cast<const u32x4*>(a.v_lsb + off);
    const float ksc = a.k_scale[row], vsc = a.v_scale[row];
    const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(a.q) +
                                                     int64_t(b) * D + h * a.dh + 32 * half);
    float d = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32x4 qw = qp[w];
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const float qv = __uint_as_float((n & 1) ? (qw[n >> 1] & 0xffff0000u) : (qw[n >> 1] << 16));
        const float code = 16.0f * msb_val(km[w], n) + float((kl[w] >> (4 * n)) & 15u);
        d = fmaf(qv, code, d);
      }
    }
    d += __shfl_xor(d, 1, 64);
    const float s = valid ? d * ksc * sc : -INFINITY;
    if (valid && half == 0) a.scores[bh * a.lc_pad + j] = s;
    float m = s;
#pragma unroll
    for (int o = 32; o > 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float p = fast_exp2(s - m);
    float l = half == 0 ? p : 0.0f;
    l = wave_sum(l);
    const float w = p * vsc;
    __syncthreads();  // previous entry's column sums are done with ob
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int n = 0; n < 8; ++n)
        ob[jl][32 * half + 8 * x + n] =
            w * (16.0f * msb_val(vm[x], n) + float((vl[x] >> (4 * n)) & 15u));
    __syncthreads();
    float acc = 0.0f;
    for (int rr = 0; rr < CH; ++rr) acc += ob[rr][t];
    a.opart[(bh * a.nchunk + chunk) * a.dh + t] = acc;
    if (t == 0) {
      a.mpart[bh * a.nchunk + chunk] = m;
      a.lpart[bh * a.nchunk + chunk] = l;
    }
  }
}

// One workgroup per sequence, one wave per head (up to 16 waves): combine
// the rows not combined yet (mode 0: every row; 1, quantized: the
// recomputed ones; 2: none, every row's lse is written), then
// a[b, j] += sum_h exp2(score[b, h, j] - lse2[b, h]) for j < lc (with
// per_head, a[b, h, j] += exp2(score[b, h, j] - lse2[b, h])).
enum { kFinishAll = 0, kFinishQuantized = 1, kFinishLseReady = 2 };
__global__ void __launch_bounds__(1024)
decode_finish(DecodeArgs a, int mode) {
  const bool quantized = mode == kFinishQuantized;
  __shared__ float lse[kMaxHeads];
  const int b = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6, nt = blockDim.x;
  const float* sp = a.scores + int64_t(b) * a.H * a.lc_pad;
  // The importance operands of this thread's first entry (per head: its
  // first eight (head, entry) pairs) are requested before the heads are
  // combined, so their latency overlaps the combine.
  const int total = a.per_head ? a.H * a.lc : a.lc;
  float* ab = a.a + int64_t(b) * (a.per_head ? a.H : 1) * a.cap;
  float sv0[kMaxHeads], av0 = 0.0f;
  float pv[8], pa[8];
  int pi[8], ph[8];
  if (a.per_head) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = threadIdx.x + u * nt;
      ph[u] = 0;
      if (i < total) {
        const int h = i / a.lc, j = i - h * a.lc;
        ph[u] = h;
        pi[u] = h * a.cap + j;
        pv[u] = sp[int64_t(h) * a.lc_pad + j];
        pa[u] = ab[pi[u]];
      }
    }
  } else if (int(threadIdx.x) < a.lc) {
#pragma unroll
    for (int h = 0; h < kMaxHeads; ++h)
      sv0[h] = h < a.H ? sp[int64_t(h) * a.lc_pad + threadIdx.x] : 0.0f;
    av0 = ab[threadIdx.x];
  }
  for (int h = wave; h < a.H; h += nw) {
    const int64_t bh = int64_t(b) * a.H + h;
    if (mode == kFinishAll || (quantized && a.flags[bh])) {
      float cmax;
      const float l2 = combine_row(a, b, h, true, &cmax);
      if (lane == 0) {
        lse[h] = l2;
        a.lse[bh] = l2;
        if (!quantized) {
          a.cmax[bh] = cmax;
          if (a.recompute) a.recompute[bh] = 0;
        }
      }
    } else if (lane == 0) {
      lse[h] = a.lse[bh];
    }
    if (lane == 0 && a.v_kept && mode != kFinishLseReady) a.v_kept[bh] = a.lc;
  }
  __syncthreads();
  if (a.per_head) {
    // a[b, h, j] += exp2(score[b, h, j] - lse2[b, h]) over the H * lc
    // (head, entry) pairs, eight pairs' loads in flight per thread
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (int(threadIdx.x) + u * nt < total) ab[pi[u]] = pa[u] + fast_exp2(pv[u] - lse[ph[u]]);
    for (int i0 = threadIdx.x + 8 * nt; i0 < total; i0 += 8 * nt) {
      float sv[8], av[8];
      int ai[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * nt;
        if (i < total) {
          const int h = i / a.lc, j = i - h * a.lc;
          ai[u] = h * a.cap + j;
          sv[u] = sp[int64_t(h) * a.lc_pad + j] - lse[h];
          av[u] = ab[ai[u]];
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u * nt < total) ab[ai[u]] = av[u] + fast_exp2(sv[u]);
    }
    return;
  }
  // a[b, j] += sum_h exp2(score[b, h, j] - lse2[b, h])
  if (int(threadIdx.x) < a.lc) {
    float acc = 0.0f;
#pragma unroll
    for (int h = 0; h < kMaxHeads; ++h)
      if (h < a.H) acc += fast_exp2(sv0[h] - lse[h]);
    ab[threadIdx.x] = av0 + acc;
  }
  for (int j = threadIdx.x + nt; j < a.lc; j += nt) {
    float acc = 0.0f;
    for (int h0 = 0; h0 < a.H; h0 += 8) {
      float sv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        sv[u] = h0 + u < a.H ? sp[int64_t(h0 + u) * a.lc_pad + j] : -INFINITY;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (h0 + u < a.H) acc += fast_exp2(sv[u] - lse[h0 + u]);
    }
    ab[j] += acc;
  }
}

}  // namespace

int launch_decode(const DecodeArgs& a, bool quantized, hipStream_t stream) {
  const int D = a.H * a.dh;
  const int V = D / 8;
  int R = 256 / V;
  if (R < 1) R = 1;
  while (R > 1 && CH % R != 0) --R;
  const int threads = V * R;
  // the partial kernel assumes whole 8-lane head groups (dh 64), at least
  // two full waves and at most 256 threads
  if (a.dh != 64 || a.H > kMaxHeads || threads > 256 || threads < 128)
    return SPATTEN_EUNSUPPORTED;
  const dim3 gp(a.nchunk, a.batch);
  const int fw = a.H < 16 ? a.H : 16;
  if (!quantized && a.v_threshold > 0.0f && a.lc_pad <= kVrowMaxRows) {
    SPATTEN_TIMED("decode_vrow", stream,
                  decode_vrow<<<a.batch * a.H, 256, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
    SPATTEN_TIMED("decode_finish", stream,
                  decode_finish<<<a.batch, 64 * fw, 0, stream>>>(a, kFinishLseReady));
    SPATTEN_LAUNCH_CHECK();
    return SPATTEN_OK;
  }
  if (!quantized && a.v_threshold > 0.0f) {
    SPATTEN_TIMED("decode_scores", stream,
                  (decode_partial<kBf16, false><<<gp, threads, 0, stream>>>(a)));
    SPATTEN_LAUNCH_CHECK();
    SPATTEN_TIMED("decode_vprune", stream, decode_vprune<<<gp, threads, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
    SPATTEN_TIMED("decode_vsum", stream, decode_vsum<<<a.batch * a.H, 64, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
    return SPATTEN_OK;
  }
  if (!quantized) {
    SPATTEN_TIMED("decode_attn", stream, decode_partial<kBf16><<<gp, threads, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
  } else {
    SPATTEN_TIMED("pq_attn_msb", stream, decode_partial<kMsb><<<gp, threads, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
    SPATTEN_TIMED("decode_flag", stream, decode_flag<<<a.batch * a.H, 64, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
    const int slots = a.batch * a.H < kRecomputeSlots ? a.batch * a.H : kRecomputeSlots;
    const dim3 gr(a.nchunk, slots);
    SPATTEN_TIMED("pq_attn_recompute", stream, decode_recompute<<<gr, 64, 0, stream>>>(a));
    SPATTEN_LAUNCH_CHECK();
  }
  SPATTEN_TIMED("decode_finish", stream,
                decode_finish<<<a.batch, 64 * fw, 0, stream>>>(
                    a, quantized ? kFinishQuantized : kFinishAll));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

}  // namespace spatten
