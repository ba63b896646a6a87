// Tile constants and workspace layout shared by the HIP-free validator and
// the kernels. Plain C++ (no HIP headers) so that the argument checks can be
// built and tested with the host compiler alone.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/spatten.h"

#if defined(__HIPCC__)
#define SPATTEN_HD __host__ __device__
#else
#define SPATTEN_HD
#endif

namespace spatten {

// Prefill token rows of Q, K, V^T are padded per (sequence, head) to this
// multiple so attention tiles never read past a head's slab.
constexpr int kTokPad = 256;
// Prefill attention (bf16 MFMA path): queries per workgroup in the forward
// (O, LSE) kernel - 32 per wave; 128 for head dim 64, 256 (eight waves
// sharing each K/V tile) for larger heads - and keys per workgroup in the
// column-sum kernel.
SPATTEN_HD constexpr int attn_qblock(int dh) { return dh == 64 ? 128 : 256; }
constexpr int kAttnKBlock = 256;
// fp32 attention: query rows per workgroup.
constexpr int kAttnF32Rows = 8;
// Decode: cache entries per chunk of the split value-pruning path, and the
// most cache rows whose scores one value-pruning workgroup keeps in LDS
// (longer caches take the split path).
constexpr int kDecChunk = 32;
constexpr int kVrowMaxRows = 4096;
// In-place compaction: most rows one call may keep per sequence (the
// selection is staged in LDS), and the longest row it moves (row units are
// counted in 32-bit integers).
constexpr int kInplaceMaxK = 8192;
constexpr int64_t kInplaceMaxRowBytes = int64_t(1) << 26;

SPATTEN_HD inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
SPATTEN_HD inline int64_t ceil_div(int64_t v, int64_t m) { return (v + m - 1) / m; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Byte offsets of every scratch array inside the caller's workspace.
struct PrefillWs {
  int64_t n_pad, nqb;
  int64_t nkb;
  int64_t nk, nk_pad;  // keys per head (per-head pruning: the kept ones)
  size_t q, k, vt, o, lse, colsum, gpart, kk, vtk, total;
};

struct DecodeWs {
  int64_t lc, lc_pad, nchunk;
  size_t q, knew, vnew, scores, mpart, lpart, opart, lse, cmax, kcount, o, total;
};

inline size_t dtype_bytes(int dt) { return dt == SPATTEN_BF16 ? 2 : 4; }

// Workspace of spatten_ada_select.
struct AdaWs {
  size_t inv, listR, listN, listV, cnt, rc, ac, total;
};
inline AdaWs ada_ws(int64_t batch, int64_t T) {
  AdaWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  const size_t n = size_t(batch) * size_t(T);
  w.inv = take(n * 4);
  w.listR = take(n * 4);
  w.listN = take(n * 4);
  w.listV = take(n * 4);
  w.cnt = take(size_t(batch) * 16);
  w.rc = take(n * 4);
  w.ac = take(n * 4);
  w.total = off;
  return w;
}

inline PrefillWs prefill_ws(const spatten_layer_desc& d) {
  PrefillWs w{};
  const int64_t B = d.batch, n = d.n_tokens, h = d.n_heads_kept, dh = d.head_dim;
  const size_t es = dtype_bytes(d.dtype);
  w.n_pad = round_up(n, kTokPad);
  const int64_t rows = d.dtype == SPATTEN_BF16 ? attn_qblock(d.head_dim) : kAttnF32Rows;
  w.nqb = ceil_div(n, rows);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  w.q = take(B * h * w.n_pad * dh * es);
  w.k = take(B * h * w.n_pad * dh * es);
  w.vt = take(B * h * w.n_pad * dh * es);
  w.o = take(B * n * h * dh * es);
  w.lse = take(B * h * w.n_pad * 4);
  w.colsum = take(B * h * w.n_pad * 4);
  w.gpart = take(B * h * w.nqb * 4);
  const bool per_head = d.per_head != 0;
  w.nk = per_head ? d.n_keys : n;
  w.nk_pad = round_up(w.nk, kTokPad);
  w.kk = take(per_head ? B * h * w.nk_pad * dh * es : 0);
  w.vtk = take(per_head ? B * h * w.nk_pad * dh * es : 0);
  w.nkb = ceil_div(w.nk, kAttnKBlock);
  w.total = off;
  return w;
}

inline DecodeWs decode_ws(const spatten_layer_desc& d) {
  DecodeWs w{};
  const int64_t B = d.batch, H = d.n_heads, dh = d.head_dim, D = H * dh;
  w.lc = int64_t(d.cache_len) + 1;
  w.lc_pad = round_up(w.lc, kDecChunk);
  w.nchunk = w.lc_pad / kDecChunk;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  w.q = take(B * D * 2);
  w.knew = take(B * D * 2);
  w.vnew = take(B * D * 2);
  w.scores = take(B * H * w.lc_pad * 4);
  // chunk statistics and partial outputs: only the split value-pruning
  // path uses them
  const bool split = d.v_threshold > 0.0f && w.lc_pad > kVrowMaxRows;
  w.mpart = take(split ? B * H * w.nchunk * 4 : 0);
  w.lpart = take(split ? B * H * w.nchunk * 4 : 0);
  w.opart = take(split ? B * H * w.nchunk * dh * 4 : 0);
  w.lse = take(B * H * 4);
  w.cmax = take(B * H * 4);
  w.kcount = take(split ? B * H * w.nchunk * 4 : 0);

  w.o = take(B * D * 2);
  w.total = off;
  return w;
}

}  // namespace spatten
