// Internal launchers (not part of the C ABI). Each enqueues on `stream` and
// returns a spatten_status.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "layout.hpp"

namespace spatten {

int launch_topk(const float* scores, int batch, int n, int64_t row_stride, int k,
                int32_t* out_idx, float* kth, hipStream_t stream);

int launch_compact(int n_tensors, const void* const* src, void* const* dst,
                   const int64_t* row_bytes, const int64_t* sbs, const int64_t* dbs,
                   const int32_t* idx, int batch, int k, hipStream_t stream);

int launch_compact_inplace(int n_tensors, void* const* base, const int64_t* row_bytes,
                           const int64_t* row_pitch, const int64_t* bs, const int32_t* idx,
                           int batch, int n, int k, hipStream_t stream);

int launch_quantize(const void* kv, int dtype, int batch, int n, int dim, int head_dim,
                    int64_t kv_bs, uint8_t* msb, uint8_t* lsb, float* scale, int64_t pbs,
                    hipStream_t stream);

// Projections. QKV: for each kept head slot s of sequence b the rows
// head_idx[b, s]*dh .. +dh of wq/wk/wv (output-major) produce Q, K and V.
//   prefill: Q, K -> [B, h, n_pad, dh]; V -> transposed [B, h, dh, n_pad]
//   decode:  q -> q_out [B, D]; k, v -> k_out/v_out + b*kv_bs + s*dh + c
struct QkvArgs {
  int dtype, mode;
  const void* x;
  const void* w[3];
  const int32_t* head_idx;
  int batch, n, n_pad, h_kept, dh, D;
  void* q;
  void* k;
  void* vt;
  int64_t kv_bs;  // decode: elements between sequences in k/v outputs
};
int launch_qkv(const QkvArgs& a, hipStream_t stream);

// Decode token importance from the score stash and row LSE of one layer
// (see importance.hpp): blocks = batch * pieces, `span` entries each.
constexpr int kImpSpan = 512;
struct ImpArgs {
  const float* scores;  // [B, H, lc_pad] log2 units
  const float* lse;     // [B, H] log2-sum-exp
  float* a;             // [B, cap], or [B, H, cap] with per_head
  int batch, H, lc, lc_pad, cap, per_head;
  int span, pieces;
  int pending;          // 0: the attention kernels already added it
};
int launch_importance(const ImpArgs& p, hipStream_t stream);

// Prefill token and head importance from the attention's column sums and
// |O| partials: a[b, j] += sum over kept heads of colsum (heads in order),
// g[b, head] += sum of the head's partials, optional natural-log LSE copy.
// Workgroup blk covers 256 entries of sequence blk / pieces.
struct PrefillImp {
  const float* colsum;      // [B, h, n_pad]
  const float* gpart;       // [B, h, nqb]
  const float* lse;         // [B, h, n_pad] (log2 units)
  float* lse_out;           // optional [B, h, n]
  float* a;                 // [B, n], or [B, h, n] with per-head pruning
  float* g;                 // [B, H]
  const int32_t* head_idx;  // [B, h]
  const int32_t* head_keys; // per-head pruning: [B, h, nk], else null
  int batch, h_kept, H, n, n_pad, nk, nqb;
  int pieces;   // ceil(n / 256)
  int pending;  // 1: still to run
};
int launch_prefill_importance(const PrefillImp& p, hipStream_t stream);

// Output projection with residual: x[b, m, :] += O[b, m, :] wo[:, gathered]^T.
// imp (decode) / pimp (prefill), optional: the layer's importance pass, run
// by extra workgroups of the projection's launch (decode: skinny path;
// prefill: tiled path), else alone before it.
struct OutArgs {
  int dtype;
  const void* o;  // [B, n, h_kept*dh]
  const void* wo;
  const int32_t* head_idx;
  int batch, n, h_kept, dh, D;
  void* x;
  const ImpArgs* imp;
  const PrefillImp* pimp;
};
int launch_out(const OutArgs& a, hipStream_t stream);

// Prefill attention with fused importance: forward (O, row LSE, |O|
// partials), key-major column sums, then a deterministic reduction into a
// and g (and an optional natural-log LSE copy).
struct AttnArgs {
  int dtype, causal;
  const void* q;
  const void* k;
  const void* vt;
  int batch, h_kept, H, n, n_pad, dh;
  void* o;          // [B, n, h_kept*dh]
  float* lse;       // [B, h, n_pad] (log2 units)
  float* colsum;    // [B, h, n_pad]
  float* gpart;     // [B, h, nqb]
  int nqb, nkb;
  const int32_t* head_idx;
  float* a;         // [B, n], or [B, h, n] with per-head pruning
  float* g;         // [B, H]
  float* lse_out;   // optional [B, h, n] (natural log)
  float v_threshold;  // local value pruning (0 = off)
  // keys: the layer's tokens (kk = k, vtk = vt, nk = n, nk_pad = n_pad), or
  // with per-head pruning each slot's gathered kept tokens
  const int32_t* head_keys;  // [B, h, nk] token of each kept key, or null
  const void* kk;            // [B, h, nk_pad, dh]
  const void* vtk;           // [B, h, dh, nk_pad]
  int nk, nk_pad;
  // non-null: the importance pass is not launched but described here, for
  // the output projection's launch to run
  PrefillImp* imp_out;
};
int launch_attention(const AttnArgs& a, hipStream_t stream);

// Decode attention over cache rows 0..lc-1 for every (b, h). Quantized
// caches: knew/vnew hold this step's k and v rows [B, D] bf16, which the
// attention codes into plane row lc-1.
struct DecodeArgs {
  const void* q;  // [B, D] bf16
  const void* k_cache;
  const void* v_cache;  // [B, cap, D] bf16
  uint8_t* k_msb;  // quantized planes [B, H, cap, dh/2] and scales [B, cap]
  uint8_t* k_lsb;
  float* k_scale;
  uint8_t* v_msb;
  uint8_t* v_lsb;
  float* v_scale;
  const void* knew;
  const void* vnew;
  int batch, H, dh, cap, lc, lc_pad, nchunk;
  float threshold;
  float v_threshold;  // local value pruning (unquantized; 0 = off)
  int per_head;       // 1: a is [B, H, cap] and takes each head's probabilities apart
  float* scores;  // [B, H, lc_pad] log2-unit scores (the importance pass reads them)
  float* mpart;
  float* lpart;   // [B, H, nchunk] chunk statistics (split value-pruning path)
  float* opart;   // [B, H, nchunk, dh]
  float* lse;     // [B, H] row log2-sum-exp
  float* cmax;    // [B, H] largest probability (MSB pass when quantized)
  int32_t* kcount;  // [B, H, nchunk] V rows kept per chunk (value pruning)
  void* o;        // [B, D] bf16
  float* a;       // [B, cap], or [B, H, cap] with per_head
  int32_t* recompute;  // optional [B, H]
  int32_t* v_kept;     // optional [B, H]
};
// Fills *imp with the importance pass the layer still needs (imp->pending).
int launch_decode(const DecodeArgs& a, bool quantized, ImpArgs* imp, hipStream_t stream);

// Representative-token selection for one layer (see ada.hip): prev null =
// full-Gram selection, else a cascade step from the flags in prev.
struct AdaArgs {
  const float* x;        // [B, T, d] activations
  int batch, T, d;
  float tau;
  const int32_t* prev;   // [B, T] flags of the inherited set, or null
  int32_t* flags;        // [B, T] out
  float* maxcos;         // [B, T] out (optional): the cosine each decision took
  int32_t* counts;       // [B, 4] out (optional): size, removed, added, Gram pairs
  // workspace
  float* inv;            // [B, T]
  int32_t* listR;        // [B, T] each
  int32_t* listN;
  int32_t* listV;
  int32_t* cnt;          // [B, 4]
  uint32_t* rc;          // [B, T] removal (full: selection) cosine keys, by R position
  uint32_t* ac;          // [B, T] addition cosine keys, by N position
};
int launch_ada_select(const AdaArgs& a, hipStream_t stream);

}  // namespace spatten
