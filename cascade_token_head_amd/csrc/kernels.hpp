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

int launch_quantize(const void* kv, int dtype, int batch, int n, int dim, int64_t kv_bs,
                    uint8_t* msb, uint8_t* lsb, float* scale, int64_t pbs, hipStream_t stream);

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

// Output projection with residual: x[b, m, :] += O[b, m, :] wo[:, gathered]^T
struct OutArgs {
  int dtype;
  const void* o;  // [B, n, h_kept*dh]
  const void* wo;
  const int32_t* head_idx;
  int batch, n, h_kept, dh, D;
  void* x;
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
  float* a;         // [B, n]
  float* g;         // [B, H]
  float* lse_out;   // optional [B, h, n] (natural log)
};
int launch_attention(const AttnArgs& a, hipStream_t stream);

// Decode attention over cache rows 0..lc-1 for every (b, h).
struct DecodeArgs {
  const void* q;  // [B, D] bf16
  const void* k_cache;
  const void* v_cache;  // [B, cap, D] bf16
  uint8_t* k_msb;  // quantized planes [B, cap, D/2] and scales [B, cap]
  uint8_t* k_lsb;
  float* k_scale;
  uint8_t* v_msb;
  uint8_t* v_lsb;
  float* v_scale;
  const void* knew;  // quantized: this step's k and v rows [B, D] bf16, coded
  const void* vnew;  // into plane row lc-1 by the MSB pass before it reads it
  int batch, H, dh, cap, lc, lc_pad, nchunk;
  float threshold;
  float v_threshold;  // local value pruning (unquantized; 0 = off)
  int per_head;       // 1: a is [B, H, cap] and takes each head's probabilities apart
  float* scores;  // [B, H, lc_pad]
  float* mpart;
  float* lpart;   // [B, H, nchunk]
  float* opart;   // [B, H, nchunk, dh]
  float* lse;     // [B, H]
  float* cmax;    // [B, H]
  int32_t* flags; // [B, H]
  int32_t* queue; // [0] = count, then entries b*H + h
  int32_t* kcount;  // [B, H, nchunk] V rows kept per chunk (value pruning)
  void* o;        // [B, D] bf16
  float* a;       // [B, cap], or [B, H, cap] with per_head
  int32_t* recompute;  // optional [B, H]
  int32_t* v_kept;     // optional [B, H]
};
int launch_decode(const DecodeArgs& a, bool quantized, hipStream_t stream);

}  // namespace spatten
