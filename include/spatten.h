/*
 * spatten.h - C ABI of libspatten.so: cascade token/head pruned attention
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations follow "SpAtten: Efficient Sparse Attention Architecture
 * with Cascade Token and Head Pruning" (Wang, Zhang, Han, arXiv 2012.09852)
 * as summarised on its paperlayer.ai page; section names below are that
 * page's, except for spatten_ada_select, which follows "Cascade Token
 * Selection for Transformer Attention Acceleration" (gist.science summary)
 * and names that page's sections.
 *
 * Conventions for every entry point
 *  - Tensor pointers are DEVICE pointers owned by the caller; the library
 *    never frees or retains them. Small descriptor arrays (the per-tensor
 *    tables of spatten_compact) are HOST memory read during the call.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream). Nothing synchronises the host; results are valid once the
 *    stream has reached the enqueued work.
 *  - Every function returns a spatten_status. Arguments are checked on the
 *    host before anything is enqueued; a rejected call enqueues nothing.
 *    SPATTEN_EHIP reports a failed launch (hipGetLastError) and leaves the
 *    outputs unspecified. No function aborts or throws.
 *  - Tensors are row-major and densely packed in their last dimension.
 *    bf16 is IEEE bfloat16 stored as uint16.
 *  - Weights use the output-major layout: w[o * D + i] multiplies input
 *    feature i into output feature o (y = x w^T). Head h owns output rows
 *    h*dh .. h*dh+dh-1 of wq, wk, wv and input columns h*dh .. h*dh+dh-1
 *    of wo.
 */
#ifndef SPATTEN_H
#define SPATTEN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPATTEN_OK = 0,
  SPATTEN_EINVAL = -1,       /* malformed argument (null pointer, size out of range, overlap) */
  SPATTEN_EUNSUPPORTED = -2, /* well-formed but outside what the kernels implement */
  SPATTEN_EWORKSPACE = -3,   /* workspace smaller than the size reported for this descriptor */
  SPATTEN_EHIP = -4          /* a HIP launch failed */
} spatten_status;

typedef enum { SPATTEN_F32 = 0, SPATTEN_BF16 = 1 } spatten_dtype;
typedef enum { SPATTEN_PREFILL = 0, SPATTEN_DECODE = 1 } spatten_mode;

/* Shape of one layer call. */
typedef struct {
  int32_t mode;          /* spatten_mode */
  int32_t dtype;         /* spatten_dtype of x, weights, caches (accumulation is fp32) */
  int32_t causal;        /* prefill: 1 = token j is masked for query i when j > i */
  int32_t batch;         /* B sequences */
  int32_t n_tokens;      /* prefill: kept tokens per sequence (n_l); decode: 1 */
  int32_t n_heads;       /* H; model dim D = H * head_dim */
  int32_t n_heads_kept;  /* h_l kept heads (decode: must equal H) */
  int32_t head_dim;      /* dh: 32, 64 or 128 */
  int32_t cache_len;     /* decode: cache entries before this step's append */
  int32_t cache_cap;     /* decode: cache rows allocated per sequence */
  int32_t kv_quantized;  /* decode: 1 = cache held as int8 MSB/LSB nibble planes */
  float pq_threshold;    /* decode, quantized: recompute rows whose max prob < this */
  float v_threshold;     /* local value pruning threshold (0 = off): prefill, decode (quantized:
                            cache_len + 1 <= 4096) */
  int32_t per_head;      /* 1 = per-head token pruning (decode: a is [B, H, cache_cap], and
                            quantized scales are [B, H, cache_cap]; prefill, bf16
                            bidirectional: see n_keys) */
  int32_t n_keys;        /* prefill with per_head: tokens each kept head keeps as keys and values */
} spatten_layer_desc;

/*
 * spatten_layer_forward - one attention-only residual layer over the kept
 * tokens and heads (section II "Attention mechanism"), with cascade token
 * and head importance accumulated on the fly (section II "Cascade
 * pruning"; "A. Cascade Token Pruning").
 *
 *   For each sequence b and kept head slot s (head h = head_idx[b, s]):
 *     Q_h, K_h, V_h = x w{q,k,v}[h rows]^T
 *     P_h = row-softmax(Q_h K_h^T / sqrt(dh))   (causal: j > i masked)
 *     O_h = P_h V_h
 *     x  += sum_s O_h wo[:, h cols]^T           (residual, in place)
 *     a[b, j] += sum_s sum_i P_h[i, j]          (token importance)
 *     g[b, h] += sum_i sum_c |O_h[i, c]|        (head importance)
 *
 * Prefill: x is [B, n_tokens, D]; a is [B, n_tokens] fp32; g is [B, H]
 *   fp32; k_cache..v_scale must be NULL. lse (optional, may be NULL) gets
 *   the per-row log-sum-exp [B, h_kept, n_tokens] fp32.
 * Decode: x is [B, 1, D] (this step's token). The token's k and v are
 *   appended at cache row cache_len, then the query attends over rows
 *   0..cache_len (no mask) and a[b, j] (a is [B, cache_cap]) accumulates
 *   for those rows. Unquantized: k_cache, v_cache are [B, cache_cap, D]
 *   in dtype. Quantized (progressive quantization, "A. Cascade
 *   Token Pruning" and "E. ... Progressive Quantization"): k_msb, k_lsb, v_msb, v_lsb are
 *   head-major [B, H, cache_cap, head_dim/2] u8 (each head's rows
 *   contiguous, so a (sequence, head) row reads whole cache lines) and
 *   k_scale, v_scale [B, cache_cap] fp32, as spatten_quantize_kv writes
 *   them with head_dim set (with per_head = 1: [B, H, cache_cap], each
 *   head holding the scale of the token in each of its own slots); this step's k and v rows are coded into
 *   row cache_len of the planes and scales with that function's arithmetic
 *   (bit for bit) before they are read; each (b, h) row is scored with MSB-only
 *   values (scale*16*msb) and, when its largest probability is below
 *   pq_threshold, recomputed with the full code scale*(16*msb + lsb) for
 *   both K and V. recompute (optional, [B, H] int32) receives 1 for
 *   recomputed rows. a accumulates the probabilities that produced O.
 *   Local value pruning ("A. Cascade Token Pruning", bullet "Local Value Pruning";
 *   v_threshold > 0): after the softmax, V row j of head h enters
 *   O_h only when P_h[j] >= v_threshold, O_h = sum over those j of
 *   P_h[j] V_h[j] (no renormalisation); the other V rows are never read.
 *   Quantized caches apply it to the probabilities of the pass that
 *   produces O_h (the recomputed ones, with both planes of V, for a
 *   recomputed row; else the MSB pass's, with MSB-only V) and need
 *   cache_len + 1 <= 4096.
 *   a still takes every probability. v_kept (optional, [B, H] int32)
 *   receives the number of V rows that entered O_h (cache_len + 1 without
 *   value pruning).
 *   Per-head token pruning (section "A. Neural Networks Pruning and Quantization", bullet "Token Pruning"; per_head = 1):
 *   a is [B, H, cache_cap] and a[b, h, j] takes head h's probabilities
 *   only, so each head can keep its own cache entries (cut with
 *   spatten_compact_inplace on the head's 128-byte slice of each row, or
 *   for quantized caches on the head's slab of plane rows and its row of
 *   scales). A quantized cache then keeps one scale per (head, slot): the
 *   new row's per-token scale (taken over the whole row) is written to
 *   every head's slot cache_len.
 *   g is not used in decode and may be NULL. Decode needs head_dim 64,
 *   H <= 32, bf16 and every head kept.
 *   Per-head token pruning in prefill (per_head = 1; bf16, bidirectional;
 *   section "A. Neural Networks Pruning and Quantization", bullet "Token
 *   Pruning"): kept head slot s of sequence b attends over its own kept
 *   tokens head_keys[b, s, 0 .. n_keys-1] (strictly ascending indices into
 *   the layer's n_tokens tokens) as keys and values, while every token
 *   queries every kept head, so x keeps all n_tokens rows; a is [B, h_kept,
 *   n_tokens] and a[b, s, t] takes slot s's probabilities only (its kept
 *   tokens' column sums). 1 <= n_keys <= n_tokens.
 * head_idx: [B, h_kept] int32, strictly ascending head ids per sequence.
 * head_keys: per-head pruning in prefill only (else NULL), as above.
 *   Device index arrays are not read on the host: ids or token indices
 *   outside their ranges are not detected and make the call's reads and
 *   writes undefined.
 * workspace: device scratch of *workspace_bytes bytes, 256-byte aligned;
 *   its contents are overwritten by every call, so calls that share one
 *   workspace must be ordered on one stream (or otherwise serialised).
 *   If workspace is NULL only *d is checked, the required size is stored in
 *   *workspace_bytes and SPATTEN_OK is returned without enqueuing anything
 *   (tensor pointers may then be NULL).
 * Supported (else SPATTEN_EUNSUPPORTED): prefill bf16 with head_dim 64 or
 *   128; prefill fp32 with head_dim 32, 64 or 128 and n_tokens <= 1024;
 *   decode bf16 with head_dim 64, n_heads <= 32 and every head kept. A
 *   v_threshold > 0 is taken by prefill and by decode (quantized caches:
 *   cache_len + 1 <= 4096), not by per-head prefill; a NaN or negative one is
 *   SPATTEN_EINVAL. per_head is 0 or 1 (else SPATTEN_EINVAL); 1 needs a
 *   decode, or a bf16 bidirectional prefill with
 *   1 <= n_keys <= n_tokens; n_keys must be 0 in every other case
 *   (SPATTEN_EINVAL).
 */
int spatten_layer_forward(const spatten_layer_desc* d, void* x,
                          const void* wq, const void* wk, const void* wv, const void* wo,
                          const int32_t* head_idx, const int32_t* head_keys, float* a, float* g,
                          void* k_cache, void* v_cache,
                          uint8_t* k_msb, uint8_t* k_lsb, float* k_scale,
                          uint8_t* v_msb, uint8_t* v_lsb, float* v_scale,
                          int32_t* recompute, int32_t* v_kept, float* lse,
                          void* workspace, size_t* workspace_bytes, void* stream);

/*
 * spatten_layer_forward_noalloc - spatten_layer_forward without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). The
 * arguments and results are those of spatten_layer_forward; the scratch it
 * needs lives in a fixed device array of SPATTEN_NOALLOC_SCRATCH_BYTES that
 * the library holds on each device it runs on until the process ends (its
 * address is taken once per device, on the first call with that device
 * current). It calls no allocating routine. A descriptor whose workspace
 * (as spatten_layer_forward reports it) exceeds the array returns
 * SPATTEN_EWORKSPACE before anything is enqueued. Nothing in the array
 * needs to start at zero: every call writes what it reads. All calls on one
 * device share the array, so calls that may overlap on one device (other
 * streams, other host threads) race and must be serialised by the caller.
 */
#define SPATTEN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int spatten_layer_forward_noalloc(const spatten_layer_desc* d, void* x,
                                  const void* wq, const void* wk, const void* wv, const void* wo,
                                  const int32_t* head_idx, const int32_t* head_keys, float* a,
                                  float* g,
                                  void* k_cache, void* v_cache,
                                  uint8_t* k_msb, uint8_t* k_lsb, float* k_scale,
                                  uint8_t* v_msb, uint8_t* v_lsb, float* v_scale,
                                  int32_t* recompute, int32_t* v_kept, float* lse, void* stream);

/*
 * spatten_topk - on-the-fly top-k ("B. Top-k Engine"): for each row b the
 * k largest of scores[b*row_stride + 0 .. n-1], ranked by fp32 value with
 * -0.0 below +0.0 and equal values broken towards the lower index
 * (NaNs rank by their bit pattern). out_idx[b*k + 0 .. k-1] receives the
 * selected indices in ascending order. kth_value (optional, [batch]) gets
 * the k-th ranked score. Requires 1 <= k <= n, row_stride >= n; batch == 0
 * is a no-op. No workspace.
 */
int spatten_topk(const float* scores, int32_t batch, int32_t n, int64_t row_stride,
                 int32_t k, int32_t* out_idx, float* kth_value, void* stream);

/*
 * spatten_compact - multi-tensor row gather that drops pruned tokens from
 * all following computation ("A. Cascade Token Pruning"):
 *   for t < n_tensors, b < batch, r < k:
 *     dst[t] + b*dst_batch_stride[t] + r*row_bytes[t]
 *       <- src[t] + b*src_batch_stride[t] + idx[b*k + r]*row_bytes[t]
 * (row_bytes bytes; strides in bytes). src, dst, row_bytes and the strides
 * are HOST arrays of n_tensors entries holding device addresses. Each
 * idx[b*k + r] must lie in [0, src rows) - the caller guarantees this
 * (typically idx comes from spatten_topk). src and dst of one tensor must
 * not overlap (checked over the span the call touches).
 */
int spatten_compact(int32_t n_tensors, const void* const* src, void* const* dst,
                    const int64_t* row_bytes, const int64_t* src_batch_stride,
                    const int64_t* dst_batch_stride, const int32_t* idx,
                    int32_t batch, int32_t k, void* stream);

/*
 * spatten_compact_inplace - the same cut done in place, for tensors whose
 * row order carries no meaning (decode caches: the query attends to every
 * kept entry without a mask), so that a cascade can cut the cache again at
 * every step (section II "Cascade pruning": pruned tokens stay pruned).
 * For each sequence b, idx[b*k + 0 .. k-1] lists k strictly ascending rows
 * below n (as spatten_topk returns them). Afterwards rows 0 .. k-1 hold
 * exactly the selected rows, as a set: a selected row below k stays where
 * it is, and the i-th selected row at or above k (in ascending order) moves
 * into the i-th unselected row below k (in ascending order). No other row
 * is read or written, so a cut from k + 1 rows to k moves at most one row.
 * Row r of sequence b of tensor t is the row_bytes[t] bytes at base[t] +
 * b*batch_stride[t] + r*row_pitch[t] (row_pitch NULL: rows are packed,
 * pitch = row_bytes; a pitch larger than the row moves one slice of each
 * row, e.g. one head of a token-major cache); base, row_bytes, row_pitch
 * and batch_stride are HOST arrays of n_tensors entries. Requires 1 <= k <= n; k > 8192 or a row longer than
 * 64 MiB returns SPATTEN_EUNSUPPORTED. Each idx entry must lie in [0, n) - the caller
 * guarantees this. row_pitch must be at least row_bytes, and sequences
 * must not overlap (batch_stride >= (n-1)*row_pitch + row_bytes when
 * batch > 1).
 */
int spatten_compact_inplace(int32_t n_tensors, void* const* base, const int64_t* row_bytes,
                            const int64_t* row_pitch, const int64_t* batch_stride,
                            const int32_t* idx, int32_t batch, int32_t n, int32_t k,
                            void* stream);

/*
 * spatten_quantize_kv - K/V rows to separately fetchable MSB and LSB
 * planes ("A. Cascade Token Pruning", bullet "Progressive Quantization"; section IV, bullet
 * "Quantization Support"). For each row of `dim` values, in fp32:
 *   s = max|x| / 127;  q = clamp(round_half_even(x / s), -127, 127)
 *   (s = 0 and q = 0 for an all-zero row)
 *   msb = q >> 4 (arithmetic, -8..7), lsb = q & 15 (0..15)
 *   msb byte j = (msb[2j] & 15) | (msb[2j+1] & 15) << 4, lsb likewise.
 * kv: [batch, n, dim] in dtype with batch stride kv_batch_stride elements.
 * msb, lsb: head_dim = 0 - token-major [batch, plane_rows, dim/2] u8;
 *   head_dim > 0 (even, dividing dim) - head-major [batch, dim/head_dim,
 *   plane_rows, head_dim/2] u8: each head's rows are contiguous, the
 *   layout spatten_layer_forward takes for quantized caches. Row r of
 *   sequence b is written at row r of its sequence's (and head's) slab.
 * scale: [batch, plane_rows] fp32. dim must be even; plane_rows >= n when
 * the slabs are more than one. Pointers may be pre-offset by the same
 * number of rows (to the first row to write).
 */
int spatten_quantize_kv(const void* kv, int32_t dtype, int32_t batch, int32_t n, int32_t dim,
                        int32_t head_dim, int64_t kv_batch_stride, uint8_t* msb, uint8_t* lsb,
                        float* scale, int64_t plane_rows, void* stream);

/*
 * spatten_ada_select - representative tokens of one layer by a Gram
 * threshold, and their cascade across layers ("Cascade Token Selection for
 * Transformer Attention Acceleration": "Probleemstelling" defines a
 * representative token, "Methodologie: Het Cascade-mechanisme" the cascade
 * steps 1-3). With theta = 1 - tau^2 and cos(t, s) the cosine of rows t and
 * s of x[b] (a zero row has cosine 0 with every row), computed in fp32:
 *   prev == NULL (full selection): flags[b, t] = 1 iff the largest cos(t,
 *     s) over s < t is below theta (token 0 always);
 *   prev != NULL (cascade step from the inherited set R = {t: prev[b, t] !=
 *     0}): a member t of R stays iff its largest cosine with a preceding
 *     member of R is below theta (the r x r product); a token u outside R
 *     joins iff its largest cosine with a preceding member that stayed is
 *     below theta (the (T - r) x r product); flags = stayed or joined.
 * x: [batch, T, d] fp32, 16-byte aligned, d a multiple of 32. prev, flags:
 *   [batch, T] int32 (flags is written whole; it must not alias prev).
 * maxcos (optional, [batch, T] fp32): the cosine each token's decision was
 *   taken on (-inf where no token precedes it in the set compared with).
 * counts (optional, [batch, 4] int32): set size, removed members, added
 *   tokens, and Gram entries evaluated (pairs s < t; saturates at 2^31-1).
 * tau in [0, 1] (else SPATTEN_EINVAL). workspace as spatten_layer_forward
 * (NULL: size query).
 */
int spatten_ada_select(const float* x, int32_t batch, int32_t T, int32_t d, float tau,
                       const int32_t* prev, int32_t* flags, float* maxcos, int32_t* counts,
                       void* workspace, size_t* workspace_bytes, void* stream);

/* Human-readable name of a status code (static string). */
const char* spatten_status_string(int status);

/*
 * Diagnostics (not part of the computation). spatten_debug_timing(1)
 * brackets every kernel the library launches with two HIP events on the
 * launching stream; spatten_debug_kernel_times() waits for them and reports,
 * per kernel name, the summed event durations and the launch count, then
 * forgets them. names receives up to max_kernels NUL-terminated names of
 * name_len bytes each. Timing state is process-wide and not thread-safe.
 */
int spatten_debug_timing(int enable);
int spatten_debug_kernel_times(int max_kernels, char* names, int name_len, double* total_ms,
                               int* launches, int* n_kernels);

#ifdef __cplusplus
}
#endif

#endif /* SPATTEN_H */
