// Host-side argument checks (no HIP). Every rejection happens here, before
// any work is enqueued.
#include "validate.hpp"

namespace spatten {

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_dtype(int32_t dt) { return dt == SPATTEN_F32 || dt == SPATTEN_BF16; }

// [p0, p0 + n0) and [p1, p1 + n1) share a byte.
bool overlap(const void* p0, int64_t n0, const void* p1, int64_t n1) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(p0), a1 = reinterpret_cast<uintptr_t>(p1);
  if (n0 <= 0 || n1 <= 0) return false;
  return a0 < a1 + uintptr_t(n1) && a1 < a0 + uintptr_t(n0);
}

}  // namespace

size_t layer_workspace_bytes(const spatten_layer_desc& d) {
  if (d.batch == 0) return 0;
  if (d.mode == SPATTEN_PREFILL) return prefill_ws(d).total;
  return decode_ws(d).total;
}

int check_layer(const spatten_layer_desc* d, const void* x, const void* wq, const void* wk,
                const void* wv, const void* wo, const int32_t* head_idx,
                const int32_t* head_keys, const float* a, const float* g,
                const void* k_cache, const void* v_cache, const uint8_t* k_msb,
                const uint8_t* k_lsb, const float* k_scale, const uint8_t* v_msb,
                const uint8_t* v_lsb, const float* v_scale, const void* workspace,
                const size_t* workspace_bytes) {
  // descriptor
  if (!d || !workspace_bytes) return SPATTEN_EINVAL;
  if (d->mode != SPATTEN_PREFILL && d->mode != SPATTEN_DECODE) return SPATTEN_EINVAL;
  if (!valid_dtype(d->dtype)) return SPATTEN_EINVAL;
  if (d->causal != 0 && d->causal != 1) return SPATTEN_EINVAL;
  if (d->kv_quantized != 0 && d->kv_quantized != 1) return SPATTEN_EINVAL;
  if (d->batch < 0 || d->n_heads < 1 || d->head_dim < 1) return SPATTEN_EINVAL;
  if (d->n_heads_kept < 1 || d->n_heads_kept > d->n_heads) return SPATTEN_EINVAL;
  if (int64_t(d->n_heads) * d->head_dim > (1 << 20)) return SPATTEN_EINVAL;
  if (!(d->v_threshold >= 0.0f)) return SPATTEN_EINVAL;  // negative or NaN
  if (d->per_head != 0 && d->per_head != 1) return SPATTEN_EINVAL;
  const bool keys_per_head = d->per_head && d->mode == SPATTEN_PREFILL;
  if (keys_per_head) {
    if (d->n_keys < 1 || d->n_keys > d->n_tokens) return SPATTEN_EINVAL;
    if (d->dtype != SPATTEN_BF16 || d->causal || d->v_threshold > 0.0f)
      return SPATTEN_EUNSUPPORTED;
  } else if (d->n_keys != 0) {
    return SPATTEN_EINVAL;
  }
  if (d->head_dim != 32 && d->head_dim != 64 && d->head_dim != 128) return SPATTEN_EUNSUPPORTED;
  // quantized value pruning keeps the row's scores in LDS: caches of at most
  // kVrowMaxRows rows (rounded up to whole chunks)
  if (d->v_threshold > 0.0f && d->kv_quantized &&
      round_up(int64_t(d->cache_len) + 1, kDecChunk) > kVrowMaxRows)
    return SPATTEN_EUNSUPPORTED;
  if (d->mode == SPATTEN_PREFILL) {
    if (d->n_tokens < 1 || d->kv_quantized != 0) return SPATTEN_EINVAL;
    if (d->dtype == SPATTEN_BF16 && d->head_dim == 32) return SPATTEN_EUNSUPPORTED;
    if (d->dtype == SPATTEN_F32 && d->n_tokens > 1024) return SPATTEN_EUNSUPPORTED;
  } else {
    if (d->n_tokens != 1 || d->causal != 0) return SPATTEN_EINVAL;
    if (d->cache_len < 0 || d->cache_cap < d->cache_len + 1) return SPATTEN_EINVAL;
    if (d->kv_quantized && !(d->pq_threshold == d->pq_threshold)) return SPATTEN_EINVAL;  // NaN
    if (d->n_heads_kept != d->n_heads) return SPATTEN_EUNSUPPORTED;
    if (d->dtype != SPATTEN_BF16 || d->head_dim != 64 || d->n_heads > 32)
      return SPATTEN_EUNSUPPORTED;
  }
  if (!workspace) return SPATTEN_OK;  // size query: pointers are not needed
  if (!aligned(workspace, 256)) return SPATTEN_EINVAL;
  if (*workspace_bytes < layer_workspace_bytes(*d)) return SPATTEN_EWORKSPACE;
  if (d->batch == 0) return SPATTEN_OK;
  // tensors
  if (!x || !wq || !wk || !wv || !wo || !head_idx || !a) return SPATTEN_EINVAL;
  if (bool(head_keys) != keys_per_head || !aligned(head_keys, 4)) return SPATTEN_EINVAL;
  if (d->mode == SPATTEN_PREFILL && !g) return SPATTEN_EINVAL;
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(wk, 16) || !aligned(wv, 16) ||
      !aligned(wo, 16) || !aligned(a, 4) || !aligned(g, 4) || !aligned(head_idx, 4))
    return SPATTEN_EINVAL;
  const bool any_plane = k_msb || k_lsb || k_scale || v_msb || v_lsb || v_scale;
  if (d->mode == SPATTEN_PREFILL) {
    if (k_cache || v_cache || any_plane) return SPATTEN_EINVAL;
  } else if (d->kv_quantized) {
    if (k_cache || v_cache) return SPATTEN_EINVAL;
    if (!k_msb || !k_lsb || !k_scale || !v_msb || !v_lsb || !v_scale) return SPATTEN_EINVAL;
    if (!aligned(k_msb, 4) || !aligned(k_lsb, 4) || !aligned(v_msb, 4) || !aligned(v_lsb, 4) ||
        !aligned(k_scale, 4) || !aligned(v_scale, 4))
      return SPATTEN_EINVAL;
  } else {
    if (any_plane || !k_cache || !v_cache) return SPATTEN_EINVAL;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16)) return SPATTEN_EINVAL;
  }
  return SPATTEN_OK;
}

int check_ada(const float* x, int32_t batch, int32_t T, int32_t d, float tau,
              const int32_t* flags, const void* workspace, const size_t* workspace_bytes) {
  if (!workspace_bytes) return SPATTEN_EINVAL;
  if (batch < 0 || T < 1 || d < 1) return SPATTEN_EINVAL;
  if (!(tau >= 0.0f && tau <= 1.0f)) return SPATTEN_EINVAL;  // also rejects NaN
  if (d % 32 != 0) return SPATTEN_EUNSUPPORTED;
  if (int64_t(T) * d > (int64_t(1) << 31)) return SPATTEN_EUNSUPPORTED;
  if (!workspace) return SPATTEN_OK;  // size query
  if (!aligned(workspace, 256)) return SPATTEN_EINVAL;
  if (*workspace_bytes < ada_ws(batch, T).total) return SPATTEN_EWORKSPACE;
  if (batch == 0) return SPATTEN_OK;
  if (!x || !flags) return SPATTEN_EINVAL;
  if (!aligned(x, 16) || !aligned(flags, 4)) return SPATTEN_EINVAL;
  return SPATTEN_OK;
}

int check_topk(const float* scores, int32_t batch, int32_t n, int64_t row_stride, int32_t k,
               const int32_t* out_idx) {
  if (batch < 0 || n < 1 || k < 1 || k > n || row_stride < n) return SPATTEN_EINVAL;
  if (batch > 0 && (!scores || !out_idx)) return SPATTEN_EINVAL;
  if (!aligned(scores, 4) || !aligned(out_idx, 4)) return SPATTEN_EINVAL;
  return SPATTEN_OK;
}

int check_compact(int32_t n_tensors, const void* const* src, void* const* dst,
                  const int64_t* row_bytes, const int64_t* src_batch_stride,
                  const int64_t* dst_batch_stride, const int32_t* idx, int32_t batch, int32_t k) {
  if (n_tensors < 0 || batch < 0 || k < 0) return SPATTEN_EINVAL;
  if (n_tensors == 0 || batch == 0 || k == 0) return SPATTEN_OK;
  if (!src || !dst || !row_bytes || !src_batch_stride || !dst_batch_stride || !idx)
    return SPATTEN_EINVAL;
  if (!aligned(idx, 4)) return SPATTEN_EINVAL;
  for (int32_t t = 0; t < n_tensors; ++t) {
    if (!src[t] || !dst[t] || row_bytes[t] <= 0) return SPATTEN_EINVAL;
    if (src_batch_stride[t] < 0 || dst_batch_stride[t] < 0) return SPATTEN_EINVAL;
    // destination rows of one sequence must not run into the next sequence's
    if (batch > 1 && dst_batch_stride[t] < int64_t(k) * row_bytes[t]) return SPATTEN_EINVAL;
    if (batch > 1 && src_batch_stride[t] < int64_t(k) * row_bytes[t]) return SPATTEN_EINVAL;
    const int64_t dspan = int64_t(batch - 1) * dst_batch_stride[t] + int64_t(k) * row_bytes[t];
    const int64_t sspan = int64_t(batch - 1) * src_batch_stride[t] + int64_t(k) * row_bytes[t];
    if (overlap(src[t], sspan, dst[t], dspan)) return SPATTEN_EINVAL;
  }
  return SPATTEN_OK;
}

int check_compact_inplace(int32_t n_tensors, void* const* base, const int64_t* row_bytes,
                          const int64_t* row_pitch, const int64_t* batch_stride,
                          const int32_t* idx, int32_t batch, int32_t n, int32_t k) {
  if (n_tensors < 0 || batch < 0 || n < 1 || k < 1 || k > n) return SPATTEN_EINVAL;
  if (k > kInplaceMaxK) return SPATTEN_EUNSUPPORTED;
  if (n_tensors == 0 || batch == 0) return SPATTEN_OK;
  if (!base || !row_bytes || !batch_stride || !idx) return SPATTEN_EINVAL;
  if (!aligned(idx, 4)) return SPATTEN_EINVAL;
  for (int32_t t = 0; t < n_tensors; ++t) {
    if (!base[t] || row_bytes[t] <= 0 || batch_stride[t] < 0) return SPATTEN_EINVAL;
    if (row_bytes[t] > kInplaceMaxRowBytes) return SPATTEN_EUNSUPPORTED;
    const int64_t pitch = row_pitch ? row_pitch[t] : row_bytes[t];
    if (pitch < row_bytes[t]) return SPATTEN_EINVAL;
    // the n rows of one sequence must not run into the next sequence's
    if (batch > 1 && batch_stride[t] < int64_t(n - 1) * pitch + row_bytes[t]) return SPATTEN_EINVAL;
  }
  return SPATTEN_OK;
}

int check_quantize(const void* kv, int32_t dtype, int32_t batch, int32_t n, int32_t dim,
                   int32_t head_dim, int64_t kv_batch_stride, const uint8_t* msb,
                   const uint8_t* lsb, const float* scale, int64_t plane_rows) {
  if (!valid_dtype(dtype)) return SPATTEN_EINVAL;
  if (batch < 0 || n < 0 || dim < 2 || (dim & 1)) return SPATTEN_EINVAL;
  if (head_dim < 0 || (head_dim > 0 && ((head_dim & 1) || dim % head_dim != 0)))
    return SPATTEN_EINVAL;
  if (batch > 1 && kv_batch_stride < int64_t(n) * dim) return SPATTEN_EINVAL;
  // sequences (and, head-major, the heads' slabs) must not overlap
  const bool slabs = batch > 1 || (head_dim > 0 && dim / head_dim > 1);
  if (slabs && plane_rows < n) return SPATTEN_EINVAL;
  if (batch == 0 || n == 0) return SPATTEN_OK;
  if (!kv || !msb || !lsb || !scale) return SPATTEN_EINVAL;
  if (!aligned(kv, dtype_bytes(dtype)) || !aligned(scale, 4)) return SPATTEN_EINVAL;
  return SPATTEN_OK;
}

}  // namespace spatten
