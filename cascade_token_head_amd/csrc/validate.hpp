// Host-side argument checks for every entry point. Plain C++ with no HIP
// dependency: the library calls these before enqueuing anything, and the
// host test builds them alone with g++ and sanitizers.
#pragma once

#include <cstddef>
#include <cstdint>

#include "layout.hpp"

namespace spatten {

// Required workspace bytes for a layer call, or 0 when none is needed.
size_t layer_workspace_bytes(const spatten_layer_desc& d);

int check_layer(const spatten_layer_desc* d, const void* x, const void* wq, const void* wk,
                const void* wv, const void* wo, const int32_t* head_idx,
                const int32_t* head_keys, const float* a, const float* g,
                const void* k_cache, const void* v_cache, const uint8_t* k_msb,
                const uint8_t* k_lsb, const float* k_scale, const uint8_t* v_msb,
                const uint8_t* v_lsb, const float* v_scale, const void* workspace,
                const size_t* workspace_bytes);

int check_ada(const float* x, int32_t batch, int32_t T, int32_t d, float tau,
              const int32_t* flags, const void* workspace, const size_t* workspace_bytes);

int check_topk(const float* scores, int32_t batch, int32_t n, int64_t row_stride, int32_t k,
               const int32_t* out_idx);

int check_compact(int32_t n_tensors, const void* const* src, void* const* dst,
                  const int64_t* row_bytes, const int64_t* src_batch_stride,
                  const int64_t* dst_batch_stride, const int32_t* idx, int32_t batch, int32_t k);

int check_compact_inplace(int32_t n_tensors, void* const* base, const int64_t* row_bytes,
                          const int64_t* row_pitch, const int64_t* batch_stride,
                          const int32_t* idx, int32_t batch, int32_t n, int32_t k);

int check_quantize(const void* kv, int32_t dtype, int32_t batch, int32_t n, int32_t dim,
                   int32_t head_dim, int64_t kv_batch_stride, const uint8_t* msb,
                   const uint8_t* lsb, const float* scale, int64_t plane_rows);

}  // namespace spatten
