// C ABI entry points of libspatten.so (declared in include/spatten.h).
// Each call validates on the host (validate.cpp), then enqueues kernels on
// the caller's stream. Nothing here allocates or synchronises; the only
// state is the per-device address of the fixed scratch array that the
// allocation-free layer entry point runs in.
#include <mutex>

#include "../../include/spatten.h"
#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

using namespace spatten;

namespace {

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

#define SPATTEN_TRY(expr)             \
  do {                                \
    const int _st = (expr);           \
    if (_st != SPATTEN_OK) return _st; \
  } while (0)

int layer_prefill(const spatten_layer_desc& d, void* x, const void* wq, const void* wk,
                  const void* wv, const void* wo, const int32_t* head_idx,
                  const int32_t* head_keys, float* a, float* g, float* lse_out, char* ws,
                  hipStream_t st) {
  const PrefillWs w = prefill_ws(d);
  const int D = d.n_heads * d.head_dim;
  QkvArgs qa{};
  qa.dtype = d.dtype;
  qa.mode = SPATTEN_PREFILL;
  qa.x = x;
  qa.w[0] = wq;
  qa.w[1] = wk;
  qa.w[2] = wv;
  qa.head_idx = head_idx;
  qa.batch = d.batch;
  qa.n = d.n_tokens;
  qa.n_pad = int(w.n_pad);
  qa.h_kept = d.n_heads_kept;
  qa.dh = d.head_dim;
  qa.D = D;
  qa.q = ws + w.q;
  qa.k = ws + w.k;
  qa.vt = ws + w.vt;
  SPATTEN_TRY(launch_qkv(qa, st));

  AttnArgs aa{};
  aa.dtype = d.dtype;
  aa.causal = d.causal;
  aa.q = ws + w.q;
  aa.k = ws + w.k;
  aa.vt = ws + w.vt;
  aa.batch = d.batch;
  aa.h_kept = d.n_heads_kept;
  aa.H = d.n_heads;
  aa.n = d.n_tokens;
  aa.n_pad = int(w.n_pad);
  aa.dh = d.head_dim;
  aa.o = ws + w.o;
  aa.lse = reinterpret_cast<float*>(ws + w.lse);
  aa.colsum = reinterpret_cast<float*>(ws + w.colsum);
  aa.gpart = reinterpret_cast<float*>(ws + w.gpart);
  aa.nqb = int(w.nqb);
  aa.nkb = int(w.nkb);
  aa.head_idx = head_idx;
  aa.a = a;
  aa.g = g;
  aa.lse_out = lse_out;
  aa.v_threshold = d.v_threshold;
  aa.head_keys = head_keys;
  aa.kk = head_keys ? ws + w.kk : aa.k;
  aa.vtk = head_keys ? ws + w.vtk : aa.vt;
  aa.nk = int(w.nk);
  aa.nk_pad = int(w.nk_pad);
  // the importance pass rides in the output projection's launch
  PrefillImp pimp{};
  aa.imp_out = &pimp;
  SPATTEN_TRY(launch_attention(aa, st));
  OutArgs oa{};
  oa.pimp = &pimp;
  oa.dtype = d.dtype;
  oa.o = ws + w.o;
  oa.wo = wo;
  oa.head_idx = head_idx;
  oa.batch = d.batch;
  oa.n = d.n_tokens;
  oa.h_kept = d.n_heads_kept;
  oa.dh = d.head_dim;
  oa.D = D;
  oa.x = x;
  return launch_out(oa, st);
}

int layer_decode(const spatten_layer_desc& d, void* x, const void* wq, const void* wk,
                 const void* wv, const void* wo, const int32_t* head_idx, float* a,
                 void* k_cache, void* v_cache, uint8_t* k_msb, uint8_t* k_lsb, float* k_scale,
                 uint8_t* v_msb, uint8_t* v_lsb, float* v_scale, int32_t* recompute,
                 int32_t* v_kept, char* ws, hipStream_t st) {
  const DecodeWs w = decode_ws(d);
  const int H = d.n_heads, dh = d.head_dim, D = H * dh;
  const int64_t cap = d.cache_cap, row = d.cache_len;
  QkvArgs qa{};
  qa.dtype = d.dtype;
  qa.mode = SPATTEN_DECODE;
  qa.x = x;
  qa.w[0] = wq;
  qa.w[1] = wk;
  qa.w[2] = wv;
  qa.head_idx = head_idx;
  qa.batch = d.batch;
  qa.n = 1;
  qa.n_pad = 1;
  qa.h_kept = H;
  qa.dh = dh;
  qa.D = D;
  qa.q = ws + w.q;
  if (d.kv_quantized) {
    qa.k = ws + w.knew;
    qa.vt = ws + w.vnew;
    qa.kv_bs = D;
  } else {
    qa.k = static_cast<bf16_t*>(k_cache) + row * D;
    qa.vt = static_cast<bf16_t*>(v_cache) + row * D;
    qa.kv_bs = cap * D;
  }
  SPATTEN_TRY(launch_qkv(qa, st));
  DecodeArgs da{};
  da.q = ws + w.q;
  da.k_cache = k_cache;
  da.v_cache = v_cache;
  da.k_msb = k_msb;
  da.k_lsb = k_lsb;
  da.k_scale = k_scale;
  da.v_msb = v_msb;
  da.v_lsb = v_lsb;
  da.v_scale = v_scale;
  if (d.kv_quantized) {
    da.knew = ws + w.knew;
    da.vnew = ws + w.vnew;
  }
  da.batch = d.batch;
  da.H = H;
  da.dh = dh;
  da.cap = int(cap);
  da.lc = int(w.lc);
  da.lc_pad = int(w.lc_pad);
  da.nchunk = int(w.nchunk);
  da.threshold = d.pq_threshold;
  da.v_threshold = d.v_threshold;
  da.per_head = d.per_head;
  da.scores = reinterpret_cast<float*>(ws + w.scores);
  da.mpart = reinterpret_cast<float*>(ws + w.mpart);
  da.lpart = reinterpret_cast<float*>(ws + w.lpart);
  da.opart = reinterpret_cast<float*>(ws + w.opart);
  da.lse = reinterpret_cast<float*>(ws + w.lse);
  da.cmax = reinterpret_cast<float*>(ws + w.cmax);
  da.kcount = reinterpret_cast<int32_t*>(ws + w.kcount);
  da.o = ws + w.o;
  da.a = a;
  da.recompute = recompute;
  da.v_kept = v_kept;
  ImpArgs imp{};
  SPATTEN_TRY(launch_decode(da, d.kv_quantized != 0, &imp, st));
  OutArgs oa{};
  oa.imp = &imp;
  oa.dtype = d.dtype;
  oa.o = ws + w.o;
  oa.wo = wo;
  oa.head_idx = head_idx;
  oa.batch = d.batch;
  oa.n = 1;
  oa.h_kept = H;
  oa.dh = dh;
  oa.D = D;
  oa.x = x;
  return launch_out(oa, st);
}

// Scratch of spatten_layer_forward_noalloc: device memory beyond the
// caller's tensors (projected Q/K/V, scores, partial results)
// for callers that cannot allocate. Each device that loads the library
// holds its own copy until the process ends. In host code `scratch` names
// a host-side stand-in; kernels get the per-device address from
// hipGetSymbolAddress, taken once per device with that device current.
__device__ __align__(256) char scratch[SPATTEN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
char* scratch_ptr[kMaxDevices] = {};

int device_scratch(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SPATTEN_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return SPATTEN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return SPATTEN_EHIP;
    }
    scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = scratch_ptr[dev];
  return SPATTEN_OK;
}

}  // namespace

extern "C" {

int spatten_layer_forward(const spatten_layer_desc* d, void* x, const void* wq, const void* wk,
                          const void* wv, const void* wo, const int32_t* head_idx,
                          const int32_t* head_keys, float* a, float* g, void* k_cache,
                          void* v_cache, uint8_t* k_msb, uint8_t* k_lsb, float* k_scale,
                          uint8_t* v_msb, uint8_t* v_lsb, float* v_scale, int32_t* recompute,
                          int32_t* v_kept, float* lse, void* workspace, size_t* workspace_bytes,
                          void* stream) {
  const int st = check_layer(d, x, wq, wk, wv, wo, head_idx, head_keys, a, g, k_cache, v_cache,
                             k_msb, k_lsb, k_scale, v_msb, v_lsb, v_scale, workspace,
                             workspace_bytes);
  if (st != SPATTEN_OK) return st;
  if (!workspace) {
    *workspace_bytes = layer_workspace_bytes(*d);
    return SPATTEN_OK;
  }
  if (d->batch == 0) return SPATTEN_OK;
  char* ws = static_cast<char*>(workspace);
  if (d->mode == SPATTEN_PREFILL)
    return layer_prefill(*d, x, wq, wk, wv, wo, head_idx, head_keys, a, g, lse, ws,
                         as_stream(stream));
  return layer_decode(*d, x, wq, wk, wv, wo, head_idx, a, k_cache, v_cache, k_msb, k_lsb, k_scale,
                      v_msb, v_lsb, v_scale, recompute, v_kept, ws, as_stream(stream));
}

int spatten_layer_forward_noalloc(const spatten_layer_desc* d, void* x, const void* wq,
                                  const void* wk, const void* wv, const void* wo,
                                  const int32_t* head_idx, const int32_t* head_keys, float* a,
                                  float* g, void* k_cache, void* v_cache, uint8_t* k_msb,
                                  uint8_t* k_lsb, float* k_scale, uint8_t* v_msb,
                                  uint8_t* v_lsb, float* v_scale, int32_t* recompute,
                                  int32_t* v_kept, float* lse, void* stream) {
  size_t bytes = SPATTEN_NOALLOC_SCRATCH_BYTES;
  // descriptor first (no workspace: only *d is checked), then the size
  int st = check_layer(d, x, wq, wk, wv, wo, head_idx, head_keys, a, g, k_cache, v_cache, k_msb,
                       k_lsb, k_scale, v_msb, v_lsb, v_scale, nullptr, &bytes);
  if (st != SPATTEN_OK) return st;
  if (layer_workspace_bytes(*d) > SPATTEN_NOALLOC_SCRATCH_BYTES) return SPATTEN_EWORKSPACE;
  if (d->batch == 0) return SPATTEN_OK;
  char* ws = nullptr;
  st = device_scratch(&ws);
  if (st != SPATTEN_OK) return st;
  st = check_layer(d, x, wq, wk, wv, wo, head_idx, head_keys, a, g, k_cache, v_cache, k_msb,
                   k_lsb, k_scale, v_msb, v_lsb, v_scale, ws, &bytes);
  if (st != SPATTEN_OK) return st;
  if (d->mode == SPATTEN_PREFILL)
    return layer_prefill(*d, x, wq, wk, wv, wo, head_idx, head_keys, a, g, lse, ws,
                         as_stream(stream));
  return layer_decode(*d, x, wq, wk, wv, wo, head_idx, a, k_cache, v_cache, k_msb, k_lsb, k_scale,
                      v_msb, v_lsb, v_scale, recompute, v_kept, ws, as_stream(stream));
}

int spatten_ada_select(const float* x, int32_t batch, int32_t T, int32_t d, float tau,
                       const int32_t* prev, int32_t* flags, float* maxcos, int32_t* counts,
                       void* workspace, size_t* workspace_bytes, void* stream) {
  const int st = check_ada(x, batch, T, d, tau, flags, workspace, workspace_bytes);
  if (st != SPATTEN_OK) return st;
  const AdaWs w = ada_ws(batch, T);
  if (!workspace) {
    *workspace_bytes = w.total;
    return SPATTEN_OK;
  }
  if (batch == 0) return SPATTEN_OK;
  char* ws = static_cast<char*>(workspace);
  AdaArgs a{};
  a.x = x;
  a.batch = batch;
  a.T = T;
  a.d = d;
  a.tau = tau;
  a.prev = prev;
  a.flags = flags;
  a.maxcos = maxcos;
  a.counts = counts;
  a.inv = reinterpret_cast<float*>(ws + w.inv);
  a.listR = reinterpret_cast<int32_t*>(ws + w.listR);
  a.listN = reinterpret_cast<int32_t*>(ws + w.listN);
  a.listV = reinterpret_cast<int32_t*>(ws + w.listV);
  a.cnt = reinterpret_cast<int32_t*>(ws + w.cnt);
  a.rc = reinterpret_cast<uint32_t*>(ws + w.rc);
  a.ac = reinterpret_cast<uint32_t*>(ws + w.ac);
  return launch_ada_select(a, as_stream(stream));
}

int spatten_topk(const float* scores, int32_t batch, int32_t n, int64_t row_stride, int32_t k,
                 int32_t* out_idx, float* kth_value, void* stream) {
  const int st = check_topk(scores, batch, n, row_stride, k, out_idx);
  if (st != SPATTEN_OK) return st;
  return launch_topk(scores, batch, n, row_stride, k, out_idx, kth_value, as_stream(stream));
}

int spatten_compact(int32_t n_tensors, const void* const* src, void* const* dst,
                    const int64_t* row_bytes, const int64_t* src_batch_stride,
                    const int64_t* dst_batch_stride, const int32_t* idx, int32_t batch, int32_t k,
                    void* stream) {
  const int st = check_compact(n_tensors, src, dst, row_bytes, src_batch_stride, dst_batch_stride,
                               idx, batch, k);
  if (st != SPATTEN_OK) return st;
  return launch_compact(n_tensors, src, dst, row_bytes, src_batch_stride, dst_batch_stride, idx,
                        batch, k, as_stream(stream));
}

int spatten_compact_inplace(int32_t n_tensors, void* const* base, const int64_t* row_bytes,
                            const int64_t* row_pitch, const int64_t* batch_stride,
                            const int32_t* idx, int32_t batch, int32_t n, int32_t k,
                            void* stream) {
  const int st = check_compact_inplace(n_tensors, base, row_bytes, row_pitch, batch_stride, idx,
                                       batch, n, k);
  if (st != SPATTEN_OK) return st;
  return launch_compact_inplace(n_tensors, base, row_bytes, row_pitch, batch_stride, idx, batch,
                                n, k, as_stream(stream));
}

int spatten_quantize_kv(const void* kv, int32_t dtype, int32_t batch, int32_t n, int32_t dim,
                        int32_t head_dim, int64_t kv_batch_stride, uint8_t* msb, uint8_t* lsb,
                        float* scale, int64_t plane_rows, void* stream) {
  const int st = check_quantize(kv, dtype, batch, n, dim, head_dim, kv_batch_stride, msb, lsb,
                                scale, plane_rows);
  if (st != SPATTEN_OK) return st;
  return launch_quantize(kv, dtype, batch, n, dim, head_dim, kv_batch_stride, msb, lsb, scale,
                         plane_rows, as_stream(stream));
}

const char* spatten_status_string(int status) {
  switch (status) {
    case SPATTEN_OK: return "ok";
    case SPATTEN_EINVAL: return "invalid argument";
    case SPATTEN_EUNSUPPORTED: return "unsupported shape or mode";
    case SPATTEN_EWORKSPACE: return "workspace too small";
    case SPATTEN_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
