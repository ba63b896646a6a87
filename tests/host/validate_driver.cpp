// Host-only driver for the argument validator (built with g++ and
// -fsanitize=address,undefined by tests/test_abi.py). Fake addresses are
// never dereferenced.
#include <cstdio>
#include <cstdlib>

#include "validate.hpp"

using namespace spatten;

static int failures = 0;
#define EXPECT(expr, want)                                                        \
  do {                                                                            \
    const int _r = (expr);                                                       \
    if (_r != (want)) {                                                          \
      std::printf("FAIL %s:%d %s -> %d, want %d\n", __FILE__, __LINE__, #expr, _r, \
                  (want));                                                        \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

int main() {
  char* P = reinterpret_cast<char*>(uintptr_t(1) << 20);
  spatten_layer_desc d{};
  d.mode = SPATTEN_PREFILL;
  d.dtype = SPATTEN_BF16;
  d.batch = 32;
  d.n_tokens = 489;
  d.n_heads = 12;
  d.n_heads_kept = 10;
  d.head_dim = 64;
  size_t need = layer_workspace_bytes(d);
  size_t got = need;
  const int32_t* hi = reinterpret_cast<const int32_t*>(P);
  const float* fp = reinterpret_cast<const float*>(P);
  EXPECT(check_layer(&d, P, P, P, P, P, hi, nullptr, fp, fp, nullptr, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, P, &got), SPATTEN_OK);
  got = need - 1;
  EXPECT(check_layer(&d, P, P, P, P, P, hi, nullptr, fp, fp, nullptr, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, P, &got), SPATTEN_EWORKSPACE);
  EXPECT(check_layer(nullptr, P, P, P, P, P, hi, nullptr, fp, fp, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, P, &got), SPATTEN_EINVAL);
  // extreme sizes must not overflow the workspace arithmetic
  d.batch = 1 << 30;
  d.n_tokens = 1 << 30;
  got = 0;
  EXPECT(check_layer(&d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, &got), SPATTEN_OK);
  d.batch = 2;
  d.n_tokens = 100;
  // decode
  d.mode = SPATTEN_DECODE;
  d.n_tokens = 1;
  d.n_heads_kept = 12;
  d.cache_len = 2048;
  d.cache_cap = 2049;
  d.kv_quantized = 1;
  d.pq_threshold = 0.1f;
  need = layer_workspace_bytes(d);
  got = need;
  const uint8_t* u8 = reinterpret_cast<const uint8_t*>(P);
  EXPECT(check_layer(&d, P, P, P, P, P, hi, nullptr, fp, nullptr, nullptr, nullptr, u8, u8, fp, u8, u8, fp,
                     P, &got), SPATTEN_OK);
  EXPECT(check_layer(&d, P, P, P, P, P, hi, nullptr, fp, nullptr, P, nullptr, u8, u8, fp, u8, u8, fp, P,
                     &got), SPATTEN_EINVAL);
  d.cache_cap = 2048;
  EXPECT(check_layer(&d, P, P, P, P, P, hi, nullptr, fp, nullptr, nullptr, nullptr, u8, u8, fp, u8, u8, fp,
                     P, &got), SPATTEN_EINVAL);
  // local value pruning: quantized caches up to 4096 rows (the scores of a
  // row stay in LDS); NaN and negative rejected
  d.cache_cap = 2049;
  d.v_threshold = 1e-4f;
  EXPECT(check_layer(&d, P, P, P, P, P, hi, nullptr, fp, nullptr, nullptr, nullptr, u8, u8, fp, u8, u8, fp,
                     P, &got), SPATTEN_OK);
  d.cache_len = 4096;
  d.cache_cap = 4097;
  got = layer_workspace_bytes(d);
  EXPECT(check_layer(&d, P, P, P, P, P, hi, nullptr, fp, nullptr, nullptr, nullptr, u8, u8, fp, u8, u8, fp,
                     P, &got), SPATTEN_EUNSUPPORTED);
  d.cache_len = 2048;
  d.cache_cap = 2049;
  got = need;
  d.kv_quantized = 0;
  EXPECT(check_layer(&d, P, P, P, P, P, hi, nullptr, fp, nullptr, P, P, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, P, &got), SPATTEN_OK);
  d.v_threshold = -1e-4f;
  EXPECT(check_layer(&d, P, P, P, P, P, hi, nullptr, fp, nullptr, P, P, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, P, &got), SPATTEN_EINVAL);
  d.v_threshold = __builtin_nanf("");
  EXPECT(check_layer(&d, P, P, P, P, P, hi, nullptr, fp, nullptr, P, P, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, P, &got), SPATTEN_EINVAL);
  d.v_threshold = 0.0f;
  // per-head token pruning in prefill: bf16 bidirectional, 1 <= n_keys <= n_tokens,
  // head_keys given exactly then
  d.mode = SPATTEN_PREFILL;
  d.n_tokens = 300;
  d.cache_len = d.cache_cap = 0;
  d.per_head = 1;
  d.n_keys = 120;
  need = layer_workspace_bytes(d);
  got = need;
  EXPECT(check_layer(&d, P, P, P, P, P, hi, hi, fp, fp, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, P, &got), SPATTEN_OK);
  EXPECT(check_layer(&d, P, P, P, P, P, hi, nullptr, fp, fp, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, P, &got), SPATTEN_EINVAL);
  d.n_keys = 301;
  EXPECT(check_layer(&d, P, P, P, P, P, hi, hi, fp, fp, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, P, &got), SPATTEN_EINVAL);
  d.n_keys = 0;
  EXPECT(check_layer(&d, P, P, P, P, P, hi, hi, fp, fp, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, P, &got), SPATTEN_EINVAL);
  d.n_keys = 120;
  d.causal = 1;
  EXPECT(check_layer(&d, P, P, P, P, P, hi, hi, fp, fp, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, P, &got), SPATTEN_EUNSUPPORTED);
  d.causal = 0;
  d.dtype = SPATTEN_F32;
  EXPECT(check_layer(&d, P, P, P, P, P, hi, hi, fp, fp, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, P, &got), SPATTEN_EUNSUPPORTED);
  d.dtype = SPATTEN_BF16;
  d.per_head = 0;
  EXPECT(check_layer(&d, P, P, P, P, P, hi, nullptr, fp, fp, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, P, &got), SPATTEN_EINVAL);  // n_keys set
  d.n_keys = 0;
  EXPECT(check_layer(&d, P, P, P, P, P, hi, hi, fp, fp, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, P, &got), SPATTEN_EINVAL);  // stray keys
  // representative-token selection
  {
    size_t need_a = ada_ws(4, 512).total, got_a = need_a;
    int32_t* fl = reinterpret_cast<int32_t*>(P);
    EXPECT(check_ada(fp, 4, 512, 768, 0.3f, fl, P, &got_a), SPATTEN_OK);
    EXPECT(check_ada(fp, 4, 512, 770, 0.3f, fl, P, &got_a), SPATTEN_EUNSUPPORTED);
    EXPECT(check_ada(fp, 4, 512, 768, 1.5f, fl, P, &got_a), SPATTEN_EINVAL);
    EXPECT(check_ada(fp, 4, 512, 768, __builtin_nanf(""), fl, P, &got_a), SPATTEN_EINVAL);
    EXPECT(check_ada(fp, 4, 0, 768, 0.3f, fl, P, &got_a), SPATTEN_EINVAL);
    got_a = need_a - 1;
    EXPECT(check_ada(fp, 4, 512, 768, 0.3f, fl, P, &got_a), SPATTEN_EWORKSPACE);
    EXPECT(check_ada(nullptr, 4, 512, 768, 0.3f, nullptr, nullptr, &got_a), SPATTEN_OK);
    got_a = need_a;
    EXPECT(check_ada(nullptr, 4, 512, 768, 0.3f, fl, P, &got_a), SPATTEN_EINVAL);
    EXPECT(check_ada(fp, 4, 512, 768, 0.3f, fl, P, nullptr), SPATTEN_EINVAL);
    // extreme sizes must not overflow the workspace arithmetic
    EXPECT(check_ada(nullptr, 1 << 30, 1 << 30, 32, 0.3f, nullptr, nullptr, &got_a),
           SPATTEN_EUNSUPPORTED);
  }
  // top-k
  EXPECT(check_topk(fp, 4, 100, 100, 100, hi), SPATTEN_OK);
  EXPECT(check_topk(fp, 4, 100, 100, 101, hi), SPATTEN_EINVAL);
  EXPECT(check_topk(fp, 4, 100, 99, 10, hi), SPATTEN_EINVAL);
  EXPECT(check_topk(nullptr, 0, 100, 100, 10, nullptr), SPATTEN_OK);
  // compact
  const void* src[2] = {P, P + 4096};
  void* dst[2] = {P + (1 << 16), P + (1 << 17)};
  int64_t rb[2] = {16, 4}, sb[2] = {1600, 400}, db[2] = {160, 40};
  EXPECT(check_compact(2, src, dst, rb, sb, db, hi, 2, 10), SPATTEN_OK);
  db[1] = 39;
  EXPECT(check_compact(2, src, dst, rb, sb, db, hi, 2, 10), SPATTEN_EINVAL);
  db[1] = 40;
  dst[0] = P + 800;
  EXPECT(check_compact(2, src, dst, rb, sb, db, hi, 2, 10), SPATTEN_EINVAL);
  // in-place compaction
  void* base[1] = {P};
  int64_t irb[1] = {16}, ibs[1] = {1600};
  EXPECT(check_compact_inplace(1, base, irb, nullptr, ibs, hi, 2, 100, 10), SPATTEN_OK);
  EXPECT(check_compact_inplace(1, base, irb, nullptr, ibs, hi, 2, 100, 101), SPATTEN_EINVAL);
  ibs[0] = 1599;
  EXPECT(check_compact_inplace(1, base, irb, nullptr, ibs, hi, 2, 100, 10), SPATTEN_EINVAL);
  ibs[0] = int64_t(16) << 20;
  EXPECT(check_compact_inplace(1, base, irb, nullptr, ibs, hi, 2, 1 << 16, 8193),
         SPATTEN_EUNSUPPORTED);
  EXPECT(check_compact_inplace(1, base, irb, nullptr, ibs, hi, 2, 1 << 16, 8192), SPATTEN_OK);
  // one 128-byte head slice of 1536-byte rows
  int64_t hrb[1] = {128}, hpitch[1] = {1536}, hbs[1] = {99 * 1536 + 128};
  EXPECT(check_compact_inplace(1, base, hrb, hpitch, hbs, hi, 2, 100, 10), SPATTEN_OK);
  hbs[0] = 99 * 1536 + 127;
  EXPECT(check_compact_inplace(1, base, hrb, hpitch, hbs, hi, 2, 100, 10), SPATTEN_EINVAL);
  hpitch[0] = 127;
  hbs[0] = 1 << 20;
  EXPECT(check_compact_inplace(1, base, hrb, hpitch, hbs, hi, 2, 100, 10), SPATTEN_EINVAL);
  // quantize
  EXPECT(check_quantize(P, SPATTEN_BF16, 2, 5, 1024, 0, 5 * 1024, u8, u8, fp, 5), SPATTEN_OK);
  EXPECT(check_quantize(P, SPATTEN_BF16, 2, 5, 1023, 0, 5 * 1023, u8, u8, fp, 5), SPATTEN_EINVAL);
  EXPECT(check_quantize(P, SPATTEN_BF16, 2, 5, 1024, 0, 4 * 1024, u8, u8, fp, 5), SPATTEN_EINVAL);
  // head-major planes: head_dim even and dividing dim; slabs of plane_rows >= n rows
  EXPECT(check_quantize(P, SPATTEN_BF16, 2, 5, 768, 64, 5 * 768, u8, u8, fp, 9), SPATTEN_OK);
  EXPECT(check_quantize(P, SPATTEN_BF16, 1, 5, 768, 64, 5 * 768, u8, u8, fp, 5), SPATTEN_OK);
  EXPECT(check_quantize(P, SPATTEN_BF16, 1, 5, 768, 64, 5 * 768, u8, u8, fp, 4), SPATTEN_EINVAL);
  EXPECT(check_quantize(P, SPATTEN_BF16, 1, 5, 768, 768, 5 * 768, u8, u8, fp, 1), SPATTEN_OK);
  EXPECT(check_quantize(P, SPATTEN_BF16, 2, 5, 768, 63, 5 * 768, u8, u8, fp, 5), SPATTEN_EINVAL);
  EXPECT(check_quantize(P, SPATTEN_BF16, 2, 5, 768, 96 * 5, 5 * 768, u8, u8, fp, 5), SPATTEN_EINVAL);
  EXPECT(check_quantize(P, SPATTEN_BF16, 2, 5, 768, -2, 5 * 768, u8, u8, fp, 5), SPATTEN_EINVAL);
  if (failures) return 1;
  std::printf("all validator cases passed\n");
  return 0;
}
