"""CPU-side checks of the C ABI: the library loads, exports every function
include/spatten.h declares, answers workspace queries, and rejects bad
arguments on the host before anything reaches the GPU. Also builds the
HIP-free validator alone with g++ and sanitizers and runs its driver."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spatten.h")


@pytest.fixture(scope="module")
def S():
    from cascade_token_head_amd import spatten
    if not os.path.exists(spatten.LIB_PATH):
        from cascade_token_head_amd import build
        build.build()
    spatten.load()
    return spatten


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spatten_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("spatten_layer_forward", "spatten_topk", "spatten_compact", "spatten_quantize_kv"):
        assert n in names


def test_library_exports_every_declared_symbol(S):
    lib = S.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], capture_output=True,
                         text=True).stdout
    for name in declared_functions():
        assert re.search(r"\bT %s\b" % name, out), name


def test_status_strings(S):
    lib = S.load()
    assert lib.spatten_status_string(0) == b"ok"
    assert lib.spatten_status_string(-3) == b"workspace too small"


def test_workspace_query_without_tensors(S):
    for desc in (S.make_desc(S.PREFILL, S.BF16, False, 32, 512, 12, 10, 64),
                 S.make_desc(S.PREFILL, S.F32, True, 1, 64, 4, 4, 32),
                 S.make_desc(S.DECODE, S.BF16, False, 64, 1, 12, 12, 64, 1024, 1056),
                 S.make_desc(S.DECODE, S.BF16, False, 16, 1, 16, 16, 64, 2048, 2080, True, 0.1)):
        assert S.workspace_bytes(desc) > 0
    # workspace grows with the cache length it must stage scores for
    small = S.workspace_bytes(S.make_desc(S.DECODE, S.BF16, False, 4, 1, 12, 12, 64, 10, 100))
    big = S.workspace_bytes(S.make_desc(S.DECODE, S.BF16, False, 4, 1, 12, 12, 64, 99, 100))
    assert big > small


FAKE = 1 << 20   # 256-aligned fake address: the validator never dereferences


def _call_layer(S, desc, ws_bytes, **kw):
    vp = ctypes.c_void_p
    names = ["x", "wq", "wk", "wv", "wo", "head_idx", "head_keys", "a", "g", "k_cache", "v_cache",
             "k_msb", "k_lsb", "k_scale", "v_msb", "v_lsb", "v_scale", "recompute", "v_kept",
             "lse"]
    args = [vp(kw[n]) if kw.get(n) else None for n in names]
    nb = ctypes.c_size_t(ws_bytes)
    return S.load().spatten_layer_forward(ctypes.byref(desc), *args, vp(kw.get("ws", FAKE)),
                                          ctypes.byref(nb), None)


def _prefill_ptrs():
    return {n: FAKE for n in ("x", "wq", "wk", "wv", "wo", "head_idx", "a", "g")}


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 48, -2), ("head_dim", 32, -2), ("n_heads_kept", 13, -1), ("n_heads_kept", 0, -1),
    ("n_tokens", 0, -1), ("mode", 7, -1), ("dtype", 5, -1), ("causal", 2, -1), ("batch", -1, -1),
])
def test_layer_rejects_bad_descriptor(S, field, value, code):
    desc = S.make_desc(S.PREFILL, S.BF16, False, 2, 100, 12, 12, 64)
    setattr(desc, field, value)
    assert _call_layer(S, desc, 1 << 40, **_prefill_ptrs()) == code


def test_layer_rejects_small_workspace_and_nulls(S):
    desc = S.make_desc(S.PREFILL, S.BF16, False, 2, 100, 12, 12, 64)
    need = S.workspace_bytes(desc)
    assert _call_layer(S, desc, need - 1, **_prefill_ptrs()) == S.EWORKSPACE
    p = _prefill_ptrs()
    p["x"] = 0
    assert _call_layer(S, desc, need, **p) == S.EINVAL
    p = _prefill_ptrs()
    p["x"] = FAKE + 2                       # misaligned
    assert _call_layer(S, desc, need, **p) == S.EINVAL
    p = _prefill_ptrs()
    p["k_cache"] = FAKE                     # caches are not prefill arguments
    assert _call_layer(S, desc, need, **p) == S.EINVAL
    assert _call_layer(S, desc, need, ws=FAKE + 16, **_prefill_ptrs()) == S.EINVAL


def test_prefill_per_head_pruning_rejections(S):
    """Per-head token pruning in prefill: bf16 bidirectional only, with
    1 <= n_keys <= n_tokens and the head_keys array given exactly then."""
    ok = S.make_desc(S.PREFILL, S.BF16, False, 2, 300, 12, 8, 64, per_head=True, n_keys=120)
    ptrs = dict(_prefill_ptrs(), head_keys=FAKE)
    # a valid call would launch; the size query stops after the descriptor
    assert _call_layer(S, ok, 0, ws=0) == S.OK
    assert S.workspace_bytes(ok) > S.workspace_bytes(
        S.make_desc(S.PREFILL, S.BF16, False, 2, 300, 12, 8, 64))
    assert _call_layer(S, ok, 1 << 40, **_prefill_ptrs()) == S.EINVAL
    for field, value, code in (("n_keys", 0, S.EINVAL), ("n_keys", 301, S.EINVAL),
                               ("causal", 1, S.EUNSUPPORTED), ("dtype", S.F32, S.EUNSUPPORTED),
                               ("v_threshold", 1e-3, S.EUNSUPPORTED)):
        d = S.make_desc(S.PREFILL, S.BF16, False, 2, 300, 12, 8, 64, per_head=True, n_keys=120)
        setattr(d, field, value)
        assert _call_layer(S, d, 1 << 40, **ptrs) == code, field
    plain = S.make_desc(S.PREFILL, S.BF16, False, 2, 300, 12, 8, 64)
    assert _call_layer(S, plain, 1 << 40, **ptrs) == S.EINVAL
    plain.n_keys = 5
    assert _call_layer(S, plain, 1 << 40, **_prefill_ptrs()) == S.EINVAL


def test_decode_rejections(S):
    base = dict(mode=S.DECODE, dtype=S.BF16, causal=False, batch=2, n_tokens=1, n_heads=12,
                n_heads_kept=12, head_dim=64, cache_len=10, cache_cap=11)
    p = _prefill_ptrs()
    p.update(k_cache=FAKE, v_cache=FAKE)
    d = S.make_desc(**{**base, "cache_cap": 10})
    assert _call_layer(S, d, 1 << 40, **p) == S.EINVAL
    d = S.make_desc(**{**base, "n_heads_kept": 10})
    assert _call_layer(S, d, 1 << 40, **p) == S.EUNSUPPORTED
    d = S.make_desc(**{**base, "n_tokens": 2})
    assert _call_layer(S, d, 1 << 40, **p) == S.EINVAL
    d = S.make_desc(**{**base, "kv_quantized": True})
    assert _call_layer(S, d, 1 << 40, **p) == S.EINVAL     # planes missing, caches given
    # local value pruning: a threshold must be a non-negative number; it is
    # taken by prefill, by unquantized caches and by quantized caches of at
    # most 4096 rows (whose scores one workgroup keeps in LDS)
    for bad in (-1e-3, float("nan")):
        d = S.make_desc(**{**base, "v_threshold": bad})
        assert _call_layer(S, d, 1 << 40, **p) == S.EINVAL
    pq = {**base, "v_threshold": 1e-3, "kv_quantized": True, "pq_threshold": 0.1}
    assert S.workspace_bytes(S.make_desc(**pq)) == S.workspace_bytes(
        S.make_desc(**{**pq, "v_threshold": 0.0}))
    d = S.make_desc(**{**pq, "cache_len": 4095, "cache_cap": 4096})
    assert S.workspace_bytes(d) > 0
    d = S.make_desc(**{**pq, "cache_len": 4096, "cache_cap": 4097})
    assert _call_layer(S, d, 1 << 40, **p) == S.EUNSUPPORTED
    d = S.make_desc(S.PREFILL, S.BF16, False, 2, 100, 12, 12, 64, v_threshold=1e-3)
    assert S.workspace_bytes(d) == S.workspace_bytes(
        S.make_desc(S.PREFILL, S.BF16, False, 2, 100, 12, 12, 64))
    # per-head importance: a flag (quantized caches included: the size query
    # accepts the descriptor); in prefill it also needs the kept key count
    # (bidirectional only)
    d = S.make_desc(**base)
    d.per_head = 2
    assert _call_layer(S, d, 1 << 40, **p) == S.EINVAL
    d = S.make_desc(**{**base, "per_head": True, "kv_quantized": True, "pq_threshold": 0.1})
    assert S.workspace_bytes(d) == S.workspace_bytes(
        S.make_desc(**{**base, "kv_quantized": True, "pq_threshold": 0.1}))
    d = S.make_desc(**{**base, "per_head": True, "n_keys": 5})
    assert _call_layer(S, d, 1 << 40, **p) == S.EINVAL
    d = S.make_desc(S.PREFILL, S.BF16, False, 2, 100, 12, 12, 64, per_head=True)
    assert _call_layer(S, d, 1 << 40, **_prefill_ptrs()) == S.EINVAL
    d = S.make_desc(S.PREFILL, S.BF16, True, 2, 100, 12, 12, 64, per_head=True, n_keys=50)
    assert _call_layer(S, d, 1 << 40, **_prefill_ptrs()) == S.EUNSUPPORTED


def test_topk_compact_quantize_rejections(S):
    lib = S.load()
    vp = ctypes.c_void_p
    assert lib.spatten_topk(vp(FAKE), 2, 10, 10, 11, vp(FAKE), None, None) == S.EINVAL
    assert lib.spatten_topk(vp(FAKE), 2, 10, 9, 5, vp(FAKE), None, None) == S.EINVAL
    assert lib.spatten_topk(vp(FAKE), 2, 0, 0, 0, vp(FAKE), None, None) == S.EINVAL
    assert lib.spatten_topk(None, 0, 10, 10, 5, None, None, None) == S.OK   # empty batch
    VP, I64 = vp * 1, ctypes.c_int64 * 1
    # overlapping src/dst
    assert lib.spatten_compact(1, VP(FAKE), VP(FAKE + 64), I64(16), I64(1600), I64(1600),
                               vp(FAKE * 2), 2, 10, None) == S.EINVAL
    # dst rows of one sequence would run into the next
    assert lib.spatten_compact(1, VP(FAKE), VP(FAKE * 4), I64(16), I64(1600), I64(32),
                               vp(FAKE * 2), 2, 10, None) == S.EINVAL
    assert lib.spatten_compact(0, None, None, None, None, None, None, 2, 10, None) == S.OK
    assert lib.spatten_quantize_kv(vp(FAKE), 1, 2, 3, 7, 0, 21, vp(FAKE), vp(FAKE), vp(FAKE), 3,
                                   None) == S.EINVAL       # odd dim
    assert lib.spatten_quantize_kv(vp(FAKE), 3, 2, 3, 8, 0, 24, vp(FAKE), vp(FAKE), vp(FAKE), 3,
                                   None) == S.EINVAL       # bad dtype
    assert lib.spatten_quantize_kv(vp(FAKE), 1, 2, 3, 8, 3, 24, vp(FAKE), vp(FAKE), vp(FAKE), 3,
                                   None) == S.EINVAL       # odd head_dim
    assert lib.spatten_quantize_kv(vp(FAKE), 1, 2, 3, 12, 8, 36, vp(FAKE), vp(FAKE), vp(FAKE), 3,
                                   None) == S.EINVAL       # head_dim does not divide dim
    assert lib.spatten_quantize_kv(vp(FAKE), 1, 1, 3, 8, 4, 24, vp(FAKE), vp(FAKE), vp(FAKE), 2,
                                   None) == S.EINVAL       # head slabs overlap
    assert lib.spatten_quantize_kv(None, 1, 0, 3, 8, 0, 24, None, None, None, 3, None) == S.OK


def test_compact_inplace_rejections(S):
    lib = S.load()
    vp = ctypes.c_void_p
    VP, I64 = vp * 1, ctypes.c_int64 * 1

    def f(nt, base, rb, bs, idx, batch, n, k, pitch=None):
        return lib.spatten_compact_inplace(nt, base, rb, pitch, bs, idx, batch, n, k, None)
    assert f(1, VP(FAKE), I64(16), I64(1600), vp(FAKE * 2), 2, 100, 101) == S.EINVAL  # k > n
    assert f(1, VP(FAKE), I64(16), I64(1600), vp(FAKE * 2), 2, 100, 0) == S.EINVAL
    assert f(1, VP(FAKE), I64(16), I64(1599), vp(FAKE * 2), 2, 100, 10) == S.EINVAL
    assert f(1, VP(FAKE), I64(0), I64(1600), vp(FAKE * 2), 2, 100, 10) == S.EINVAL
    assert f(1, VP(FAKE), I64(16), I64(1600), vp(FAKE * 2 + 2), 2, 100, 10) == S.EINVAL
    assert f(1, VP(0), I64(16), I64(1600), vp(FAKE * 2), 2, 100, 10) == S.EINVAL
    # a pitch below the row, and sequences that would overlap at the pitch
    assert f(1, VP(FAKE), I64(16), I64(1 << 20), vp(FAKE * 2), 2, 100, 10, I64(8)) == S.EINVAL
    assert f(1, VP(FAKE), I64(128), I64(99 * 1536), vp(FAKE * 2), 2, 100, 10,
             I64(1536)) == S.EINVAL
    # the selection is staged on chip: at most 8192 kept rows per sequence
    assert f(1, VP(FAKE), I64(16), I64(16 * 9000), vp(FAKE * 2), 1, 9000, 8193) == S.EUNSUPPORTED
    assert f(1, VP(FAKE), I64((1 << 26) + 16), I64(1 << 40), vp(FAKE * 2), 2, 100,
             10) == S.EUNSUPPORTED
    assert f(0, None, None, None, None, 2, 100, 10) == S.OK
    assert f(1, VP(FAKE), I64(16), I64(1600), vp(FAKE * 2), 0, 100, 10) == S.OK


def test_validator_standalone_with_sanitizers(tmp_path):
    """Build validate.cpp alone with g++ -fsanitize=address,undefined and run
    a driver over edge cases (no HIP involved)."""
    csrc = os.path.join(ROOT, "cascade_token_head_amd", "csrc")
    drv = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host", "validate_driver.cpp")
    exe = str(tmp_path / "vdrv")
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-I", csrc, drv,
                        os.path.join(csrc, "validate.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all validator cases passed" in r.stdout


def test_noalloc_rejects_oversized_and_malformed_calls_on_the_host(S):
    """The allocation-free entry point checks the descriptor, then its fixed
    scratch size, before it touches a device: a bert_base-sized prefill
    layer needs more than the scratch holds."""
    lib = S.load()
    big = S.make_desc(S.PREFILL, S.BF16, False, 32, 512, 12, 12, 64)
    assert S.workspace_bytes(big) > S.NOALLOC_SCRATCH_BYTES
    args = [ctypes.byref(big)] + [None] * 21
    assert lib.spatten_layer_forward_noalloc(*args) == S.EWORKSPACE
    bad = S.make_desc(S.PREFILL, S.BF16, False, 2, 64, 12, 13, 64)   # more kept heads than H
    assert lib.spatten_layer_forward_noalloc(ctypes.byref(bad), *([None] * 21)) == S.EINVAL
    dec = S.make_desc(S.DECODE, S.BF16, False, 64, 1, 12, 12, 64, 1024, 1056)
    assert S.workspace_bytes(dec) <= S.NOALLOC_SCRATCH_BYTES
    with open(HEADER) as f:
        assert "#define SPATTEN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in f.read()
    assert S.NOALLOC_SCRATCH_BYTES == 64 << 20
