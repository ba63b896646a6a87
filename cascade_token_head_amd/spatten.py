"""Thin ctypes binding over libspatten.so (include/spatten.h).

Argument marshalling only: torch tensors supply device addresses and the
current HIP stream; every step runs in the library's kernels. Raises
SpattenError on any non-zero status, and RuntimeError if the library has
not been built (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspatten.so")

F32, BF16 = 0, 1
PREFILL, DECODE = 0, 1

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4

EXPORTED = ("spatten_layer_forward", "spatten_layer_forward_noalloc", "spatten_topk", "spatten_compact", "spatten_compact_inplace",
            "spatten_quantize_kv", "spatten_ada_select", "spatten_status_string")


class SpattenError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib().spatten_status_string(status).decode()
        super().__init__("%s failed: %s (%d)" % (fn, msg, status))


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32), ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("n_tokens", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("n_heads_kept", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("cache_len", ctypes.c_int32), ("cache_cap", ctypes.c_int32),
        ("kv_quantized", ctypes.c_int32), ("pq_threshold", ctypes.c_float),
        ("v_threshold", ctypes.c_float), ("per_head", ctypes.c_int32),
        ("n_keys", ctypes.c_int32),
    ]


_L = None


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libspatten.so is not built: run `python -m cascade_token_head_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.spatten_layer_forward.restype = ctypes.c_int
        lib.spatten_layer_forward.argtypes = [ctypes.POINTER(LayerDesc)] + [vp] * 21 + \
            [ctypes.POINTER(ctypes.c_size_t), vp]
        lib.spatten_layer_forward_noalloc.restype = ctypes.c_int
        lib.spatten_layer_forward_noalloc.argtypes = [ctypes.POINTER(LayerDesc)] + [vp] * 21
        lib.spatten_topk.restype = ctypes.c_int
        lib.spatten_topk.argtypes = [vp, i32, i32, i64, i32, vp, vp, vp]
        lib.spatten_compact.restype = ctypes.c_int
        lib.spatten_compact.argtypes = [i32, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                        ctypes.POINTER(i64), ctypes.POINTER(i64),
                                        ctypes.POINTER(i64), vp, i32, i32, vp]
        lib.spatten_compact_inplace.restype = ctypes.c_int
        lib.spatten_compact_inplace.argtypes = [i32, ctypes.POINTER(vp), ctypes.POINTER(i64),
                                                ctypes.POINTER(i64), ctypes.POINTER(i64), vp,
                                                i32, i32, i32, vp]
        lib.spatten_quantize_kv.restype = ctypes.c_int
        lib.spatten_quantize_kv.argtypes = [vp, i32, i32, i32, i32, i32, i64, vp, vp, vp, i64, vp]
        lib.spatten_ada_select.restype = ctypes.c_int
        lib.spatten_ada_select.argtypes = [vp, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp,
                                           ctypes.POINTER(ctypes.c_size_t), vp]
        lib.spatten_status_string.restype = ctypes.c_char_p
        lib.spatten_status_string.argtypes = [ctypes.c_int]
        _L = lib
    return _L


def load() -> ctypes.CDLL:
    """Load the library (raises if it is missing)."""
    return _lib()


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, st):
    if st != OK:
        raise SpattenError(fn, st)


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise ValueError("unsupported dtype %s" % dt)


def make_desc(mode=PREFILL, dtype=BF16, causal=False, batch=1, n_tokens=1, n_heads=1,
              n_heads_kept=None, head_dim=64, cache_len=0, cache_cap=0, kv_quantized=False,
              pq_threshold=0.0, v_threshold=0.0, per_head=False, n_keys=0) -> LayerDesc:
    return LayerDesc(mode, dtype, int(causal), batch, n_tokens, n_heads,
                     n_heads if n_heads_kept is None else n_heads_kept, head_dim, cache_len,
                     cache_cap, int(kv_quantized), float(pq_threshold), float(v_threshold),
                     int(per_head), int(n_keys))


def workspace_bytes(desc: LayerDesc) -> int:
    """Workspace size the library needs for `desc` (query mode)."""
    nb = ctypes.c_size_t(0)
    st = _lib().spatten_layer_forward(ctypes.byref(desc), *([None] * 21), ctypes.byref(nb), None)
    _check("spatten_layer_forward(query)", st)
    return nb.value


def layer_forward(desc: LayerDesc, x, wq, wk, wv, wo, head_idx, a, g, workspace,
                  k_cache=None, v_cache=None, k_msb=None, k_lsb=None, k_scale=None,
                  v_msb=None, v_lsb=None, v_scale=None, recompute=None, v_kept=None, lse=None,
                  head_keys=None, stream=None):
    nb = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    st = _lib().spatten_layer_forward(
        ctypes.byref(desc), _p(x), _p(wq), _p(wk), _p(wv), _p(wo), _p(head_idx), _p(head_keys),
        _p(a), _p(g),
        _p(k_cache), _p(v_cache), _p(k_msb), _p(k_lsb), _p(k_scale), _p(v_msb), _p(v_lsb),
        _p(v_scale), _p(recompute), _p(v_kept), _p(lse), _p(workspace), ctypes.byref(nb),
        _stream(stream))
    _check("spatten_layer_forward", st)


def layer_forward_noalloc(desc: LayerDesc, x, wq, wk, wv, wo, head_idx, a, g,
                          k_cache=None, v_cache=None, k_msb=None, k_lsb=None, k_scale=None,
                          v_msb=None, v_lsb=None, v_scale=None, recompute=None, v_kept=None,
                          lse=None, head_keys=None, stream=None):
    """layer_forward in the library's fixed per-device scratch (no workspace)."""
    st = _lib().spatten_layer_forward_noalloc(
        ctypes.byref(desc), _p(x), _p(wq), _p(wk), _p(wv), _p(wo), _p(head_idx), _p(head_keys),
        _p(a), _p(g),
        _p(k_cache), _p(v_cache), _p(k_msb), _p(k_lsb), _p(k_scale), _p(v_msb), _p(v_lsb),
        _p(v_scale), _p(recompute), _p(v_kept), _p(lse), _stream(stream))
    _check("spatten_layer_forward_noalloc", st)


NOALLOC_SCRATCH_BYTES = 64 << 20


def topk(scores: torch.Tensor, k: int, n: Optional[int] = None, out: Optional[torch.Tensor] = None,
         kth: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Top-k of scores[:, :n] per row; returns int32 [B, k] ascending indices."""
    assert scores.dtype == torch.float32 and scores.dim() == 2 and scores.stride(1) == 1
    B = scores.shape[0]
    n = scores.shape[1] if n is None else n
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=scores.device)
    st = _lib().spatten_topk(_p(scores), B, n, scores.stride(0), k, _p(out), _p(kth),
                             _stream(stream))
    _check("spatten_topk", st)
    return out


def compact(pairs: Sequence, idx: torch.Tensor, k: int, stream=None):
    """Row gather for several tensors at once.

    pairs: (src, dst, row_bytes, src_batch_stride_bytes, dst_batch_stride_bytes)
    idx:   int32 [B, k] device tensor of source row indices.
    """
    n = len(pairs)
    VP = ctypes.c_void_p * max(n, 1)
    I64 = ctypes.c_int64 * max(n, 1)
    src = VP(*[p[0].data_ptr() for p in pairs])
    dst = VP(*[p[1].data_ptr() for p in pairs])
    rb = I64(*[p[2] for p in pairs])
    sb = I64(*[p[3] for p in pairs])
    db = I64(*[p[4] for p in pairs])
    B = idx.shape[0]
    st = _lib().spatten_compact(n, src, dst, rb, sb, db, _p(idx), B, k, _stream(stream))
    _check("spatten_compact", st)


def quantize_kv(kv: torch.Tensor, msb: torch.Tensor, lsb: torch.Tensor, scale: torch.Tensor,
                n: Optional[int] = None, stream=None):
    """kv [B, n, D] (bf16/fp32) -> planes and scale [B, cap] (rows 0..n-1).

    Planes [B, H, cap, dh/2] u8 are head-major (the layout the quantized
    decode reads); [B, cap, D/2] u8 planes are token-major.
    """
    B, rows, D = kv.shape
    n = rows if n is None else n
    if msb.dim() == 4:
        H, hd2 = msb.shape[1], msb.shape[3]
        head_dim = 2 * hd2
        plane_rows = msb.stride(1) // msb.stride(2)
        assert msb.stride(3) == 1 and msb.stride(2) == hd2 and H * head_dim == D
        assert msb.stride(0) == H * msb.stride(1) and lsb.stride() == msb.stride()
    else:
        head_dim = 0
        plane_rows = msb.stride(0) // msb.stride(1)
        assert msb.stride(2) == 1 and msb.stride(1) == D // 2 and lsb.stride() == msb.stride()
    assert scale.stride(0) == plane_rows or B == 1
    st = _lib().spatten_quantize_kv(_p(kv), dtype_code(kv.dtype), B, n, D, head_dim,
                                    kv.stride(0), _p(msb), _p(lsb), _p(scale), plane_rows,
                                    _stream(stream))
    _check("spatten_quantize_kv", st)


def compact_inplace(tensors: Sequence, idx: torch.Tensor, n: int, k: int, stream=None):
    """In-place cut of rows whose order carries no meaning.

    tensors: (base, row_bytes, batch_stride_bytes[, row_pitch_bytes]) per
             tensor; base may be a view (its data_ptr is the first row).
    idx:     int32 [B, k] ascending selected rows, each below n.
    """
    m = len(tensors)
    VP = ctypes.c_void_p * max(m, 1)
    I64 = ctypes.c_int64 * max(m, 1)
    base = VP(*[t[0].data_ptr() for t in tensors])
    rb = I64(*[t[1] for t in tensors])
    bs = I64(*[t[2] for t in tensors])
    rp = I64(*[t[3] if len(t) > 3 else t[1] for t in tensors])
    B = idx.shape[0]
    st = _lib().spatten_compact_inplace(m, base, rb, rp, bs, _p(idx), B, n, k, _stream(stream))
    _check("spatten_compact_inplace", st)


def ada_workspace_bytes(batch: int, T: int, d: int) -> int:
    nb = ctypes.c_size_t(0)
    st = _lib().spatten_ada_select(None, batch, T, d, ctypes.c_float(0.3), None, None, None, None,
                                   None, ctypes.byref(nb), None)
    _check("spatten_ada_select(query)", st)
    return nb.value


def ada_select(x: torch.Tensor, tau: float, flags: torch.Tensor, workspace: torch.Tensor,
               prev: Optional[torch.Tensor] = None, maxcos: Optional[torch.Tensor] = None,
               counts: Optional[torch.Tensor] = None, stream=None):
    """Representative tokens of one layer: x [B, T, d] fp32; flags [B, T]
    int32 out; prev [B, T] int32 (None = full-Gram selection)."""
    assert x.dtype == torch.float32 and x.dim() == 3 and x.is_contiguous()
    B, T, d = x.shape
    nb = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    st = _lib().spatten_ada_select(_p(x), B, T, d, ctypes.c_float(tau), _p(prev), _p(flags),
                                   _p(maxcos), _p(counts), _p(workspace), ctypes.byref(nb),
                                   _stream(stream))
    _check("spatten_ada_select", st)
