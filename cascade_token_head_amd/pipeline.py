"""Cascade drivers: sequences the C-ABI calls over a stack of layers.

All device memory is allocated up front (constructors), so `run()` /
`step()` only enqueue library calls and can be captured in a HIP graph.

Prefill (SpAtten section II "Cascade pruning"; "A. Cascade Token
Pruning"): after layer l (l < L) the next layer keeps the top n_{l+1}
tokens by cumulative importance; x, the importance scores and the original
positions are compacted together, so pruned tokens are gone from every
later layer. When the head count drops, the kept heads are re-ranked by
cumulative head importance.

Per-head token pruning in prefill ("A. Neural Networks Pruning and
Quantization", bullet "Token Pruning"): every token keeps its row of x;
each kept head attends over its own kept tokens and cuts them by its own
cumulative importance after every layer.

Decode (section II, generation): one token per step against per-layer K/V
caches; after every layer of step 1 the caches of all layers are pruned to
the top cache_keep entries by cumulative importance, and with prune_every
= r > 0 cut back to cache_keep again after every r-th later step. Local
value pruning ("A. Cascade Token Pruning", bullet "Local Value Pruning")
is a per-layer option of the attention call.
"""
from __future__ import annotations

from typing import List, Optional

import torch

from . import spatten as S


def weights_to_device(layers: List[dict], dtype: torch.dtype, device="cuda") -> List[dict]:
    """Per-layer x @ W weights ([D_in, D_out] arrays) -> output-major device
    tensors (w[o, i]), the layout the library takes."""
    out = []
    for w in layers:
        out.append({k: torch.as_tensor(w[k]).t().contiguous().to(device=device, dtype=dtype)
                    for k in ("wq", "wk", "wv", "wo")})
    return out


class PrefillStack:
    def __init__(self, n_layers: int, batch: int, n_heads: int, head_dim: int, tokens, heads,
                 dtype: torch.dtype, causal: bool, weights: List[dict], device="cuda",
                 v_threshold: float = 0.0):
        assert len(tokens) == n_layers and len(heads) == n_layers
        self.L, self.B, self.H, self.dh = n_layers, batch, n_heads, head_dim
        self.D = n_heads * head_dim
        self.tokens, self.heads = list(tokens), list(heads)
        self.dtype, self.causal, self.w = dtype, causal, weights
        self.es = torch.tensor([], dtype=dtype).element_size()
        B, T, D, H = batch, tokens[0], self.D, n_heads
        dev = device
        self.xbuf = [torch.empty(B * T * D, dtype=dtype, device=dev) for _ in range(2)]
        self.abuf = [torch.zeros(B * T, dtype=torch.float32, device=dev) for _ in range(2)]
        self.pbuf = [torch.empty(B * T, dtype=torch.int32, device=dev) for _ in range(2)]
        self.hbuf = [torch.empty(B * H, dtype=torch.int32, device=dev) for _ in range(2)]
        self.g = torch.zeros(B, H, dtype=torch.float32, device=dev)
        self.g_kept = torch.empty(B * H, dtype=torch.float32, device=dev)
        self.tok_idx = torch.empty(B * T, dtype=torch.int32, device=dev)
        self.head_sel = torch.empty(B * H, dtype=torch.int32, device=dev)
        self.descs = [S.make_desc(S.PREFILL, S.dtype_code(dtype), causal, B, tokens[l], H,
                                  heads[l], head_dim, v_threshold=v_threshold)
                      for l in range(n_layers)]
        ws = max(S.workspace_bytes(d) for d in self.descs)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.lse = None
        self.trace: Optional[list] = None

    def load(self, x: torch.Tensor):
        """Reset the cascade state and load x [B, T, D]."""
        B, T, H = self.B, self.tokens[0], self.H
        self.xbuf[0][: B * T * self.D].copy_(x.reshape(-1))
        self.abuf[0].zero_()
        self.g.zero_()
        self.pbuf[0].copy_(torch.arange(T, dtype=torch.int32, device=self.g.device).repeat(B))
        self.hbuf[0].copy_(torch.arange(H, dtype=torch.int32, device=self.g.device).repeat(B))

    def run(self, record: bool = False, layer_hook=None):
        """Run all layers; returns (x [B, n_L, D], pos [B, n_L], heads [B, h_L]).
        layer_hook(l), if given, is called after layer l's calls (its
        forward, and the head and token selection and compaction that
        follow it) have been enqueued."""
        B, D, es = self.B, self.D, self.es
        cur_t, cur_h = 0, 0
        self.trace = [] if record else None
        for l in range(self.L):
            n, h = self.tokens[l], self.heads[l]
            x = self.xbuf[cur_t][: B * n * D].view(B, n, D)
            a = self.abuf[cur_t][: B * n].view(B, n)
            hidx = self.hbuf[cur_h][: B * h].view(B, h)
            lse = None
            if record:
                lse = torch.empty(B, h, n, dtype=torch.float32, device=x.device)
                rec = {"x_in": x.clone(), "a_in": a.clone(), "g_in": self.g.clone(),
                       "heads": hidx.clone(),
                       "pos": self.pbuf[cur_t][: B * n].view(B, n).clone()}
            w = self.w[l]
            S.layer_forward(self.descs[l], x, w["wq"], w["wk"], w["wv"], w["wo"], hidx, a, self.g,
                            self.ws, lse=lse)
            if record:
                rec.update({"x_out": x.clone(), "a_out": a.clone(), "g_out": self.g.clone(),
                            "lse": lse, "ws": self.ws.clone()})
            if l + 1 < self.L:
                h2, n2 = self.heads[l + 1], self.tokens[l + 1]
                if h2 != h:
                    gk = self.g_kept[: B * h].view(B, h)
                    S.compact([(self.g, gk, 4, self.H * 4, h * 4)], hidx, h)
                    sel = self.head_sel[: B * h2].view(B, h2)
                    S.topk(gk, h2, out=sel)
                    hnew = self.hbuf[cur_h ^ 1][: B * h2].view(B, h2)
                    S.compact([(hidx, hnew, 4, h * 4, h2 * 4)], sel, h2)
                    cur_h ^= 1
                    if record:
                        rec["head_sel"] = sel.clone()
                idx = self.tok_idx[: B * n2].view(B, n2)
                S.topk(a, n2, out=idx)
                nt = cur_t ^ 1
                S.compact([
                    (x, self.xbuf[nt], D * es, n * D * es, n2 * D * es),
                    (a, self.abuf[nt], 4, n * 4, n2 * 4),
                    (self.pbuf[cur_t], self.pbuf[nt], 4, n * 4, n2 * 4),
                ], idx, n2)
                cur_t = nt
                if record:
                    rec["tok_sel"] = idx.clone()
            if record:
                self.trace.append(rec)
            if layer_hook is not None:
                layer_hook(l)
        nL, hL = self.tokens[-1], self.heads[-1]
        self.final = (self.xbuf[cur_t][: B * nL * D].view(B, nL, D),
                      self.pbuf[cur_t][: B * nL].view(B, nL),
                      self.hbuf[cur_h][: B * hL].view(B, hL),
                      self.abuf[cur_t][: B * nL].view(B, nL))
        return self.final


class PerHeadPrefillStack:
    """Prefill stack with per-head token pruning (bf16, bidirectional):
    every token keeps its row of x through all layers; each kept head slot
    attends over its own kept tokens, key_keep[l] of them at layer l, and
    after each layer keeps the top key_keep[l + 1] of them by its own
    cumulative importance a[b, slot, token]. Heads are cut by cumulative
    head importance as in PrefillStack; the slot rows of a and of the key
    lists follow the kept heads."""

    def __init__(self, n_layers: int, batch: int, n_heads: int, head_dim: int, n_tokens: int,
                 heads, key_keep, weights: List[dict], device="cuda"):
        assert len(heads) == n_layers and len(key_keep) == n_layers
        assert key_keep[0] == n_tokens, "every head starts with every token"
        assert all(1 <= m <= n_tokens for m in key_keep)
        assert all(b <= a for a, b in zip(key_keep, key_keep[1:]))
        self.L, self.B, self.H, self.dh, self.n = n_layers, batch, n_heads, head_dim, n_tokens
        self.D = n_heads * head_dim
        self.heads, self.keep, self.w = list(heads), list(key_keep), weights
        B, H, n, dev = batch, n_heads, n_tokens, device
        self.x = torch.empty(B, n, self.D, dtype=torch.bfloat16, device=dev)
        self.abuf = [torch.zeros(B * H * n, dtype=torch.float32, device=dev) for _ in range(2)]
        self.kbuf = [torch.empty(B * H * n, dtype=torch.int32, device=dev) for _ in range(2)]
        self.hbuf = [torch.empty(B * H, dtype=torch.int32, device=dev) for _ in range(2)]
        self.g = torch.zeros(B, H, dtype=torch.float32, device=dev)
        self.g_kept = torch.empty(B * H, dtype=torch.float32, device=dev)
        self.head_sel = torch.empty(B * H, dtype=torch.int32, device=dev)
        self.key_scores = torch.empty(B * H * n, dtype=torch.float32, device=dev)
        self.key_sel = torch.empty(B * H * n, dtype=torch.int32, device=dev)
        self.descs = [S.make_desc(S.PREFILL, S.BF16, False, B, n, H, heads[l], head_dim,
                                  per_head=True, n_keys=key_keep[l]) for l in range(n_layers)]
        ws = max(S.workspace_bytes(d) for d in self.descs)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.trace: Optional[list] = None

    def load(self, x: torch.Tensor):
        """Reset the cascade state and load x [B, n, D]; every head keeps
        every token at the first layer."""
        B, H, n = self.B, self.H, self.n
        self.x.copy_(x.reshape(B, n, self.D))
        self.abuf[0].zero_()
        self.g.zero_()
        dev = self.g.device
        self.hbuf[0].copy_(torch.arange(H, dtype=torch.int32, device=dev).repeat(B))
        self.kbuf[0][: B * H * n].copy_(
            torch.arange(n, dtype=torch.int32, device=dev).repeat(B * H))

    def run(self, record: bool = False, layer_hook=None):
        """Run all layers; returns (x [B, n, D], heads [B, h_L], keys
        [B, h_L, m_L], a [B, h_L, n])."""
        B, n, D = self.B, self.n, self.D
        cur_a, cur_h, cur_k = 0, 0, 0
        self.trace = [] if record else None
        for l in range(self.L):
            h, m = self.heads[l], self.keep[l]
            a = self.abuf[cur_a][: B * h * n].view(B, h, n)
            keys = self.kbuf[cur_k][: B * h * m].view(B, h, m)
            hidx = self.hbuf[cur_h][: B * h].view(B, h)
            lse = None
            if record:
                lse = torch.empty(B, h, n, dtype=torch.float32, device=self.x.device)
                rec = {"x_in": self.x.clone(), "a_in": a.clone(), "g_in": self.g.clone(),
                       "heads": hidx.clone(), "keys": keys.clone()}
            w = self.w[l]
            S.layer_forward(self.descs[l], self.x, w["wq"], w["wk"], w["wv"], w["wo"], hidx, a,
                            self.g, self.ws, lse=lse, head_keys=keys)
            if record:
                rec.update({"x_out": self.x.clone(), "a_out": a.clone(),
                            "g_out": self.g.clone(), "lse": lse, "ws": self.ws.clone()})
            if l + 1 < self.L:
                h2, m2 = self.heads[l + 1], self.keep[l + 1]
                if h2 != h:
                    gk = self.g_kept[: B * h].view(B, h)
                    S.compact([(self.g, gk, 4, self.H * 4, h * 4)], hidx, h)
                    sel = self.head_sel[: B * h2].view(B, h2)
                    S.topk(gk, h2, out=sel)
                    hnew = self.hbuf[cur_h ^ 1][: B * h2].view(B, h2)
                    anew = self.abuf[cur_a ^ 1][: B * h2 * n].view(B, h2, n)
                    knew = self.kbuf[cur_k ^ 1][: B * h2 * m].view(B, h2, m)
                    S.compact([(hidx, hnew, 4, h * 4, h2 * 4),
                               (a, anew, n * 4, h * n * 4, h2 * n * 4),
                               (keys, knew, m * 4, h * m * 4, h2 * m * 4)], sel, h2)
                    hidx, a, keys = hnew, anew, knew
                    cur_h, cur_a, cur_k = cur_h ^ 1, cur_a ^ 1, cur_k ^ 1
                    if record:
                        rec["head_sel"] = sel.clone()
                if m2 != m:
                    # each slot's importance at its own kept tokens, top m2 of
                    # those (positions in the key list), then the key list cut
                    rows = B * h2
                    sc = self.key_scores[: rows * m].view(rows, m)
                    S.compact([(a, sc, 4, n * 4, m * 4)], keys.view(rows, m), m)
                    ksel = self.key_sel[: rows * m2].view(rows, m2)
                    S.topk(sc, m2, out=ksel)
                    knew = self.kbuf[cur_k ^ 1][: rows * m2].view(B, h2, m2)
                    S.compact([(keys, knew, 4, m * 4, m2 * 4)], ksel, m2)
                    cur_k ^= 1
                    if record:
                        rec["key_sel"] = ksel.view(B, h2, m2).clone()
            if record:
                self.trace.append(rec)
            if layer_hook is not None:
                layer_hook(l)
        hL, mL = self.heads[-1], self.keep[-1]
        self.final = (self.x, self.hbuf[cur_h][: B * hL].view(B, hL),
                      self.kbuf[cur_k][: B * hL * mL].view(B, hL, mL),
                      self.abuf[cur_a][: B * hL * n].view(B, hL, n))
        return self.final


def _row_views(t: torch.Tensor):
    """Views of t whose dim 1 is the cache row: t itself for [B, cap, ...],
    one [B, cap, dh/2] view per head for head-major planes [B, H, cap, dh/2]."""
    if t.dim() == 4:
        return [t[:, h] for h in range(t.shape[1])]
    return [t]


class DecodeStack:
    def __init__(self, n_layers: int, batch: int, n_heads: int, head_dim: int, cache_len: int,
                 cache_keep: int, steps: int, weights: List[dict], quantized: bool = False,
                 threshold: float = 0.0, dtype: torch.dtype = torch.bfloat16, device="cuda",
                 v_threshold: float = 0.0, prune_every: int = 0, per_head: bool = False):
        self.L, self.B, self.H, self.dh = n_layers, batch, n_heads, head_dim
        self.D = D = n_heads * head_dim
        self.L0, self.keep, self.steps = cache_len, cache_keep, steps
        self.cap = cap = cache_len + steps
        self.quantized, self.threshold, self.w, self.dtype = quantized, threshold, weights, dtype
        self.v_threshold, self.prune_every, self.per_head = v_threshold, prune_every, per_head
        # repeated and per-head cuts run in place on one copy of the caches;
        # a single shared cut gathers the survivors, in order, into the
        # second copy
        self.inplace = prune_every > 0 or per_head
        sides = 1 if self.inplace else 2
        B, dev = batch, device
        self.caches = [[] for _ in range(sides)]
        for side in range(sides):
            for _ in range(n_layers):
                if quantized:
                    # head-major planes: each (sequence, head) slab contiguous;
                    # per-head pruning keeps a scale per (head, slot)
                    pl = (B, n_heads, cap, head_dim // 2)
                    sc = (B, n_heads, cap) if per_head else (B, cap)
                    c = {"k_msb": torch.empty(pl, dtype=torch.uint8, device=dev),
                         "k_lsb": torch.empty(pl, dtype=torch.uint8, device=dev),
                         "k_scale": torch.empty(sc, dtype=torch.float32, device=dev),
                         "v_msb": torch.empty(pl, dtype=torch.uint8, device=dev),
                         "v_lsb": torch.empty(pl, dtype=torch.uint8, device=dev),
                         "v_scale": torch.empty(sc, dtype=torch.float32, device=dev)}
                else:
                    c = {"k_cache": torch.empty(B, cap, D, dtype=dtype, device=dev),
                         "v_cache": torch.empty(B, cap, D, dtype=dtype, device=dev)}
                self.caches[side].append(c)
        # per-token scales of the initial cache, copied to every head's slots
        # when each head keeps its own entries
        self.scale_tok = (torch.empty(B, cap, dtype=torch.float32, device=dev)
                          if quantized and per_head else None)
        ashape = (B, n_heads, cap) if per_head else (B, cap)
        self.abuf = [torch.zeros(ashape, dtype=torch.float32, device=dev) for _ in range(sides)]
        self.x = torch.empty(B, 1, D, dtype=dtype, device=dev)
        self.head_idx = torch.arange(n_heads, dtype=torch.int32, device=dev).repeat(B, 1).contiguous()
        self.g = torch.zeros(B, n_heads, dtype=torch.float32, device=dev)
        self.recompute = torch.zeros(n_layers, B, n_heads, dtype=torch.int32, device=dev)
        self.v_kept = torch.zeros(n_layers, B, n_heads, dtype=torch.int32, device=dev)
        self.cache_sel = torch.empty((n_heads, B, cache_keep) if per_head else (B, cache_keep),
                                     dtype=torch.int32, device=dev)
        dmax = S.make_desc(S.DECODE, S.dtype_code(dtype), False, B, 1, n_heads, n_heads, head_dim,
                           cap - 1, cap, quantized, threshold, v_threshold, per_head)
        self.ws = torch.empty(max(S.workspace_bytes(dmax), 256), dtype=torch.uint8, device=dev)
        self.side, self.len, self.s = 0, cache_len, 0
        self.trace = []

    def load(self, k0: List[torch.Tensor], v0: List[torch.Tensor]):
        """Initial caches, per layer [B, L0, H, dh] in dtype on the device."""
        B, L0, D = self.B, self.L0, self.D
        for l in range(self.L):
            c = self.caches[0][l]
            if self.quantized and self.per_head:
                for kv, name in ((k0[l], "k"), (v0[l], "v")):
                    S.quantize_kv(kv.reshape(B, L0, D), c[name + "_msb"], c[name + "_lsb"],
                                  self.scale_tok)
                    c[name + "_scale"].copy_(self.scale_tok[:, None, :].expand(B, self.H,
                                                                                self.cap))
            elif self.quantized:
                S.quantize_kv(k0[l].reshape(B, L0, D), c["k_msb"], c["k_lsb"], c["k_scale"])
                S.quantize_kv(v0[l].reshape(B, L0, D), c["v_msb"], c["v_lsb"], c["v_scale"])
            else:
                c["k_cache"][:, :L0].copy_(k0[l].reshape(B, L0, D))
                c["v_cache"][:, :L0].copy_(v0[l].reshape(B, L0, D))
        for a in self.abuf:
            a.zero_()
        self.side, self.len, self.s = 0, L0, 0
        self.trace = []

    def step(self, x: torch.Tensor, record: bool = False, hook=None) -> torch.Tensor:
        """One decode step for x [B, D]; returns the step's output x [B, D].
        With record=True the per-layer recompute flags of this step are kept
        in self.trace. hook(phase, layer), if given, is called before
        ("pre") and after ("post") each layer call."""
        B, H = self.B, self.H
        self.x.view(B, self.D).copy_(x)
        desc = S.make_desc(S.DECODE, S.dtype_code(self.dtype), False, B, 1, H, H, self.dh,
                           self.len, self.cap, self.quantized, self.threshold, self.v_threshold,
                           self.per_head)
        a = self.abuf[self.side]
        for l in range(self.L):
            w, c = self.w[l], self.caches[self.side][l]
            if hook is not None:
                hook("pre", l)
            S.layer_forward(desc, self.x, w["wq"], w["wk"], w["wv"], w["wo"], self.head_idx, a,
                            self.g, self.ws, recompute=self.recompute[l], v_kept=self.v_kept[l],
                            **c)
            if hook is not None:
                hook("post", l)
        self.len += 1
        if record:
            self.trace.append({"recompute": self.recompute.clone(),
                               "v_kept": self.v_kept.clone()})
        if self.cut_due():
            if record:
                self.trace[-1]["a_before_cut"] = self.abuf[self.side][..., :self.len].clone()
            self.prune()
            if record:
                self.trace[-1]["cache_sel"] = self.cache_sel.clone()
        self.s += 1
        return self.x.view(B, self.D)

    def cut_due(self) -> bool:
        """After the first step, and after every prune_every-th later one,
        when the cache holds more than `keep` entries."""
        r = self.prune_every
        return (self.s == 0 or (r > 0 and self.s % r == 0)) and self.len > self.keep

    def prune(self):
        """Keep the top `keep` cache entries (by cumulative importance) in
        every layer: a gather into the second copy of the caches, in order,
        or for repeated cuts an in-place move of the survivors that sit past
        the kept range into the dropped rows."""
        B, cap, k = self.B, self.cap, self.keep
        a = self.abuf[self.side]
        if self.per_head:
            # each head: its own top-k, then an in-place cut of its 128-byte
            # slice of every layer's cache rows (quantized: its slab of plane
            # rows and its row of scales) and of its importance row
            H, dh, D = self.H, self.dh, self.D
            for h in range(H):
                sel = self.cache_sel[h]
                S.topk(a[:, h, :], k, n=self.len, out=sel)
                tensors = [(a[:, h, :], 4, H * cap * 4)]
                for c in self.caches[0]:
                    for t in c.values():
                        es = t.element_size()
                        if t.dim() == 4:    # planes [B, H, cap, dh/2]
                            tensors.append((t[:, h], t.shape[3], H * cap * t.shape[3]))
                        elif t.dim() == 3 and self.quantized:   # scales [B, H, cap]
                            tensors.append((t[:, h], es, H * cap * es))
                        else:               # rows [B, cap, D]
                            tensors.append((t[:, :, h * dh:(h + 1) * dh], dh * es,
                                            cap * D * es, D * es))
                S.compact_inplace(tensors, sel, self.len, k)
            a[:, :, k:self.len].zero_()
            self.len = k
            return
        S.topk(a, k, n=self.len, out=self.cache_sel)
        if self.inplace:
            tensors = [(a, 4, cap * 4)]
            for c in self.caches[0]:
                for t in c.values():
                    for v in _row_views(t):
                        es = v.element_size()
                        rb = v.stride(1) * es if v.dim() == 3 else es
                        tensors.append((v, rb, v.stride(0) * es))
            S.compact_inplace(tensors, self.cache_sel, self.len, k)
            # rows past the kept range take the next entries, whose
            # importance starts at 0
            a[:, k:self.len].zero_()
            self.len = k
            return
        a2 = self.abuf[self.side ^ 1]
        pairs = [(a, a2, 4, cap * 4, cap * 4)]
        for l in range(self.L):
            src, dst = self.caches[self.side][l], self.caches[self.side ^ 1][l]
            for name, t in src.items():
                for v, w in zip(_row_views(t), _row_views(dst[name])):
                    es = v.element_size()
                    rb = v.stride(1) * es if v.dim() == 3 else es
                    pairs.append((v, w, rb, v.stride(0) * es, w.stride(0) * es))
        S.compact(pairs, self.cache_sel, k)
        self.side ^= 1
        self.len = k


class AdaStack:
    """Representative-token selection over a stack of layer activations
    (page 5, "Cascade Token Selection for Transformer Attention
    Acceleration"): the first layer takes the full-Gram selection, every
    later one a cascade step from the previous layer's set. All buffers are
    allocated here; run() only enqueues library calls."""

    def __init__(self, n_layers: int, batch: int, seq_len: int, dim: int, tau: float,
                 device="cuda"):
        self.L, self.B, self.T, self.d, self.tau = n_layers, batch, seq_len, dim, tau
        self.flags = torch.zeros(n_layers, batch, seq_len, dtype=torch.int32, device=device)
        self.maxcos = torch.empty(n_layers, batch, seq_len, dtype=torch.float32, device=device)
        self.counts = torch.zeros(n_layers, batch, 4, dtype=torch.int32, device=device)
        self.ws = torch.empty(max(S.ada_workspace_bytes(batch, seq_len, dim), 256),
                              dtype=torch.uint8, device=device)

    def run(self, layers, full_every_layer: bool = False):
        """layers: per-layer activations [B, T, d] fp32 device tensors.
        full_every_layer selects every layer independently (the baseline
        the cascade is compared with)."""
        for l, x in enumerate(layers):
            prev = None if (l == 0 or full_every_layer) else self.flags[l - 1]
            S.ada_select(x, self.tau, self.flags[l], self.ws, prev=prev, maxcos=self.maxcos[l],
                         counts=self.counts[l])
        return self.flags
