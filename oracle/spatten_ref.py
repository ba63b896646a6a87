"""Plain fp64 CPU oracle for cascade token/head pruned attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
run this module: only the tests, the smoke entry and the benchmark's CPU
baseline leg use it. It shares no code with the HIP library.

Source: "SpAtten: Efficient Sparse Attention Architecture with Cascade Token
and Head Pruning" (Wang, Zhang, Han; arXiv 2012.09852), as summarised on the
paperlayer.ai page for that paper. Section names below are that page's.

Every function follows a definition directly, with numpy doing the
arithmetic in float64. Where a value is stored in bf16 by the GPU path
(x between layers, Q, K, V, the head outputs O and the K/V cache), the
`bf16` flag rounds to bf16 (round to nearest even) at exactly those points
and nowhere else. Decisions that turn a float into an integer are taken in
the precision the kernels take them in: top-k compares fp32 keys, and the
int8 quantizer runs in fp32.
"""
from __future__ import annotations

import math
from typing import Callable, Optional

import numpy as np

# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------


def bf16_round(a) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even).

    bf16 keeps 8 significant bits and fp32's exponent range. For normal
    numbers the quantum is 2**(e - 8) where frexp gives a = m * 2**e,
    m in [0.5, 1); below 2**-126 the quantum is fixed at 2**-133.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    e = np.maximum(e, -125)
    q = np.ldexp(np.ones_like(a), e - 8)
    return np.rint(a / q) * q


def _store(a, bf16: bool):
    return bf16_round(a) if bf16 else np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# attention (page: section II, "Attention mechanism")
# --------------------------------------------------------------------------


def softmax_rows(S: np.ndarray) -> np.ndarray:
    """Row-wise softmax; -inf entries get probability 0."""
    m = np.max(S, axis=-1, keepdims=True)
    E = np.exp(S - m)
    return E / np.sum(E, axis=-1, keepdims=True)


def head_attention(Q, K, V, causal: bool, row_block: int = 512, v_threshold: float = 0.0):
    """One head: S = Q K^T / sqrt(dh), causal mask j > i (indices are in
    ascending original-position order, so this is the positional mask),
    P = row softmax(S), O = P V.

    v_threshold > 0 applies local value pruning ("A. Cascade Token
    Pruning", bullet "Local Value Pruning") to every query row: V row j
    enters O[i] only when P[i, j] >= v_threshold, with no renormalisation;
    the column sums still take every probability.

    Returns O [n, dh], column sums of P [n], row log-sum-exp [n].
    Works in row blocks so that n x n is never held for long sequences.
    """
    n, dh = Q.shape
    scale = 1.0 / math.sqrt(dh)
    O = np.empty((n, V.shape[1]))
    col = np.zeros(K.shape[0])
    lse = np.empty(n)
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        S = (Q[r0:r1] @ K.T) * scale
        if causal:
            i = np.arange(r0, r1)[:, None]
            j = np.arange(K.shape[0])[None, :]
            S = np.where(j > i, -np.inf, S)
        m = np.max(S, axis=1, keepdims=True)
        E = np.exp(S - m)
        l = np.sum(E, axis=1, keepdims=True)
        P = E / l
        O[r0:r1] = (np.where(P >= v_threshold, P, 0.0) if v_threshold > 0 else P) @ V
        col += P.sum(axis=0)
        lse[r0:r1] = (m + np.log(l))[:, 0]
    return O, col, lse


def attention_rows(Q, K, V, rows, causal: bool, v_threshold: float = 0.0):
    """Selected query rows of one head, each from its own full row of scores
    (the definition head_attention applies to every row): for query i,
    S_i = Q_i K^T / sqrt(dh) over the keys it sees (j <= i when causal),
    P_i = softmax(S_i), O_i = P_i V.

    Returns O [len(rows), dh] and the natural-log LSE [len(rows)]. Used to
    check long sequences on a sample of rows. v_threshold as in
    head_attention.
    """
    rows = np.asarray(rows, dtype=np.int64)
    dh = Q.shape[1]
    S = (np.asarray(Q, np.float64)[rows] @ np.asarray(K, np.float64).T) / math.sqrt(dh)
    if causal:
        S = np.where(np.arange(K.shape[0])[None, :] > rows[:, None], -np.inf, S)
    m = np.max(S, axis=1, keepdims=True)
    E = np.exp(S - m)
    l = np.sum(E, axis=1, keepdims=True)
    P = E / l
    if v_threshold > 0:
        P = np.where(P >= v_threshold, P, 0.0)
    return P @ np.asarray(V, np.float64), (m + np.log(l))[:, 0]


def column_sums(Q, K, lse, cols, causal: bool):
    """Column sums of one head's P at selected key columns, given every
    row's natural-log LSE: sum over the queries i that see key j (all i, or
    i >= j when causal) of exp(Q_i . K_j / sqrt(dh) - lse_i).

    This is the token-importance contribution of the head (section II
    "Cascade pruning": importance is the probability mass a key receives),
    evaluated column by column so that n x n is never formed.
    """
    cols = np.asarray(cols, dtype=np.int64)
    dh = Q.shape[1]
    S = (np.asarray(Q, np.float64) @ np.asarray(K, np.float64)[cols].T) / math.sqrt(dh)
    E = np.exp(S - np.asarray(lse, np.float64)[:, None])
    if causal:
        E = np.where(np.arange(Q.shape[0])[:, None] < cols[None, :], 0.0, E)
    return E.sum(axis=0)


# --------------------------------------------------------------------------
# cascade token and head pruning (page: section II "Cascade pruning",
# "B. Motivation" token pruning, "A. Cascade Token Pruning")
# --------------------------------------------------------------------------


def prefill_layer(x, w: dict, heads, head_dim: int, causal: bool, bf16: bool,
                  extras: Optional[dict] = None, v_threshold: float = 0.0):
    """One attention-only residual layer over the kept tokens and heads of
    one sequence.

    x:     [n, D] kept token rows (values already in storage precision)
    w:     dict of wq, wk, wv, wo, each [D, D] in x @ W layout
    heads: kept head ids, ascending

    Returns (x_new [n, D], token-importance increment [n] = sum over kept
    heads and queries of P, head-importance increment {h: sum |O_h|},
    per-head LSE {h: [n]}). If `extras` is given it also receives the
    stored per-head Q, K, V and O under extras[h]. v_threshold > 0 applies
    local value pruning inside every head; head importance then takes the
    pruned output (the output the head hands on).
    """
    x = np.asarray(x, dtype=np.float64)
    n, D = x.shape
    dh = head_dim
    delta = np.zeros((n, D))
    dcol = np.zeros(n)
    dg = {}
    lse = {}
    for h in heads:
        c = slice(h * dh, (h + 1) * dh)
        Q = _store(x @ w["wq"][:, c].astype(np.float64), bf16)
        K = _store(x @ w["wk"][:, c].astype(np.float64), bf16)
        V = _store(x @ w["wv"][:, c].astype(np.float64), bf16)
        O, col, l = head_attention(Q, K, V, causal, v_threshold=v_threshold)
        if extras is not None:
            extras[h] = {"q": Q, "k": K, "v": V, "o": _store(O, bf16)}
        dcol += col
        dg[h] = float(np.abs(O).sum())
        lse[h] = l
        delta += _store(O, bf16) @ w["wo"][c, :].astype(np.float64)
    return _store(x + delta, bf16), dcol, dg, lse


# --------------------------------------------------------------------------
# top-k (page: "B. Top-k Engine"): the k largest scores, reported in input
# order. Ranking is on the fp32 value, ties broken towards the lower index.
# --------------------------------------------------------------------------


def order_key(v) -> np.ndarray:
    """Monotone map from fp32 to uint32: larger value -> larger key.
    Negative numbers have all bits flipped, non-negative ones the sign bit
    set, so -0.0 orders just below +0.0."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    neg = (u >> 31) == 1
    return np.where(neg, u ^ 0xFFFFFFFF, u ^ 0x80000000).astype(np.int64)


def topk(scores, k: int) -> np.ndarray:
    """Indices of the k largest fp32 scores by (key desc, index asc),
    returned in ascending index order."""
    key = order_key(scores)
    n = key.shape[0]
    assert 0 < k <= n
    order = np.lexsort((np.arange(n), -key))
    return np.sort(order[:k]).astype(np.int32)


def kth_value(scores, k: int) -> np.float32:
    """The score of the k-th ranked element (fp32)."""
    s = np.asarray(scores, dtype=np.float32)
    key = order_key(s)
    order = np.lexsort((np.arange(s.shape[0]), -key))
    return s[order[k - 1]]


def compact(arr, idx) -> np.ndarray:
    """Rows of arr at the survivor indices, in the given order."""
    return np.asarray(arr)[np.asarray(idx)]


# --------------------------------------------------------------------------
# progressive quantization (page: "A. Cascade Token Pruning", bullet "Progressive Quantization",
# IV "Quantization Support", E "Progressive Quantization")
# --------------------------------------------------------------------------


def quantize_rows(x):
    """Per-row symmetric int8 in fp32 arithmetic.

    s = fp32(max |x|) / 127; q = clamp(round_half_even(x / s), -127, 127);
    a row of zeros gets s = 0 and q = 0.
    Returns (q int8 [..., D], s float32 [...]).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    q = np.rint(x / safe[..., None]).astype(np.float32)
    q = np.where(s[..., None] == 0, np.float32(0.0), q)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, s


def split_planes(q):
    """int8 code -> (msb, lsb): msb = q >> 4 (arithmetic, -8..7),
    lsb = q & 15 (0..15); 16*msb + lsb == q."""
    q = np.asarray(q, dtype=np.int8).astype(np.int16)
    msb = (q >> 4).astype(np.int8)
    lsb = (q & 15).astype(np.uint8)
    return msb, lsb


def pack_nibbles(v):
    """Two 4-bit fields per byte: element 2j in the low nibble, element
    2j+1 in the high nibble (two's complement bits kept as is)."""
    b = (np.asarray(v).astype(np.int16) & 0xF).astype(np.uint8)
    return (b[..., 0::2] | (b[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(p, signed: bool):
    p = np.asarray(p, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    if signed:
        lo = np.where(lo >= 8, lo - 16, lo)
        hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int16)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def quantize_kv(x):
    """Full quantization of K or V rows [..., D] into the two planes.
    Returns packed msb [..., D/2] u8, packed lsb [..., D/2] u8, scale [...] f32."""
    q, s = quantize_rows(x)
    msb, lsb = split_planes(q)
    return pack_nibbles(msb), pack_nibbles(lsb), s


def dequant(msb_p, lsb_p, scale, full: bool):
    """Value of the stored cache: scale*16*msb (MSBs only, LSBs taken as
    zero) or scale*(16*msb + lsb) (both planes)."""
    m = unpack_nibbles(msb_p, signed=True).astype(np.float64)
    v = 16.0 * m
    if full:
        v = v + unpack_nibbles(lsb_p, signed=False).astype(np.float64)
    return v * np.asarray(scale, dtype=np.float64)[..., None]


def pq_head_attention(q, Kmsb, Kfull, Vmsb, Vfull, threshold: float,
                      decide: Optional[Callable] = None, v_threshold: float = 0.0):
    """One decode query row of one head under progressive quantization.

    First pass scores against the MSB-only keys. If the largest probability
    is below the threshold the distribution is flat: the row is recomputed
    with both planes for K and V. Returns (o, p, recomputed, max_p_msb).
    decide(c, default) may override the decision (tests use it to follow
    the GPU among rows whose confidence is at the threshold). v_threshold
    > 0 applies local value pruning to the probabilities that produce o
    (the recomputed ones for a flat row) and the V values of the same pass.
    """
    dh = q.shape[0]
    p = softmax_rows((Kmsb @ q) / math.sqrt(dh))
    c = float(np.max(p))
    flat = c < threshold
    if decide is not None:
        flat = decide(c, flat)
    if flat:
        p = softmax_rows((Kfull @ q) / math.sqrt(dh))
        return value_pruned_output(p, Vfull, v_threshold)[0], p, True, c
    return value_pruned_output(p, Vmsb, v_threshold)[0], p, False, c


# --------------------------------------------------------------------------
# whole stacks
# --------------------------------------------------------------------------


def run_prefill(cfg, inputs: dict, seqs=None,
                adopt: Optional[Callable] = None) -> dict:
    """Cascade over cfg.n_layers layers for each sequence in `seqs`.

    Start: all tokens and heads kept, token importance a = 0, head
    importance g = 0. After layer l (l < L) the next layer keeps
    topk(a, n_{l+1}) tokens, with x, a and the original positions compacted
    to them; when the head count drops, kept heads become
    heads[topk(g[heads], h_{l+1})].

    adopt(kind, b, l, oracle_idx, scores) may return another valid selection
    (used by tests to follow the GPU's choice among near-ties).
    """
    bf16 = cfg.dtype == "bf16"
    B = cfg.batch
    seqs = range(B) if seqs is None else seqs
    D, dh = cfg.model_dim, cfg.head_dim
    out = {}
    for b in seqs:
        x = np.asarray(inputs["x"][b], dtype=np.float64)
        pos = np.arange(cfg.tokens[0], dtype=np.int32)
        heads = np.arange(cfg.n_heads, dtype=np.int32)
        a = np.zeros(cfg.tokens[0])
        g = np.zeros(cfg.n_heads)
        trace = []
        for l in range(cfg.n_layers):
            assert x.shape[0] == cfg.tokens[l] and len(heads) == cfg.heads[l]
            x, dcol, dg, lse = prefill_layer(x, inputs["layers"][l], heads, dh, cfg.causal, bf16,
                                             v_threshold=getattr(cfg, "v_threshold", 0.0))
            a = a + dcol
            for h, v in dg.items():
                g[h] += v
            rec = {"pos": pos.copy(), "heads": heads.copy(), "a": a.copy(), "g": g.copy(),
                   "x": x.copy()}
            if l + 1 < cfg.n_layers:
                if cfg.heads[l + 1] != len(heads):
                    gk = g[heads].astype(np.float32)
                    sel = topk(gk, cfg.heads[l + 1])
                    if adopt is not None:
                        sel = adopt("head", b, l, sel, gk)
                    heads = heads[sel]
                a32 = a.astype(np.float32)
                idx = topk(a32, cfg.tokens[l + 1])
                if adopt is not None:
                    idx = adopt("token", b, l, idx, a32)
                rec["sel"] = idx
                x, a, pos = compact(x, idx), compact(a, idx), compact(pos, idx)
            trace.append(rec)
        out[b] = {"x": x, "pos": pos, "heads": heads, "a": a, "g": g, "trace": trace}
    return out


def perhead_prefill_layer(x, w: dict, heads, keys: dict, head_dim: int, bf16: bool,
                          extras: Optional[dict] = None):
    """One attention-only residual layer with per-head token pruning
    (section "A. Neural Networks Pruning and Quantization", bullet "Token
    Pruning": each head keeps its own tokens). Reading: head h attends over
    its own kept tokens keys[h] (ascending token indices) as keys and
    values; every token still queries every head, so O_h has a row for
    every token and x keeps all rows. Bidirectional.

    Returns (x_new [n, D], {h: column sums of P_h over its keys [len(keys[h])]},
    {h: sum |O_h|}). extras, if given, receives each head's stored Q, K, V
    (all tokens) and O."""
    x = np.asarray(x, dtype=np.float64)
    n, D = x.shape
    dh = head_dim
    delta = np.zeros((n, D))
    cols, dg = {}, {}
    for h in heads:
        c = slice(h * dh, (h + 1) * dh)
        Q = _store(x @ w["wq"][:, c].astype(np.float64), bf16)
        K = _store(x @ w["wk"][:, c].astype(np.float64), bf16)
        V = _store(x @ w["wv"][:, c].astype(np.float64), bf16)
        kk = np.asarray(keys[h], dtype=np.int64)
        S = (Q @ K[kk].T) / math.sqrt(dh)
        P = softmax_rows(S)
        O = P @ V[kk]
        if extras is not None:
            extras[h] = {"q": Q, "k": K, "v": V, "o": _store(O, bf16), "p": P}
        cols[h] = P.sum(axis=0)
        dg[h] = float(np.abs(O).sum())
        delta += _store(O, bf16) @ w["wo"][c, :].astype(np.float64)
    return _store(x + delta, bf16), cols, dg


def run_prefill_perhead(cfg, inputs: dict, seqs=None,
                        adopt: Optional[Callable] = None) -> dict:
    """Per-head token pruning over a prefill stack (bidirectional). Every
    token keeps its row of x; head h keeps its own key/value tokens: all
    of them at layer 1, then after layer l the top cfg.key_keep[l+1] of its
    own cumulative importance a_h among the tokens it kept so far (a token
    a head dropped stays dropped for that head). a_h[j] accumulates the
    probability mass head h gives token j. When the head count drops, kept
    heads are re-ranked by cumulative head importance as in run_prefill.

    adopt(kind, b, l, idx, scores) may return another valid selection.
    Returns per sequence the final x, heads, {h: keys} and {h: a_h} and a
    per-layer trace."""
    bf16 = cfg.dtype == "bf16"
    seqs = range(cfg.batch) if seqs is None else seqs
    n, dh, H = cfg.tokens[0], cfg.head_dim, cfg.n_heads
    out = {}
    for b in seqs:
        x = np.asarray(inputs["x"][b], dtype=np.float64)
        heads = np.arange(H, dtype=np.int32)
        keys = {h: np.arange(n, dtype=np.int64) for h in range(H)}
        a = {h: np.zeros(n) for h in range(H)}
        g = np.zeros(H)
        trace = []
        for l in range(cfg.n_layers):
            assert len(heads) == cfg.heads[l]
            assert all(len(keys[h]) == cfg.key_keep[l] for h in heads)
            x, cols, dg = perhead_prefill_layer(x, inputs["layers"][l], heads, keys, dh, bf16)
            for h in heads:
                a[h][keys[h]] += cols[h]
                g[h] += dg[h]
            rec = {"heads": heads.copy(), "keys": {h: keys[h].copy() for h in heads},
                   "a": {h: a[h].copy() for h in heads}, "g": g.copy(), "x": x.copy()}
            if l + 1 < cfg.n_layers:
                if cfg.heads[l + 1] != len(heads):
                    gk = g[heads].astype(np.float32)
                    sel = topk(gk, cfg.heads[l + 1])
                    if adopt is not None:
                        sel = adopt("head", b, l, sel, gk)
                    heads = heads[sel]
                m = cfg.key_keep[l + 1]
                for h in heads:
                    sc = a[h][keys[h]].astype(np.float32)
                    sel = topk(sc, m)
                    if adopt is not None:
                        sel = adopt("key", b, (l, int(h)), sel, sc)
                    keys[h] = keys[h][sel]
            trace.append(rec)
        out[b] = {"x": x, "heads": heads, "keys": keys, "a": a, "g": g, "trace": trace}
    return out


def value_pruned_output(p, V, tau: float):
    """Local value pruning ("A. Cascade Token Pruning", bullet "Local Value Pruning"): once the
    softmax has produced a head's probabilities p [Lc], the V rows whose
    probability is below tau are dropped for this head only, so
    o = sum over j with p_j >= tau of p_j V_j. The kept probabilities are
    not renormalised (the softmax already normalised them) and the token
    importance still takes every p_j. tau = 0 keeps every row. Returns
    (o [dh], number of V rows kept)."""
    keep = np.asarray(p) >= tau
    return np.asarray(p)[keep] @ np.asarray(V, dtype=np.float64)[keep], int(keep.sum())


def decode_attention(q, cache: dict, heads_n: int, head_dim: int, quantized: bool,
                     threshold: float, decide: Optional[Callable] = None,
                     v_threshold: float = 0.0):
    """Attention of one decode query q [H, dh] over every entry of a cache
    (no mask). Unquantized caches hold k, v [Lc, H, dh]; quantized ones the
    packed planes and scales of K and V rows: planes [Lc, D/2] with scales
    [Lc] (one scale per token, shared by the heads), or under per-head
    pruning planes [Lc, H, dh/2] with scales [Lc, H] (slot r of head h holds
    head h's r-th kept entry and that token's scale). v_threshold > 0 applies local
    value pruning (quantized caches: to the probabilities and V values of the
    pass that produces o, the recomputed one for a flat row). Returns (o [H, dh], p [H, Lc],
    recompute flags [H], MSB-pass max probability [H], V rows kept [H])."""
    H, dh = heads_n, head_dim
    if quantized:

        def planes(kv, full):
            m, l_, sc = cache[kv + "_msb"], cache[kv + "_lsb"], np.asarray(cache[kv + "_scale"])
            if sc.ndim == 2:  # per-head slots: each head's planes carry their own scale
                m = np.asarray(m).reshape(sc.shape[0], H, dh // 2)
                l_ = np.asarray(l_).reshape(sc.shape[0], H, dh // 2)
            return dequant(m, l_, sc, full).reshape(-1, H, dh)
        Km, Kf, Vm, Vf = planes("k", False), planes("k", True), planes("v", False), planes("v", True)
        Lc = Km.shape[0]
    else:
        Lc = cache["k"].shape[0]
    O = np.zeros((H, dh))
    P = np.zeros((H, Lc))
    rec = np.zeros(H, dtype=bool)
    cmax = np.zeros(H)
    kept = np.full(H, Lc, dtype=np.int64)
    for h in range(H):
        if quantized:
            dec = None if decide is None else (lambda c_, d_, h_=h: decide(h_, c_, d_))
            O[h], P[h], rec[h], cmax[h] = pq_head_attention(q[h], Km[:, h], Kf[:, h], Vm[:, h],
                                                            Vf[:, h], threshold, dec, v_threshold)
            kept[h] = int(np.sum(P[h] >= v_threshold))
        else:
            P[h] = softmax_rows((cache["k"][:, h] @ q[h]) / math.sqrt(dh))
            O[h], kept[h] = value_pruned_output(P[h], cache["v"][:, h], v_threshold)
    return O, P, rec, cmax, kept


def decode_layer(x, w: dict, cache: dict, heads_n: int, head_dim: int, bf16: bool,
                 quantized: bool, threshold: float, decide: Optional[Callable] = None,
                 v_threshold: float = 0.0):
    """One decode layer for one sequence. The new token's k and v are
    appended to the cache, then the query attends over every cache entry
    (no mask). Returns (x_new, p [H, Lc], recompute flags [H], MSB-pass max
    probability [H], V rows kept [H]). decide(h, c, default) may override a
    PQ decision."""
    H, dh = heads_n, head_dim
    x = np.asarray(x, dtype=np.float64)
    q = _store(x @ w["wq"].astype(np.float64), bf16).reshape(H, dh)
    k = _store(x @ w["wk"].astype(np.float64), bf16)
    v = _store(x @ w["wv"].astype(np.float64), bf16)
    if quantized:
        km, kl, ks = quantize_kv(k.astype(np.float32))
        vm, vl, vs = quantize_kv(v.astype(np.float32))
        for name, val in (("k_msb", km), ("k_lsb", kl), ("k_scale", ks),
                          ("v_msb", vm), ("v_lsb", vl), ("v_scale", vs)):
            # per-head slots: the row's planes split by head, its scale
            # copied to every head
            row = np.broadcast_to(val, cache[name].shape[1:]) if name.endswith("scale") \
                else np.asarray(val).reshape(cache[name].shape[1:])
            cache[name] = np.concatenate([cache[name], row[None]], axis=0)
    else:
        cache["k"] = np.concatenate([cache["k"], k.reshape(1, H, dh)], axis=0)
        cache["v"] = np.concatenate([cache["v"], v.reshape(1, H, dh)], axis=0)
    O, P, rec, cmax, kept = decode_attention(q, cache, H, dh, quantized, threshold, decide,
                                             v_threshold)
    delta = np.zeros(x.shape[0])
    for h in range(H):
        delta += _store(O[h], bf16) @ w["wo"][h * dh:(h + 1) * dh, :].astype(np.float64)
    return _store(x + delta, bf16), P, rec, cmax, kept


def prune_after_step(cfg, s: int) -> bool:
    """Whether the cache is pruned after 0-based step s: always after the
    first step; with prune_every = r > 0 again after every r-th later step
    (r = 1 re-prunes after every step, a rolling keep budget)."""
    r = getattr(cfg, "prune_every", 0)
    return s == 0 or (r > 0 and s % r == 0)


def run_decode(cfg, inputs: dict, seqs=None, adopt: Optional[Callable] = None,
               steps: Optional[int] = None, pq_adopt: Optional[Callable] = None) -> dict:
    """Generation (page: section II, attention-based NLP models): one new
    token per step against cached K/V. Token importance a accumulates the
    probabilities each cache entry receives, over heads, layers and steps;
    a new entry starts at 0. After every layer of step 1 has run, the cache
    of every layer keeps topk(a over L0+1 entries, cache_keep) entries
    (section II "Cascade pruning": a pruned token stays pruned); with
    cfg.prune_every = r > 0 the same cut back to cache_keep entries is
    repeated after every r-th later step, over the entries kept so far plus
    the new ones. cfg.v_threshold > 0 adds local value pruning inside each
    head's attention. With cfg.per_head (per-head token pruning, page
    section "A. Neural Networks Pruning and Quantization", bullet "Token Pruning" names it) each head h keeps its own entries:
    a_h[j] accumulates only head h's probabilities and every cut keeps
    topk(a_h, cache_keep) for that head in every layer's K and V. All heads
    keep the same count, so slot r of head h holds head h's r-th entry; a
    quantized cache then holds its token scales per head as well (each head
    keeps a copy of the scale of every token it keeps; the scale itself is
    still the token's, taken over the whole row).
    pq_adopt(b, s, l, h, c, default) may override a recompute decision.

    Per sequence the result holds the step outputs, the final a, the first
    selection (indices into the L0+1 entries), "kept_ids" after every step
    (original entry ids, prior tokens 0..L0-1 and step s's token L0+s, in
    cache order), "before_prune" (ids and a after each step, before its
    cut), the recompute records and the V rows kept [step, layer, head]."""
    bf16 = cfg.dtype == "bf16"
    seqs = range(cfg.batch) if seqs is None else seqs
    steps = cfg.steps if steps is None else steps
    H, dh = cfg.n_heads, cfg.head_dim
    vthr = getattr(cfg, "v_threshold", 0.0)
    per_head = getattr(cfg, "per_head", False)
    out = {}
    for b in seqs:
        caches = []
        for l in range(cfg.n_layers):
            Lw = inputs["layers"][l]
            K0 = np.asarray(Lw["k_cache"][b], dtype=np.float64)
            V0 = np.asarray(Lw["v_cache"][b], dtype=np.float64)
            if cfg.quantized:
                km, kl, ks = quantize_kv(K0.reshape(K0.shape[0], -1).astype(np.float32))
                vm, vl, vs = quantize_kv(V0.reshape(V0.shape[0], -1).astype(np.float32))
                c = {"k_msb": km, "k_lsb": kl, "k_scale": ks,
                     "v_msb": vm, "v_lsb": vl, "v_scale": vs}
                if per_head:
                    # per-head slots: planes [L0, H, dh/2], the token's
                    # scale copied to every head [L0, H]
                    L0 = K0.shape[0]
                    c = {k_: (np.repeat(np.asarray(v_)[:, None], H, axis=1)
                              if k_.endswith("scale") else
                              np.asarray(v_).reshape(L0, H, dh // 2)) for k_, v_ in c.items()}
                caches.append(c)
            else:
                caches.append({"k": K0, "v": V0})
        shape = (H, cfg.cache_len) if per_head else (cfg.cache_len,)
        a = np.zeros(shape)
        ids = np.broadcast_to(np.arange(cfg.cache_len, dtype=np.int64), shape).copy()
        xs, recs, kept, sel, kept_ids, pre = [], [], [], None, [], []
        for s in range(steps):
            x = np.asarray(inputs["x_steps"][s][b], dtype=np.float64)
            a = np.concatenate([a, np.zeros(shape[:-1] + (1,))], axis=-1)
            ids = np.concatenate([ids, np.full(shape[:-1] + (1,), cfg.cache_len + s)], axis=-1)
            step_rec, step_kept = [], []
            for l in range(cfg.n_layers):
                dec = None
                if pq_adopt is not None:
                    dec = (lambda h_, c_, d_, b_=b, s_=s, l_=l: pq_adopt(b_, s_, l_, h_, c_, d_))
                x, P, rec, cmax, kv = decode_layer(x, inputs["layers"][l], caches[l], H, dh,
                                                   bf16, cfg.quantized, cfg.pq_threshold, dec,
                                                   vthr)
                a = a + (P if per_head else P.sum(axis=0))
                step_rec.append((rec, cmax))
                step_kept.append(kv)
            xs.append(x)
            recs.append(step_rec)
            kept.append(step_kept)
            pre.append((ids.copy(), a.copy()))
            if prune_after_step(cfg, s) and a.shape[-1] > cfg.cache_keep:
                if per_head:
                    idx = np.stack([topk(a[h].astype(np.float32), cfg.cache_keep)
                                    for h in range(H)])
                    if adopt is not None:
                        idx = np.stack([adopt("cache_head", b, s, idx[h], a[h].astype(np.float32))
                                        for h in range(H)])
                    for c in caches:
                        for name in c:
                            c[name] = np.stack([c[name][idx[h], h] for h in range(H)], axis=1)
                    a = np.stack([a[h][idx[h]] for h in range(H)])
                    ids = np.stack([ids[h][idx[h]] for h in range(H)])
                else:
                    a32 = a.astype(np.float32)
                    idx = topk(a32, cfg.cache_keep)
                    if adopt is not None:
                        idx = adopt("cache", b, s, idx, a32)
                    for c in caches:
                        for name in c:
                            c[name] = compact(c[name], idx)
                    a, ids = compact(a, idx), compact(ids, idx)
                if s == 0:
                    sel = idx
            kept_ids.append(ids.copy())
        out[b] = {"x_steps": np.stack(xs), "a": a, "sel": sel, "recompute": recs,
                  "kept_ids": kept_ids, "before_prune": pre, "v_kept": np.array(kept)}
    return out
