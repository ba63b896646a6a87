"""Workload definitions for cascade token/head pruned attention.

Five workloads are defined, each a stack of attention-only residual layers
(x += softmax(Q K^T / sqrt(dh)) V Wo, no FFN, no LayerNorm):

  tiny        2 layers, B=1, T=64, H=4, dh=32, D=128, fp32; layer 2 keeps the
              top-32 tokens by layer-1 cumulative importance.
  bert_base   12 layers, B=32, T=512, H=12, dh=64, D=768, bf16 storage,
              bidirectional; token keep fraction falls linearly from 1.0 at
              layer 1 to 0.5 at layer 12; heads cut to the top-10 of 12 from
              layer 4 by |O_h| importance.
  gpt2_decode 12 layers, H=12, dh=64, B=64, 1024 cached tokens, 32 decode
              steps; the cache is pruned to 40% of its length after step 1.
  pq_decode   24 layers, H=16, dh=64, B=16, 2048 cached tokens, K/V stored as
              4-bit MSB and LSB planes of a per-token int8 code; MSB-only
              scoring first, recompute with LSBs for rows whose max
              probability is below 0.1; cache keep 50%.
  long_causal 4 layers, B=1, T=32768, H=32, dh=128, D=4096, bf16, causal;
              25% of tokens kept after layer 1, heads top-24 of 32 from
              layer 2.

Three extensions of gpt2_decode: gpt2_decode_vprune (local value pruning,
threshold 1e-4), gpt2_decode_rolling (the cache cut back to 410 entries
after every step) and gpt2_decode_perhead (each head keeps its own 410
entries by its own importance); pq_decode_perhead does the same for the
quantized cache (1024 entries per head) and pq_decode_vprune adds value
pruning at 1e-4 to it.

This module holds shapes and schedules only. Keep counts follow
k = floor(f * N + 1/2) with N the original length, so fractions are absolute
along the cascade.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from fractions import Fraction
from typing import List, Optional


def keep_count(frac: Fraction, n: int) -> int:
    """floor(frac * n + 1/2), exact."""
    v = Fraction(frac) * n + Fraction(1, 2)
    return v.numerator // v.denominator


@dataclass(frozen=True)
class Config:
    name: str
    kind: str                 # "prefill" or "decode"
    n_layers: int
    batch: int
    n_heads: int
    head_dim: int
    dtype: str                # "f32" or "bf16" (storage type; accumulation is fp32 on the GPU)
    causal: bool = False
    # prefill: tokens and heads processed by each layer
    tokens: tuple = ()
    heads: tuple = ()
    # decode
    cache_len: int = 0        # prior tokens in the cache (L0)
    cache_keep: int = 0       # entries kept after step 1
    steps: int = 0
    quantized: bool = False
    pq_threshold: float = 0.0
    # local value pruning: V rows with probability below this are dropped
    # for the current head (0 = off)
    v_threshold: float = 0.0
    # re-prune the cache back to cache_keep after every prune_every-th step
    # following the first (0 = prune once, after step 1)
    prune_every: int = 0
    # per-head token pruning: each head keeps its own cache entries by its
    # own cumulative importance (unquantized decode)
    per_head: bool = False
    # prefill per-head token pruning: keys (and values) each head keeps per
    # layer (empty: no per-head pruning); every token keeps its row of x
    key_keep: tuple = ()
    heavy_frac: float = 0.05
    heavy_scale: float = 3.0

    @property
    def model_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def seq_len(self) -> int:
        return self.tokens[0] if self.kind == "prefill" else self.cache_len

    @property
    def cache_cap(self) -> int:
        """Cache rows needed per sequence: L0 prior entries + one per step."""
        return self.cache_len + self.steps

    def token_layers(self) -> int:
        """Tokens processed summed over layers (and steps for decode)."""
        # (per-head pruning keeps every token's row: tokens stays n per layer)
        if self.kind == "prefill":
            return self.batch * sum(self.tokens)
        return self.batch * self.n_layers * self.steps


def _linear_schedule(T: int, L: int, last_frac: Fraction) -> tuple:
    # f_l = 1 - (1 - last_frac) * (l - 1) / (L - 1), l = 1..L
    out = []
    for l in range(1, L + 1):
        f = 1 - (1 - last_frac) * Fraction(l - 1, L - 1)
        out.append(keep_count(f, T))
    return tuple(out)


TINY = Config(
    name="tiny", kind="prefill", n_layers=2, batch=1, n_heads=4, head_dim=32,
    dtype="f32", causal=False, tokens=(64, 32), heads=(4, 4))

BERT_BASE = Config(
    name="bert_base", kind="prefill", n_layers=12, batch=32, n_heads=12, head_dim=64,
    dtype="bf16", causal=False,
    tokens=_linear_schedule(512, 12, Fraction(1, 2)),
    heads=(12, 12, 12) + (10,) * 9)

GPT2_DECODE = Config(
    name="gpt2_decode", kind="decode", n_layers=12, batch=64, n_heads=12, head_dim=64,
    dtype="bf16", cache_len=1024, cache_keep=keep_count(Fraction(2, 5), 1024), steps=32)

PQ_DECODE = Config(
    name="pq_decode", kind="decode", n_layers=24, batch=16, n_heads=16, head_dim=64,
    dtype="bf16", cache_len=2048, cache_keep=keep_count(Fraction(1, 2), 2048), steps=32,
    quantized=True, pq_threshold=0.1)

LONG_CAUSAL = Config(
    name="long_causal", kind="prefill", n_layers=4, batch=1, n_heads=32, head_dim=128,
    dtype="bf16", causal=True,
    tokens=(32768,) + (keep_count(Fraction(1, 4), 32768),) * 3,
    heads=(32,) + (24,) * 3)

# Extensions of the GPT-2-small decode workload: local value pruning with a
# probability threshold of 1e-4, a rolling cascade that cuts the cache back
# to 410 entries after every step, and per-head cache pruning.
GPT2_DECODE_VPRUNE = replace(GPT2_DECODE, name="gpt2_decode_vprune", v_threshold=1e-4)
GPT2_DECODE_ROLLING = replace(GPT2_DECODE, name="gpt2_decode_rolling", prune_every=1)
GPT2_DECODE_PERHEAD = replace(GPT2_DECODE, name="gpt2_decode_perhead", per_head=True)
# Per-head cache pruning under progressive quantization: each head keeps its
# own 1024 entries of the pq_decode cache (with a copy of each kept token's
# scales), recomputing flat rows from both planes as pq_decode does.
PQ_DECODE_PERHEAD = replace(PQ_DECODE, name="pq_decode_perhead", per_head=True)
# Local value pruning under progressive quantization, threshold 1e-4 as in
# gpt2_decode_vprune: V rows are read (MSB plane, or both for a recomputed
# row) only where the final probability reaches it.
PQ_DECODE_VPRUNE = replace(PQ_DECODE, name="pq_decode_vprune", v_threshold=1e-4)
# Local value pruning in prefill: the bert_base stack with a probability
# threshold of 1e-3 (about half of a 512-token row's uniform share).
BERT_BASE_VPRUNE = replace(BERT_BASE, name="bert_base_vprune", v_threshold=1e-3)
# Per-head token pruning in prefill: every token keeps its row (512 per
# layer) and each head keeps its own keys and values, falling from 512 to
# 256 like bert_base's token schedule; heads 12 -> 10 from layer 4.
BERT_BASE_PERHEAD = replace(BERT_BASE, name="bert_base_perhead", per_head=True,
                            tokens=(512,) * 12, key_keep=BERT_BASE.tokens)

CONFIGS = [TINY, BERT_BASE, GPT2_DECODE, PQ_DECODE, LONG_CAUSAL]
EXTENSIONS = [GPT2_DECODE_VPRUNE, GPT2_DECODE_ROLLING, GPT2_DECODE_PERHEAD, PQ_DECODE_PERHEAD,
              PQ_DECODE_VPRUNE, BERT_BASE_VPRUNE, BERT_BASE_PERHEAD]
BY_NAME = {c.name: c for c in CONFIGS + EXTENSIONS}


@dataclass(frozen=True)
class AdaConfig:
    """Cascade representative-token selection over a stack of per-layer
    activations (page 5): T tokens of dimension d per sequence and layer,
    threshold tau on the Gram (cosine) product.

    Synthetic activations: a token is a cluster centre (round(clusters_frac
    * T) centres, N(0, I)) plus spread * N(0, I); every later layer adds
    drift * N(0, I) to the previous layer's activations (a residual stream
    whose near-duplicates slowly come apart)."""
    name: str
    batch: int
    seq_len: int
    dim: int
    n_layers: int
    tau: float = 0.30
    clusters_frac: float = 0.25
    spread: float = 0.2
    drift: float = 0.07
    kind: str = "ada"

    def token_layers(self) -> int:
        return self.batch * self.seq_len * self.n_layers


# the page's measured setting (T = 512, tau = 0.30) on GPT-2-small-shaped
# activations (d = 768, 12 layers), and its projected long sequence (T =
# 8192) at d = 4096; a small case for oracle pins and parity tests
ADA_GPT2 = AdaConfig(name="ada_gpt2", batch=16, seq_len=512, dim=768, n_layers=12)
ADA_LONG = AdaConfig(name="ada_long", batch=1, seq_len=8192, dim=4096, n_layers=4)
ADA_SMALL = AdaConfig(name="ada_small", batch=2, seq_len=96, dim=32, n_layers=4)
ADA_CONFIGS = [ADA_GPT2, ADA_LONG]
BY_NAME.update({c.name: c for c in ADA_CONFIGS})


def scaled(cfg: Config, **kw) -> Config:
    """A smaller variant of a workload for parity tests (same structure)."""
    return replace(cfg, **kw)
