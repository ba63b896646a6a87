"""Seeded synthetic inputs shared by the oracle and the GPU path.

Only random draws and storage-format casts live here; none of the method's
arithmetic does. Draw order from one numpy PCG64 generator:

  prefill: x [B, T, D] ~ N(0, 1); then for each sequence round(0.05*T) rows,
           drawn without replacement, are scaled by 3; then for each layer
           Wq, Wk, Wv, Wo, each [D, D] ~ N(0, 1/D) (x @ W layout: column block
           h*dh:(h+1)*dh of Wq/Wk/Wv and the same row block of Wo belong to
           head h).
  decode:  for each layer: Wq, Wk, Wv, Wo; then cached K [B, L0, H, dh] and
           V [B, L0, H, dh] ~ N(0, 1); then for each sequence round(0.05*L0)
           token indices, drawn without replacement, whose K and V rows (all
           heads) are scaled by 3. After all layers: one x row [B, D] ~ N(0, 1)
           per decode step.

Values are drawn in fp64 and cast to fp32; for bf16 workloads the fp32 value
is then rounded to bf16 (round to nearest even) and returned as an fp32 array
holding exactly that bf16 value.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import AdaConfig, Config


def _cast(a64: np.ndarray, dtype: str) -> np.ndarray:
    a32 = a64.astype(np.float32)
    if dtype == "f32":
        return a32
    t = torch.from_numpy(a32).to(torch.bfloat16).to(torch.float32)
    return t.numpy()


def _heavy_count(n: int, frac: float) -> int:
    return int(np.floor(frac * n + 0.5))


def _weights(rng: np.random.Generator, D: int, dtype: str) -> dict:
    out = {}
    for name in ("wq", "wk", "wv", "wo"):
        out[name] = _cast(rng.standard_normal((D, D)) / np.sqrt(D), dtype)
    return out


def make_prefill_inputs(cfg: Config, seed: int = 0) -> dict:
    """x [B, T, D] and per-layer weights, as fp32 arrays."""
    assert cfg.kind == "prefill"
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, D = cfg.batch, cfg.tokens[0], cfg.model_dim
    x = rng.standard_normal((B, T, D))
    nh = _heavy_count(T, cfg.heavy_frac)
    heavy = []
    for b in range(B):
        rows = rng.choice(T, size=nh, replace=False)
        x[b, rows, :] *= cfg.heavy_scale
        heavy.append(np.sort(rows))
    layers = [_weights(rng, D, cfg.dtype) for _ in range(cfg.n_layers)]
    return {"x": _cast(x, cfg.dtype), "layers": layers, "heavy": heavy}


def make_decode_inputs(cfg: Config, seed: int = 0) -> dict:
    """Per-layer weights and initial caches, then one x row per step."""
    assert cfg.kind == "decode"
    rng = np.random.Generator(np.random.PCG64(seed))
    B, L0, H, dh, D = cfg.batch, cfg.cache_len, cfg.n_heads, cfg.head_dim, cfg.model_dim
    nh = _heavy_count(L0, cfg.heavy_frac)
    layers = []
    for _ in range(cfg.n_layers):
        w = _weights(rng, D, cfg.dtype)
        K = rng.standard_normal((B, L0, H, dh))
        V = rng.standard_normal((B, L0, H, dh))
        for b in range(B):
            rows = rng.choice(L0, size=nh, replace=False)
            K[b, rows] *= cfg.heavy_scale
            V[b, rows] *= cfg.heavy_scale
        w["k_cache"] = _cast(K, cfg.dtype)
        w["v_cache"] = _cast(V, cfg.dtype)
        del K, V
        layers.append(w)
    xs = np.stack([_cast(rng.standard_normal((B, D)), cfg.dtype) for _ in range(cfg.steps)])
    return {"layers": layers, "x_steps": xs}


def make_inputs(cfg: Config, seed: int = 0) -> dict:
    if cfg.kind == "prefill":
        return make_prefill_inputs(cfg, seed)
    return make_decode_inputs(cfg, seed)


def random_scores(shape, seed: int = 0, kind: str = "normal") -> np.ndarray:
    """fp32 score arrays for top-k tests: 'normal', 'ties' (few distinct
    values), 'signed_zero' (mix of +0.0, -0.0 and small values)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "normal":
        return rng.standard_normal(shape).astype(np.float32)
    if kind == "ties":
        return rng.integers(0, 4, size=shape).astype(np.float32)
    if kind == "signed_zero":
        choice = rng.integers(0, 4, size=shape)
        vals = np.array([0.0, -0.0, 1e-40, -1e-40], dtype=np.float32)
        return vals[choice]
    if kind == "uniform":
        return rng.random(shape).astype(np.float32)
    raise ValueError(kind)


def ada_layers(cfg: AdaConfig, seq: int, seed: int = 0):
    """Per-layer activations [T, d] (float32) of sequence `seq`, one layer
    at a time: layer 0 = cluster centre + spread noise, layer l = layer l-1
    + drift noise. Each sequence has its own generator (PCG64 seeded with
    (seed, seq)), so sequences can be generated independently."""
    rng = np.random.Generator(np.random.PCG64([seed, seq]))
    T, d = cfg.seq_len, cfg.dim
    K = max(1, int(np.floor(cfg.clusters_frac * T + 0.5)))
    centres = rng.standard_normal((K, d))
    x = centres[rng.integers(0, K, T)] + cfg.spread * rng.standard_normal((T, d))
    del centres
    for l in range(cfg.n_layers):
        if l > 0:
            x += cfg.drift * rng.standard_normal((T, d))
        yield x.astype(np.float32)


def ada_batch_layers(cfg: AdaConfig, seed: int = 0):
    """Per-layer activations [B, T, d] (float32) of every sequence."""
    gens = [ada_layers(cfg, b, seed) for b in range(cfg.batch)]
    for _ in range(cfg.n_layers):
        yield np.stack([next(g) for g in gens])
