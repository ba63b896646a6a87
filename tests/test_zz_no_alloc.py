"""The allocation-free layer entry point (fixed per-device scratch) against
spatten_layer_forward with a caller workspace: identical kernels on
identical inputs, so every output must match bit for bit. Two calls in a
row per mode, the second with a smaller input, so the second runs in
scratch that still holds the first call's data."""
import numpy as np
import pytest
import torch

from cascade_token_head_amd import pipeline
from cascade_token_head_amd import spatten as S
from workloads import BERT_BASE, GPT2_DECODE, PQ_DECODE, make_decode_inputs, make_prefill_inputs
from workloads import scaled
from workloads.configs import BERT_BASE_PERHEAD

pytestmark = pytest.mark.gpu


def _prefill_pair(cfg, noalloc):
    inp = make_prefill_inputs(cfg)
    w = pipeline.weights_to_device(inp["layers"][:1], torch.bfloat16)[0]
    B, n, H, dh = cfg.batch, cfg.tokens[0], cfg.n_heads, cfg.head_dim
    x = torch.from_numpy(inp["x"]).to(torch.bfloat16).cuda()
    ashape = (B, H, n) if cfg.per_head else (B, n)
    a = torch.linspace(0, 1, int(np.prod(ashape)), device="cuda").reshape(ashape).contiguous()
    g = torch.ones(B, H, device="cuda")
    hidx = torch.arange(H, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
    lse = torch.empty(B, H, n, device="cuda")
    keys, m = None, 0
    if cfg.per_head:
        m = cfg.key_keep[0]
        rng = np.random.default_rng(n)
        keys = torch.from_numpy(np.stack([np.sort(rng.choice(n, m, replace=False))
                                          for _ in range(B * H)]).astype(np.int32))
        keys = keys.reshape(B, H, m).cuda()
    desc = S.make_desc(S.PREFILL, S.BF16, cfg.causal, B, n, H, H, dh,
                       v_threshold=cfg.v_threshold, per_head=cfg.per_head, n_keys=m)
    if noalloc:
        S.layer_forward_noalloc(desc, x, w["wq"], w["wk"], w["wv"], w["wo"], hidx, a, g, lse=lse,
                                head_keys=keys)
    else:
        ws = torch.empty(S.workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        S.layer_forward(desc, x, w["wq"], w["wk"], w["wv"], w["wo"], hidx, a, g, ws, lse=lse,
                        head_keys=keys)
    torch.cuda.synchronize()
    return [t.cpu() for t in (x, a, g, lse)]


def _decode_pair(cfg, noalloc):
    inp = make_decode_inputs(cfg)
    dt = torch.bfloat16
    w = pipeline.weights_to_device(inp["layers"][:1], dt)[0]
    B, H, dh, L0 = cfg.batch, cfg.n_heads, cfg.head_dim, cfg.cache_len
    D, cap = H * dh, L0 + 3
    k0 = torch.from_numpy(inp["layers"][0]["k_cache"]).to(dt).cuda().reshape(B, L0, D)
    v0 = torch.from_numpy(inp["layers"][0]["v_cache"]).to(dt).cuda().reshape(B, L0, D)
    x = torch.from_numpy(inp["x_steps"][0]).to(dt).cuda().reshape(B, 1, D).contiguous()
    a = torch.zeros(B, cap, device="cuda")
    a[:, :L0] = torch.linspace(0, 1, L0, device="cuda")
    hidx = torch.arange(H, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
    g = torch.zeros(B, H, device="cuda")
    rec = torch.full((B, H), -1, dtype=torch.int32, device="cuda")
    kept = torch.full((B, H), -1, dtype=torch.int32, device="cuda")
    if cfg.quantized:
        c = {n: torch.zeros(B, H, cap, D // H // 2, dtype=torch.uint8, device="cuda")
             for n in ("k_msb", "k_lsb", "v_msb", "v_lsb")}
        c["k_scale"] = torch.zeros(B, cap, device="cuda")
        c["v_scale"] = torch.zeros(B, cap, device="cuda")
        S.quantize_kv(k0, c["k_msb"], c["k_lsb"], c["k_scale"])
        S.quantize_kv(v0, c["v_msb"], c["v_lsb"], c["v_scale"])
    else:
        c = {"k_cache": torch.zeros(B, cap, D, dtype=dt, device="cuda"),
             "v_cache": torch.zeros(B, cap, D, dtype=dt, device="cuda")}
        c["k_cache"][:, :L0] = k0
        c["v_cache"][:, :L0] = v0
    desc = S.make_desc(S.DECODE, S.BF16, False, B, 1, H, H, dh, L0, cap, cfg.quantized,
                       cfg.pq_threshold, cfg.v_threshold)
    if noalloc:
        S.layer_forward_noalloc(desc, x, w["wq"], w["wk"], w["wv"], w["wo"], hidx, a, g,
                                recompute=rec, v_kept=kept, **c)
    else:
        ws = torch.empty(S.workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        S.layer_forward(desc, x, w["wq"], w["wk"], w["wv"], w["wo"], hidx, a, g, ws,
                        recompute=rec, v_kept=kept, **c)
    torch.cuda.synchronize()
    return [t.cpu() for t in [x, a, rec, kept] + [c[k] for k in sorted(c)]]


def _same(got, want, what):
    for i, (p, q) in enumerate(zip(got, want)):
        assert p.dtype == q.dtype and p.shape == q.shape, (what, i)
        assert torch.equal(p.view(torch.uint8) if p.dtype == torch.bfloat16 else p,
                           q.view(torch.uint8) if q.dtype == torch.bfloat16 else q), (what, i)


CASES = [
    ("prefill", scaled(BERT_BASE, batch=4, n_layers=1, tokens=(300,), heads=(12,)),
     scaled(BERT_BASE, batch=2, n_layers=1, tokens=(77,), heads=(12,))),
    ("prefill_causal", scaled(BERT_BASE, batch=2, n_layers=1, tokens=(500,), heads=(12,),
                              causal=True),
     scaled(BERT_BASE, batch=1, n_layers=1, tokens=(130,), heads=(12,), causal=True)),
    ("prefill_vprune", scaled(BERT_BASE, batch=3, n_layers=1, tokens=(260,), heads=(12,),
                              v_threshold=1e-3),
     scaled(BERT_BASE, batch=2, n_layers=1, tokens=(64,), heads=(12,), v_threshold=1e-3)),
    ("prefill_perhead", scaled(BERT_BASE_PERHEAD, batch=3, n_layers=1, tokens=(300,),
                               heads=(12,), key_keep=(140,)),
     scaled(BERT_BASE_PERHEAD, batch=2, n_layers=1, tokens=(90,), heads=(12,), key_keep=(33,))),
    ("decode", scaled(GPT2_DECODE, batch=8, n_layers=1, cache_len=700, steps=1),
     scaled(GPT2_DECODE, batch=3, n_layers=1, cache_len=90, steps=1)),
    ("decode_pq", scaled(PQ_DECODE, batch=4, n_layers=1, cache_len=900, steps=1),
     scaled(PQ_DECODE, batch=2, n_layers=1, cache_len=200, steps=1)),
    ("decode_vprune", scaled(GPT2_DECODE, batch=4, n_layers=1, cache_len=500, steps=1,
                             v_threshold=1e-3),
     scaled(GPT2_DECODE, batch=2, n_layers=1, cache_len=64, steps=1, v_threshold=1e-3)),
    ("decode_pq_vprune", scaled(PQ_DECODE, batch=4, n_layers=1, cache_len=900, steps=1,
                                v_threshold=1e-3),
     scaled(PQ_DECODE, batch=2, n_layers=1, cache_len=200, steps=1, v_threshold=1e-3)),
]


@pytest.mark.parametrize("name,big,small", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_entry_point(name, big, small):
    print("noalloc", name, flush=True)
    run = _prefill_pair if big.kind == "prefill" else _decode_pair
    for cfg in (big, small):
        want = run(cfg, noalloc=False)
        got = run(cfg, noalloc=True)
        _same(got, want, "%s %s" % (name, cfg.name))


def test_noalloc_rejects_a_layer_beyond_its_scratch():
    big = S.make_desc(S.PREFILL, S.BF16, False, 32, 512, 12, 12, 64)
    x = torch.zeros(1, device="cuda")
    with pytest.raises(S.SpattenError) as e:
        S.layer_forward_noalloc(big, x, x, x, x, x, x, x, x)
    assert e.value.status == S.EWORKSPACE
