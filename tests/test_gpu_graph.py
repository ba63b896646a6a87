"""HIP graph capture of whole passes. The stacks allocate every buffer up
front and their passes only enqueue library kernels (no allocation, memset
or host synchronisation), so one pass captures into a graph. Every replay,
each from a freshly loaded state and with unrelated eager work and
synchronisations between replays, must reproduce the eager pass bit for bit
(the kernels are deterministic)."""
import numpy as np
import pytest
import torch

from cascade_token_head_amd import pipeline
from workloads import BERT_BASE, GPT2_DECODE, LONG_CAUSAL, PQ_DECODE, make_decode_inputs, \
    make_prefill_inputs, scaled

pytestmark = pytest.mark.gpu


def _capture(pass_fn, reset_fn):
    # warm up on a side stream, as graph capture expects
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset_fn()
        pass_fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    reset_fn()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        pass_fn()
    torch.cuda.synchronize()
    return g


def _replays_match(g, reset_fn, outputs, ref):
    for rep in range(3):
        reset_fn()
        junk = torch.randn(4096, device="cuda").cumsum(0)   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outputs(), ref)):
            # bytes, not values: cache rows past the kept range are never
            # written and may hold NaN patterns
            assert torch.equal(o.contiguous().view(torch.uint8), r.contiguous().view(torch.uint8)), (
                "replay", rep, "output", i)
        del junk


PREFILL = {
    "bert_small": scaled(BERT_BASE, batch=4, n_layers=5, tokens=(512, 470, 430, 390, 350),
                         heads=(12, 12, 10, 10, 10)),
    "causal_small": scaled(LONG_CAUSAL, n_heads=8, n_layers=3, tokens=(2048, 1024, 1024),
                           heads=(8, 6, 6)),
}


@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_stack_graph_replays_match_eager(name):
    cfg = PREFILL[name]
    print("graph prefill", name, flush=True)
    dt = torch.bfloat16
    inputs = make_prefill_inputs(cfg)
    w = pipeline.weights_to_device(inputs["layers"], dt)
    st = pipeline.PrefillStack(cfg.n_layers, cfg.batch, cfg.n_heads, cfg.head_dim, cfg.tokens,
                               cfg.heads, dt, cfg.causal, w)
    x0 = torch.from_numpy(inputs["x"]).to(dt).cuda()
    st.load(x0)
    st.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in st.final] + [st.g.clone()]
    g = _capture(st.run, lambda: st.load(x0))
    _replays_match(g, lambda: st.load(x0), lambda: list(st.final) + [st.g], ref)


DECODE = {
    "gpt2_small": scaled(GPT2_DECODE, batch=4, n_layers=4, cache_len=256, cache_keep=102,
                         steps=4),
    "pq_small": scaled(PQ_DECODE, batch=3, n_layers=3, cache_len=300, cache_keep=150, steps=3),
    "perhead_rolling_vprune": scaled(GPT2_DECODE, batch=3, n_layers=3, cache_len=200,
                                     cache_keep=80, steps=5, prune_every=1, per_head=True,
                                     v_threshold=1e-3),
    # the configurations bench.py times as graph replays, at full size
    "gpt2_decode": GPT2_DECODE,
    "pq_decode": PQ_DECODE,
}


@pytest.mark.parametrize("name", list(DECODE))
def test_decode_pass_graph_replays_match_eager(name):
    cfg = DECODE[name]
    print("graph decode", name, flush=True)
    dt = torch.bfloat16
    inputs = make_decode_inputs(cfg)
    w = pipeline.weights_to_device(inputs["layers"], dt)
    st = pipeline.DecodeStack(cfg.n_layers, cfg.batch, cfg.n_heads, cfg.head_dim, cfg.cache_len,
                              cfg.cache_keep, cfg.steps, w, cfg.quantized, cfg.pq_threshold, dt,
                              v_threshold=cfg.v_threshold, prune_every=cfg.prune_every,
                              per_head=cfg.per_head)
    k0 = [torch.from_numpy(l["k_cache"]).to(dt).cuda() for l in inputs["layers"]]
    v0 = [torch.from_numpy(l["v_cache"]).to(dt).cuda() for l in inputs["layers"]]
    xs = torch.from_numpy(inputs["x_steps"]).to(dt).cuda()
    outs = torch.empty(cfg.steps, cfg.batch, cfg.model_dim, dtype=dt, device="cuda")

    def pass_():
        for s in range(cfg.steps):
            outs[s].copy_(st.step(xs[s]))

    def reset():
        st.load(k0, v0)

    end = {}

    def outputs():
        # the buffers the pass ends in (a replay does not advance the
        # stack's host-side state, which reset() returns to the start)
        c = st.caches[end["side"]][0]
        return [outs, st.abuf[end["side"]]] + [c[k] for k in sorted(c)]

    reset()
    pass_()
    torch.cuda.synchronize()
    end["side"] = st.side
    ref = [t.clone() for t in outputs()]
    assert np.isfinite(outs.float().cpu().numpy()).all()
    g = _capture(pass_, reset)
    _replays_match(g, reset, outputs, ref)


def test_perhead_prefill_graph_replays_match_eager():
    """Per-head token pruning in prefill: the head cut, each slot's key cut
    and the layer calls of a whole pass replay from one graph."""
    from workloads.configs import BERT_BASE_PERHEAD
    cfg = scaled(BERT_BASE_PERHEAD, batch=3, n_layers=4, n_heads=6, tokens=(300,) * 4,
                 heads=(6, 6, 4, 4), key_keep=(300, 200, 120, 120))
    print("graph per-head prefill", flush=True)
    inputs = make_prefill_inputs(cfg)
    w = pipeline.weights_to_device(inputs["layers"], torch.bfloat16)
    st = pipeline.PerHeadPrefillStack(cfg.n_layers, cfg.batch, cfg.n_heads, cfg.head_dim,
                                      cfg.tokens[0], cfg.heads, cfg.key_keep, w)
    x0 = torch.from_numpy(inputs["x"]).to(torch.bfloat16).cuda()
    st.load(x0)
    st.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in st.final] + [st.g.clone()]
    g = _capture(st.run, lambda: st.load(x0))
    _replays_match(g, lambda: st.load(x0), lambda: list(st.final) + [st.g], ref)


def test_selection_stack_graph_replays_match_eager():
    """Page-5 representative selection over a stack of layers (full Gram
    product at layer 1, cascade steps after) replays from one graph."""
    from workloads import ada_batch_layers
    from workloads.configs import ADA_SMALL
    cfg = scaled(ADA_SMALL, batch=3, seq_len=300, dim=64, n_layers=4)
    print("graph selection", flush=True)
    layers = [torch.from_numpy(x).cuda() for x in ada_batch_layers(cfg)]
    st = pipeline.AdaStack(cfg.n_layers, cfg.batch, cfg.seq_len, cfg.dim, cfg.tau)

    def reset():
        st.flags.zero_()
        st.counts.zero_()

    def pass_():
        st.run(layers)

    reset()
    pass_()
    torch.cuda.synchronize()
    ref = [st.flags.clone(), st.maxcos.clone(), st.counts.clone()]
    assert 0 < int(ref[2][:, :, 0].min()) < cfg.seq_len
    g = _capture(pass_, reset)
    _replays_match(g, reset, lambda: [st.flags, st.maxcos, st.counts], ref)
