#!/usr/bin/env python3
"""Pruned-attention throughput on one MI355X.

A step is one pass of the whole cascade over one batch of synthetic input.
The headline workload is long_causal (4 attention-only layers, batch 1,
T = 32768, H = 32, dh = 128, D = 4096, bf16, causal; 25% of tokens kept
after layer 1, heads top-24 of 32 from layer 2), the largest configuration
that fits one GPU: per layer a QKV projection, a row log-sum-exp pass with
the attention output, a column-sum pass for token importance, the output
projection + residual, then head and token top-k and compaction. Inputs are
resident on the GPU before timing starts.

Prints one JSON line. `value` is token-layers per second (sum over layers
of B * n_l per step, divided by the step time). `roofline` describes the
kernel with the largest share of GPU time, timed with HIP events on the
library's stream in a second, instrumented pass over the same steps;
`roofline.attention` adds the attention kernels' combined rate (prefill:
algorithmic and executed MFMA work; decode: attention bytes) and
`roofline.step` the whole step against the same roof. `per_layer` gives each
layer's tokens/s including its selection and compaction. `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of the same workload.
Without --config the line also carries `workloads`: the same measurements
(no CPU baseline) for bert_base, bert_base_perhead, gpt2_decode and
pq_decode (the last with the fraction of rows the progressive quantization
recomputed), and for the
cascade representative-token selection workloads ada_gpt2 and ada_long
(fp32 Gram products; their line compares the cascade with a full-Gram
selection at every layer).

Launch mode (--launch): decode workloads replay one pass captured into a
HIP graph by default (the stacks allocate nothing and only enqueue kernels;
replays match the eager pass bit for bit), since a decode pass is thousands
of short launches and the host would otherwise pace the quantized one;
prefill and selection passes launch eagerly. --launch graph / eager forces
one mode for every workload (--graph = --launch graph). Each workload's
object names its mode in `launch`. The per-kernel pass is always eager.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu]
                    [--launch auto|graph|eager]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "pruned-attention tokens/s per layer + MFMA util / HBM GB/s vs peak, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def _cache_lengths(cfg):
    """Cache entries each decode step attends over (its own entry included):
    the cache is cut to cache_keep after step 1 and, with prune_every = r,
    after every r-th later step."""
    out, n = [], cfg.cache_len
    for s in range(cfg.steps):
        n += 1
        out.append(n)
        r = cfg.prune_every
        if (s == 0 or (r > 0 and s % r == 0)) and n > cfg.cache_keep:
            n = cfg.cache_keep
    return out


def _keys(cfg, l):
    """Keys each head attends over at prefill layer l."""
    return cfg.key_keep[l] if cfg.key_keep else cfg.tokens[l]


def _kernel_work(cfg, v_kept=None, recompute_frac=None):
    """Algorithmic work per kernel name for one step: (flops, bytes).
    v_kept[s][l]: V rows read at step s, layer l (value pruning);
    recompute_frac: fraction of (step, layer, sequence, head) rows that
    progressive quantization recomputed with both planes."""
    B, H, dh = cfg.batch, cfg.n_heads, cfg.head_dim
    D = H * dh
    es = 2 if cfg.dtype == "bf16" else 4
    w = {}

    def add(name, flops=0.0, nbytes=0.0):
        f, b = w.get(name, (0.0, 0.0))
        w[name] = (f + flops, b + nbytes)

    if cfg.kind == "prefill":
        for l in range(cfg.n_layers):
            n, h = cfg.tokens[l], cfg.heads[l]
            m = _keys(cfg, l)
            pairs = n * (n + 1) / 2 if cfg.causal else float(n) * m
            add("qkv_gemm", 2.0 * B * n * 3 * h * dh * D,
                es * (B * n * D + 3 * h * dh * D + 3 * B * n * h * dh))
            # the output projection's launch also runs the importance
            # reduction (bf16): column sums read, a read and written
            add("out_gemm", 2.0 * B * n * D * h * dh,
                es * (B * n * h * dh + D * h * dh + 2 * B * n * D) + 4.0 * B * h * m + 8.0 * B * n)
            # Q and O per query, K and V per key
            add("attn_fwd", 4.0 * B * h * dh * pairs, es * 2 * B * h * (n + m) * dh)
            add("attn_colsum", 2.0 * B * h * dh * pairs,
                es * B * h * (n + m) * dh + 4 * B * h * m)
            if cfg.key_keep:
                # each head's kept K rows and V columns, read and written
                add("gather_keys", 0.0, es * 4 * B * h * m * dh)
    else:
        for s, lc in enumerate(_cache_lengths(cfg)):
            for l in range(cfg.n_layers):
                add("qkv_gemm", 2.0 * B * 3 * D * D, es * 3 * D * D)
                # the output projection's launch also runs the importance
                # pass: a[b, j] read and written once per layer
                add("out_gemm", 2.0 * B * D * D, es * D * D + 8.0 * B * lc)
                if cfg.quantized:
                    # MSB planes and scales of K and V; a recomputed
                    # (sequence, head) row also needs the LSB halves of its
                    # head slice of K and V (dh / 2 bytes each; the kernel
                    # re-reads the MSB halves too, which the method does not
                    # need)
                    r = recompute_frac or 0.0
                    if cfg.v_threshold > 0:
                        # value pruning: K planes and scales, then the MSB
                        # half (and scale) of each kept V head row only; the
                        # fp32 scores the importance pass reads
                        kept = v_kept[s][l] if v_kept is not None else 0
                        add("pq_attn_vprune", 2.0 * B * H * dh * lc * (1 + r) + 2.0 * dh * kept,
                            B * lc * (D // 2 + 4) + r * B * H * lc * dh // 2
                            + kept * (dh // 2 + 4) + 4 * B * H * lc)
                    else:
                        add("pq_attn", 4.0 * B * H * dh * lc * (1 + r),
                            2 * B * lc * (D // 2 + 4) + r * B * H * lc * dh)
                elif cfg.v_threshold > 0:
                    # K rows once, the kept V rows (a 128-byte head slice
                    # each) and the fp32 scores the importance pass reads
                    kept = v_kept[s][l] if v_kept is not None else 0
                    fl = 2.0 * B * H * dh * lc + 2.0 * dh * kept
                    by = B * lc * D * es + kept * dh * es + 4 * B * H * lc
                    if -(-lc // 32) * 32 <= 4096:
                        add("decode_vrow", fl, by)
                    else:
                        add("decode_scores", 2.0 * B * H * dh * lc,
                            B * lc * D * es + 4 * B * H * lc)
                        add("decode_vprune", 2.0 * dh * kept,
                            kept * dh * es + 4 * B * H * lc + 8 * B * lc)
                else:
                    add("decode_attn", 4.0 * B * H * dh * lc, 2 * B * lc * D * es)
    return w


def _read_kernel_times(lib):
    maxk, nl = 64, 64
    names = ctypes.create_string_buffer(maxk * nl)
    ms = (ctypes.c_double * maxk)()
    cnt = (ctypes.c_int * maxk)()
    nk = ctypes.c_int(0)
    st = lib.spatten_debug_kernel_times(maxk, names, nl, ms, cnt, ctypes.byref(nk))
    if st != 0:
        raise RuntimeError("kernel timing failed (%d)" % st)
    out = {}
    for i in range(nk.value):
        nm = names.raw[i * nl:(i + 1) * nl].split(b"\0", 1)[0].decode()
        out[nm] = (ms[i], cnt[i])
    return out


def _traffic(kernel, workload, launches):
    """HBM bytes per launch from a committed counter summary for this kernel
    and workload, if its source hash still matches the current sources."""
    path = os.path.join(ROOT, "profiles", "pmc_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from cascade_token_head_amd.traffic import source_sha1
    if rec.get("source_sha1") != source_sha1(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def _mfma_counters(kernel, workload):
    """Executed MFMA rate of a kernel from a committed SQ_INSTS_MFMA summary
    for this workload (counter-measured), if its source hash still matches."""
    path = os.path.join(ROOT, "profiles", "mfma_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from cascade_token_head_amd.traffic import source_sha1
    if rec.get("source_sha1") != source_sha1(kernel):
        return None
    return {"executed_tflops": rec["executed_tflops"], "executed_frac": rec["executed_frac"],
            "avg_us": rec["avg_duration_us"]}


def _cpu_baseline(cfg, inputs, budget_s: float):
    """Time the fp64 oracle on whole sequences until `budget_s` is spent."""
    from oracle import spatten_ref as R
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    done, t0 = 0, time.perf_counter()
    if cfg.kind == "prefill" and cfg.tokens[0] > 4096:
        # A whole sequence is hours of fp64 work: time the oracle's first
        # layer on causal prefixes of sequence 0 (rows of a causal prefix see
        # only its own keys), doubling the prefix until the budget is spent.
        # Later rows of the full layer see more keys, so this rate is an
        # upper bound on the oracle's rate for the whole workload.
        assert cfg.causal
        W = inputs["layers"][0]
        heads = list(range(cfg.heads[0]))
        rows, el, S = 0, 0.0, 256
        while S <= cfg.tokens[0]:
            ts = time.perf_counter()
            R.prefill_layer(inputs["x"][0, :S], W, heads, cfg.head_dim, True, True)
            dt = time.perf_counter() - ts
            rows, el = S, dt
            if time.perf_counter() - t0 + 2.2 * dt > budget_s:
                break
            S *= 2
        sample = ("layer 1 of sequence 0 on its first %d tokens (a causal prefix), all %d heads; "
                  "rows of the full %d-token layer see up to %dx more keys, so this is an upper "
                  "bound on the oracle's rate" % (rows, cfg.heads[0], cfg.tokens[0],
                                                  cfg.tokens[0] // rows))
        return {"value": rows / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": sample, "seconds": round(el, 2)}
    if cfg.kind == "prefill":
        per_seq = sum(cfg.tokens)
        while done < cfg.batch:
            R.run_prefill(cfg, inputs, seqs=[done])
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
        sample = "sequences 0..%d of %d, all %d layers" % (done - 1, cfg.batch, cfg.n_layers)
        return {"value": done * per_seq / el, "unit": "tokens/s", "cores": threads,
                "kind": "oracle", "sample": sample, "seconds": round(el, 2)}
    steps = 2
    while done < cfg.batch:
        R.run_decode(cfg, inputs, seqs=[done], steps=steps)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    sample = "sequences 0..%d of %d, first %d decode steps, all %d layers" % (
        done - 1, cfg.batch, steps, cfg.n_layers)
    return {"value": done * steps * cfg.n_layers / el, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "sample": sample, "seconds": round(el, 2)}


ATTN_KERNELS = {
    "prefill": ("gather_keys", "attn_fwd", "attn_fwd_vprune", "attn_colsum", "importance"),
    "decode": ("decode_attn", "pq_attn", "pq_attn_vprune", "decode_vrow", "decode_scores",
               "decode_vprune",
               "decode_vsum", "decode_importance"),
}


def _attention_roof(cfg, ktimes, work, steps):
    """Combined rate of the attention kernels of one step."""
    names = [n for n in ATTN_KERNELS[cfg.kind] if n in ktimes]
    ms = sum(ktimes[n][0] for n in names) / steps
    if ms <= 0:
        return None
    if cfg.kind == "prefill":
        B, dh = cfg.batch, cfg.head_dim
        alg = 0.0
        for l in range(cfg.n_layers):
            n, h = cfg.tokens[l], cfg.heads[l]
            pairs = n * (n + 1) / 2 if cfg.causal else float(n) * _keys(cfg, l)
            alg += 4.0 * B * h * dh * pairs
        # the column-sum pass recomputes Q K^T: 6 instead of 4 flops per
        # (pair, dim); value pruning runs the forward pass twice (8)
        executed = (2.0 if cfg.v_threshold > 0 else 1.5) * alg
        a = alg / (ms / 1e3) / 1e12
        e = executed / (ms / 1e3) / 1e12
        return {"kernels": names, "ms_per_step": round(ms, 4), "bound": "mfma", "unit": "TFLOP/s",
                "achieved_alg": round(a, 2), "frac_alg": round(a / PEAK_BF16_TFLOPS, 4),
                "achieved_executed": round(e, 2),
                "frac_executed": round(e / PEAK_BF16_TFLOPS, 4)}
    by = sum(work.get(n, (0.0, 0.0))[1] for n in names)
    a = by / (ms / 1e3) / 1e9
    return {"kernels": names, "ms_per_step": round(ms, 4), "bound": "hbm", "unit": "GB/s",
            "achieved": round(a, 1), "frac": round(a / PEAK_HBM_GBS, 4)}


def _step_roof(cfg, work, ms_per_step):
    """The whole step's algorithmic work against the config's roof."""
    fl = sum(v[0] for v in work.values())
    by = sum(v[1] for v in work.values())
    sec = ms_per_step / 1e3
    if cfg.kind == "prefill":
        a = fl / sec / 1e12
        return {"bound": "mfma", "unit": "TFLOP/s", "alg_tflop": round(fl / 1e12, 4),
                "achieved": round(a, 2), "frac": round(a / PEAK_BF16_TFLOPS, 4)}
    a = by / sec / 1e9
    return {"bound": "hbm", "unit": "GB/s", "alg_gb": round(by / 1e9, 3),
            "achieved": round(a, 1), "frac": round(a / PEAK_HBM_GBS, 4)}


def use_graph(cfg, args) -> bool:
    """Whether the timed passes of this workload replay a captured graph."""
    return args.launch == "graph" or (args.launch == "auto" and cfg.kind == "decode")


def measure(cfg, args, lib, with_cpu: bool) -> dict:
    import torch

    from cascade_token_head_amd import pipeline
    from workloads import make_inputs

    dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    inputs = make_inputs(cfg)
    w = pipeline.weights_to_device(inputs["layers"], dtype)

    if cfg.kind == "prefill":
        if cfg.key_keep:
            stack = pipeline.PerHeadPrefillStack(cfg.n_layers, cfg.batch, cfg.n_heads,
                                                 cfg.head_dim, cfg.tokens[0], cfg.heads,
                                                 cfg.key_keep, w)
        else:
            stack = pipeline.PrefillStack(cfg.n_layers, cfg.batch, cfg.n_heads, cfg.head_dim,
                                          cfg.tokens, cfg.heads, dtype, cfg.causal, w,
                                          v_threshold=cfg.v_threshold)
        x0 = torch.from_numpy(inputs["x"]).to(dtype).cuda()

        def reset():
            stack.load(x0)

        def body(layer_hook=None):
            stack.run(layer_hook=layer_hook)

        def run_pass():
            reset()
            body()

        def timed_pass(ev0, ev1):
            ev0.record()
            reset()
            replay_or(body)
            ev1.record()
    else:
        stack = pipeline.DecodeStack(cfg.n_layers, cfg.batch, cfg.n_heads, cfg.head_dim,
                                     cfg.cache_len, cfg.cache_keep, cfg.steps, w, cfg.quantized,
                                     cfg.pq_threshold, dtype, v_threshold=cfg.v_threshold,
                                     prune_every=cfg.prune_every, per_head=cfg.per_head)
        k0 = [torch.from_numpy(l["k_cache"]).to(dtype).cuda() for l in inputs["layers"]]
        v0 = [torch.from_numpy(l["v_cache"]).to(dtype).cuda() for l in inputs["layers"]]
        xs = torch.from_numpy(inputs["x_steps"]).to(dtype).cuda()

        def reset():
            stack.load(k0, v0)

        def body(hook=None, record=False):
            for s in range(cfg.steps):
                stack.step(xs[s], hook=hook, record=record)

        def run_pass():
            reset()
            body()

        def timed_pass(ev0, ev1):
            reset()                # cache reset is not part of the decode work
            ev0.record()
            replay_or(body)
            ev1.record()

    for _ in range(args.warmup):
        run_pass()
    torch.cuda.synchronize()
    # With --graph, one pass is captured into a HIP graph (the stacks allocate
    # nothing and only enqueue kernels once constructed) and each timed step
    # replays it from a freshly loaded state.
    graph = None
    if use_graph(cfg, args):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run_pass()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        reset()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            body()
        torch.cuda.synchronize()

    def replay_or(fn):
        if graph is not None:
            graph.replay()
        else:
            fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        timed_pass(e0, e1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs)
    ms_per_step = wall * 1e3 / args.steps if cfg.kind == "prefill" else gpu_ms / args.steps
    tokens = cfg.token_layers()
    value = tokens / (ms_per_step / 1e3)

    # per-layer pass: events at layer boundaries (decode: around each layer
    # call of every step; the cache cut after a step is timed on its own)
    per_layer = []
    if cfg.kind == "prefill":
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(cfg.n_layers + 1)]
        reset()
        marks[0].record()
        body(layer_hook=lambda l: marks[l + 1].record())
        torch.cuda.synchronize()
        for l in range(cfg.n_layers):
            us = marks[l].elapsed_time(marks[l + 1]) * 1e3
            n = cfg.batch * cfg.tokens[l]
            per_layer.append({"layer": l + 1, "tokens": n, "heads": cfg.heads[l],
                              "us": round(us, 2), "tokens_per_s": round(n / (us / 1e6), 1)})
    else:
        ev = {}

        def hook(phase, l):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            ev[(stack.s, l, phase)] = e
        reset()
        cut_us = []
        for s in range(cfg.steps):
            stack.step(xs[s], hook=hook)
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            ev[(s, "end")] = e
        torch.cuda.synchronize()
        for s in range(cfg.steps):
            cut_us.append(ev[(s, cfg.n_layers - 1, "post")].elapsed_time(ev[(s, "end")]) * 1e3)
        for l in range(cfg.n_layers):
            us = sum(ev[(s, l, "pre")].elapsed_time(ev[(s, l, "post")])
                     for s in range(cfg.steps)) * 1e3 / cfg.steps
            per_layer.append({"layer": l + 1, "tokens": cfg.batch, "us": round(us, 2),
                              "tokens_per_s": round(cfg.batch / (us / 1e6), 1)})
        per_layer.append({"cache_cuts_us_per_step": round(sum(cut_us) / cfg.steps, 2)})

    # instrumented pass: per-kernel HIP-event durations over the same steps
    _read_kernel_times(lib)
    lib.spatten_debug_timing(1)
    for _ in range(args.steps):
        run_pass()
    torch.cuda.synchronize()
    lib.spatten_debug_timing(0)
    ktimes = _read_kernel_times(lib)
    v_kept, kept_frac, recompute_frac = None, None, None
    if cfg.kind == "decode" and (cfg.v_threshold > 0 or cfg.quantized):
        # V rows each layer read and rows recomputed, from one more (untimed)
        # pass over the steps
        reset()
        body(record=True)
        if cfg.v_threshold > 0:
            v_kept = [[int(n) for n in t["v_kept"].sum(dim=(1, 2)).tolist()]
                      for t in stack.trace]
            rows = sum(cfg.batch * cfg.n_heads * lc * cfg.n_layers for lc in _cache_lengths(cfg))
            kept_frac = round(sum(map(sum, v_kept)) / rows, 4)
        if cfg.quantized:
            rc = sum(int(t["recompute"].sum()) for t in stack.trace)
            recompute_frac = round(rc / (cfg.steps * cfg.n_layers * cfg.batch * cfg.n_heads), 5)
    work = _kernel_work(cfg, v_kept, recompute_frac)
    per_kernel = {}
    for name, (ms, cnt) in ktimes.items():
        fl, by = work.get(name, (0.0, 0.0))
        sec = ms / 1e3
        per_kernel[name] = {
            "total_ms": round(ms / args.steps, 4), "launches_per_step": cnt // args.steps,
            "avg_us": round(ms * 1e3 / max(cnt, 1), 3),
            "tflops": round(fl * args.steps / sec / 1e12, 2) if fl and sec > 0 else None,
            "gbs": round(by * args.steps / sec / 1e9, 1) if by and sec > 0 else None}
    dom = max(ktimes, key=lambda k: ktimes[k][0])
    fl, by = work.get(dom, (0.0, 0.0))
    dms, dcnt = ktimes[dom]
    if cfg.kind == "prefill":
        achieved = fl * args.steps / (dms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = by * args.steps / (dms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    traffic = _traffic(dom, cfg.name, dcnt // args.steps)
    avg_us = dms * 1e3 / max(dcnt, 1)
    roof.update({"kernel": dom, "avg_us": round(avg_us, 3),
                 "launches_per_step": dcnt // args.steps,
                 "traffic": traffic,
                 "attention": _attention_roof(cfg, ktimes, work, args.steps),
                 "step": _step_roof(cfg, work, ms_per_step)})
    if traffic is not None and cfg.kind == "decode":
        # the same launch's HBM rate from counter-measured bytes
        roof["frac_counters"] = round(traffic / (avg_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    if cfg.kind == "prefill" and roof["attention"] is not None:
        roof["attention"]["mfma_counters"] = {
            k: _mfma_counters(k, cfg.name) for k in ("attn_fwd", "attn_colsum")}

    cpu = _cpu_baseline(cfg, inputs, args.cpu_seconds) if with_cpu else None

    if cfg.kind == "prefill":
        conf = {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.tokens[0],
                "layers": cfg.n_layers, "heads": cfg.n_heads, "head_dim": cfg.head_dim,
                "tokens_per_layer": list(cfg.tokens), "heads_per_layer": list(cfg.heads),
                "causal": cfg.causal}
        if cfg.key_keep:
            conf["keys_per_head_per_layer"] = list(cfg.key_keep)
        if cfg.v_threshold > 0:
            conf["v_threshold"] = cfg.v_threshold
    else:
        conf = {"workload": cfg.name, "batch": cfg.batch, "cache_len": cfg.cache_len,
                "cache_keep": cfg.cache_keep, "decode_steps": cfg.steps, "layers": cfg.n_layers,
                "heads": cfg.n_heads, "head_dim": cfg.head_dim, "quantized": cfg.quantized,
                "pq_threshold": cfg.pq_threshold, "prune_every": cfg.prune_every,
                "v_threshold": cfg.v_threshold, "per_head": cfg.per_head,
                "v_rows_kept_frac": kept_frac, "pq_recompute_frac": recompute_frac}
    del stack, w, inputs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"value": round(value, 1), "ms_per_step": round(ms_per_step, 4),
            "gpu_ms_per_step": round(gpu_ms / args.steps, 4),
            "launch": "hip_graph" if use_graph(cfg, args) else "eager",
            "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "config": conf,
            "roofline": roof, "per_layer": per_layer, "kernels": per_kernel,
            "cpu_baseline": cpu}


PEAK_FP32_TFLOPS = 157.3     # MI355X dense fp32 (MFMA and vector)


def measure_ada(cfg, args, lib, with_cpu: bool) -> dict:
    """Cascade representative-token selection (page 5) over a stack of
    synthetic layer activations: a step is one pass over every layer (the
    full-Gram selection of layer 1, then a cascade step per layer)."""
    import torch

    from cascade_token_head_amd import pipeline
    from workloads import ada_batch_layers

    layers = [torch.from_numpy(x).cuda() for x in ada_batch_layers(cfg)]
    st = pipeline.AdaStack(cfg.n_layers, cfg.batch, cfg.seq_len, cfg.dim, cfg.tau)
    for _ in range(args.warmup):
        st.run(layers)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        st.run(layers)
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    gpu_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
    value = cfg.token_layers() / (ms_per_step / 1e3)
    counts = st.counts.cpu().numpy().astype(np.int64)   # [L, B, 4]
    pairs = counts[:, :, 3].sum(axis=1)                  # Gram entries per layer
    sizes = counts[:, :, 0].sum(axis=1)
    # per-layer times, and the same layers selected independently (full
    # Gram product at every layer) for comparison
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(cfg.n_layers + 1)]
    from cascade_token_head_amd import spatten as S
    marks[0].record()
    for l, x in enumerate(layers):
        S.ada_select(x, cfg.tau, st.flags[l], st.ws, prev=None if l == 0 else st.flags[l - 1],
                     maxcos=st.maxcos[l], counts=st.counts[l])
        marks[l + 1].record()
    torch.cuda.synchronize()
    per_layer = []
    for l in range(cfg.n_layers):
        us = marks[l].elapsed_time(marks[l + 1]) * 1e3
        n = cfg.batch * cfg.seq_len
        per_layer.append({"layer": l + 1, "tokens": n, "representatives": int(sizes[l]),
                          "gram_pairs": int(pairs[l]), "us": round(us, 2),
                          "tokens_per_s": round(n / (us / 1e6), 1)})
    full = pipeline.AdaStack(cfg.n_layers, cfg.batch, cfg.seq_len, cfg.dim, cfg.tau)
    full.run(layers, full_every_layer=True)
    torch.cuda.synchronize()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    for _ in range(args.steps):
        full.run(layers, full_every_layer=True)
    f1.record()
    torch.cuda.synchronize()
    full_ms = f0.elapsed_time(f1) / args.steps
    full_pairs = cfg.batch * cfg.n_layers * cfg.seq_len * (cfg.seq_len - 1) // 2
    # per-kernel times over the same steps
    _read_kernel_times(lib)
    lib.spatten_debug_timing(1)
    for _ in range(args.steps):
        st.run(layers)
    torch.cuda.synchronize()
    lib.spatten_debug_timing(0)
    ktimes = _read_kernel_times(lib)
    gram_flops = 2.0 * cfg.dim * float(pairs.sum())   # per step
    per_kernel = {n: {"total_ms": round(ms / args.steps, 4), "launches_per_step": c // args.steps,
                      "avg_us": round(ms * 1e3 / max(c, 1), 3)} for n, (ms, c) in ktimes.items()}
    gms, gcnt = ktimes["ada_gram"]
    achieved = gram_flops * args.steps / (gms / 1e3) / 1e12
    per_kernel["ada_gram"]["tflops"] = round(achieved, 2)
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4), "kernel": "ada_gram",
            "dtype": "f32", "avg_us": round(gms * 1e3 / max(gcnt, 1), 3),
            "launches_per_step": gcnt // args.steps,
            "traffic": _traffic("ada_gram", cfg.name, gcnt // args.steps),
            "step": {"gram_tflop": round(gram_flops / 1e12, 5),
                     "achieved": round(gram_flops / (ms_per_step / 1e3) / 1e12, 2)}}
    cpu = None
    if with_cpu:
        from oracle import ada_ref as R
        from workloads import ada_layers
        t0 = time.perf_counter()
        done = 0
        while done < cfg.batch and time.perf_counter() - t0 < args.cpu_seconds:
            R.run_cascade(ada_layers(cfg, done), cfg.tau)
            done += 1
        el = time.perf_counter() - t0
        cpu = {"value": round(done * cfg.seq_len * cfg.n_layers / el, 1), "unit": "tokens/s",
               "cores": os.cpu_count(), "kind": "oracle",
               "sample": "sequences 0..%d of %d, all %d layers" % (done - 1, cfg.batch,
                                                                   cfg.n_layers),
               "seconds": round(el, 2)}
    del layers, st, full
    torch.cuda.empty_cache()
    return {"value": round(value, 1), "ms_per_step": round(ms_per_step, 4),
            "gpu_ms_per_step": round(gpu_ms, 4), "launch": "eager", "dtype": "f32",
            "config": {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.seq_len,
                       "dim": cfg.dim, "layers": cfg.n_layers, "tau": cfg.tau},
            "roofline": roof, "per_layer": per_layer, "kernels": per_kernel,
            "cascade_vs_full": {"gram_pairs": int(pairs.sum()), "full_gram_pairs": full_pairs,
                                "pair_ratio": round(float(pairs.sum()) / full_pairs, 4),
                                "full_ms_per_step": round(full_ms, 4),
                                "speedup": round(full_ms / gpu_ms, 3)},
            "cpu_baseline": cpu}


HEADLINE = "long_causal"
OTHERS = ("bert_base", "bert_base_perhead", "gpt2_decode", "pq_decode", "ada_gpt2", "ada_long")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None,
                    help="measure only this workload (default: long_causal as the headline, "
                         "plus " + ", ".join(OTHERS) + ")")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=30.0)
    ap.add_argument("--launch", choices=("auto", "graph", "eager"), default="auto",
                    help="auto: decode passes replay a captured HIP graph, the others launch "
                         "every kernel from the host; graph / eager: that mode everywhere")
    ap.add_argument("--graph", action="store_true", help="same as --launch graph")
    args = ap.parse_args()
    if args.graph:
        args.launch = "graph"
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(the sequences of a batch are independent, so a batch would shard by sequence)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from cascade_token_head_amd import spatten as S
    from workloads import BY_NAME

    lib = S.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    head = args.config or HEADLINE
    print("measuring %s" % head, file=sys.stderr, flush=True)
    run = measure_ada if BY_NAME[head].kind == "ada" else measure
    r = run(BY_NAME[head], args, lib, with_cpu=not args.no_cpu)
    out = {"metric": METRIC, "value": r["value"], "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
           "gpu_ms_per_step": r["gpu_ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": r["dtype"], "data": "synthetic (seeded)",
           "config": r["config"], "launch": r["launch"],
           "roofline": r["roofline"], "per_layer": r["per_layer"], "kernels": r["kernels"],
           "cpu_baseline": r["cpu_baseline"]}
    if "cascade_vs_full" in r:
        out["cascade_vs_full"] = r["cascade_vs_full"]
    if args.config is None:
        out["workloads"] = {}
        for name in OTHERS:
            print("measuring %s" % name, file=sys.stderr, flush=True)
            cfg = BY_NAME[name]
            o = (measure_ada if cfg.kind == "ada" else measure)(cfg, args, lib, with_cpu=False)
            o.pop("cpu_baseline")
            out["workloads"][name] = o
    print(json.dumps(out))


if __name__ == "__main__":
    main()
