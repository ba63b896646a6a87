#!/usr/bin/env python3
"""Pruned-attention throughput on one MI355X.

A step is one pass of the whole cascade over one batch of synthetic input:
for the default workload (bert_base: 12 attention-only layers, batch 32,
T=512, H=12, dh=64, bf16, token keep 1.0 -> 0.5, heads 12 -> 10 from layer
4) that is QKV projection, attention with fused token/head importance,
output projection + residual, head and token top-k and compaction, for
every layer. Inputs are resident on the GPU before timing starts.

Prints one JSON line. `value` is token-layers per second (sum over layers
of B * n_l per step, divided by the step time). `roofline` describes the
kernel with the largest share of GPU time, timed with HIP events on its own
stream in a second, instrumented pass over the same steps. `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of the same workload.

With --graph the timed steps replay one pass captured into a HIP graph (the
stacks allocate nothing and only enqueue kernels; replays match the eager
pass bit for bit). On MI355X both time the same: the host already keeps the
kernels back to back. The per-kernel pass is always eager.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu] [--graph]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

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


def _kernel_work(cfg, v_kept=None):
    """Algorithmic work per kernel name for one step: (flops, bytes).
    v_kept[s][l]: V rows read at step s, layer l (value pruning)."""
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
            pairs = n * (n + 1) / 2 if cfg.causal else float(n) * n
            add("qkv_gemm", 2.0 * B * n * 3 * h * dh * D, es * (B * n * D + 3 * h * dh * D + 3 * B * n * h * dh))
            add("out_gemm", 2.0 * B * n * D * h * dh, es * (B * n * h * dh + D * h * dh + 2 * B * n * D))
            add("attn_fwd", 4.0 * B * h * dh * pairs, es * 4 * B * h * n * dh)
            add("attn_colsum", 2.0 * B * h * dh * pairs, es * 2 * B * h * n * dh + 4 * B * h * n)
    else:
        for s, lc in enumerate(_cache_lengths(cfg)):
            for l in range(cfg.n_layers):
                add("qkv_gemm", 2.0 * B * 3 * D * D, es * 3 * D * D)
                add("out_gemm", 2.0 * B * D * D, es * D * D)
                if cfg.quantized:
                    add("pq_attn_msb", 4.0 * B * H * dh * lc, 2 * B * lc * (D // 2 + 4))
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="bert_base")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one pass captured into a HIP graph instead of "
                         "launching every kernel from the host")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(sequences are independent; see the sharding notes in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch

    from cascade_token_head_amd import pipeline
    from cascade_token_head_amd import spatten as S
    from workloads import BY_NAME, make_inputs

    cfg = BY_NAME[args.config]
    lib = S.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    inputs = make_inputs(cfg)
    w = pipeline.weights_to_device(inputs["layers"], dtype)

    if cfg.kind == "prefill":
        stack = pipeline.PrefillStack(cfg.n_layers, cfg.batch, cfg.n_heads, cfg.head_dim,
                                      cfg.tokens, cfg.heads, dtype, cfg.causal, w)
        x0 = torch.from_numpy(inputs["x"]).to(dtype).cuda()

        def reset():
            stack.load(x0)

        def body():
            stack.run()

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

        def body():
            for s in range(cfg.steps):
                stack.step(xs[s])

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
    if args.graph:
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
    t0 = time.perf_counter()
    for e0, e1 in evs:
        timed_pass(e0, e1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs)
    ms_per_step = wall * 1e3 / args.steps if cfg.kind == "prefill" else gpu_ms / args.steps
    tokens = cfg.token_layers()
    value = tokens / (ms_per_step / 1e3)

    # instrumented pass: per-kernel HIP-event durations over the same steps
    _read_kernel_times(lib)
    lib.spatten_debug_timing(1)
    for _ in range(args.steps):
        run_pass()
    torch.cuda.synchronize()
    lib.spatten_debug_timing(0)
    ktimes = _read_kernel_times(lib)
    v_kept, kept_frac = None, None
    if cfg.kind == "decode" and cfg.v_threshold > 0:
        # V rows each layer read, from one more (untimed) pass over the steps
        stack.load(k0, v0)
        for s in range(cfg.steps):
            stack.step(xs[s], record=True)
        v_kept = [[int(n) for n in t["v_kept"].sum(dim=(1, 2)).tolist()] for t in stack.trace]
        rows = sum(cfg.batch * cfg.n_heads * lc * cfg.n_layers for lc in _cache_lengths(cfg))
        kept_frac = round(sum(map(sum, v_kept)) / rows, 4)
    work = _kernel_work(cfg, v_kept)
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
    roof.update({"kernel": dom, "avg_us": round(dms * 1e3 / max(dcnt, 1), 3),
                 "launches_per_step": dcnt // args.steps,
                 "traffic": _traffic(dom, cfg.name, dcnt // args.steps)})

    cpu = None
    if not args.no_cpu:
        cpu = _cpu_baseline(cfg, inputs, args.cpu_seconds)

    if cfg.kind == "prefill":
        conf = {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.tokens[0],
                "layers": cfg.n_layers, "heads": cfg.n_heads, "head_dim": cfg.head_dim,
                "tokens_per_layer": list(cfg.tokens), "heads_per_layer": list(cfg.heads),
                "causal": cfg.causal}
    else:
        conf = {"workload": cfg.name, "batch": cfg.batch, "cache_len": cfg.cache_len,
                "cache_keep": cfg.cache_keep, "decode_steps": cfg.steps, "layers": cfg.n_layers,
                "heads": cfg.n_heads, "head_dim": cfg.head_dim, "quantized": cfg.quantized,
                "prune_every": cfg.prune_every, "v_threshold": cfg.v_threshold,
                "per_head": cfg.per_head,
                "v_rows_kept_frac": kept_frac}
    out = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "gpu_ms_per_step": round(gpu_ms / args.steps, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic (seeded)",
           "config": conf, "launch": "hip_graph" if args.graph else "eager",
           "roofline": roof, "kernels": per_kernel, "cpu_baseline": cpu}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
