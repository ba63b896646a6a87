"""HBM traffic and executed MFMA work of a kernel from rocprofv3 counter runs.

    # a plain device-to-device copy of known size, for the counter scale
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR -o copy_fetch -- \\
        python3 -m cascade_token_head_amd.traffic copy --mib 1024
    # the same with WRITE_SIZE; the same pair on a second known-traffic
    # kernel (`triad`, c = a + b) to cross-check the scales; then both
    # counters on the benchmark command
    python3 -m cascade_token_head_amd.traffic summarize --label qkv_gemm \\
        --workload bert_base --kernel-regex 'gemm_tile_kernel<0,' \\
        --fetch run_fetch.csv --write run_write.csv \\
        --copy-fetch copy_fetch.csv --copy-write copy_write.csv \\
        --triad-fetch triad_fetch.csv --triad-write triad_write.csv \\
        --command '...' --out profiles/

The mfma subcommand reads SQ_INSTS_MFMA (wave-level MFMA instructions per
dispatch; every prefill MFMA here is a 32x32x16 bf16 one, 32768 flops) and
the kernel's average duration from a kernel-trace statistics file of the
same command, and writes profiles/mfma_<label>_<workload>.{json,md} with the
executed flops per launch and their rate against the bf16 dense peak.

FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch. Each is scaled by
known bytes / counted bytes of the copy kernel (so a counter that reads
high or low on this part is corrected), then averaged per launch of the
kernel. The result, with the hash of the sources that kernel is built from
(its .hip file and the shared headers), goes to
profiles/pmc_<label>_<workload>.json (read by bench.py) and a short .md
summary beside it.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "cascade_token_head_amd", "csrc")
COPY_KERNEL = r"copyBuffer"

# The source file each timed kernel is built from; every kernel also
# depends on the shared headers.
KERNEL_SOURCE = {
    "qkv_gemm": "gemm.hip", "out_gemm": "gemm.hip",
    "attn_fwd": "attn.hip", "attn_colsum": "attn.hip", "importance": "attn.hip",
    "attn_fwd_vprune": "attn.hip", "gather_keys": "attn.hip",
    "decode_attn": "decode.hip", "pq_attn": "decode.hip", "pq_attn_vprune": "decode.hip",
    "decode_vrow": "decode.hip",
    "decode_scores": "decode.hip", "decode_vprune": "decode.hip", "decode_vsum": "decode.hip",
    "decode_importance": "decode.hip",
    "topk": "topk.hip", "compact": "compact.hip", "compact_inplace": "compact.hip",
    "quantize": "quant.hip",
    "ada_gram": "ada.hip", "ada_invnorm": "ada.hip", "ada_lists": "ada.hip",
    "ada_valid": "ada.hip", "ada_finish": "ada.hip",
}
SHARED_HEADERS = ("common.hpp", "importance.hpp", "kernels.hpp", "layout.hpp", "timing.hpp")


def source_sha1(kernel: str) -> str:
    """Hash of the sources a kernel is built from: its .hip file and the
    shared headers (bench.py checks the same hash before it reports a
    counter summary). Unknown kernels hash every source file."""
    files = ([KERNEL_SOURCE[kernel]] + list(SHARED_HEADERS) if kernel in KERNEL_SOURCE
             else sorted(os.listdir(CSRC)))
    h = hashlib.sha1()
    for fn in files:
        with open(os.path.join(CSRC, fn), "rb") as f:
            h.update(fn.encode() + f.read())
    return h.hexdigest()


def per_dispatch(path: str, counter: str, kernel_regex: str):
    """{dispatch id: counter value} for kernels whose name matches."""
    rx = re.compile(kernel_regex)
    vals = defaultdict(float)
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter or not rx.search(row.get("Kernel_Name", "")):
                continue
            vals[row.get("Dispatch_Id") or row.get("Correlation_Id")] += float(row["Counter_Value"])
    return dict(vals)


def copy_main(mib: int) -> None:
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}))


def triad_main(mib: int) -> None:
    """c = a + b over fp32 vectors of `mib` MiB each: a second kernel of
    known traffic (2 x mib read, mib written per dispatch)."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.ones(n, dtype=torch.float32, device="cuda")
    c = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.add(a, b, out=c)
    torch.cuda.synchronize()
    print(json.dumps({"triad_bytes_each": n * 4, "dispatches": 3}))


TRIAD_KERNEL = r"CUDAFunctor_add|AddFunctor|add_kernel"


def _scale(path, counter, regex, expected):
    """known bytes / counted bytes over the dispatches that carry the bulk
    (counted at above a quarter of the expected bytes: a counter that reads
    half of them, as FETCH_SIZE does here, still qualifies; fills and small
    copies do not)."""
    vals = per_dispatch(path, counter, regex)
    big = [v for v in vals.values() if v * 1024 > 0.25 * expected]
    if not big:
        sys.exit("no %s dispatch of the expected size in %s" % (counter, path))
    return expected / (sum(big) / len(big) * 1024)


def summarize_main(a) -> None:
    copy_bytes = a.copy_mib * (1 << 20)
    # the copy kernel moves copy_bytes in and out per dispatch
    f_scale = _scale(a.copy_fetch, "FETCH_SIZE", COPY_KERNEL, copy_bytes)
    w_scale = _scale(a.copy_write, "WRITE_SIZE", COPY_KERNEL, copy_bytes)
    check = None
    if a.triad_fetch and a.triad_write:
        # a second known-traffic kernel: the scales must agree
        tb = a.triad_mib * (1 << 20)
        tf = _scale(a.triad_fetch, "FETCH_SIZE", TRIAD_KERNEL, 2 * tb)
        tw = _scale(a.triad_write, "WRITE_SIZE", TRIAD_KERNEL, tb)
        check = {"triad_fetch_scale": round(tf, 4), "triad_write_scale": round(tw, 4),
                 "fetch_scale_rel_diff": round(abs(tf - f_scale) / f_scale, 4),
                 "write_scale_rel_diff": round(abs(tw - w_scale) / w_scale, 4)}
    kf = per_dispatch(a.fetch, "FETCH_SIZE", a.kernel_regex)
    kw = per_dispatch(a.write, "WRITE_SIZE", a.kernel_regex)
    if not kf or not kw:
        sys.exit("kernel %r not found in the counter runs" % a.kernel_regex)
    fetch = sum(kf.values()) / len(kf) * 1024 * f_scale
    write = sum(kw.values()) / len(kw) * 1024 * w_scale
    rec = {"kernel": a.label, "workload": a.workload, "kernel_regex": a.kernel_regex,
           "dispatches": len(kf), "fetch_bytes_per_launch": round(fetch),
           "write_bytes_per_launch": round(write),
           "hbm_bytes_per_launch": round(fetch + write),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "copy_bytes": copy_bytes, "calibration_check": check,
           "source_sha1": source_sha1(a.label), "command": a.command}
    os.makedirs(a.out, exist_ok=True)
    base = os.path.join(a.out, "pmc_%s_%s" % (a.label, a.workload))
    with open(base + ".json", "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    with open(base + ".md", "w") as f:
        f.write("# HBM traffic: %s on %s\n\n" % (a.label, a.workload))
        f.write("Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch), one rocprofv3 "
                "--pmc run each, scaled by known/counted bytes of a %d MiB device copy.\n\n"
                % a.copy_mib)
        f.write("| quantity | value |\n|---|---|\n")
        for k in ("dispatches", "fetch_bytes_per_launch", "write_bytes_per_launch",
                  "hbm_bytes_per_launch", "fetch_scale", "write_scale"):
            f.write("| %s | %s |\n" % (k, rec[k]))
        if check:
            f.write("\nCalibration cross-check with a second kernel of known traffic "
                    "(c = a + b, %d MiB per vector: 2x read, 1x written):\n\n"
                    "| quantity | value |\n|---|---|\n" % a.triad_mib)
            for k, v in check.items():
                f.write("| %s | %s |\n" % (k, v))
        f.write("\nkernel symbol regex: `%s`\n\nsource sha1: `%s`\n\ncommand:\n\n```\n%s\n```\n"
                % (a.kernel_regex, rec["source_sha1"], a.command))
    print(json.dumps(rec))


MFMA_FLOPS = {"32x32x16": 2 * 32 * 32 * 16}
PEAK_BF16_TFLOPS = 2500.0


def mfma_main(a) -> None:
    counts = per_dispatch(a.counters, "SQ_INSTS_MFMA", a.kernel_regex)
    if not counts:
        sys.exit("kernel %r not found in the counter run" % a.kernel_regex)
    rx = re.compile(a.kernel_regex)
    durs = []
    with open(a.stats, newline="") as f:
        for row in csv.DictReader(f):
            if rx.search(row["Name"]):
                durs.append((int(row["Calls"]), float(row["TotalDurationNs"])))
    if not durs:
        sys.exit("kernel %r not found in the trace statistics" % a.kernel_regex)
    avg_ns = sum(t for _, t in durs) / sum(c for c, _ in durs)
    insts = sum(counts.values()) / len(counts)
    flops = insts * MFMA_FLOPS[a.shape]
    rate = flops / (avg_ns * 1e-9) / 1e12
    rec = {"kernel": a.label, "workload": a.workload, "kernel_regex": a.kernel_regex,
           "dispatches": len(counts), "mfma_insts_per_launch": round(insts),
           "mfma_shape": a.shape, "executed_flops_per_launch": flops,
           "avg_duration_us": round(avg_ns / 1e3, 3), "executed_tflops": round(rate, 1),
           "peak_tflops": PEAK_BF16_TFLOPS, "executed_frac": round(rate / PEAK_BF16_TFLOPS, 4),
           "source_sha1": source_sha1(a.label), "command": a.command}
    os.makedirs(a.out, exist_ok=True)
    base = os.path.join(a.out, "mfma_%s_%s" % (a.label, a.workload))
    with open(base + ".json", "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    with open(base + ".md", "w") as f:
        f.write("# Executed MFMA work: %s on %s\n\n" % (a.label, a.workload))
        f.write("SQ_INSTS_MFMA per dispatch (one rocprofv3 --pmc run) times %d flops per "
                "v_mfma_f32_%s_bf16, over the kernel's average duration from a "
                "rocprofv3 --kernel-trace --stats run of the same command.\n\n"
                % (MFMA_FLOPS[a.shape], a.shape))
        f.write("| quantity | value |\n|---|---|\n")
        for k in ("dispatches", "mfma_insts_per_launch", "executed_flops_per_launch",
                  "avg_duration_us", "executed_tflops", "peak_tflops", "executed_frac"):
            f.write("| %s | %s |\n" % (k, rec[k]))
        f.write("\nkernel symbol regex: `%s`\n\nsource sha1: `%s`\n\ncommand:\n\n```\n%s\n```\n"
                % (a.kernel_regex, rec["source_sha1"], a.command))
    print(json.dumps(rec))


# Issue-level SQ counters summarised per kernel, and the ratios read from
# them (counts are summed over the shader engines; the ratios of two counts
# of one run do not depend on that).
SQ_RATIOS = (
    ("valu_insts_per_mfma", "SQ_INSTS_VALU", "SQ_INSTS_MFMA"),
    ("trans_insts_per_mfma", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA"),
    ("lds_insts_per_mfma", "SQ_INSTS_LDS", "SQ_INSTS_MFMA"),
    ("wave_cycles_waiting_on_dependencies", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
    ("wave_cycles_issuing_valu", "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES"),
    ("wave_cycles_issuing_lds", "SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES"),
    ("wave_cycles_waiting_on_lds", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"),
    ("mfma_busy_with_valu_coissued", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES"),
    ("lds_bank_conflicts_per_lds_inst", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS"),
)


def sq_main(a) -> None:
    kernels = [kv.split("=", 1) for kv in a.kernel]
    per = {}
    for label, rx in kernels:
        vals = {}
        for path in a.counters:
            names = set()
            with open(path, newline="") as f:
                for row in csv.DictReader(f):
                    names.add(row["Counter_Name"])
            for c in sorted(names):
                d = per_dispatch(path, c, rx)
                if d:
                    vals[c] = sum(d.values()) / len(d)
        if not vals:
            sys.exit("kernel %r not found in the counter runs" % rx)
        per[label] = vals
    rec = {"workload": a.workload, "kernels": {k: v for k, v in per.items()},
           "ratios": {}, "command": a.command,
           "source_sha1": {label: source_sha1(label) for label, _ in kernels}}
    for label, vals in per.items():
        rec["ratios"][label] = {name: round(vals[n] / vals[d], 4)
                                for name, n, d in SQ_RATIOS if n in vals and vals.get(d)}
    os.makedirs(a.out, exist_ok=True)
    base = os.path.join(a.out, "sq_%s_%s" % (a.name, a.workload))
    with open(base + ".json", "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    labels = [k for k, _ in kernels]
    with open(base + ".md", "w") as f:
        f.write("# Issue counters: %s on %s\n\n" % (", ".join(labels), a.workload))
        f.write("SQ counters per dispatch (averages over the matching dispatches of each "
                "rocprofv3 --pmc pass; counts summed over the shader engines), and the "
                "ratios read from them.\n\n")
        f.write("| ratio | " + " | ".join(labels) + " |\n|---|" + "---|" * len(labels) + "\n")
        for name, _, _ in SQ_RATIOS:
            f.write("| %s | %s |\n" % (name, " | ".join(
                str(rec["ratios"][l].get(name, "")) for l in labels)))
        f.write("\n| counter | " + " | ".join(labels) + " |\n|---|" + "---|" * len(labels) + "\n")
        names = sorted(set().union(*[set(v) for v in per.values()]))
        for c in names:
            f.write("| %s | %s |\n" % (c, " | ".join(
                "%.4g" % per[l][c] if c in per[l] else "" for l in labels)))
        f.write("\nkernel symbol regexes: %s\n\nsource sha1: %s\n\ncommand:\n\n```\n%s\n```\n"
                % (", ".join("%s `%s`" % (l, r) for l, r in kernels),
                   ", ".join("%s `%s`" % (l, rec["source_sha1"][l]) for l in labels), a.command))
    print(json.dumps(rec["ratios"]))


def trace_main(a) -> None:
    """Markdown summary of a rocprofv3 --kernel-trace --stats run: the
    kernels by share of GPU time, with the command that produced it."""
    rows = list(csv.DictReader(open(a.stats, newline="")))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    os.makedirs(a.out, exist_ok=True)
    path = os.path.join(a.out, "%s_%s_kernel_trace.md" % (a.label, a.workload))
    with open(path, "w") as f:
        f.write("# Kernel trace: %s workload (dominant kernel %s)\n\n" % (a.workload, a.label))
        f.write("rocprofv3 kernel-trace statistics: every dispatch of the command (the "
                "warm-up, timed and instrumented passes bench.py runs).\n\nCommand:\n\n"
                "```\n%s\n```\n\n" % a.command)
        f.write("| kernel | calls | avg us | min us | max us | share |\n|---|---|---|---|---|---|\n")
        for r in rows[: a.top]:
            name = r["Name"] if len(r["Name"]) <= 90 else r["Name"][:87] + "..."
            f.write("| `%s` | %s | %.2f | %.2f | %.2f | %.1f%% |\n" % (
                name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3, 100.0 * float(r["TotalDurationNs"]) / total))
        if a.bench_json:
            # bench.py's own HIP-event average for the same kernel, printed
            # by the traced run itself
            with open(a.bench_json) as bj:
                line = json.loads(bj.read().strip().splitlines()[-1])
            rec = line if line["config"]["workload"] == a.workload else \
                line.get("workloads", {}).get(a.workload)
            if rec is not None and rec["roofline"].get("kernel") == a.label:
                tr = [r for r in rows if re.search(a.kernel_regex, r["Name"])] if \
                    a.kernel_regex else []
                f.write("\nbench.py's HIP-event average for %s in the traced run: %.2f us "
                        "over %d launches per step" % (a.label, rec["roofline"]["avg_us"],
                                                        rec["roofline"]["launches_per_step"]))
                if tr:
                    calls = sum(int(r["Calls"]) for r in tr)
                    avg = sum(float(r["TotalDurationNs"]) for r in tr) / calls / 1e3
                    f.write("; the trace's average for `%s`: %.2f us over %d dispatches"
                            % (a.kernel_regex, avg, calls))
                f.write(".\n")
        f.write("\nsource sha1 of %s: `%s`\n" % (a.label, source_sha1(a.label)))
    print(path)


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    t = sub.add_parser("triad")
    t.add_argument("--mib", type=int, default=512)
    tr = sub.add_parser("trace")
    tr.add_argument("--label", required=True)
    tr.add_argument("--workload", required=True)
    tr.add_argument("--stats", required=True)
    tr.add_argument("--top", type=int, default=12)
    tr.add_argument("--command", default="")
    tr.add_argument("--bench-json", default=None,
                    help="bench.py's output line from the traced run")
    tr.add_argument("--kernel-regex", default=None,
                    help="symbol regex of the dominant kernel in the trace")
    tr.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    s = sub.add_parser("summarize")
    s.add_argument("--label", required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--kernel-regex", required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--copy-fetch", required=True)
    s.add_argument("--copy-write", required=True)
    s.add_argument("--copy-mib", type=int, default=1024)
    s.add_argument("--triad-fetch", default=None)
    s.add_argument("--triad-write", default=None)
    s.add_argument("--triad-mib", type=int, default=512)
    s.add_argument("--command", default="")
    s.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    m = sub.add_parser("mfma")
    m.add_argument("--label", required=True)
    m.add_argument("--workload", required=True)
    m.add_argument("--kernel-regex", required=True)
    m.add_argument("--counters", required=True)
    m.add_argument("--stats", required=True)
    m.add_argument("--shape", default="32x32x16", choices=sorted(MFMA_FLOPS))
    m.add_argument("--command", default="")
    m.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    q = sub.add_parser("sq")
    q.add_argument("--name", required=True, help="file name stem, e.g. attention")
    q.add_argument("--workload", required=True)
    q.add_argument("--kernel", action="append", required=True, help="label=symbol regex")
    q.add_argument("--counters", nargs="+", required=True, help="counter CSVs, one per pass")
    q.add_argument("--command", default="")
    q.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args()
    if a.cmd == "copy":
        copy_main(a.mib)
    elif a.cmd == "triad":
        triad_main(a.mib)
    elif a.cmd == "trace":
        trace_main(a)
    elif a.cmd == "mfma":
        mfma_main(a)
    elif a.cmd == "sq":
        sq_main(a)
    else:
        summarize_main(a)


if __name__ == "__main__":
    main()
