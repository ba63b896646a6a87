"""HBM traffic and executed MFMA work of a kernel from rocprofv3 counter runs.

    # a plain device-to-device copy of known size, for the counter scale
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR -o copy_fetch -- \\
        python3 -m cascade_token_head_amd.traffic copy --mib 1024
    # the same with WRITE_SIZE, then both counters on the benchmark command
    python3 -m cascade_token_head_amd.traffic summarize --label qkv_gemm \\
        --workload bert_base --kernel-regex 'gemm_tile_kernel<0,' \\
        --fetch run_fetch.csv --write run_write.csv \\
        --copy-fetch copy_fetch.csv --copy-write copy_write.csv \\
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
    "decode_attn": "decode.hip", "pq_attn": "decode.hip", "decode_vrow": "decode.hip",
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


def summarize_main(a) -> None:
    copy_bytes = a.copy_mib * (1 << 20)
    cf = per_dispatch(a.copy_fetch, "FETCH_SIZE", COPY_KERNEL)
    cw = per_dispatch(a.copy_write, "WRITE_SIZE", COPY_KERNEL)
    # the copy kernel moves copy_bytes in and out per dispatch; take the
    # dispatches that carry the bulk (fills and small copies excluded)
    big_f = [v for v in cf.values() if v * 1024 > 0.5 * copy_bytes]
    big_w = [v for v in cw.values() if v * 1024 > 0.5 * copy_bytes]
    if not big_f or not big_w:
        sys.exit("no copy dispatch of the expected size in the calibration runs")
    f_scale = copy_bytes / (sum(big_f) / len(big_f) * 1024)
    w_scale = copy_bytes / (sum(big_w) / len(big_w) * 1024)
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
           "copy_bytes": copy_bytes, "source_sha1": source_sha1(a.label), "command": a.command}
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


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    s = sub.add_parser("summarize")
    s.add_argument("--label", required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--kernel-regex", required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--copy-fetch", required=True)
    s.add_argument("--copy-write", required=True)
    s.add_argument("--copy-mib", type=int, default=1024)
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
    a = ap.parse_args()
    if a.cmd == "copy":
        copy_main(a.mib)
    elif a.cmd == "mfma":
        mfma_main(a)
    else:
        summarize_main(a)


if __name__ == "__main__":
    main()
