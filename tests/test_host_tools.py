"""Host-side tools, no GPU: the benchmark's algorithmic-work accounting
against totals worked out independently from the workload definitions
(projection and attention FLOPs of the prefill stacks, cache and weight
bytes of the decode passes, the per-step cache lengths), and the counter
and kernel-trace summarisers on synthetic profiler output."""
import csv
import json
import os

import pytest

import bench
from cascade_token_head_amd import traffic
from workloads.configs import BY_NAME


def _sums(w):
    return ({k: v[0] for k, v in w.items()}, {k: v[1] for k, v in w.items()})


def test_prefill_work_matches_the_workload_totals():
    # bert_base: 617 GF of projections (8 B n_l h_l dh D per layer) and
    # 163 GF of attention (4 h dh per kept pair, every pair)
    fl, _ = _sums(bench._kernel_work(BY_NAME["bert_base"]))
    assert fl["qkv_gemm"] + fl["out_gemm"] == pytest.approx(617e9, rel=2e-3)
    assert fl["attn_fwd"] == pytest.approx(163e9, rel=2e-3)
    assert fl["attn_colsum"] == pytest.approx(fl["attn_fwd"] / 2)
    # long_causal: 6.9 TF of projections, 10.0 TF of causal attention
    # (unmasked pairs n (n + 1) / 2)
    fl, _ = _sums(bench._kernel_work(BY_NAME["long_causal"]))
    assert fl["qkv_gemm"] + fl["out_gemm"] == pytest.approx(6.87e12, rel=5e-3)
    assert fl["attn_fwd"] == pytest.approx(10.03e12, rel=5e-3)
    # layer 1 alone: 8.8 TF of attention
    n, h, dh = 32768, 32, 128
    assert 4.0 * h * dh * n * (n + 1) / 2 == pytest.approx(8.8e12, rel=5e-3)


def test_decode_cache_lengths():
    """Step 1 attends over the prior cache plus its own entry; the cut after
    step 1 keeps cache_keep, and later steps add one entry each (a rolling
    cascade cuts back after every step)."""
    g = BY_NAME["gpt2_decode"]
    lens = bench._cache_lengths(g)
    assert lens[0] == 1025 and lens[1:] == [410 + s for s in range(1, 32)]
    q = BY_NAME["pq_decode"]
    lens = bench._cache_lengths(q)
    assert lens[0] == 2049 and lens[1:] == [1024 + s for s in range(1, 32)]
    r = bench._cache_lengths(BY_NAME["gpt2_decode_rolling"])
    assert r[0] == 1025 and set(r[1:]) == {411}


def test_decode_bytes_match_the_workload_totals():
    # gpt2_decode: K and V rows read once per layer and step, plus the
    # weights and the small terms: 35.5 GB for the 32 steps
    _, by = _sums(bench._kernel_work(BY_NAME["gpt2_decode"]))
    assert sum(by.values()) == pytest.approx(35.5e9, rel=1e-2)
    D, B, L = 768, 64, 12
    kv = sum(2 * B * lc * D * 2 for lc in bench._cache_lengths(BY_NAME["gpt2_decode"])) * L
    assert by["decode_attn"] == kv
    # pq_decode: MSB planes, scales and weights, 20.1 GB; a recomputed row
    # adds the LSB halves, 13.5 GB if every row were recomputed
    cfg = BY_NAME["pq_decode"]
    _, b0 = _sums(bench._kernel_work(cfg, recompute_frac=0.0))
    _, b1 = _sums(bench._kernel_work(cfg, recompute_frac=1.0))
    assert sum(b0.values()) == pytest.approx(20.1e9, rel=1e-2)
    assert sum(b1.values()) - sum(b0.values()) == pytest.approx(13.5e9, rel=1e-2)


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_summary_scales_by_the_calibration_kernels(tmp_path):
    """FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by known
    bytes over what the copy kernel read, averaged per launch of the
    kernel, and cross-checked against the triad kernel's scales."""
    mib = 1024
    copy_b = mib << 20
    # the counters read half of the copy's fetched bytes and all of its writes
    _counter_csv(tmp_path / "cf.csv", [
        {"Dispatch_Id": i, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
         "Counter_Value": copy_b / 2 / 1024} for i in range(3)] + [
        {"Dispatch_Id": 9, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
         "Counter_Value": 4}])   # a small copy, ignored
    _counter_csv(tmp_path / "cw.csv", [
        {"Dispatch_Id": i, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE",
         "Counter_Value": copy_b / 1024} for i in range(3)])
    tb = 512 << 20
    _counter_csv(tmp_path / "tf.csv", [
        {"Dispatch_Id": i, "Kernel_Name": "vectorized_elementwise_kernel<4, CUDAFunctor_add<float>>",
         "Counter_Name": "FETCH_SIZE", "Counter_Value": 2 * tb / 2 / 1024} for i in range(3)])
    _counter_csv(tmp_path / "tw.csv", [
        {"Dispatch_Id": i, "Kernel_Name": "vectorized_elementwise_kernel<4, CUDAFunctor_add<float>>",
         "Counter_Name": "WRITE_SIZE", "Counter_Value": tb / 1024} for i in range(3)])
    # two launches of the kernel: 100 and 300 KiB counted fetch, 50 KiB written
    _counter_csv(tmp_path / "kf.csv", [
        {"Dispatch_Id": 1, "Kernel_Name": "decode_bh<1>(args)", "Counter_Name": "FETCH_SIZE",
         "Counter_Value": 100},
        {"Dispatch_Id": 2, "Kernel_Name": "decode_bh<1>(args)", "Counter_Name": "FETCH_SIZE",
         "Counter_Value": 300},
        {"Dispatch_Id": 3, "Kernel_Name": "gemm(args)", "Counter_Name": "FETCH_SIZE",
         "Counter_Value": 7}])
    _counter_csv(tmp_path / "kw.csv", [
        {"Dispatch_Id": d, "Kernel_Name": "decode_bh<1>(args)", "Counter_Name": "WRITE_SIZE",
         "Counter_Value": 50} for d in (1, 2)])

    class A:
        label, workload, kernel_regex = "pq_attn", "synthetic", r"decode_bh<1>"
        fetch, write = str(tmp_path / "kf.csv"), str(tmp_path / "kw.csv")
        copy_fetch, copy_write = str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv")
        triad_fetch, triad_write = str(tmp_path / "tf.csv"), str(tmp_path / "tw.csv")
        copy_mib, triad_mib, command, out = mib, 512, "synthetic", str(tmp_path / "out")
    traffic.summarize_main(A)
    rec = json.load(open(tmp_path / "out" / "pmc_pq_attn_synthetic.json"))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_bytes_per_launch"] == 2 * 200 * 1024
    assert rec["write_bytes_per_launch"] == 50 * 1024
    assert rec["hbm_bytes_per_launch"] == (400 + 50) * 1024
    assert rec["calibration_check"]["fetch_scale_rel_diff"] == 0.0
    assert rec["calibration_check"]["write_scale_rel_diff"] == 0.0
    assert rec["source_sha1"] == traffic.source_sha1("pq_attn")
    assert os.path.exists(tmp_path / "out" / "pmc_pq_attn_synthetic.md")


def test_trace_summary_orders_kernels_by_time(tmp_path):
    path = tmp_path / "stats.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow({"Name": "small_kernel", "Calls": 10, "TotalDurationNs": 1000,
                    "AverageNs": 100, "Percentage": 10, "MinNs": 90, "MaxNs": 110, "StdDev": 1})
        w.writerow({"Name": "big_kernel", "Calls": 3, "TotalDurationNs": 9000,
                    "AverageNs": 3000, "Percentage": 90, "MinNs": 2900, "MaxNs": 3100, "StdDev": 5})

    class A:
        label, workload, stats, top, command = "attn_fwd", "synthetic", str(path), 12, "cmd"
        out, bench_json, kernel_regex = str(tmp_path), None, None
    traffic.trace_main(A)
    text = open(tmp_path / "attn_fwd_synthetic_kernel_trace.md").read()
    assert text.index("big_kernel") < text.index("small_kernel")
    assert "| `big_kernel` | 3 | 3.00 | 2.90 | 3.10 | 90.0% |" in text
    assert "cmd" in text


def test_issue_counter_summary_ratios(tmp_path):
    """SQ counters average over a kernel's dispatches across several pass
    files, and the ratios are quotients of those averages."""
    _counter_csv(tmp_path / "p1.csv", [
        {"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v}
        for d, k, c, v in [
            (1, "attn_fwd_bf16<128, true, 1, 1, false>", "SQ_INSTS_MFMA", 100),
            (2, "attn_fwd_bf16<128, true, 1, 1, false>", "SQ_INSTS_MFMA", 300),
            (1, "attn_fwd_bf16<128, true, 1, 1, false>", "SQ_WAVE_CYCLES", 1000),
            (2, "attn_fwd_bf16<128, true, 1, 1, false>", "SQ_WAVE_CYCLES", 3000),
            (3, "other_kernel", "SQ_INSTS_MFMA", 7)]])
    _counter_csv(tmp_path / "p2.csv", [
        {"Dispatch_Id": d, "Kernel_Name": "attn_fwd_bf16<128, true, 1, 1, false>",
         "Counter_Name": c, "Counter_Value": v}
        for d, c, v in [(4, "SQ_INSTS_VALU", 1400), (5, "SQ_INSTS_VALU", 1400),
                        (4, "SQ_WAIT_INST_ANY", 500), (5, "SQ_WAIT_INST_ANY", 700)]])
    class A:
        name, workload, kernel = "attention", "w", ["attn_fwd=attn_fwd_bf16<128, true"]
        counters = [str(tmp_path / "p1.csv"), str(tmp_path / "p2.csv")]
        command, out = "cmd", str(tmp_path)
    traffic.sq_main(A)
    rec = json.load(open(tmp_path / "sq_attention_w.json"))
    k = rec["kernels"]["attn_fwd"]
    assert k["SQ_INSTS_MFMA"] == 200 and k["SQ_WAVE_CYCLES"] == 2000 and k["SQ_INSTS_VALU"] == 1400
    rt = rec["ratios"]["attn_fwd"]
    assert rt["valu_insts_per_mfma"] == 7.0
    assert rt["wave_cycles_waiting_on_dependencies"] == 0.3
    assert "trans_insts_per_mfma" not in rt      # its counter was not collected
    md = open(tmp_path / "sq_attention_w.md").read()
    assert "| valu_insts_per_mfma | 7.0 |" in md and "cmd" in md
