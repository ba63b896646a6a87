"""Pins for the CPU oracle: values and properties fixed by the pages and by
mathematics, independent of the oracle's own formulas.

Cited definitions (SpAtten, paperlayer.ai summary of arXiv 2012.09852):
attention = section II "Attention mechanism"; token importance = column
sums of probabilities ("B. Motivation", "A. Cascade Token Pruning"); head
importance = cumulative |attention output| (section II "Cascade pruning");
top-k = "B. Top-k Engine"; MSB/LSB planes = section III "Progressive
Quantization" and IV "Quantization Support".
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import spatten_ref as R
from oracle.topk_engine import topk_engine, zero_eliminate
from workloads import TINY, make_prefill_inputs, random_scores, scaled

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _sdpa(Q, K, V, causal):
    """torch's attention in fp64 on the CPU (library cross-check)."""
    q = torch.from_numpy(np.asarray(Q, np.float64))[None, None]
    k = torch.from_numpy(np.asarray(K, np.float64))[None, None]
    v = torch.from_numpy(np.asarray(V, np.float64))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    return o[0, 0].numpy()


def _torch_probs(Q, K, causal):
    q = torch.from_numpy(np.asarray(Q, np.float64))
    k = torch.from_numpy(np.asarray(K, np.float64))
    s = q @ k.T / math.sqrt(Q.shape[1])
    if causal:
        s = s.masked_fill(torch.ones_like(s, dtype=torch.bool).triu(1), float("-inf"))
    return torch.softmax(s, dim=-1).numpy(), torch.logsumexp(s, dim=-1).numpy()


# ----------------------------------------------------------------- bf16


def test_bf16_golden():
    for c in _gold("bf16_ties.json")["cases"]:
        assert R.bf16_round(c["x"]) == c["r"], c


def test_bf16_matches_torch_cast_on_fp32_inputs():
    rng = np.random.default_rng(1)
    a = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(2000) * 1e-39]).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(R.bf16_round(a.astype(np.float64)), ref)


# ----------------------------------------------------------------- attention


def test_attention_golden_two_tokens():
    g = _gold("attention_2tok.json")
    Q, K, V = (np.array(g[k]) for k in ("Q", "K", "V"))
    for mode, causal in (("bidirectional", False), ("causal", True)):
        O, col, lse = R.head_attention(Q, K, V, causal)
        np.testing.assert_allclose(O, g[mode]["O"], atol=1e-12)
        np.testing.assert_allclose(col, g[mode]["colsum"], atol=1e-12)
        np.testing.assert_allclose(lse, g[mode]["lse"], atol=1e-12)
        assert abs(np.abs(O).sum() - g[mode]["abs_o_sum"]) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,dh", [(1, 8), (7, 4), (37, 16), (130, 32)])
def test_attention_vs_torch_sdpa(n, dh, causal):
    rng = np.random.default_rng(n * 100 + dh)
    Q, K, V = (rng.standard_normal((n, dh)) * 2 for _ in range(3))
    O, col, lse = R.head_attention(Q, K, V, causal, row_block=16)
    np.testing.assert_allclose(O, _sdpa(Q, K, V, causal), rtol=1e-12, atol=1e-12)
    P, L = _torch_probs(Q, K, causal)
    np.testing.assert_allclose(col, P.sum(axis=0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, L, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)


def test_attention_brute_force_loops():
    rng = np.random.default_rng(5)
    for n, dh in ((1, 1), (3, 2), (8, 4)):
        Q, K, V = (rng.standard_normal((n, dh)) for _ in range(3))
        O, col, _ = R.head_attention(Q, K, V, causal=False)
        for i in range(n):
            e = [math.exp(sum(Q[i, c] * K[j, c] for c in range(dh)) / math.sqrt(dh))
                 for j in range(n)]
            z = sum(e)
            for c in range(dh):
                assert abs(O[i, c] - sum(e[j] / z * V[j, c] for j in range(n))) < 1e-12


def test_attention_closed_forms():
    rng = np.random.default_rng(6)
    n, dh = 23, 8
    K, V = rng.standard_normal((n, dh)), rng.standard_normal((n, dh))
    Z = np.zeros((n, dh))
    # Q = 0: uniform probabilities; bidirectional column sums are n_q / n = 1
    O, col, lse = R.head_attention(Z, K, V, causal=False)
    np.testing.assert_allclose(O, np.tile(V.mean(axis=0), (n, 1)), atol=1e-12)
    np.testing.assert_allclose(col, 1.0, atol=1e-12)
    np.testing.assert_allclose(lse, math.log(n), atol=1e-12)
    # causal, Q = 0: row i is uniform over j <= i, so column j sums to H_n - H_j
    O, col, _ = R.head_attention(Z, K, V, causal=True)
    harm = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    np.testing.assert_allclose(col, harm[n] - harm[np.arange(n)], atol=1e-12)
    np.testing.assert_allclose(O[0], V[0], atol=1e-12)           # causal row 0 sees only key 0
    # n = 1: O = V
    O, col, _ = R.head_attention(K[:1], K[:1], V[:1], causal=False)
    np.testing.assert_allclose(O, V[:1], atol=1e-15)
    np.testing.assert_allclose(col, [1.0], atol=1e-15)


def test_attention_permutation_equivariance():
    rng = np.random.default_rng(7)
    n, dh = 19, 8
    Q, K, V = (rng.standard_normal((n, dh)) for _ in range(3))
    perm = rng.permutation(n)
    O, col, _ = R.head_attention(Q, K, V, causal=False)
    O2, col2, _ = R.head_attention(Q[perm], K[perm], V[perm], causal=False)
    np.testing.assert_allclose(O2, O[perm], atol=1e-12)
    np.testing.assert_allclose(col2, col[perm], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_rows_and_column_sums_vs_torch(causal):
    rng = np.random.default_rng(11)
    n, dh = 97, 16
    Q, K, V = (rng.standard_normal((n, dh)) * 2 for _ in range(3))
    P, L = _torch_probs(Q, K, causal)
    rows = np.array([0, 1, 31, 32, 64, 96])
    O, lse = R.attention_rows(Q, K, V, rows, causal)
    np.testing.assert_allclose(O, P[rows] @ V, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, L[rows], rtol=1e-12, atol=1e-12)
    cols = np.array([0, 5, 63, 95, 96])
    np.testing.assert_allclose(R.column_sums(Q, K, L, cols, causal), P[:, cols].sum(axis=0),
                               rtol=1e-12, atol=1e-12)
    # every row's probabilities sum to one, so all columns add up to n
    assert abs(R.column_sums(Q, K, L, np.arange(n), causal).sum() - n) < 1e-9


def test_attention_rows_and_column_sums_closed_forms():
    rng = np.random.default_rng(12)
    n, dh = 41, 8
    K, V = rng.standard_normal((n, dh)), rng.standard_normal((n, dh))
    Z = np.zeros((n, dh))
    rows = np.array([0, 7, 40])
    # causal, Q = 0: row i averages V over keys 0..i and has LSE log(i + 1)
    O, lse = R.attention_rows(Z, K, V, rows, causal=True)
    for t, i in enumerate(rows):
        np.testing.assert_allclose(O[t], V[:i + 1].mean(axis=0), atol=1e-12)
    np.testing.assert_allclose(lse, np.log(rows + 1.0), atol=1e-12)
    # column j then sums 1/(i+1) over i >= j: H_n - H_j
    cols = np.array([0, 3, 40])
    harm = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    got = R.column_sums(Z, K, np.log(np.arange(n) + 1.0), cols, causal=True)
    np.testing.assert_allclose(got, harm[n] - harm[cols], atol=1e-12)
    # bidirectional, Q = 0: every column sums to exactly one
    np.testing.assert_allclose(R.column_sums(Z, K, np.full(n, math.log(n)), cols, causal=False),
                               1.0, atol=1e-12)


# ----------------------------------------------------------------- layer


def _tiny_weights(D, rng):
    return {k: rng.standard_normal((D, D)) / math.sqrt(D) for k in ("wq", "wk", "wv", "wo")}


@pytest.mark.parametrize("causal", [False, True])
def test_layer_matches_torch_dense_mha(causal):
    rng = np.random.default_rng(8)
    n, H, dh = 29, 4, 8
    D = H * dh
    x = rng.standard_normal((n, D))
    w = _tiny_weights(D, rng)
    xn, dcol, dg, _ = R.prefill_layer(x, w, range(H), dh, causal, bf16=False)
    # the same layer through torch: per-head SDPA, concatenate, project
    t = {k: torch.from_numpy(v) for k, v in w.items()}
    tx = torch.from_numpy(x)
    q = (tx @ t["wq"]).reshape(n, H, dh).transpose(0, 1).contiguous()
    k = (tx @ t["wk"]).reshape(n, H, dh).transpose(0, 1).contiguous()
    v = (tx @ t["wv"]).reshape(n, H, dh).transpose(0, 1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    ref = tx + o.transpose(0, 1).reshape(n, D) @ t["wo"]
    np.testing.assert_allclose(xn, ref.numpy(), rtol=1e-11, atol=1e-11)
    assert abs(dcol.sum() - H * n) < 1e-9                        # each row sums to 1
    gref = o.abs().sum(dim=(1, 2)).numpy()
    np.testing.assert_allclose([dg[h] for h in range(H)], gref, rtol=1e-12)


def test_layer_q_zero_closed_form_and_kept_heads():
    rng = np.random.default_rng(9)
    n, H, dh = 17, 4, 8
    D = H * dh
    x = rng.standard_normal((n, D))
    w = _tiny_weights(D, rng)
    w["wq"] = np.zeros((D, D))
    heads = [1, 3]
    _, dcol, dg, _ = R.prefill_layer(x, w, heads, dh, False, bf16=False)
    np.testing.assert_allclose(dcol, len(heads), atol=1e-12)      # h * n_q / n per column
    assert sorted(dg) == heads
    _, dcol, _, _ = R.prefill_layer(x, w, heads, dh, True, bf16=False)
    harm = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    np.testing.assert_allclose(dcol, len(heads) * (harm[n] - harm[np.arange(n)]), atol=1e-12)


def test_layer_constant_v_head_importance():
    rng = np.random.default_rng(10)
    n, H, dh = 11, 2, 4
    D = H * dh
    row = rng.standard_normal(D)
    x = np.tile(row, (n, 1))                                     # identical rows
    w = _tiny_weights(D, rng)
    _, _, dg, _ = R.prefill_layer(x, w, range(H), dh, False, bf16=False)
    v = row @ w["wv"]
    for h in range(H):
        assert abs(dg[h] - n * np.abs(v[h * dh:(h + 1) * dh]).sum()) < 1e-10


def test_layer_bf16_storage_points_are_bf16():
    rng = np.random.default_rng(11)
    n, H, dh = 9, 2, 8
    D = H * dh
    x = R.bf16_round(rng.standard_normal((n, D)))
    w = {k: R.bf16_round(v) for k, v in _tiny_weights(D, rng).items()}
    xn, _, _, _ = R.prefill_layer(x, w, range(H), dh, False, bf16=True)
    np.testing.assert_array_equal(xn, R.bf16_round(xn))


# ----------------------------------------------------------------- top-k


def test_topk_golden():
    g = _gold("topk_ties.json")
    s = np.array(g["scores"], dtype=np.float32)
    for c in g["cases"]:
        idx = R.topk(s, c["k"])
        assert idx.tolist() == c["idx"]
        kv = R.kth_value(s, c["k"])
        assert kv == c["kth"] and math.copysign(1.0, kv) == math.copysign(1.0, c["kth"])
        assert topk_engine(s, c["k"]).tolist() == c["idx"]


def _ranks_above(a, i, j):
    """True if element i outranks element j: larger value, -0.0 below +0.0,
    equal values broken by lower index. Uses float comparisons only."""
    vi, vj = float(a[i]), float(a[j])
    if vi != vj:
        return vi > vj
    si, sj = math.copysign(1.0, vi), math.copysign(1.0, vj)
    if si != sj:
        return si > sj
    return i < j


def test_topk_brute_force_subsets():
    rng = np.random.default_rng(12)
    for trial in range(60):
        n = int(rng.integers(1, 10))
        kind = ["normal", "ties", "signed_zero"][trial % 3]
        a = random_scores(n, seed=trial, kind=kind)
        for k in range(1, n + 1):
            valid = [S for S in itertools.combinations(range(n), k)
                     if all(_ranks_above(a, i, j) for i in S for j in range(n) if j not in S)]
            assert len(valid) == 1
            assert R.topk(a, k).tolist() == list(valid[0])


@pytest.mark.parametrize("kind", ["normal", "ties", "signed_zero", "uniform"])
def test_topk_matches_engine_and_properties(kind):
    rng = np.random.default_rng(13)
    for trial in range(12):
        n = int(rng.integers(1, 300))
        a = random_scores(n, seed=100 + trial, kind=kind)
        for k in sorted({1, n, int(rng.integers(1, n + 1))}):
            idx = R.topk(a, k)
            assert idx.tolist() == topk_engine(a, k).tolist()
            assert len(idx) == k and np.all(np.diff(idx) > 0)
            rest = np.setdiff1d(np.arange(n), idx)
            if len(rest):
                key = R.order_key(a)
                assert key[idx].min() >= key[rest].max()


def test_zero_eliminator_keeps_order():
    rng = np.random.default_rng(14)
    for n in (1, 2, 5, 16, 33, 100):
        keep = rng.random(n) < 0.4
        assert zero_eliminate(list(range(n)), keep) == list(np.flatnonzero(keep))


def test_order_key_monotone():
    vals = np.array([-np.inf, -3.0, -1e-40, -0.0, 0.0, 1e-40, 2.0, np.inf], dtype=np.float32)
    k = R.order_key(vals)
    assert np.all(np.diff(k) > 0)


def test_compact_is_fancy_indexing():
    a = np.arange(30).reshape(10, 3)
    idx = np.array([1, 4, 9])
    np.testing.assert_array_equal(R.compact(a, idx), a[[1, 4, 9]])
    np.testing.assert_array_equal(R.compact(a, np.arange(10)), a)


# ----------------------------------------------------------------- quantizer


def test_quantize_golden_rows():
    for row in _gold("quantize_rows.json")["rows"]:
        x = np.array(row["x"], dtype=np.float32)[None]
        q, s = R.quantize_rows(x)
        assert float(s[0]) == row["scale"]
        assert q[0].tolist() == row["q"]
        msb, lsb = R.split_planes(q[0])
        assert msb.tolist() == row["msb"] and lsb.tolist() == row["lsb"]
        pm, pl, ps = R.quantize_kv(x)
        assert pm[0].tolist() == row["msb_bytes"] and pl[0].tolist() == row["lsb_bytes"]


def test_nibble_round_trip_exhaustive():
    q = np.arange(-128, 128, dtype=np.int16).astype(np.int8)
    msb, lsb = R.split_planes(q)
    assert np.all((msb >= -8) & (msb <= 7)) and np.all((lsb >= 0) & (lsb <= 15))
    np.testing.assert_array_equal(16 * msb.astype(np.int32) + lsb.astype(np.int32), q.astype(np.int32))
    # packing: every pair of codes survives pack/unpack
    a, b = np.meshgrid(q, q)
    pairs = np.stack([a.ravel(), b.ravel()], axis=1)
    m, l = R.split_planes(pairs)
    um = R.unpack_nibbles(R.pack_nibbles(m), signed=True)
    ul = R.unpack_nibbles(R.pack_nibbles(l), signed=False)
    np.testing.assert_array_equal(16 * um + ul, pairs.astype(np.int16))


def test_quantizer_error_bound_and_extremes():
    rng = np.random.default_rng(15)
    x = (rng.standard_normal((500, 64)) * rng.random((500, 1)) * 10).astype(np.float32)
    q, s = R.quantize_rows(x)
    err = np.abs(x.astype(np.float64) - s[:, None].astype(np.float64) * q)
    assert np.all(err <= s[:, None].astype(np.float64) * 0.5 * (1 + 1e-6))
    amax_at = np.argmax(np.abs(x), axis=1)
    np.testing.assert_array_equal(np.abs(q[np.arange(500), amax_at]), 127)
    assert q.min() >= -127


# ----------------------------------------------------------------- progressive quantization


def test_pq_threshold_extremes():
    rng = np.random.default_rng(16)
    Lc, dh = 57, 16
    K = rng.standard_normal((Lc, dh)).astype(np.float32)
    V = rng.standard_normal((Lc, dh)).astype(np.float32)
    km, kl, ks = R.quantize_kv(K)
    vm, vl, vs = R.quantize_kv(V)
    Km, Kf = R.dequant(km, kl, ks, False), R.dequant(km, kl, ks, True)
    Vm, Vf = R.dequant(vm, vl, vs, False), R.dequant(vm, vl, vs, True)
    # full dequantisation is exactly scale * int8 code
    q8, s8 = R.quantize_rows(K)
    np.testing.assert_array_equal(Kf, q8.astype(np.float64) * s8[:, None].astype(np.float64))
    q = rng.standard_normal(dh) * 2
    o, p, rec, _ = R.pq_head_attention(q, Km, Kf, Vm, Vf, threshold=0.0)
    assert not rec
    np.testing.assert_allclose(o, _sdpa(q[None], Km, Vm, False)[0], atol=1e-12)
    o, p, rec, _ = R.pq_head_attention(q, Km, Kf, Vm, Vf, threshold=1.01)
    assert rec
    np.testing.assert_allclose(o, _sdpa(q[None], Kf, Vf, False)[0], atol=1e-12)
    np.testing.assert_allclose(p.sum(), 1.0, atol=1e-12)


# ----------------------------------------------------------------- stacks


def test_run_prefill_keep_all_equals_repeated_dense_layers():
    cfg = scaled(TINY, tokens=(64, 64), heads=(4, 4))
    inp = make_prefill_inputs(cfg)
    out = R.run_prefill(cfg, inp)[0]
    x = inp["x"][0].astype(np.float64)
    for l in range(2):
        x, _, _, _ = R.prefill_layer(x, inp["layers"][l], range(4), 32, False, False)
    np.testing.assert_allclose(out["x"], x, atol=1e-12)
    np.testing.assert_array_equal(out["pos"], np.arange(64))
    assert abs(out["a"].sum() - 2 * 4 * 64) < 1e-9


def test_run_prefill_tiny_cascade_invariants():
    cfg = TINY
    inp = make_prefill_inputs(cfg)
    out = R.run_prefill(cfg, inp)[0]
    t0, t1 = out["trace"]
    assert abs(t0["a"].sum() - 4 * 64) < 1e-9
    sel = t0["sel"]
    assert len(sel) == 32 and np.all(np.diff(sel) > 0)
    np.testing.assert_array_equal(t1["pos"], sel)
    # layer-2 mass = kept layer-1 mass + heads * kept queries
    assert abs(out["a"].sum() - (t0["a"][sel].sum() + 4 * 32)) < 1e-9
    # the kept tokens are the 32 largest of layer-1 importance
    rest = np.setdiff1d(np.arange(64), sel)
    assert t0["a"][sel].min() >= t0["a"][rest].max()


def test_run_prefill_head_cut():
    cfg = scaled(TINY, n_layers=3, tokens=(48, 40, 32), heads=(4, 4, 2))
    inp = make_prefill_inputs(cfg)
    out = R.run_prefill(cfg, inp)[0]
    t1 = out["trace"][1]
    heads = out["trace"][2]["heads"]
    assert len(heads) == 2 and np.all(np.diff(heads) > 0)
    rest = np.setdiff1d(np.arange(4), heads)
    assert t1["g"][heads].min() >= t1["g"][rest].max()


def test_run_decode_small_invariants():
    from workloads import GPT2_DECODE, make_decode_inputs
    cfg = scaled(GPT2_DECODE, n_layers=2, batch=2, n_heads=2, head_dim=8, cache_len=20,
                 cache_keep=8, steps=3)
    inp = make_decode_inputs(cfg)
    out = R.run_decode(cfg, inp)
    for b in range(2):
        o = out[b]
        assert o["x_steps"].shape == (3, 16)
        assert len(o["sel"]) == 8 and np.all(np.diff(o["sel"]) > 0)
        # every step adds heads x layers probability mass; step 1 mass is 2x2
        # over 21 entries, then compaction keeps part of it
        assert o["a"].shape == (8 + 2,)


def test_run_decode_pq_threshold_zero_never_recomputes():
    from workloads import PQ_DECODE, make_decode_inputs
    cfg = scaled(PQ_DECODE, n_layers=1, batch=1, n_heads=2, head_dim=8, cache_len=16,
                 cache_keep=8, steps=2, pq_threshold=0.0)
    out = R.run_decode(cfg, make_decode_inputs(cfg))[0]
    assert not any(r.any() for step in out["recompute"] for r, _ in step)
    cfg2 = scaled(cfg, pq_threshold=1.01)
    out2 = R.run_decode(cfg2, make_decode_inputs(cfg2))[0]
    assert all(r.all() for step in out2["recompute"] for r, _ in step)


def test_stack_amplifies_one_ulp_perturbation():
    """The synthetic random-weight stack is chaotic: one bf16 step on one
    input element grows by orders of magnitude within a few layers. This is
    why stack parity is checked layer by layer on identical inputs."""
    from workloads import BERT_BASE
    cfg = scaled(BERT_BASE, batch=1, n_layers=6, tokens=(512,) * 6, heads=(12,) * 6)
    inp = make_prefill_inputs(cfg)
    base = R.run_prefill(cfg, inp)[0]
    x2 = inp["x"].copy()
    x2[0, 5, 7] = np.float32(R.bf16_round(x2[0, 5, 7] * (1 + 2.0 ** -7)))
    pert = R.run_prefill(cfg, dict(inp, x=x2))[0]

    def nrmse(l):
        a, b = base["trace"][l]["x"], pert["trace"][l]["x"]
        return np.sqrt(np.mean((a - b) ** 2) / np.mean(a * a))
    assert nrmse(0) < 1e-3
    assert nrmse(5) > 100 * nrmse(0)


# ----------------------------------------------------------------- local value pruning
# (section III "Local Value Pruning": after the softmax, low-probability V
# vectors are dropped for the current head only)


def test_value_pruning_one_hot_values_expose_each_probability():
    """With V = I (one V row per output dim) o_j is p_j when row j is kept
    and 0 otherwise, so a wrong pairing of p with V rows, a wrong comparison
    or renormalisation shows up entry by entry. Thresholds at the m-th
    largest probability keep exactly m rows."""
    rng = np.random.default_rng(31)
    n = 24
    q = rng.standard_normal(16) * 2
    K = rng.standard_normal((n, 16))
    p, _ = _torch_probs(q[None], K, False)
    p = p[0]
    order = np.sort(p)[::-1]
    assert np.all(np.diff(order) < 0)
    for m in (1, 5, 12, 24):
        tau = order[m - 1]
        o, kept = R.value_pruned_output(p, np.eye(n), tau)
        assert kept == m
        ref = np.where(p >= tau, p, 0.0)
        np.testing.assert_array_equal(o, ref)
        assert o.sum() <= 1.0 + 1e-15


def test_value_pruning_threshold_extremes_and_uniform_rows():
    rng = np.random.default_rng(32)
    n, dh = 40, 8
    q = rng.standard_normal(dh)
    K, V = rng.standard_normal((n, dh)), rng.standard_normal((n, dh))
    p, _ = _torch_probs(q[None], K, False)
    o, kept = R.value_pruned_output(p[0], V, 0.0)
    assert kept == n
    np.testing.assert_allclose(o, _sdpa(q[None], K, V, False)[0], atol=1e-13)
    o, kept = R.value_pruned_output(p[0], V, 1.01)
    assert kept == 0 and np.all(o == 0.0)
    # q = 0: every probability is exactly 1/8
    p0 = R.softmax_rows(np.zeros((1, 8)))[0]
    V8 = V[:8]
    o, kept = R.value_pruned_output(p0, V8, 0.125)
    assert kept == 8
    np.testing.assert_allclose(o, V8.mean(axis=0), atol=1e-15)
    o, kept = R.value_pruned_output(p0, V8, 0.125 * (1 + 2.0 ** -40))
    assert kept == 0


def test_run_decode_value_pruning_leaves_importance_whole():
    """Token importance takes every probability, so one layer's importance
    is the same with and without value pruning while its output is not;
    every layer still adds H to the total importance."""
    from workloads import GPT2_DECODE, make_decode_inputs
    cfg = scaled(GPT2_DECODE, n_layers=1, batch=1, n_heads=3, head_dim=8, cache_len=30,
                 cache_keep=31, steps=1)
    inp = make_decode_inputs(cfg)
    dense = R.run_decode(cfg, inp)[0]
    vp = R.run_decode(scaled(cfg, v_threshold=0.02), inp)[0]
    np.testing.assert_array_equal(vp["a"], dense["a"])
    assert abs(vp["a"].sum() - 3) < 1e-12
    assert np.all(dense["v_kept"] == 31)
    assert np.all(vp["v_kept"] < 31) and np.all(vp["v_kept"] >= 1)
    assert np.max(np.abs(vp["x_steps"] - dense["x_steps"])) > 1e-6
    cfg3 = scaled(cfg, n_layers=3, v_threshold=0.02)
    out = R.run_decode(cfg3, make_decode_inputs(cfg3))[0]
    assert abs(out["a"].sum() - 3 * 3) < 1e-12


# ----------------------------------------------------------------- repeated decode cascade


def test_prune_schedule():
    from workloads import GPT2_DECODE
    once = GPT2_DECODE
    every = scaled(GPT2_DECODE, prune_every=1)
    third = scaled(GPT2_DECODE, prune_every=3)
    assert [R.prune_after_step(once, s) for s in range(7)] == [True] + [False] * 6
    assert all(R.prune_after_step(every, s) for s in range(7))
    assert [R.prune_after_step(third, s) for s in range(7)] == [True, False, False, True,
                                                               False, False, True]


@pytest.mark.parametrize("every", [1, 2])
def test_run_decode_rolling_cut_keeps_the_largest(every):
    """After each cut the cache holds cache_keep entries: the largest by
    importance among the entries kept so far plus the new ones (checked by
    brute force over the candidates), each id at most once, and a pruned
    entry never comes back."""
    from workloads import GPT2_DECODE, make_decode_inputs
    cfg = scaled(GPT2_DECODE, n_layers=2, batch=1, n_heads=2, head_dim=8, cache_len=20,
                 cache_keep=9, steps=6, prune_every=every)
    out = R.run_decode(cfg, make_decode_inputs(cfg))[0]
    gone = set()
    for s, (ids_pre, a_pre) in enumerate(out["before_prune"]):
        ids = out["kept_ids"][s]
        assert len(set(ids.tolist())) == len(ids)
        assert not (set(ids.tolist()) & gone)
        if R.prune_after_step(cfg, s):
            assert len(ids) == 9
            keep = np.isin(ids_pre, ids)
            assert keep.sum() == 9
            assert a_pre[keep].astype(np.float32).min() >= a_pre[~keep].astype(np.float32).max()
            gone |= set(ids_pre[~keep].tolist())
        else:
            np.testing.assert_array_equal(ids, ids_pre)
    if every == 1:
        assert all(len(k) == 9 for k in out["kept_ids"])


def test_run_decode_rolling_without_cuts_is_the_dense_run():
    """A keep budget at least the final cache length never cuts, so the
    rolling schedule reproduces the plain run that never prunes."""
    from workloads import GPT2_DECODE, make_decode_inputs
    cfg = scaled(GPT2_DECODE, n_layers=2, batch=1, n_heads=2, head_dim=8, cache_len=12,
                 cache_keep=12 + 4, steps=4)
    inp = make_decode_inputs(cfg)
    plain = R.run_decode(cfg, inp)[0]
    roll = R.run_decode(scaled(cfg, prune_every=1), inp)[0]
    np.testing.assert_array_equal(roll["x_steps"], plain["x_steps"])
    np.testing.assert_array_equal(roll["kept_ids"][-1], np.arange(16))


# ----------------------------------------------------------------- per-head token pruning
# (page section VI "Token Pruning": per-head token pruning; reading: in
# decode each head keeps its own cache entries by its own importance)


def _small_decode(**kw):
    from workloads import GPT2_DECODE
    base = dict(n_layers=2, batch=1, n_heads=2, head_dim=8, cache_len=20, cache_keep=9, steps=4)
    base.update(kw)
    return scaled(GPT2_DECODE, **base)


def test_per_head_with_one_head_is_the_shared_cut():
    from workloads import make_decode_inputs
    cfg = _small_decode(n_heads=1, head_dim=16, prune_every=1)
    inp = make_decode_inputs(cfg)
    shared = R.run_decode(cfg, inp)[0]
    ph = R.run_decode(scaled(cfg, per_head=True), inp)[0]
    np.testing.assert_array_equal(ph["x_steps"], shared["x_steps"])
    np.testing.assert_array_equal(ph["a"][0], shared["a"])
    for k1, k2 in zip(ph["kept_ids"], shared["kept_ids"]):
        np.testing.assert_array_equal(k1[0], k2)


def test_per_head_with_identical_heads_is_the_shared_cut():
    """Two heads with identical weights and caches see identical
    probabilities: each head's importance is half the shared one (exact in
    binary), so every head keeps the shared selection and the outputs
    match."""
    from workloads import make_decode_inputs
    cfg = _small_decode(n_heads=2, head_dim=8, prune_every=2)
    inp = make_decode_inputs(cfg)
    dh = 8
    for L in inp["layers"]:
        for name in ("wq", "wk", "wv"):
            L[name][:, dh:] = L[name][:, :dh]
        L["wo"][dh:, :] = L["wo"][:dh, :]
        for name in ("k_cache", "v_cache"):
            L[name][:, :, 1] = L[name][:, :, 0]
    shared = R.run_decode(cfg, inp)[0]
    ph = R.run_decode(scaled(cfg, per_head=True), inp)[0]
    np.testing.assert_array_equal(ph["x_steps"], shared["x_steps"])
    for k1, k2 in zip(ph["kept_ids"], shared["kept_ids"]):
        np.testing.assert_array_equal(k1[0], k2)
        np.testing.assert_array_equal(k1[1], k2)


def test_per_head_cut_keeps_each_heads_largest():
    from workloads import make_decode_inputs
    cfg = _small_decode(n_heads=3, head_dim=8, prune_every=1, steps=5, per_head=True)
    out = R.run_decode(cfg, make_decode_inputs(cfg))[0]
    differ = False
    for s, (ids_pre, a_pre) in enumerate(out["before_prune"]):
        assert ids_pre.shape[0] == 3
        if s == 0:
            # before the first cut every head holds L0 + 1 entries whose
            # importance adds up to one per layer
            np.testing.assert_allclose(a_pre.sum(axis=1), [2.0] * 3, atol=1e-12)
        ids = out["kept_ids"][s]
        for h in range(3):
            keep = np.isin(ids_pre[h], ids[h])
            assert keep.sum() == 9 and len(set(ids[h].tolist())) == 9
            assert (a_pre[h][keep].astype(np.float32).min()
                    >= a_pre[h][~keep].astype(np.float32).max())
        differ |= not (np.array_equal(ids[0], ids[1]) and np.array_equal(ids[1], ids[2]))
    assert differ, "heads never chose different entries"
