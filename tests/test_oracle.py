"""Pins for the CPU oracle: values and properties fixed by the pages and by
mathematics, independent of the oracle's own formulas.

Cited definitions (SpAtten, paperlayer.ai summary of arXiv 2012.09852):
attention = section II "Attention mechanism"; token importance = column
sums of probabilities ("B. Motivation", "A. Cascade Token Pruning"); head
importance = cumulative |attention output| (section II "Cascade pruning");
top-k = "B. Top-k Engine"; MSB/LSB planes = "A. Cascade Token Pruning", bullet
"Progressive Quantization", and section IV, bullet "Quantization Support".
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
# ("A. Cascade Token Pruning", bullet "Local Value Pruning": after the softmax, low-probability V
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
# (page section "A. Neural Networks Pruning and Quantization", bullet "Token Pruning": per-head token pruning; reading: in
# decode each head keeps its own cache entries by its own importance)


def _small_decode(**kw):
    from workloads import GPT2_DECODE
    base = dict(n_layers=2, batch=1, n_heads=2, head_dim=8, cache_len=20, cache_keep=9, steps=4)
    base.update(kw)
    return scaled(GPT2_DECODE, **base)


@pytest.mark.parametrize("quantized", [False, True])
def test_per_head_with_one_head_is_the_shared_cut(quantized):
    from workloads import make_decode_inputs
    cfg = _small_decode(n_heads=1, head_dim=16, prune_every=1, quantized=quantized,
                        pq_threshold=0.2 if quantized else 0.0)
    inp = make_decode_inputs(cfg)
    shared = R.run_decode(cfg, inp)[0]
    ph = R.run_decode(scaled(cfg, per_head=True), inp)[0]
    np.testing.assert_array_equal(ph["x_steps"], shared["x_steps"])
    np.testing.assert_array_equal(ph["a"][0], shared["a"])
    for k1, k2 in zip(ph["kept_ids"], shared["kept_ids"]):
        np.testing.assert_array_equal(k1[0], k2)
    for r1, r2 in zip(ph["recompute"], shared["recompute"]):
        for (f1, c1), (f2, c2) in zip(r1, r2):
            np.testing.assert_array_equal(f1, f2)
            np.testing.assert_array_equal(c1, c2)
    if quantized:
        flags = [bool(f.any()) for step in shared["recompute"] for f, _ in step]
        assert any(flags) and not all(flags)  # the case reaches both sides of the threshold


@pytest.mark.parametrize("quantized", [False, True])
def test_per_head_with_identical_heads_is_the_shared_cut(quantized):
    """Two heads with identical weights and caches see identical
    probabilities: each head's importance is half the shared one (exact in
    binary), so every head keeps the shared selection and the outputs
    match."""
    from workloads import make_decode_inputs
    cfg = _small_decode(n_heads=2, head_dim=8, prune_every=2, quantized=quantized,
                        pq_threshold=0.2 if quantized else 0.0)
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


# ----------------------------------------------------------------- generation-mode attention
# (SpAtten page, section II "Attention-based NLP models": generation takes one
# new token per iteration and combines it with the cached keys and values;
# "E. Query-Key Multiplication Module", bullet "Progressive Quantization":
# LSBs are fetched and the probabilities recomputed when the largest
# probability is below the threshold)


def _decode_case(seed, H=3, dh=8, L0=11):
    rng = np.random.default_rng(seed)
    D = H * dh
    w = _tiny_weights(D, rng)
    x = rng.standard_normal(D) * 1.5
    K0 = rng.standard_normal((L0, H, dh))
    V0 = rng.standard_normal((L0, H, dh))
    return w, x, K0, V0


def _torch_decode_reference(w, x, K0, V0, H, dh):
    """The new token's query is the last row of causal attention over the
    old cache followed by the new token itself: torch SDPA in fp64 on
    [cache; new] keys and values, written from the definition with torch's
    own projections (nothing from the oracle)."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    xt = t(x)
    q = (xt @ t(w["wq"])).reshape(H, dh)
    k = (xt @ t(w["wk"])).reshape(1, H, dh)
    v = (xt @ t(w["wv"])).reshape(1, H, dh)
    Kc = torch.cat([t(K0), k], 0)           # [L0+1, H, dh]
    Vc = torch.cat([t(V0), v], 0)
    L = Kc.shape[0]
    # the new token sits at position L-1 of a causal sequence: as the last
    # query it sees every key, so SDPA's causal mask on a full query block
    # gives its row exactly; the other queries are placeholders
    Qfull = torch.zeros(H, L, dh, dtype=torch.float64)
    Qfull[:, L - 1] = q
    o = torch.nn.functional.scaled_dot_product_attention(
        Qfull[None], Kc.permute(1, 0, 2)[None], Vc.permute(1, 0, 2)[None], is_causal=True)[0]
    o = o[:, L - 1]                          # [H, dh]
    p = torch.softmax((Kc.permute(1, 0, 2) @ q[:, :, None])[:, :, 0] / math.sqrt(dh), dim=-1)
    x_new = xt + o.reshape(-1) @ t(w["wo"])
    return x_new.numpy(), p.numpy(), k.numpy(), v.numpy()


def test_decode_layer_is_the_last_row_of_causal_attention_over_cache_and_new_token():
    H, dh = 3, 8
    w, x, K0, V0 = _decode_case(31, H, dh)
    cache = {"k": K0.copy(), "v": V0.copy()}
    x_new, P, rec, _, kept = R.decode_layer(x, w, cache, H, dh, bf16=False, quantized=False,
                                            threshold=0.0)
    x_ref, p_ref, k_ref, v_ref = _torch_decode_reference(w, x, K0, V0, H, dh)
    np.testing.assert_allclose(x_new, x_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(P, p_ref, rtol=1e-12, atol=1e-14)
    # the appended entry is the new token's own key and value, in that order
    assert cache["k"].shape == (K0.shape[0] + 1, H, dh)
    np.testing.assert_allclose(cache["k"][-1], k_ref[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(cache["v"][-1], v_ref[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(cache["k"][:-1], K0)
    np.testing.assert_array_equal(cache["v"][:-1], V0)
    assert not rec.any() and np.all(kept == K0.shape[0] + 1)


def test_decode_attention_zero_query_is_uniform_over_the_cache():
    """q = 0: every score is 0, so p = 1/Lc exactly and o is the mean of
    the cached values (closed form, independent of the score scale)."""
    rng = np.random.default_rng(32)
    H, dh, Lc = 2, 4, 13
    cache = {"k": rng.standard_normal((Lc, H, dh)), "v": rng.standard_normal((Lc, H, dh))}
    O, P, _, _, _ = R.decode_attention(np.zeros((H, dh)), cache, H, dh, False, 0.0)
    np.testing.assert_allclose(P, 1.0 / Lc, rtol=0, atol=1e-16)
    np.testing.assert_allclose(O, cache["v"].mean(axis=0), atol=1e-14)


def test_decode_attention_scale_is_inverse_sqrt_head_dim():
    """Two cached keys whose scores differ by exactly sqrt(dh) * ln 3 under
    q . k: with the 1/sqrt(dh) scale the probabilities are 3/4 and 1/4
    (closed form)."""
    H, dh = 1, 16
    q = np.zeros((H, dh))
    q[0, 0] = 1.0
    K = np.zeros((2, H, dh))
    K[0, 0, 0] = math.sqrt(dh) * math.log(3.0)
    V = np.array([[[1.0] + [0.0] * (dh - 1)], [[0.0] * (dh - 1) + [1.0]]])
    O, P, _, _, _ = R.decode_attention(q, {"k": K, "v": V}, H, dh, False, 0.0)
    np.testing.assert_allclose(P[0], [0.75, 0.25], atol=1e-15)
    np.testing.assert_allclose(O[0, 0], 0.75, atol=1e-15)
    np.testing.assert_allclose(O[0, -1], 0.25, atol=1e-15)


def _quantized_cache(K, V):
    km, kl, ks = R.quantize_kv(K.reshape(K.shape[0], -1).astype(np.float32))
    vm, vl, vs = R.quantize_kv(V.reshape(V.shape[0], -1).astype(np.float32))
    return {"k_msb": km, "k_lsb": kl, "k_scale": ks, "v_msb": vm, "v_lsb": vl, "v_scale": vs}


def test_pq_confidence_exactly_at_threshold_is_not_recomputed():
    """Ten cached keys with identical codes give a uniform MSB-pass row:
    max p = 1/10, which is the double nearest 0.1, the workload's
    threshold. The test is strict (recompute only when max p < threshold),
    so that row keeps its MSB result; just above the threshold it is
    recomputed."""
    rng = np.random.default_rng(33)
    H, dh, Lc = 2, 8, 10
    # integer-valued rows with amax 127 have scale 1 and exact codes, and an
    # integer query makes every score exact in any summation order
    row = rng.integers(-127, 128, H * dh).astype(np.float32)
    row[0] = 127.0
    K = np.tile(row, (Lc, 1)).reshape(Lc, H, dh)
    V = rng.standard_normal((Lc, H, dh)).astype(np.float32)
    cache = _quantized_cache(K, V)
    assert np.all(cache["k_scale"] == 1.0)
    q = rng.integers(-3, 4, (H, dh)).astype(np.float64)
    O, P, rec, cmax, _ = R.decode_attention(q, cache, H, dh, True, 0.1)
    assert np.all(cmax == 0.1), cmax
    assert not rec.any()
    _, _, rec2, _, _ = R.decode_attention(q, cache, H, dh, True, np.nextafter(0.1, 1.0))
    assert rec2.all()


def test_pq_importance_takes_the_probabilities_that_produced_the_output():
    """At a middle threshold one head is confident and one is flat. The flat
    head's returned p and o must be the full-code softmax (both planes),
    the confident head's the MSB-only one; each is checked against torch's
    softmax over values dequantised from the int8 codes directly."""
    rng = np.random.default_rng(34)
    H, dh, Lc = 2, 16, 40
    K = rng.standard_normal((Lc, H, dh)).astype(np.float32)
    V = rng.standard_normal((Lc, H, dh)).astype(np.float32)
    # head 0 sharp (its query aligned with one key), head 1 flat
    q = np.zeros((H, dh))
    q[0] = K[7, 0] * 3.0
    q[1] = rng.standard_normal(dh) * 0.05
    cache = _quantized_cache(K, V)
    q8k, sk = R.quantize_rows(K.reshape(Lc, -1))
    q8v, sv = R.quantize_rows(V.reshape(Lc, -1))
    kf = (q8k.astype(np.float64) * sk[:, None]).reshape(Lc, H, dh)
    vf = (q8v.astype(np.float64) * sv[:, None]).reshape(Lc, H, dh)
    # MSB-only values: the code with its low four bits cleared
    km = ((q8k.astype(np.int16) >> 4) * 16 * sk[:, None].astype(np.float64)).reshape(Lc, H, dh)
    vm = ((q8v.astype(np.int16) >> 4) * 16 * sv[:, None].astype(np.float64)).reshape(Lc, H, dh)

    def tsoft(Kh, qh):
        s = torch.from_numpy(Kh @ qh / math.sqrt(dh))
        return torch.softmax(s, dim=0).numpy()

    p_msb = [tsoft(km[:, h], q[h]) for h in range(H)]
    p_full = [tsoft(kf[:, h], q[h]) for h in range(H)]
    assert p_msb[0].max() > 0.5 and p_msb[1].max() < 0.1
    # the two planes must disagree on the flat head, or the pin is empty
    assert np.max(np.abs(p_full[1] - p_msb[1])) > 1e-4
    O, P, rec, cmax, _ = R.decode_attention(q, cache, H, dh, True, 0.1)
    np.testing.assert_array_equal(rec, [False, True])
    np.testing.assert_allclose(cmax, [p_msb[0].max(), p_msb[1].max()], rtol=1e-12)
    np.testing.assert_allclose(P[0], p_msb[0], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(P[1], p_full[1], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(O[0], p_msb[0] @ vm[:, 0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(O[1], p_full[1] @ vf[:, 1], rtol=1e-12, atol=1e-14)


def test_run_decode_pq_importance_accumulates_recomputed_probabilities():
    """Through the stack: the importance after step 1 (before the cut) is
    the sum over layers and heads of the probabilities that produced each
    head's output; with threshold 1.01 every row is recomputed, so it must
    equal the sum of full-code softmaxes, which differ from MSB-only ones."""
    from workloads import PQ_DECODE, make_decode_inputs
    cfg = scaled(PQ_DECODE, n_layers=1, batch=1, n_heads=2, head_dim=8, cache_len=24,
                 cache_keep=12, steps=1, pq_threshold=1.01)
    inp = make_decode_inputs(cfg)
    out = R.run_decode(cfg, inp)[0]
    _, a_pre = out["before_prune"][0]
    L = inp["layers"][0]
    H, dh = 2, 8
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    x = t(inp["x_steps"][0][0].astype(np.float64))
    q = R.bf16_round((x @ t(L["wq"])).numpy()).reshape(H, dh)
    k = R.bf16_round((x @ t(L["wk"])).numpy())
    Kc = np.concatenate([np.asarray(L["k_cache"][0], np.float64).reshape(24, -1), k[None]], 0)
    q8, s = R.quantize_rows(Kc.astype(np.float32))
    kf = (q8.astype(np.float64) * s[:, None]).reshape(25, H, dh)
    km = ((q8.astype(np.int16) >> 4) * 16 * s[:, None].astype(np.float64)).reshape(25, H, dh)
    want = sum(torch.softmax(t(kf[:, h] @ q[h] / math.sqrt(dh)), 0).numpy() for h in range(H))
    msb = sum(torch.softmax(t(km[:, h] @ q[h] / math.sqrt(dh)), 0).numpy() for h in range(H))
    assert np.max(np.abs(want - msb)) > 1e-4
    np.testing.assert_allclose(a_pre, want, rtol=1e-10, atol=1e-14)


# ----------------------------------------------------------------- value pruning in prefill
# ("A. Cascade Token Pruning", bullet "Local Value Pruning": after the
# softmax, a head drops its low-probability V vectors for the current head;
# reading: for every query row, V row j enters only when P[i, j] >= tau)


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_value_pruning_one_hot_values(causal):
    """V = identity rows: O[i, j] is P[i, j] when it reaches the threshold
    and 0 otherwise, with P from torch's softmax; the column sums keep every
    probability."""
    rng = np.random.default_rng(51)
    n, dh = 24, 32
    Q, K = rng.standard_normal((n, dh)) * 1.5, rng.standard_normal((n, dh)) * 1.5
    V = np.eye(n, dh)
    P, _ = _torch_probs(Q, K, causal)
    for tau in (1e-3, 0.05, 0.2):
        O, col, _ = R.head_attention(Q, K, V, causal, v_threshold=tau)
        np.testing.assert_allclose(O[:, :n], np.where(P >= tau, P, 0.0), atol=1e-14)
        np.testing.assert_allclose(col, P.sum(axis=0), atol=1e-12)
        rows = np.array([0, 5, n - 1])
        Or, _ = R.attention_rows(Q, K, V, rows, causal, v_threshold=tau)
        np.testing.assert_allclose(Or[:, :n], np.where(P[rows] >= tau, P[rows], 0.0), atol=1e-14)


def test_prefill_value_pruning_extremes():
    rng = np.random.default_rng(52)
    n, dh = 17, 8
    Q, K, V = (rng.standard_normal((n, dh)) for _ in range(3))
    # a threshold below every probability keeps torch's attention
    O, _, _ = R.head_attention(Q, K, V, True, v_threshold=1e-300)
    np.testing.assert_allclose(O, _sdpa(Q, K, V, True), atol=1e-12)
    # above one nothing is kept, except nothing: O = 0
    O, col, _ = R.head_attention(Q, K, V, False, v_threshold=1.01)
    np.testing.assert_array_equal(O, 0.0)
    assert abs(col.sum() - n) < 1e-9
    # causal row 0 has p = 1 on key 0, kept for any threshold <= 1
    O, _, _ = R.head_attention(Q, K, V, True, v_threshold=1.0)
    np.testing.assert_allclose(O[0], V[0], atol=1e-15)
    # uniform rows (Q = 0): p = 1/n, kept at tau = 1/n exactly, dropped above
    Z = np.zeros((n, dh))
    O, _, _ = R.head_attention(Z, K, V, False, v_threshold=1.0 / n)
    np.testing.assert_allclose(O, np.tile(V.mean(axis=0), (n, 1)), atol=1e-12)
    O, _, _ = R.head_attention(Z, K, V, False, v_threshold=np.nextafter(1.0 / n, 1.0))
    np.testing.assert_array_equal(O, 0.0)


def test_prefill_layer_value_pruning_head_importance_takes_pruned_output():
    rng = np.random.default_rng(53)
    D, dh, n = 32, 8, 12
    w = _tiny_weights(D, rng)
    x = rng.standard_normal((n, D))
    ex = {}
    _, dcol, dg, _ = R.prefill_layer(x, w, range(4), dh, False, False, extras=ex, v_threshold=0.1)
    _, dcol0, _, _ = R.prefill_layer(x, w, range(4), dh, False, False)
    np.testing.assert_allclose(dcol, dcol0, atol=1e-12)
    for h in range(4):
        P, _ = _torch_probs(ex[h]["q"], ex[h]["k"], False)
        O = np.where(P >= 0.1, P, 0.0) @ ex[h]["v"]
        assert abs(dg[h] - np.abs(O).sum()) < 1e-12


# ----------------------------------------------------------------- per-head token pruning, prefill
# (section "A. Neural Networks Pruning and Quantization", bullet "Token
# Pruning"; reading: each head attends over its own kept tokens as keys and
# values, every token keeps its row and queries every head)


def _perhead_cfg(**kw):
    from workloads.configs import BERT_BASE_PERHEAD
    base = dict(n_layers=3, batch=1, n_heads=3, head_dim=8, tokens=(24,) * 3, heads=(3, 3, 3),
                key_keep=(24, 16, 10), dtype="f32")
    base.update(kw)
    return scaled(BERT_BASE_PERHEAD, **base)


def test_perhead_prefill_keeping_every_key_is_the_dense_stack():
    cfg = _perhead_cfg(key_keep=(24, 24, 24))
    inp = make_prefill_inputs(cfg)
    ph = R.run_prefill_perhead(cfg, inp)[0]
    dense = R.run_prefill(scaled(cfg, per_head=False, key_keep=()), inp)[0]
    np.testing.assert_allclose(ph["x"], dense["x"], atol=1e-12)
    # the summed per-head importance is the shared importance
    np.testing.assert_allclose(sum(ph["a"][h] for h in range(3)), dense["a"], atol=1e-12)


def test_perhead_prefill_layer_matches_torch_attention_over_each_heads_keys():
    rng = np.random.default_rng(61)
    D, dh, n = 24, 8, 15
    w = _tiny_weights(D, rng)
    x = rng.standard_normal((n, D))
    keys = {0: np.array([0, 3, 4, 9, 14]), 1: np.arange(n), 2: np.array([7])}
    ex = {}
    xn, cols, dg = R.perhead_prefill_layer(x, w, [0, 1, 2], keys, dh, False, extras=ex)
    delta = np.zeros((n, D))
    for h in range(3):
        c = slice(h * dh, (h + 1) * dh)
        Q, K, V = x @ w["wq"][:, c], x @ w["wk"][:, c], x @ w["wv"][:, c]
        q = torch.from_numpy(Q)[None, None]
        k = torch.from_numpy(K[keys[h]])[None, None]
        v = torch.from_numpy(V[keys[h]])[None, None]
        O = torch.nn.functional.scaled_dot_product_attention(q, k, v)[0, 0].numpy()
        np.testing.assert_allclose(ex[h]["o"], O, atol=1e-12)
        assert abs(cols[h].sum() - n) < 1e-9          # every query row sums to one
        assert abs(dg[h] - np.abs(O).sum()) < 1e-9
        delta += O @ w["wo"][c, :]
    np.testing.assert_allclose(cols[2], [n], atol=1e-12)   # one key takes all the mass
    np.testing.assert_allclose(ex[2]["o"], np.tile(x[7] @ w["wv"][:, 16:24], (n, 1)), atol=1e-12)
    np.testing.assert_allclose(xn, x + delta, atol=1e-12)


def test_perhead_prefill_cuts_keep_each_heads_largest_and_never_revive():
    cfg = _perhead_cfg(n_layers=4, tokens=(30,) * 4, key_keep=(30, 20, 12, 7), heads=(3, 3, 2, 2))
    out = R.run_prefill_perhead(cfg, make_prefill_inputs(cfg))[0]
    tr = out["trace"]
    differ = False
    for l in range(cfg.n_layers - 1):
        nxt_heads = tr[l + 1]["heads"]
        for h in nxt_heads:
            before, after = tr[l]["keys"][h], tr[l + 1]["keys"][h]
            assert np.all(np.isin(after, before)) and np.all(np.diff(after) > 0)
            a = tr[l]["a"][h][before].astype(np.float32)
            kept = np.isin(before, after)
            assert a[kept].min() >= a[~kept].max()
        ks = [tuple(tr[l + 1]["keys"][h]) for h in nxt_heads]
        differ |= len(set(ks)) > 1
    assert differ, "heads never chose different keys"
    # the head cut before layer 3 keeps the largest cumulative |O|
    g = tr[1]["g"]
    assert len(tr[2]["heads"]) == 2
    rest = np.setdiff1d(tr[1]["heads"], tr[2]["heads"])
    assert g[tr[2]["heads"]].min() >= g[rest].max()


# ------------------------------------------------- closed-form cascades
#
# Inputs under which every query of a head sees the same scores: x[:, 0] = 1
# for every token, Wq is zero outside row 0 and Wo writes nothing into
# column 0, so column 0 stays 1 through every layer and head h's query is
# row 0 of its Wq columns for every token. The score of key j is then a
# function of the key alone, each probability row is one vector softmax
# (bidirectional) or its prefix-normalised form (causal), and the whole
# cascade - importance accumulated over layers, token and head cuts,
# compaction of x, a and positions - has a closed form that never builds a
# score matrix.


def _rank_one_inputs(cfg, seed=0):
    inp = make_prefill_inputs(cfg, seed=seed)
    inp["x"][:, :, 0] = 1.0
    for w in inp["layers"]:
        w["wq"][1:, :] = 0.0
        w["wo"][:, 0] = 0.0
    return inp


def _rank_one_head(e, V, causal):
    """Column sums and output rows of a head whose probability of key j in
    row i is proportional to e_j (keys j <= i when causal).
    Bidirectional: every row is e / sum(e), so column j sums to
    n e_j / sum(e) and every output row is e V / sum(e).
    Causal: row i is e_j / Z_i with Z_i = e_0 + ... + e_i, so column j sums
    to e_j (1/Z_j + ... + 1/Z_{n-1}) and output row i is
    (e_0 V_0 + ... + e_i V_i) / Z_i."""
    n = e.shape[0]
    if not causal:
        Z = e.sum()
        return n * e / Z, np.broadcast_to(e @ V / Z, V.shape)
    Z = np.cumsum(e)
    tail = np.cumsum((1.0 / Z)[::-1])[::-1]
    return e * tail, np.cumsum(e[:, None] * V, axis=0) / Z[:, None]


def _largest(v, k):
    """Indices of the k largest fp32 values (lower index first on ties),
    ascending, by a plain sort."""
    v32 = np.asarray(v, np.float32)
    order = sorted(range(v32.shape[0]), key=lambda j: (-float(v32[j]), j))
    return np.sort(np.array(order[:k], dtype=np.int64))


def _closed_form_cascade(cfg, inp, b):
    dh = cfg.head_dim
    x = inp["x"][b].astype(np.float64)
    n0 = x.shape[0]
    pos, heads = np.arange(n0), np.arange(cfg.n_heads)
    a, g = np.zeros(n0), np.zeros(cfg.n_heads)
    trace = []
    for l in range(cfg.n_layers):
        w = {k_: v_.astype(np.float64) for k_, v_ in inp["layers"][l].items()}
        delta, dcol, dg = np.zeros_like(x), np.zeros(x.shape[0]), np.zeros(cfg.n_heads)
        for h in heads:
            c = slice(h * dh, (h + 1) * dh)
            s = (x @ w["wk"][:, c]) @ w["wq"][0, c] / math.sqrt(dh)
            col, O = _rank_one_head(np.exp(s - s.max()), x @ w["wv"][:, c], cfg.causal)
            dcol += col
            dg[h] = np.abs(O).sum()
            delta += O @ w["wo"][c, :]
        x, a, g = x + delta, a + dcol, g + dg
        rec = {"pos": pos, "heads": heads, "a": a, "g": g, "x": x, "dcol": dcol, "dg": dg}
        if l + 1 < cfg.n_layers:
            if cfg.heads[l + 1] != len(heads):
                heads = heads[_largest(g[heads], cfg.heads[l + 1])]
            keep = _largest(a, cfg.tokens[l + 1])
            x, a, pos = x[keep], a[keep], pos[keep]
        trace.append(rec)
    return trace


@pytest.mark.parametrize("causal", [False, True])
def test_run_prefill_matches_closed_form_cascade(causal):
    cfg = scaled(TINY, n_layers=4, tokens=(40, 30, 22, 16), heads=(4, 4, 3, 2), causal=causal,
                 batch=4)
    inp = _rank_one_inputs(cfg)
    out = R.run_prefill(cfg, inp)
    sensitive_tok = sensitive_head = False
    for b in range(cfg.batch):
        want = _closed_form_cascade(cfg, inp, b)
        got = out[b]["trace"]
        for l, (wr, gr) in enumerate(zip(want, got)):
            np.testing.assert_array_equal(gr["pos"], wr["pos"])
            np.testing.assert_array_equal(gr["heads"], wr["heads"])
            np.testing.assert_allclose(gr["a"], wr["a"], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(gr["g"], wr["g"], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(gr["x"], wr["x"], rtol=1e-10, atol=1e-10)
            if l + 1 < cfg.n_layers:
                k = cfg.tokens[l + 1]
                sensitive_tok |= not np.array_equal(_largest(wr["a"], k),
                                                    _largest(wr["dcol"], k))
                if cfg.heads[l + 1] != len(wr["heads"]):
                    hk = wr["heads"]
                    sensitive_head |= not np.array_equal(
                        _largest(wr["g"][hk], cfg.heads[l + 1]),
                        _largest(wr["dg"][hk], cfg.heads[l + 1]))
    # the case tells cumulative importance from the last layer's alone (a
    # causal layer's column sums fall with position so steeply that its own
    # token ranking already agrees with the cumulative one here)
    assert sensitive_head and (sensitive_tok or causal)


def _uniform_decode(cfg, inp, b):
    """The decode stack in closed form when every query is zero (Wq = 0):
    each head spreads probability 1/Lc over the Lc entries of the cache
    (the new token's entry included), so a layer adds the mean of the cache's
    V rows times Wo, every entry present gains layers x heads / Lc per step
    (layers / Lc per head under per-head pruning), and a cut keeps the entries that have been present longest (ties go to
    the lower cache slot). Quantized caches hold the rows' int8 values;
    a row whose largest probability 1/Lc is below the threshold reads both
    planes, otherwise the MSB plane alone."""
    L0, D = cfg.cache_len, cfg.model_dim
    vals = []
    for l in range(cfg.n_layers):
        V0 = inp["layers"][l]["v_cache"][b].reshape(L0, D)
        vals.append(R.quantize_kv(V0.astype(np.float32)) if cfg.quantized else V0)
    full = []
    a, ids = np.zeros(L0), list(range(L0))
    xs, kept, flat = [], [], []
    for s in range(cfg.steps):
        x = inp["x_steps"][s][b].astype(np.float64)
        ids.append(L0 + s)
        a = np.append(a, 0.0)
        Lc = len(ids)
        use_full = cfg.quantized and 1.0 / Lc < cfg.pq_threshold
        for l in range(cfg.n_layers):
            w = {k_: v_.astype(np.float64) for k_, v_ in inp["layers"][l].items()
                 if k_ in ("wv", "wo")}
            v = x @ w["wv"]
            if cfg.quantized:
                planes = R.quantize_kv(v.astype(np.float32)[None])
                vals[l] = tuple(np.concatenate([p_, n_]) for p_, n_ in zip(vals[l], planes))
                V = R.dequant(*vals[l], use_full)
            else:
                vals[l] = np.concatenate([vals[l], v[None]])
                V = vals[l]
            x = x + V.mean(axis=0) @ w["wo"]
        # per-head pruning: head h's importance takes head h's share only
        a = a + cfg.n_layers * (1 if cfg.per_head else cfg.n_heads) / Lc
        xs.append(x)
        flat.append(use_full)
        if R.prune_after_step(cfg, s) and Lc > cfg.cache_keep:
            keep = _largest(a, cfg.cache_keep)
            a, ids = a[keep], [ids[j] for j in keep]
            vals = [tuple(p_[keep] for p_ in c) if cfg.quantized else c[keep] for c in vals]
        kept.append(np.array(ids))
    return np.stack(xs), a, kept, flat


@pytest.mark.parametrize("variant", ["once", "rolling", "perhead", "pq", "pq_perhead"])
def test_run_decode_matches_zero_query_closed_form(variant):
    from workloads import GPT2_DECODE, PQ_DECODE, make_decode_inputs
    base = PQ_DECODE if variant.startswith("pq") else GPT2_DECODE
    cfg = scaled(base, dtype="f32", n_layers=3, batch=2, n_heads=2, head_dim=8, cache_len=12,
                 cache_keep=7, steps=5, prune_every=1 if variant == "rolling" else 0,
                 per_head=variant.endswith("perhead"))
    inp = make_decode_inputs(cfg)
    for w in inp["layers"]:
        w["wq"][:] = 0.0
    out = R.run_decode(cfg, inp)
    for b in range(cfg.batch):
        xs, a, kept, flat = _uniform_decode(cfg, inp, b)
        o = out[b]
        np.testing.assert_allclose(o["x_steps"], xs, rtol=1e-10, atol=1e-10)
        for s in range(cfg.steps):
            ids = np.asarray(o["kept_ids"][s])
            want = np.broadcast_to(kept[s], ids.shape) if cfg.per_head else kept[s]
            np.testing.assert_array_equal(ids, want)
            if cfg.quantized:
                assert all(bool(r.all()) == flat[s] and bool(r.any()) == flat[s]
                           for r, _ in o["recompute"][s])
        np.testing.assert_allclose(o["a"], np.broadcast_to(a, o["a"].shape), rtol=1e-12)
    if cfg.quantized:
        # the case crosses the threshold: rows of 12 and 13 entries read both
        # planes, the pruned cache of 8 entries only the MSBs
        assert flat[0] and not flat[1]


def test_run_prefill_perhead_matches_closed_form_cascade():
    """Per-head token pruning on the equal-query inputs: head h's rows are
    one softmax over its own keys, so its column sums are n p_h and every
    output row is p_h V[keys_h]; each head's cut keeps its own largest
    cumulative importance, and the head cut ranks cumulative |O_h|."""
    from workloads.configs import BERT_BASE_PERHEAD
    cfg = scaled(BERT_BASE_PERHEAD, dtype="f32", n_layers=4, batch=3, n_heads=4, head_dim=8,
                 tokens=(24,) * 4, key_keep=(24, 17, 12, 9), heads=(4, 4, 3, 2))
    inp = _rank_one_inputs(cfg)
    out = R.run_prefill_perhead(cfg, inp)
    dh, n = cfg.head_dim, cfg.tokens[0]
    differ = False
    for b in range(cfg.batch):
        x = inp["x"][b].astype(np.float64)
        heads = np.arange(cfg.n_heads)
        keys = {h: np.arange(n) for h in heads}
        a = {h: np.zeros(n) for h in heads}
        g = np.zeros(cfg.n_heads)
        for l in range(cfg.n_layers):
            w = {k_: v_.astype(np.float64) for k_, v_ in inp["layers"][l].items()}
            delta = np.zeros_like(x)
            for h in heads:
                c = slice(h * dh, (h + 1) * dh)
                kk = keys[h]
                s = (x[kk] @ w["wk"][:, c]) @ w["wq"][0, c] / math.sqrt(dh)
                e = np.exp(s - s.max())
                p = e / e.sum()
                o = p @ (x[kk] @ w["wv"][:, c])
                a[h][kk] += n * p
                g[h] += n * np.abs(o).sum()
                delta += o @ w["wo"][c, :]
            x = x + delta
            rec = out[b]["trace"][l]
            np.testing.assert_array_equal(rec["heads"], heads)
            np.testing.assert_allclose(rec["x"], x, rtol=1e-10, atol=1e-10)
            np.testing.assert_allclose(rec["g"], g, rtol=1e-10, atol=1e-12)
            for h in heads:
                np.testing.assert_array_equal(rec["keys"][h], keys[h])
                np.testing.assert_allclose(rec["a"][h], a[h], rtol=1e-10, atol=1e-12)
            if l + 1 < cfg.n_layers:
                if cfg.heads[l + 1] != len(heads):
                    heads = heads[_largest(g[heads], cfg.heads[l + 1])]
                for h in heads:
                    keys[h] = keys[h][_largest(a[h][keys[h]], cfg.key_keep[l + 1])]
                differ |= len({tuple(keys[h]) for h in heads}) > 1
    assert differ  # the heads keep different tokens


@pytest.mark.parametrize("threshold,full", [(0.0, False), (1.01, True)])
def test_pq_value_pruning_one_hot_values(threshold, full):
    """Quantized caches: V rows 127 e_j (scale 1, code 127 in one dim) make
    every kept probability show up in its own output element, as 127 p_j
    from both planes (a recomputed row) or 16 * 7 p_j = 112 p_j from the MSB
    plane alone (127 >> 4 = 7); probabilities from torch's softmax of the
    dequantized keys of the pass. A threshold just below the m-th largest
    probability keeps exactly m rows."""
    rng = np.random.default_rng(61)
    H, dh, Lc = 1, 16, 12
    K = rng.standard_normal((Lc, dh)).astype(np.float32)
    V = np.zeros((Lc, dh), np.float32)
    V[np.arange(Lc), np.arange(Lc)] = 127.0
    km, kl, ks = R.quantize_kv(K)
    vm, vl, vs = R.quantize_kv(V)
    np.testing.assert_array_equal(vs, 1.0)
    cache = {"k_msb": km, "k_lsb": kl, "k_scale": ks, "v_msb": vm, "v_lsb": vl, "v_scale": vs}
    q = rng.standard_normal((H, dh)) * 2.0
    Kd = R.dequant(km, kl, ks, full)
    p = torch.softmax(torch.from_numpy(Kd @ q[0]) / math.sqrt(dh), dim=0).numpy()
    amp = 127.0 if full else 112.0
    for m in (1, 4, Lc):
        ps = np.sort(p)[::-1]
        tau = float(ps[m - 1]) * (1 - 1e-9)   # just below the m-th largest
        assert m == Lc or ps[m] < tau
        o, P, rec, _, kept = R.decode_attention(q, cache, H, dh, True, threshold, v_threshold=tau)
        assert bool(rec[0]) == full and kept[0] == m
        np.testing.assert_allclose(P[0], p, atol=1e-12)
        want = np.zeros(dh)
        want[:Lc] = np.where(p >= tau, amp * p, 0.0)
        np.testing.assert_allclose(o[0], want, atol=1e-10)
    # tau = 0 is the unpruned progressive quantization
    o0, _, _, _, kept0 = R.decode_attention(q, cache, H, dh, True, threshold)
    o1, _, _, _, kept1 = R.decode_attention(q, cache, H, dh, True, threshold, v_threshold=0.0)
    np.testing.assert_array_equal(o0, o1)
    assert kept0[0] == kept1[0] == Lc
