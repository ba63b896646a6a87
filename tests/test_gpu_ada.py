"""GPU parity of cascade representative-token selection (page 5) against
the fp64 oracle, through the C ABI.

Each layer is compared on identical inputs (the oracle takes the GPU's
previous set): the cosine every decision was taken on must match the
oracle's within the fp32 error of a d-term dot product of unit vectors
(2 d u for the dot and both inverse norms, u = 2^-24, plus a few units);
decisions must agree except for tokens whose oracle cosine lies within that
bound of the threshold, where the oracle follows the GPU; the counts must
match the sets exactly. Proposition 4 (the cascade set contains the
independent set) holds bit for bit on the GPU's own cosines, since a pair's
fp32 cosine is the same in every product.
"""
import math

import numpy as np
import pytest
import torch

from cascade_token_head_amd import pipeline
from oracle import ada_ref as A
from workloads import ADA_GPT2, ADA_LONG, ADA_SMALL, ada_batch_layers, ada_layers
from workloads.configs import AdaConfig

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def cos_bound(d):
    return (2 * d + 16) * U32


def _check_layer(cfg, l, x_np, gpu_flags, gpu_cos, gpu_counts, prev_flags, stats, rows=None):
    """One layer of one sequence. rows: the tokens to check (None = all)."""
    T, d = x_np.shape
    theta = 1.0 - cfg.tau * cfg.tau
    bnd = cos_bound(d)
    gset = np.nonzero(gpu_flags)[0]
    if rows is None:
        if prev_flags is None:
            ind, mc = A.independent_selection(x_np, cfg.tau)
            want_cos, want_set = mc, ind
            decided = {}
            for t in range(T):
                o = mc[t] < theta
                if bool(gpu_flags[t]) != o:
                    assert abs(mc[t] - theta) <= bnd, ("full decision outside the band", l, t, mc[t])
                    decided[t] = bool(gpu_flags[t])
                    stats["in_band"] += 1
            want_set = np.array([t for t in range(T) if decided.get(t, mc[t] < theta)])
            pairs = T * (T - 1) // 2
            removed = added = 0
        else:
            def decide(kind, t, c, dflt):
                g = bool(gpu_flags[t])
                if g != dflt:
                    assert abs(c - theta) <= bnd, ("%s decision outside the band" % kind, l, t, c)
                    stats["in_band"] += 1
                return g
            st = A.cascade_step(x_np, np.nonzero(prev_flags)[0], cfg.tau, decide)
            want_set = st["set"]
            want_cos = np.full(T, np.nan)
            R = np.nonzero(prev_flags)[0]
            want_cos[R] = st["remove_cos"]
            want_cos[st["others"]] = st["add_cos"]
            pairs = st["gram_pairs"]
            removed, added = st["removed"].size, st["added"].size
        np.testing.assert_array_equal(gset, want_set, err_msg="layer %d set" % l)
        fin = np.isfinite(want_cos)
        np.testing.assert_array_equal(np.isfinite(gpu_cos), fin)
        err = np.max(np.abs(gpu_cos[fin] - want_cos[fin])) if fin.any() else 0.0
        assert err <= bnd, ("cosine error", l, err, bnd)
        stats["cos_err_over_bound"] = max(stats["cos_err_over_bound"], err / bnd)
        assert list(gpu_counts) == [gset.size, removed, added, min(pairs, 2 ** 31 - 1)], (
            l, list(gpu_counts), [gset.size, removed, added, pairs])
        return
    # sampled rows (full-size long sequences): each row's cosine over the set
    # it was compared with, recomputed from the definition for that row only
    rows = np.asarray(rows)
    if prev_flags is None:
        want = A.max_preceding_cosine(x_np, rows, np.arange(T))
        pairs = T * (T - 1) // 2
    else:
        R = np.nonzero(prev_flags)[0]
        # the members that stayed are the GPU's flags restricted to R
        V = R[gpu_flags[R] != 0]
        N = np.setdiff1d(np.arange(T), R)
        pairs = R.size * (R.size - 1) // 2 + int(np.searchsorted(V, N).sum())
        member = prev_flags[rows] != 0
        want = np.empty(rows.size)
        want[member] = A.max_preceding_cosine(x_np, rows[member], R)
        want[~member] = A.max_preceding_cosine(x_np, rows[~member], V)
    for t, c in zip(rows, want):
        if np.isfinite(c):
            assert abs(gpu_cos[t] - c) <= bnd, ("cosine error", l, t, gpu_cos[t], c)
            stats["cos_err_over_bound"] = max(stats["cos_err_over_bound"], abs(gpu_cos[t] - c) / bnd)
        else:
            assert gpu_cos[t] == -np.inf
        g = bool(gpu_flags[t])
        if g != (c < 1.0 - cfg.tau ** 2):
            assert abs(c - (1.0 - cfg.tau ** 2)) <= bnd
            stats["in_band"] += 1
    assert gpu_counts[0] == gset.size and gpu_counts[3] == min(pairs, 2 ** 31 - 1)


def run_checked(cfg, rows=None):
    st = pipeline.AdaStack(cfg.n_layers, cfg.batch, cfg.seq_len, cfg.dim, cfg.tau)
    full = pipeline.AdaStack(cfg.n_layers, cfg.batch, cfg.seq_len, cfg.dim, cfg.tau)
    layers_np = list(ada_batch_layers(cfg))
    layers = [torch.from_numpy(x).cuda() for x in layers_np]
    st.run(layers)
    full.run(layers, full_every_layer=True)
    torch.cuda.synchronize()
    flags = st.flags.cpu().numpy()
    cosv = st.maxcos.cpu().numpy()
    counts = st.counts.cpu().numpy()
    fflags = full.flags.cpu().numpy()
    stats = {"in_band": 0, "cos_err_over_bound": 0.0, "extra": 0, "cascade_pairs": 0,
             "full_pairs": 0}
    for l in range(cfg.n_layers):
        for b in range(cfg.batch):
            prev = None if l == 0 else flags[l - 1, b]
            _check_layer(cfg, l, layers_np[l][b].astype(np.float64), flags[l, b], cosv[l, b],
                         counts[l, b], prev, stats, rows)
            # Proposition 4 on the GPU's own cosines: cascade contains full
            assert np.all(flags[l, b][fflags[l, b] != 0] != 0), (l, b)
            stats["extra"] += int(flags[l, b].sum() - fflags[l, b].sum())
        stats["cascade_pairs"] += int(counts[l, :, 3].astype(np.int64).sum())
        stats["full_pairs"] += cfg.batch * cfg.seq_len * (cfg.seq_len - 1) // 2
        print("  layer %d checked" % l, flush=True)
    return stats


CASES = {
    "small": ADA_SMALL,
    "ragged": AdaConfig(name="ada_ragged", batch=3, seq_len=701, dim=96, n_layers=4),
    "one_token": AdaConfig(name="ada_one", batch=2, seq_len=1, dim=32, n_layers=2),
    "tight": AdaConfig(name="ada_tight", batch=2, seq_len=300, dim=64, n_layers=5, tau=0.15,
                       drift=0.1),
    "gpt2_full": ADA_GPT2,
}


@pytest.mark.parametrize("name", list(CASES))
def test_ada_cascade_parity(name):
    cfg = CASES[name]
    print("ada", name, flush=True)
    stats = run_checked(cfg)
    print(name, stats, flush=True)
    if cfg.seq_len > 1 and cfg.n_layers > 1:
        assert stats["cascade_pairs"] < stats["full_pairs"]


def test_ada_long_sampled_rows():
    """T = 8192, d = 4096: every layer's cosines and decisions on 48 sampled
    tokens (first, last, spread) against the definition, the counts against
    the sets, and Proposition 4 on every token."""
    cfg = ADA_LONG
    rows = np.unique(np.concatenate([[0, 1, 2, 63, 64, 8191], np.linspace(0, 8191, 42).astype(int)]))
    print("ada long", flush=True)
    stats = run_checked(cfg, rows=rows)
    print(stats, flush=True)


def test_ada_rejects_bad_arguments():
    from cascade_token_head_amd import spatten as S
    x = torch.zeros(1, 8, 33, device="cuda")
    f = torch.zeros(1, 8, dtype=torch.int32, device="cuda")
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(S.SpattenError) as e:
        S.ada_select(x, 0.3, f, ws)
    assert e.value.status == S.EUNSUPPORTED
    x = torch.zeros(1, 8, 32, device="cuda")
    with pytest.raises(S.SpattenError) as e:
        S.ada_select(x, 1.5, f, ws)
    assert e.value.status == S.EINVAL
