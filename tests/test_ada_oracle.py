"""Pins for the cascade representative-selection oracle (page 5, "Cascade
Token Selection for Transformer Attention Acceleration"): values fixed by
the page's definitions and by mathematics, independent of the oracle's own
formulas.

  * the Gram threshold ("Probleemstelling"): brute-force scalar loops on
    tiny inputs, and closed forms (identical directions, orthogonal rows,
    pairs whose cosine is set on either side of 1 - tau^2);
  * the cascade ("Methodologie", steps 1-3): inheriting every token
    reproduces the full-Gram selection; inheriting nothing makes every
    token representative; a hand-worked five-token case;
  * Proposition 4 ("Belangrijkste Bijdragen"): the cascade set contains
    the independent set, on random clustered activations.
"""
import math

import numpy as np
import pytest

from oracle import ada_ref as A
from workloads import ada_layers
from workloads.configs import ADA_SMALL


def _brute_selection(X, tau):
    theta = 1.0 - tau * tau
    T, d = len(X), len(X[0])
    norms = [math.sqrt(sum(v * v for v in X[t])) for t in range(T)]
    sel = []
    for t in range(T):
        best = -math.inf
        for s in range(t):
            dot = sum(X[t][c] * X[s][c] for c in range(d))
            cs = dot / (norms[t] * norms[s]) if norms[t] > 0 and norms[s] > 0 else 0.0
            best = max(best, cs)
        if best < theta:
            sel.append(t)
    return sel


def test_independent_selection_matches_brute_force():
    rng = np.random.default_rng(41)
    for T, d in ((1, 3), (5, 2), (9, 4), (13, 3)):
        base = rng.standard_normal((max(2, T // 3), d))
        X = base[rng.integers(0, base.shape[0], T)] + 0.15 * rng.standard_normal((T, d))
        for tau in (0.1, 0.3, 0.6):
            sel, mc = A.independent_selection(X, tau)
            assert sel.tolist() == _brute_selection(X.tolist(), tau), (T, d, tau)
            assert mc[0] == -np.inf


def test_closed_forms():
    rng = np.random.default_rng(42)
    # one direction at different scales: only the first token is representative
    v = rng.standard_normal(16)
    X = np.outer(rng.uniform(0.5, 3.0, 10), v)
    sel, mc = A.independent_selection(X, 0.3)
    assert sel.tolist() == [0]
    np.testing.assert_allclose(mc[1:], 1.0, atol=1e-12)
    # orthogonal rows: every token is representative, all cosines 0
    X = np.eye(12)[:7] * 2.5
    sel, mc = A.independent_selection(X, 0.3)
    assert sel.tolist() == list(range(7))
    np.testing.assert_array_equal(mc[1:], 0.0)
    # a pair whose cosine is cos(phi): representative iff cos(phi) < 1 - tau^2
    tau = 0.3
    theta = 1.0 - tau * tau
    for c in (theta - 1e-9, theta + 1e-9, 0.5, 0.99):
        phi = math.acos(c)
        X = np.array([[1.0, 0.0], [math.cos(phi), math.sin(phi)]])
        sel, mc = A.independent_selection(X, tau)
        assert abs(mc[1] - c) < 1e-12
        assert sel.tolist() == ([0, 1] if c < theta else [0]), c


def test_zero_row_has_cosine_zero():
    X = np.array([[1.0, 2.0], [0.0, 0.0], [2.0, 4.0]])
    sel, mc = A.independent_selection(X, 0.3)
    assert mc[1] == 0.0
    assert sel.tolist() == [0, 1]


def test_cascade_from_every_token_is_the_full_selection():
    """Inheriting all T tokens: the r x r product is the full Gram, the
    removal keeps exactly the independent set and nothing is left to add."""
    rng = np.random.default_rng(43)
    for _ in range(5):
        X = rng.standard_normal((40, 6))
        X[10:20] = X[:10] + 0.05 * rng.standard_normal((10, 6))
        ind, _ = A.independent_selection(X, 0.3)
        st = A.cascade_step(X, np.arange(40), 0.3)
        np.testing.assert_array_equal(st["set"], ind)
        assert st["added"].size == 0
        assert st["gram_pairs"] == 40 * 39 // 2


def test_cascade_from_nothing_adds_every_token():
    rng = np.random.default_rng(44)
    X = rng.standard_normal((17, 5))
    st = A.cascade_step(X, np.array([], dtype=np.int64), 0.3)
    np.testing.assert_array_equal(st["set"], np.arange(17))
    assert st["gram_pairs"] == 0


def test_cascade_hand_worked_case():
    """Five tokens in the plane, tau = 0.3 (threshold 0.91), inherited set
    {0, 2, 3}. Angles 0, 5, 90, 93 and 10 degrees:
      removal: 2 vs 0 -> cos 90 = 0 (stays); 3 vs {0, 2} -> cos 3 deg =
               0.9986 with token 2 (removed);
      addition against {0, 2}: token 1 (5 deg) vs 0 -> 0.996 (not added);
               token 4 (10 deg) vs 0 -> 0.985, vs 2 -> cos 80 (not added);
      result {0, 2}; the independent set is {0, 2} as well."""
    ang = np.radians([0.0, 5.0, 90.0, 93.0, 10.0])
    X = np.stack([np.cos(ang), np.sin(ang)], axis=1)
    st = A.cascade_step(X, [0, 2, 3], 0.3)
    assert st["removed"].tolist() == [3]
    assert st["added"].tolist() == []
    assert st["set"].tolist() == [0, 2]
    np.testing.assert_allclose(st["remove_cos"], [-np.inf, 0.0, math.cos(math.radians(3))],
                               atol=1e-12)
    # now inherit {0, 3}: token 2 (90 deg) was not inherited; against the
    # valid {0} it has cosine 0 and is added; token 3 stays (93 deg vs 0)
    st = A.cascade_step(X, [0, 3], 0.3)
    assert st["removed"].tolist() == []
    assert st["added"].tolist() == [2]
    assert st["set"].tolist() == [0, 2, 3]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_proposition_4_cascade_contains_the_independent_set(seed):
    cfg = ADA_SMALL
    layers = list(ada_layers(cfg, seq=0, seed=seed))
    recs = A.run_cascade(layers, cfg.tau)
    extra = 0
    for l, r in enumerate(recs):
        assert np.all(np.isin(r["independent"], r["set"])), l
        extra += r["set"].size - r["independent"].size
        if l > 0:
            # the validation reads fewer Gram entries than the full product
            assert r["gram_pairs"] < r["full_pairs"]
    assert recs[0]["set"].tolist() == recs[0]["independent"].tolist()


def test_synthetic_activations_keep_a_coherent_set():
    """The generator's drift keeps most representatives from one layer to
    the next (the depth coherence the method relies on)."""
    cfg = ADA_SMALL
    recs = A.run_cascade(list(ada_layers(cfg, seq=0)), cfg.tau)
    for a, b in zip(recs, recs[1:]):
        inter = np.intersect1d(a["set"], b["set"]).size
        union = np.union1d(a["set"], b["set"]).size
        assert inter / union > 0.5
    assert 0 < recs[0]["set"].size < cfg.seq_len


def _brute_cos(X, t, s):
    nt = math.sqrt(sum(v * v for v in X[t]))
    ns = math.sqrt(sum(v * v for v in X[s]))
    if nt == 0 or ns == 0:
        return 0.0
    return sum(X[t][c] * X[s][c] for c in range(len(X[t]))) / (nt * ns)


def _brute_cascade(layers, tau):
    """The page's three steps over a stack, written as scalar loops: layer 1
    keeps the full-Gram selection; each later layer drops the inherited
    members that come close to an earlier inherited member, then adds the
    other tokens that come close to no earlier member that stayed. Returns
    per layer (set, Gram pairs read)."""
    theta = 1.0 - tau * tau
    out, prev = [], None
    for X in layers:
        X = np.asarray(X, dtype=np.float64).tolist()
        T = len(X)
        if prev is None:
            sel = _brute_selection(X, tau)
            out.append((sel, T * (T - 1) // 2))
        else:
            R = sorted(prev)
            valid = [t for t in R if all(_brute_cos(X, t, s) < theta for s in R if s < t)]
            others = [u for u in range(T) if u not in R]
            added = [u for u in others
                     if all(_brute_cos(X, u, s) < theta for s in valid if s < u)]
            pairs = sum(1 for t in R for s in R if s < t)
            pairs += sum(1 for u in others for s in valid if s < u)
            sel = sorted(valid + added)
            out.append((sel, pairs))
        prev = out[-1][0]
    return out


@pytest.mark.parametrize("seed", [3, 4])
def test_run_cascade_matches_brute_force_loops(seed):
    """The whole stack: sets and Gram pairs of every layer against scalar
    loops over the definitions, on clustered activations small enough for
    them (18 tokens, 4 layers, a drift that turns some tokens over)."""
    rng = np.random.default_rng(seed)
    centres = rng.standard_normal((5, 4))
    X = centres[rng.integers(0, 5, 18)] + 0.25 * rng.standard_normal((18, 4))
    layers = []
    for _ in range(4):
        layers.append(X.copy())
        X = X + 0.3 * rng.standard_normal(X.shape)
    recs = A.run_cascade(layers, 0.3)
    want = _brute_cascade(layers, 0.3)
    changed = False
    for l, (r, (sel, pairs)) in enumerate(zip(recs, want)):
        assert r["set"].tolist() == sel, l
        assert r["gram_pairs"] == pairs, l
        if l > 0:
            changed |= (r["set"].tolist() != recs[l - 1]["set"].tolist())
    assert changed  # some layer removes or adds a token
