"""Plain fp64 CPU oracle for cascade representative-token selection.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
run this module: only the tests, the smoke entry and the benchmark's CPU
baseline leg use it. It shares no code with the HIP library.

Source: "Cascade Token Selection for Transformer Attention Acceleration"
(gist.science summary, in Dutch), sections "Probleemstelling" (the Gram
threshold that defines a representative token), "Methodologie: Het
Cascade-mechanisme" (steps 1-3: inherit, validate with an r x r and a
(T - r) x r Gram product, update) and "Belangrijkste Bijdragen"
(Proposition 4: the cascade set contains the independent set).

Definitions used here (the page gives no formulas; the readings are listed
with the rest of the design notes):
  cos(t, s) = x_t . x_s / (|x_t| |x_s|), in float64; a zero row has cosine 0
              with everything.
  theta     = 1 - tau**2.
  independent (full-Gram) selection: token t is representative iff the
              largest cosine between t and any preceding token s < t is
              below theta (token 0 always is: the maximum over no tokens is
              -inf).
  cascade step, given the set R inherited from the previous layer and this
              layer's activations:
    1. removal (the r x r product among R): t in R stays iff its largest
       cosine with a preceding member of R is below theta;
    2. addition (the (T - r) x r product between the other tokens and the
       members that stayed, R_valid): u not in R joins iff its largest
       cosine with a preceding member of R_valid is below theta;
    3. the layer's set is R_valid plus the added tokens.
  The first layer takes the independent selection.

Every decision that turns a cosine into a set membership is returned
together with the cosine it was taken on, so tests can compare decisions
away from the threshold and check the rest against each side's own values.
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np


def unit_rows(X) -> np.ndarray:
    """Rows scaled to unit length (zero rows stay zero), float64."""
    X = np.asarray(X, dtype=np.float64)
    n = np.sqrt(np.sum(X * X, axis=1, keepdims=True))
    return np.divide(X, n, out=np.zeros_like(X), where=n > 0)


def max_preceding_cosine(X, rows, cols) -> np.ndarray:
    """For each token i in `rows`, the largest cos(i, j) over tokens j in
    `cols` with j < i (-inf when there is none). rows and cols are token
    indices into X; the result follows the order of `rows`."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    out = np.full(rows.shape[0], -np.inf)
    if rows.size == 0 or cols.size == 0:
        return out
    U = unit_rows(X)
    G = U[rows] @ U[cols].T                       # the Gram product of the two sets
    G = np.where(cols[None, :] < rows[:, None], G, -np.inf)
    return G.max(axis=1)


def independent_selection(X, tau: float):
    """Full-Gram selection ("Probleemstelling"): returns (sorted index array
    of representatives, per-token largest preceding cosine [T])."""
    X = np.asarray(X, dtype=np.float64)
    T = X.shape[0]
    theta = 1.0 - tau * tau
    allt = np.arange(T)
    mc = max_preceding_cosine(X, allt, allt)
    return allt[mc < theta], mc


def cascade_step(X, R_prev, tau: float,
                 decide: Optional[Callable[[str, int, float, bool], bool]] = None) -> dict:
    """One cascade validation ("Methodologie", steps 1-3) of the inherited
    set R_prev against this layer's activations X [T, d].

    decide(kind, token, cosine, default) may override a decision (tests use
    it to follow the GPU among tokens whose cosine is at the threshold).
    Returns the new set and every intermediate: the removal cosines of the
    inherited members, the addition cosines of the other tokens, the
    removed and added tokens and the number of Gram entries each product
    evaluated (pairs s < t only)."""
    X = np.asarray(X, dtype=np.float64)
    T = X.shape[0]
    theta = 1.0 - tau * tau
    R = np.unique(np.asarray(R_prev, dtype=np.int64))
    assert R.size == 0 or (R[0] >= 0 and R[-1] < T)
    # step 2a: r x r among the inherited members
    rc = max_preceding_cosine(X, R, R)
    keep = rc < theta
    if decide is not None:
        keep = np.array([decide("remove", int(t), float(c), bool(k))
                         for t, c, k in zip(R, rc, keep)], dtype=bool)
    R_valid = R[keep]
    # step 2b: (T - r) x r between the other tokens and the valid members
    others = np.setdiff1d(np.arange(T), R)
    ac = max_preceding_cosine(X, others, R_valid)
    add = ac < theta
    if decide is not None:
        add = np.array([decide("add", int(u), float(c), bool(k))
                        for u, c, k in zip(others, ac, add)], dtype=bool)
    added = others[add]
    new = np.union1d(R_valid, added)
    pairs_rr = int(np.sum(R[None, :] < R[:, None]))
    pairs_cross = int(np.sum(R_valid[None, :] < others[:, None]))
    return {"set": new, "removed": R[~keep], "added": added, "kept": R_valid,
            "remove_cos": rc, "add_cos": ac, "others": others,
            "gram_pairs": pairs_rr + pairs_cross}


def run_cascade(layers, tau: float, decide=None, adopt=None) -> list:
    """Selection over a stack of per-layer activations (an iterable of
    [T, d] arrays): the first layer takes the independent selection, every
    later layer a cascade step from the previous layer's set.

    decide(layer, kind, token, cosine, default) overrides decisions;
    adopt(layer, set) may replace the set a layer hands on (tests pass the
    GPU's set so every layer is compared on identical inputs).
    Returns one record per layer with the set, the independent set of the
    same layer and the Gram pairs each method evaluated."""
    out = []
    prev = None
    for l, X in enumerate(layers):
        X = np.asarray(X, dtype=np.float64)
        T = X.shape[0]
        ind, mc = independent_selection(X, tau)
        full_pairs = T * (T - 1) // 2
        if prev is None:
            sel = ind
            if decide is not None:
                theta = 1.0 - tau * tau
                keep = np.array([decide(l, "full", t, float(mc[t]), bool(mc[t] < theta))
                                 for t in range(T)], dtype=bool)
                sel = np.arange(T)[keep]
            rec = {"set": sel, "independent": ind, "full_cos": mc, "gram_pairs": full_pairs}
        else:
            d = None if decide is None else (lambda k, t, c, dflt, l_=l: decide(l_, k, t, c, dflt))
            step = cascade_step(X, prev, tau, d)
            rec = dict(step)
            rec["independent"] = ind
            rec["full_cos"] = mc
        rec["full_pairs"] = full_pairs
        if adopt is not None:
            rec["set"] = np.asarray(adopt(l, rec["set"]), dtype=np.int64)
        out.append(rec)
        prev = rec["set"]
    return out
