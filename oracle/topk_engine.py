"""Second, independent top-k: threshold, filter, order-preserving zero
elimination.

TEST INFRASTRUCTURE ONLY (used to pin the sort-based top-k of the oracle).

Follows the top-k engine of the SpAtten paper (paperlayer.ai summary,
"B. Top-k Engine"): find the k-th largest value with quick-select and use it
as a threshold, keep the elements that pass it (zeroing the rest), then
remove the zeros with a shifter whose stages move each survivor by 1, 2,
4, ... places according to the bits of the count of zeros before it. The
summary leaves ties at the threshold open; here equal keys rank by lower
index, so only the first (k - #above) elements equal to the threshold pass.
"""
from __future__ import annotations

import numpy as np


def _key(v):
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    neg = (u >> 31) == 1
    return np.where(neg, u ^ 0xFFFFFFFF, u ^ 0x80000000).astype(np.int64)


def quickselect_kth_largest(keys, k: int) -> int:
    """k-th largest (1-based) of a list of ints by Hoare-style partitioning."""
    a = [int(x) for x in keys]
    lo, hi = 0, len(a) - 1
    target = k - 1                   # index in descending order
    while True:
        if lo == hi:
            return a[lo]
        pivot = a[(lo + hi) // 2]
        gt = [x for x in a[lo:hi + 1] if x > pivot]
        eq = [x for x in a[lo:hi + 1] if x == pivot]
        lt = [x for x in a[lo:hi + 1] if x < pivot]
        a[lo:hi + 1] = gt + eq + lt
        if target < lo + len(gt):
            hi = lo + len(gt) - 1
        elif target < lo + len(gt) + len(eq):
            return pivot
        else:
            lo = lo + len(gt) + len(eq)


def zero_eliminate(vals, keep):
    """Order-preserving compaction by a log-stage shifter: survivor i moves
    left by z_i (the number of dropped entries before it), applying bit s of
    z_i at stage s. Returns the survivors in their original order."""
    n = len(vals)
    z = np.cumsum(~np.asarray(keep, dtype=bool)) - (~np.asarray(keep, dtype=bool))
    lane_val = list(vals)
    lane_ok = list(bool(x) for x in keep)
    lane_z = [int(x) for x in z]
    s = 0
    while (1 << s) < max(n, 1):
        step = 1 << s
        nv, nok, nz = [None] * n, [False] * n, [0] * n
        for i in range(n):
            if not lane_ok[i]:
                continue
            d = step if (lane_z[i] >> s) & 1 else 0
            j = i - d
            assert not nok[j], "shifter collision"
            nv[j], nok[j], nz[j] = lane_val[i], True, lane_z[i]
        lane_val, lane_ok, lane_z = nv, nok, nz
        s += 1
    cnt = int(np.sum(keep))
    return [lane_val[i] for i in range(cnt)]


def topk_engine(scores, k: int) -> np.ndarray:
    key = _key(scores)
    n = key.shape[0]
    thr = quickselect_kth_largest(key, k)
    above = int(np.sum(key > thr))
    need_eq = k - above
    keep = np.zeros(n, dtype=bool)
    for i in range(n):
        if key[i] > thr:
            keep[i] = True
        elif key[i] == thr and need_eq > 0:
            keep[i] = True
            need_eq -= 1
    return np.asarray(zero_eliminate(list(range(n)), keep), dtype=np.int32)
