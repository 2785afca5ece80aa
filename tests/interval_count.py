"""Visible-key counts per query row by interval arithmetic (test helper).

An independent second derivation of the window definition used to pin the oracle's
element-wise mask: for a query at key position p = i + (Lk - Lq) the visible keys are
the union of at most three key intervals (sink, near, band), whose size follows from
inclusion-exclusion.  It evaluates O(rows) numbers instead of O(rows x keys) booleans,
so it also reaches the 32K- and 128K-token shapes.
"""

import numpy as np


def _band(h, near, gap, lr, mode):
    start = near + gap
    if mode == "dense":
        return start, None
    slot = h if mode == "complementary" else 0
    return start + slot * lr, start + slot * lr + lr


def row_intervals(rows, Lq, Lk, h, sink, near, gap, lr, mode):
    """Half-open key intervals [a, b) of the three windows for each row."""
    p = np.asarray(rows, dtype=np.int64) + (Lk - Lq)
    lo, hi = _band(h, near, gap, lr, mode)
    # sink: keys [0, sink) that are causal (j <= p)
    s = (np.zeros_like(p), np.minimum(sink, p + 1))
    # near: distances [0, near) -> keys (p - near, p]
    n = (np.maximum(0, p - near + 1), p + 1)
    # band: distances [lo, hi) -> keys (p - hi, p - lo]
    b_hi = p - lo + 1
    b_lo = np.zeros_like(p) if hi is None else np.maximum(0, p - hi + 1)
    b = (b_lo, np.maximum(b_lo, b_hi))
    return s, n, b


def _len(a, b):
    return np.maximum(0, b - a)


def row_counts(rows, Lq, Lk, h, sink, near, gap, lr, mode):
    (a1, b1), (a2, b2), (a3, b3) = row_intervals(rows, Lq, Lk, h, sink, near, gap, lr, mode)
    tot = _len(a1, b1) + _len(a2, b2) + _len(a3, b3)
    tot -= _len(np.maximum(a1, a2), np.minimum(b1, b2))
    tot -= _len(np.maximum(a1, a3), np.minimum(b1, b3))
    tot -= _len(np.maximum(a2, a3), np.minimum(b2, b3))
    tot += _len(np.maximum(np.maximum(a1, a2), a3), np.minimum(np.minimum(b1, b2), b3))
    return tot


def head_edges(Lq, Lk, Hkv, sink, near, gap, lr, mode):
    rows = np.arange(Lq, dtype=np.int64)
    return [int(row_counts(rows, Lq, Lk, h, sink, near, gap, lr, mode).sum())
            for h in range(Hkv)]
