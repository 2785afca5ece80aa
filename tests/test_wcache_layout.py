"""Layout of the window-only decode cache (cowa_wcache_layout), pinned against the
oracle's element-wise mask: head h must hold the prefix sink and every key it can still
see, i.e. keys up to one less than the largest distance at which it sees a key past the
sink, and no more (slinene.github.io ai-papers-daily page, practical note 3: each rank
keeps only its window's cache)."""

import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))
import oracle  # noqa: E402

api = pytest.importorskip("structured_sparse_attention_plan_amd.api")


def _capacities(win, Hkv, Lmax):
    slots, offs = api.wcache_layout(win, Hkv, Lmax)
    assert offs[0] == 0 and offs[-1] == slots
    return [offs[h + 1] - offs[h] for h in range(Hkv)]


def _reach_from_mask(ow, h, L):
    """1 + the largest distance at which head h sees a key past the sink, read off the
    oracle mask of the last row of a length-L sequence (the longest history)."""
    m = oracle.mask_rows([L - 1], L, L, h, ow)[0]
    j = np.nonzero(m)[0]
    j = j[j >= ow.sink]
    return int((L - 1 - j).max()) + 1 if len(j) else 0


@pytest.mark.parametrize("L,Hkv,sink,near,mode", [
    (3000, 8, 16, 64, "complementary"),
    (3000, 8, 16, 64, "duplicated"),
    (3000, 8, 16, 64, "dense"),
    (5000, 4, 0, 100, "complementary"),
    (4096, 2, 7, 0, "complementary"),
])
def test_capacity_is_sink_plus_reach(L, Hkv, sink, near, mode):
    ow = oracle.Window.for_length(L, Hkv, sink, near, 0, mode=mode)
    win = api.window(ow.sink, ow.near, ow.gap, ow.lr, mode)
    caps = _capacities(win, Hkv, L)
    for h in range(Hkv):
        reach = _reach_from_mask(ow, h, L)
        # either the whole history (the ring would reach back to the sink), or the sink
        # keys plus a ring of exactly `reach` positions
        want = L if reach + min(sink, L) >= L else min(sink, L) + reach
        assert caps[h] == want, (h, caps[h], want, reach)


def test_128k_capacities_and_saving():
    """At 131072 positions (sink 128, near 4096, 8 bands of 15872): head h < 7 holds
    sink + near + (h + 1) * 15872 rows, head 7 (whose band reaches the sink) the whole
    history; 605056 rows in all against 8 * 131072 for full caches (1.73x less), and
    head 0, the smallest, 6.5x less than a full cache."""
    L, Hkv = 131072, 8
    win = api.make_window(L, Hkv, 128, 4096)
    caps = _capacities(win, Hkv, L)
    assert caps == [128 + 4096 + (h + 1) * 15872 for h in range(7)] + [L]
    assert sum(caps) == 605056
    assert L / caps[0] == pytest.approx(6.52, abs=0.01)
