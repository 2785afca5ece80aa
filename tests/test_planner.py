"""Host planner (cowa_plan_blocks) against the oracle's explicit mask — bit-exact tile
lists, FULL/PARTIAL flags, column lists, work orders and counters.  CPU only."""

import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))
import oracle  # noqa: E402
from interval_count import head_edges  # noqa: E402

api = pytest.importorskip("structured_sparse_attention_plan_amd.api")


def _lib_lists(plan, Hkv):
    a = plan.arrays
    nqb, nkb = plan.info.nqb, plan.info.nkb
    rows = [[[(int(e) >> 1, not (int(e) & 1)) for e in a["row_ent"][a["row_ptr"][h * nqb + qb]:
                                                                  a["row_ptr"][h * nqb + qb + 1]]]
             for qb in range(nqb)] for h in range(Hkv)]
    cols = [[[(int(e) >> 1, not (int(e) & 1)) for e in a["col_ent"][a["col_ptr"][h * nkb + kb]:
                                                                  a["col_ptr"][h * nkb + kb + 1]]]
             for kb in range(nkb)] for h in range(Hkv)]
    return rows, cols


CASES = [
    # (Lq, Lk, Hkv, Bq, Bk, sink, near, gap, mode)
    (1024, 1024, 2, 64, 64, 64, 128, 0, "complementary"),
    (1024, 1024, 2, 64, 64, 64, 128, 0, "duplicated"),
    (1024, 1024, 2, 64, 64, 64, 128, 0, "dense"),
    (1000, 1000, 8, 51, 64, 16, 100, 0, "complementary"),
    (777, 1500, 4, 25, 128, 7, 33, 5, "complementary"),
    (300, 300, 3, 64, 32, 0, 1, 0, "complementary"),
    (1, 4096, 8, 1, 64, 128, 256, 0, "complementary"),
    (1, 5000, 8, 1, 64, 100, 300, 0, "duplicated"),
    (2048, 2048, 8, 25, 128, 128, 512, 0, "complementary"),
    (130, 130, 2, 64, 64, 200, 0, 0, "complementary"),
    (500, 200, 2, 64, 64, 3, 10, 0, "complementary"),  # Lq > Lk: early rows see nothing
]


@pytest.mark.parametrize("Lq,Lk,Hkv,Bq,Bk,sink,near,gap,mode", CASES)
def test_plan_matches_oracle_mask(Lq, Lk, Hkv, Bq, Bk, sink, near, gap, mode):
    owin = oracle.Window.for_length(max(Lk, 1), Hkv, sink, near, gap, mode=mode)
    win = api.window(owin.sink, owin.near, owin.gap, owin.lr, mode)
    plan = api.plan_blocks(Lq, Lk, Hkv, Bq, Bk, win)
    want = oracle.tile_lists(Lq, Lk, Hkv, Bq, Bk, owin)
    rows, cols = _lib_lists(plan, Hkv)
    assert rows == want
    # column lists are the transpose, q-blocks ascending
    nkb = plan.info.nkb
    for h in range(Hkv):
        tr = [[] for _ in range(nkb)]
        for qb, ent in enumerate(want[h]):
            for kb, full in ent:
                tr[kb].append((qb, full))
        assert cols[h] == tr
    info = plan.info
    nnz = sum(len(e) for hl in want for e in hl)
    assert info.nnz == nnz and info.visited == nnz
    assert info.n_partial == sum(1 for hl in want for e in hl for _, f in e if not f)
    assert info.edges == sum(oracle.edge_counts(Lq, Lk, Hkv, owin))
    # launch orders: permutations; items with a list over twice the mean length first,
    # longest first; after them the items dealt to one XCD (positions b % 8 == x) walk
    # runs of consecutive blocks of one head
    a = plan.arrays
    for key, ptr_key, nblk in (("row_order", "row_ptr", plan.info.nqb),
                               ("col_order", "col_ptr", plan.info.nkb)):
        order = a[key]
        n = Hkv * nblk
        assert sorted(order.tolist()) == list(range(n))
        lens = np.diff(a[ptr_key])
        heavy = [int(i) for i in np.argsort(-lens, kind="stable") if lens[i] > 2.0 * lens.mean()]
        assert order[:len(heavy)].tolist() == heavy
        for x in range(8):
            seq = np.array([order[p] for p in range(len(heavy), n) if p % 8 == x])
            if len(seq) < 2:
                continue
            runs = 1 + int(np.sum(seq[1:] - seq[:-1] != 1))
            # parts of at least 16 blocks when a head has 16 or more and an XCD's share is
            # at least 64 items (heavy items and parts split between XCDs break a few runs)
            if nblk >= 16 and n // 8 >= 64:
                assert len(seq) / runs >= 4, (key, x, len(seq), runs)


def test_info_only_call_matches_full_call():
    win = api.make_window(4096, 8, 128, 512)
    info = api.plan_info(4096, 4096, 8, 51, 64, win)
    full = api.plan_blocks(4096, 4096, 8, 51, 64, win)
    for f in ("nqb", "nkb", "nnz", "n_partial", "visited", "edges"):
        assert getattr(info, f) == getattr(full.info, f)


@pytest.mark.parametrize("L,sink,near,Bq,Bk,tiles,partial", [
    # tile counts at the 32K and 128K workloads with 128x128 tiles (also derivable by hand
    # from the band edges)
    (32768, 128, 2048, 128, 128, 64914, 5387),
    (131072, 128, 4096, 128, 128, 768050, 22059),
])
def test_large_tile_counts(L, sink, near, Bq, Bk, tiles, partial):
    win = api.make_window(L, 8, sink, near)
    info = api.plan_info(L, L, 8, Bq, Bk, win)
    assert info.nnz == tiles and info.n_partial == partial and info.visited == tiles


@pytest.mark.parametrize("L,sink,near", [(32768, 128, 2048), (131072, 128, 4096)])
@pytest.mark.parametrize("mode", ["complementary", "duplicated", "dense"])
def test_large_edge_counts_match_interval_count(L, sink, near, mode):
    win = api.make_window(L, 8, sink, near, 0, mode)
    info = api.plan_info(L, L, 8, 64, 64, win)
    assert info.edges == sum(head_edges(L, L, 8, sink, near, 0, win.lr, mode))


def _greedy_makespan(order, cost, workers=256):
    """Finish time of list scheduling: items start in launch order on the first free worker."""
    import heapq
    free = [0.0] * workers
    for it in order:
        t = heapq.heappop(free)
        heapq.heappush(free, t + cost[it])
    return max(free)


def test_backward_column_order_balances_the_sink_columns():
    # 131072 tokens, 25-token q-blocks x 128-key blocks (the dK/dV launch): the 8 columns
    # holding the prefix sink are seen by all 5243 q-blocks, ~11x the mean; launched first
    # they no longer set the finish time of a 256-CU launch
    L = 131072
    win = api.make_window(L, 8, 128, 4096)
    plan = api.plan_blocks(L, L, 8, 25, 128, win)
    nkb = plan.info.nkb
    order = plan.arrays["col_order"]
    assert order[:8].tolist() == [h * nkb for h in range(8)]
    cost = np.diff(plan.arrays["col_ptr"]).astype(np.float64) + 8.0  # per-item start-up
    ideal = cost.sum() / 256
    assert _greedy_makespan(order, cost) < 1.01 * ideal


def _xcd_makespan(order, cost, xcds=8, cus=32):
    """Finish time when work group b goes to XCD b % 8 and each XCD's CUs take its work
    groups in order, each on the first free CU."""
    import heapq
    end = 0.0
    for x in range(xcds):
        free = [0.0] * cus
        for it in order[x::xcds]:
            t = heapq.heappop(free)
            heapq.heappush(free, t + cost[it])
        end = max(end, max(free))
    return end


@pytest.mark.parametrize("L,sink,near", [(32768, 128, 2048), (131072, 128, 4096)])
@pytest.mark.parametrize("Bq,Bk,key,ptr_key", [
    (51, 64, "row_order", "row_ptr"),    # the forward's launch
    (25, 128, "row_order", "row_ptr"),   # the dQ launch
    (25, 128, "col_order", "col_ptr"),   # the dK/dV launch
])
def test_launch_orders_balance_the_xcds(L, sink, near, Bq, Bk, key, ptr_key):
    # every XCD runs its own queue, so the launch ends with the XCD that has the most
    # work: with work = list length + 4 per item, 8 XCDs x 32 CUs end within 1% (131072
    # tokens) or 3% (32768, where a prefix-sink column alone is 98% of the even share of
    # the dK/dV launch) of the even share
    win = api.make_window(L, 8, sink, near)
    plan = api.plan_blocks(L, L, 8, Bq, Bk, win)
    cost = np.diff(plan.arrays[ptr_key]).astype(np.float64) + 4.0
    ideal = cost.sum() / 256
    bound = 1.01 if L == 131072 else 1.03
    order = plan.arrays[key]
    assert _xcd_makespan(order, cost) < bound * ideal
    # and each XCD still runs neighbouring blocks together: runs of 12 or more on average
    for x in range(8):
        seq = order[x::8]
        runs = 1 + int(np.sum(seq[1:] - seq[:-1] != 1))
        assert len(seq) / runs >= 12, (x, len(seq), runs)


def test_decode_plan_reads_only_visible_blocks():
    # 131072-token cache, query at the last position: per head sink + near + band blocks
    win = api.make_window(131072, 8, 128, 4096)
    plan = api.plan_blocks(1, 131072, 8, 1, 64, win)
    rl = np.diff(plan.arrays["row_ptr"])
    # blocks of 64: sink 2 + band 248 + near 64; head 7's band [0, 15872) holds the sink
    assert rl.tolist() == [314] * 7 + [312]
    owin = oracle.Window.for_length(131072, 8, 128, 4096)
    want = oracle.tile_lists(1, 131072, 8, 1, 64, owin)
    assert rl.tolist() == [len(want[h][0]) for h in range(8)]
    assert plan.info.edges == 7 * 20096 + 19968


def test_planner_rejects_bad_arguments():
    from structured_sparse_attention_plan_amd import _cowa as C
    import ctypes
    win = api.window(1, 2, 0, 3)
    info = C.cowa_plan_info()
    assert C.lib.cowa_plan_blocks(0, 10, 1, 8, 8, ctypes.byref(win), ctypes.byref(info),
                                  None, None, None, None, None, None) == C.COWA_ERR_INVALID_ARG
    bad = api.window(-1, 2, 0, 3)
    assert C.lib.cowa_plan_blocks(10, 10, 1, 8, 8, ctypes.byref(bad), ctypes.byref(info),
                                  None, None, None, None, None, None) == C.COWA_ERR_INVALID_ARG
    arr = (ctypes.c_int32 * 16)()
    # some but not all output arrays
    assert C.lib.cowa_plan_blocks(10, 10, 1, 8, 8, ctypes.byref(win), ctypes.byref(info),
                                  arr, None, None, None, None, None) == C.COWA_ERR_INVALID_ARG
    w = C.cowa_window()
    assert C.lib.cowa_window_make(100, 0, 1, 2, 0, 0, ctypes.byref(w)) == C.COWA_ERR_INVALID_ARG
    assert C.lib.cowa_window_make(131072, 8, 128, 4096, 0, 0, ctypes.byref(w)) == C.COWA_OK
    assert (w.sink, w.near_w, w.gap, w.lr, w.band_mode) == (128, 4096, 0, 15872, 0)
