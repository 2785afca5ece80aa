"""Pins of the CPU oracle against facts that do not come from the oracle itself.

* Mask: the collective-coverage property (union over KV heads == causal history),
  disjoint and equal-width bands, shared sink/near windows, the 1/Hkv coverage of
  duplicated bands, dense mode == causal, one bottom-right distance for prefill and
  decode (CoWindow Attention: Full Causal Coverage Is a Collective Property — abstract,
  and the slinene.github.io ai-papers-daily page, method key points 1-3 and key
  result 1), plus edge counts from an independent interval-arithmetic count and
  closed forms.
* Attention: textbook attention (torch SDPA, float64) with the oracle's mask as an
  explicit boolean mask, and without a mask in dense mode; closed forms for q = 0.
* Gradients: central finite differences, autograd of textbook attention, and the exact
  column-sum identities.
"""

import math
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))
import oracle  # noqa: E402
from interval_count import head_edges, row_counts  # noqa: E402

W = oracle.Window


def causal(Lq, Lk):
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    return j <= i + (Lk - Lq)


# ----------------------------------------------------------------------------- mask

SHAPES = [
    # (Lq, Lk, Hkv, sink, near, gap)
    (1024, 1024, 2, 64, 128, 0),
    (777, 777, 8, 16, 40, 0),
    (300, 700, 4, 3, 17, 0),
    (1, 4096, 8, 128, 256, 0),
    (513, 513, 3, 0, 1, 0),
]


@pytest.mark.parametrize("Lq,Lk,Hkv,sink,near,gap", SHAPES)
def test_collective_coverage_is_causal(Lq, Lk, Hkv, sink, near, gap):
    win = W.for_length(Lk, Hkv, sink, near, gap)
    union = np.zeros((Lq, Lk), dtype=bool)
    for h in range(Hkv):
        union |= oracle.full_mask(Lq, Lk, h, win)
    assert np.array_equal(union, causal(Lq, Lk))


@pytest.mark.parametrize("Lq,Lk,Hkv,sink,near,gap", SHAPES)
def test_bands_disjoint_equal_width_shared_windows(Lq, Lk, Hkv, sink, near, gap):
    win = W.for_length(Lk, Hkv, sink, near, gap)
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    d = i + (Lk - Lq) - j
    shared = (d >= 0) & ((j < sink) | (d < near))
    mult = np.zeros((Lq, Lk), dtype=np.int32)
    for h in range(Hkv):
        m = oracle.full_mask(Lq, Lk, h, win)
        # the shared windows are the same for every head
        assert np.array_equal(m & shared, shared)
        band_only = m & ~shared
        mult += band_only
        # the band of head h, as distances, is one run of exactly lr distances
        dist = np.unique(d[band_only])
        if len(dist):
            assert dist.max() - dist.min() + 1 == len(dist)
    assert mult.max() <= 1  # pairwise disjoint


def test_band_width_is_exact_on_long_row():
    # on the last row of a long sequence (no sink overlap with most bands), each band
    # contributes exactly lr distances
    Lk, Hkv, near = 4096, 8, 256
    win = W.for_length(Lk, Hkv, 0, near, 0)
    d = (Lk - 1) - np.arange(Lk)
    for h in range(Hkv):
        m = oracle.mask_rows([Lk - 1], Lk, Lk, h, win)[0]
        band = m & (d >= near)
        assert band.sum() == min(win.lr, Lk - near - h * win.lr)
        assert d[band].min() == near + h * win.lr


def test_duplicated_bands_cover_one_over_hkv():
    # key result 1 of the ai-papers-daily page: duplicated windows cover 12.5%-50%;
    # with 8 KV heads sharing one band, 1/8 of the long-range distances
    L, Hkv, near = 4096, 8, 256
    win = W.for_length(L, Hkv, 0, near, 0, mode=oracle.DUPLICATED)
    union = np.zeros((L, L), dtype=bool)
    for h in range(Hkv):
        union |= oracle.full_mask(L, L, h, win)
    d = (L - 1) - np.arange(L)
    last = union[L - 1]
    frac = last[d >= near].sum() / (L - near)
    assert frac == pytest.approx(1 / Hkv, abs=1 / (L - near))


@pytest.mark.parametrize("Lq,Lk", [(257, 257), (100, 900)])
def test_dense_mode_is_causal(Lq, Lk):
    win = W.for_length(Lk, 4, 5, 9, 0, mode=oracle.DENSE)
    for h in range(4):
        assert np.array_equal(oracle.full_mask(Lq, Lk, h, win), causal(Lq, Lk))


def test_bottom_right_alignment_prefill_decode():
    # one distance definition for training, prefill and decoding (method key point 2):
    # the mask of the last Lq rows of a length-L prefill equals the (Lq, L) mask
    L, Hkv = 600, 4
    win = W.for_length(L, Hkv, 8, 32, 0)
    for h in range(Hkv):
        full = oracle.full_mask(L, L, h, win)
        for Lq in (1, 7, 128):
            assert np.array_equal(oracle.full_mask(Lq, L, h, win), full[L - Lq:])


@pytest.mark.parametrize("mode", oracle.MODES)
@pytest.mark.parametrize("Lq,Lk,Hkv,sink,near,gap", SHAPES + [(600, 600, 4, 10, 50, 7)])
def test_edge_counts_match_interval_arithmetic(mode, Lq, Lk, Hkv, sink, near, gap):
    win = W.for_length(Lk, Hkv, sink, near, gap, mode=mode)
    got = oracle.edge_counts(Lq, Lk, Hkv, win)
    want = head_edges(Lq, Lk, Hkv, sink, near, gap, win.lr, mode)
    assert got == want


def test_edge_count_closed_forms():
    # dense causal with Lq == Lk: L (L + 1) / 2 per head
    L = 1024
    win = W.for_length(L, 2, 64, 128, 0, mode=oracle.DENSE)
    assert oracle.edge_counts(L, L, 2, win) == [L * (L + 1) // 2] * 2
    # decode row at position Lk - 1: sink + near + lr keys while the band stays clear of
    # the sink, and lr + near when the last band reaches key 0
    Lk, Hkv, sink, near = 131072, 8, 128, 4096
    win = W.for_length(Lk, Hkv, sink, near, 0)
    assert win.lr == 15872
    counts = [int(row_counts([0], 1, Lk, h, sink, near, 0, win.lr, "complementary")[0])
              for h in range(Hkv)]
    assert counts == [sink + near + win.lr] * 7 + [near + win.lr]
    assert oracle.edge_counts(1, Lk, Hkv, win) == counts


def test_golden_edge_counts_file():
    import json
    path = os.path.join(os.path.dirname(__file__), "golden", "edge_counts.json")
    with open(path) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        win = W(case["sink"], case["near"], case["gap"], case["lr"], case["mode"])
        want = head_edges(case["Lq"], case["Lk"], case["Hkv"], case["sink"], case["near"],
                          case["gap"], case["lr"], case["mode"])
        assert want == case["per_head"], case
        if case["Lq"] * case["Lk"] <= 2 ** 22:
            assert oracle.edge_counts(case["Lq"], case["Lk"], case["Hkv"], win) == want


# ----------------------------------------------------------------------------- forward

def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


def _sdpa(q, k, v, mask_per_head, scale):
    """Textbook attention (torch SDPA, float64) with explicit boolean masks [Hq, Lq, Lk]."""
    B, Lq, Hq, D = q.shape
    G = Hq // k.shape[2]
    qt = q.permute(0, 2, 1, 3)
    kt = k.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vt = v.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    m = torch.as_tensor(mask_per_head)[None] if mask_per_head is not None else None
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o.permute(0, 2, 1, 3)


def _masks(Lq, Lk, Hq, Hkv, win):
    G = Hq // Hkv
    return np.stack([oracle.full_mask(Lq, Lk, qh // G, win) for qh in range(Hq)])


@pytest.mark.parametrize("Lq,Lk,Hq,Hkv,D,sink,near,mode", [
    (96, 96, 4, 2, 16, 5, 9, oracle.COMPLEMENTARY),
    (96, 96, 6, 3, 8, 0, 4, oracle.DUPLICATED),
    (40, 130, 10, 2, 16, 7, 11, oracle.COMPLEMENTARY),
    (1, 200, 10, 2, 16, 7, 11, oracle.COMPLEMENTARY),
])
def test_fwd_matches_textbook_masked_attention(Lq, Lk, Hq, Hkv, D, sink, near, mode):
    win = W.for_length(Lk, Hkv, sink, near, 0, mode=mode)
    q, k, v = _rand((2, Lq, Hq, D), 1), _rand((2, Lk, Hkv, D), 2), _rand((2, Lk, Hkv, D), 3)
    scale = 1 / math.sqrt(D)
    O, LSE = oracle.attn_fwd(q, k, v, win, scale)
    ref = _sdpa(q, k, v, _masks(Lq, Lk, Hq, Hkv, win), scale)
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)
    # LSE: textbook logsumexp of the masked scores
    G = Hq // Hkv
    for qh in range(Hq):
        s = scale * torch.einsum("bid,bjd->bij", q[:, :, qh], k[:, :, qh // G])
        s = s.masked_fill(~torch.as_tensor(oracle.full_mask(Lq, Lk, qh // G, win)), -math.inf)
        np.testing.assert_allclose(LSE[:, qh], torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


def test_fwd_dense_mode_is_causal_sdpa():
    L, Hq, Hkv, D = 128, 4, 2, 16
    win = W.for_length(L, Hkv, 3, 5, 0, mode=oracle.DENSE)
    q, k, v = _rand((1, L, Hq, D), 4), _rand((1, L, Hkv, D), 5), _rand((1, L, Hkv, D), 6)
    O, _ = oracle.attn_fwd(q, k, v, win, 0.25)
    qt = q.permute(0, 2, 1, 3)
    kt = k.repeat_interleave(2, dim=2).permute(0, 2, 1, 3)
    vt = v.repeat_interleave(2, dim=2).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           scale=0.25)
    np.testing.assert_allclose(O, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)


@pytest.mark.parametrize("variant", ["near_ge_L", "sink_ge_L", "one_head_full_band"])
def test_windows_that_reduce_to_dense(variant):
    L, D = 90, 8
    Hkv = 1 if variant == "one_head_full_band" else 2
    Hq = 2 * Hkv
    if variant == "near_ge_L":
        win = W(0, L, 0, 3)
    elif variant == "sink_ge_L":
        win = W(L, 1, 0, 3)
    else:
        win = W.for_length(L, 1, 2, 7, 0)
    q, k, v = _rand((1, L, Hq, D), 7), _rand((1, L, Hkv, D), 8), _rand((1, L, Hkv, D), 9)
    O, _ = oracle.attn_fwd(q, k, v, win, 0.3)
    Od, _ = oracle.attn_fwd(q, k, v, W(0, 0, 0, 0, oracle.DENSE), 0.3)
    np.testing.assert_allclose(O, Od, atol=1e-12)


def test_zero_query_closed_form():
    # q = 0: every visible score is 0, so LSE_i = log(#visible keys) and O_i is the mean
    # of the visible values (counts from interval arithmetic, not from the mask)
    Lq, Lk, Hq, Hkv, D = 70, 150, 4, 2, 8
    sink, near = 6, 13
    win = W.for_length(Lk, Hkv, sink, near, 0)
    q = torch.zeros((1, Lq, Hq, D), dtype=torch.float64)
    k, v = _rand((1, Lk, Hkv, D), 10), _rand((1, Lk, Hkv, D), 11)
    O, LSE = oracle.attn_fwd(q, k, v, win, 1.0)
    for qh in range(Hq):
        h = qh // 2
        n = row_counts(np.arange(Lq), Lq, Lk, h, sink, near, 0, win.lr, "complementary")
        np.testing.assert_allclose(LSE[0, qh], np.log(n), atol=1e-13)
    # mean of the visible values, checked on a few rows by explicit index lists
    for i in (0, 33, Lq - 1):
        p = i + Lk - Lq
        for h in range(Hkv):
            lo = near + h * win.lr
            keys = sorted(set(range(min(sink, p + 1))) | set(range(max(0, p - near + 1), p + 1))
                          | set(range(max(0, p - lo - win.lr + 1), max(0, p - lo + 1))))
            want = v[0, keys, h].mean(dim=0).numpy()
            np.testing.assert_allclose(O[0, i, 2 * h], want, atol=1e-13)


def test_empty_rows_when_near_is_zero():
    L, D = 50, 4
    win = W(0, 0, 0, 10)  # band 0 starts at distance 0; head 1 sees nothing near
    q, k, v = _rand((1, L, 2, D), 12), _rand((1, L, 2, D), 13), _rand((1, L, 2, D), 14)
    O, LSE = oracle.attn_fwd(q, k, v, win, 1.0)
    # head 1's band is distances [10, 20): rows 0..9 see nothing
    assert np.all(O[0, :10, 1] == 0) and np.all(np.isneginf(LSE[0, 1, :10]))
    assert np.all(np.isfinite(LSE[0, 1, 10:]))


# ----------------------------------------------------------------------------- backward

def _loss(q, k, v, do, win, scale):
    O, _ = oracle.attn_fwd(q, k, v, win, scale)
    return float((O * do.numpy()).sum())


def test_bwd_finite_differences():
    Lq, Lk, Hq, Hkv, D = 12, 12, 4, 2, 4
    win = W.for_length(Lk, Hkv, 2, 3, 0)
    scale = 0.7
    q, k, v = _rand((1, Lq, Hq, D), 20), _rand((1, Lk, Hkv, D), 21), _rand((1, Lk, Hkv, D), 22)
    do = _rand((1, Lq, Hq, D), 23)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, win, scale)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros(x.shape)
        flat = x.reshape(-1)
        for idx in range(flat.numel()):
            old = float(flat[idx])
            flat[idx] = old + eps
            fp = _loss(q, k, v, do, win, scale)
            flat[idx] = old - eps
            fm = _loss(q, k, v, do, win, scale)
            flat[idx] = old
            num.reshape(-1)[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=2e-8, err_msg=name)


def test_bwd_matches_autograd_of_textbook_attention():
    Lq, Lk, Hq, Hkv, D = 64, 64, 6, 2, 8
    win = W.for_length(Lk, Hkv, 4, 8, 0)
    scale = 1 / math.sqrt(D)
    q, k, v = _rand((1, Lq, Hq, D), 30), _rand((1, Lk, Hkv, D), 31), _rand((1, Lk, Hkv, D), 32)
    do = _rand((1, Lq, Hq, D), 33)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, win, scale)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = _sdpa(qa, ka, va, _masks(Lq, Lk, Hq, Hkv, win), scale)
    (o * do).sum().backward()
    np.testing.assert_allclose(dq, qa.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, ka.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, va.grad.numpy(), atol=1e-12)


def test_bwd_column_sum_identities():
    # sum_j dS_ij = 0 for every row, so sum_j dK_j = 0; sum_j P_ij = 1, so
    # sum_j dV_j = sum over the head's query heads and rows of dO_i
    Lq, Lk, Hq, Hkv, D = 80, 80, 6, 3, 8
    win = W.for_length(Lk, Hkv, 4, 8, 0)
    q, k, v = _rand((1, Lq, Hq, D), 40), _rand((1, Lk, Hkv, D), 41), _rand((1, Lk, Hkv, D), 42)
    do = _rand((1, Lq, Hq, D), 43)
    _, dk, dv = oracle.attn_bwd(q, k, v, do, win, 0.35)
    np.testing.assert_allclose(dk.sum(axis=1), 0, atol=1e-11)
    want = do.numpy().reshape(1, Lq, Hkv, Hq // Hkv, D).sum(axis=(1, 3))
    np.testing.assert_allclose(dv.sum(axis=1), want, atol=1e-11)


def test_bwd_row_and_column_subsets_match_full():
    Lq, Lk, Hq, Hkv, D = 70, 70, 4, 2, 8
    win = W.for_length(Lk, Hkv, 3, 9, 0)
    q, k, v = _rand((1, Lq, Hq, D), 50), _rand((1, Lk, Hkv, D), 51), _rand((1, Lk, Hkv, D), 52)
    do = _rand((1, Lq, Hq, D), 53)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, win, 0.5)
    rows = [0, 5, 33, 69]
    cols = [0, 2, 3, 40, 69]
    np.testing.assert_allclose(oracle.attn_bwd_dq_rows(q, k, v, do, win, 0.5, rows),
                               dq[:, rows], atol=1e-12)
    for chunk, workers in ((16, 1), (7, 4), (256, 1)):
        dkc, dvc = oracle.attn_bwd_dkdv_cols(q, k, v, do, win, 0.5, cols, row_chunk=chunk,
                                             workers=workers)
        np.testing.assert_allclose(dkc, dk[:, cols], atol=1e-12)
        np.testing.assert_allclose(dvc, dv[:, cols], atol=1e-12)


# ----------------------------------------------------------------------------- decode

def test_decode_is_last_row_of_prefill_and_textbook():
    Lk, Hq, Hkv, D = 300, 8, 4, 16
    win = W.for_length(Lk, Hkv, 4, 20, 0)
    q, k, v = _rand((2, Lk, Hq, D), 60), _rand((2, Lk, Hkv, D), 61), _rand((2, Lk, Hkv, D), 62)
    O, LSE = oracle.attn_fwd(q, k, v, win, 0.25)
    Od, LSEd = oracle.decode(q[:, -1:], k, v, win, 0.25)
    np.testing.assert_allclose(Od[:, 0], O[:, -1], atol=1e-13)
    np.testing.assert_allclose(LSEd[:, :, 0], LSE[:, :, -1], atol=1e-13)
    ref = _sdpa(q[:, -1:], k, v, _masks(1, Lk, Hq, Hkv, win), 0.25)
    np.testing.assert_allclose(Od, ref.numpy(), atol=1e-12)


# ----------------------------------------------------------------------------- tiles

@pytest.mark.parametrize("Lq,Lk,Hkv,Bq,Bk,sink,near", [
    (1024, 1024, 2, 64, 64, 64, 128),
    (300, 300, 4, 64, 32, 5, 70),
    (1, 1000, 8, 64, 64, 16, 100),
    (200, 450, 2, 16, 128, 0, 1),
])
def test_tile_lists_cover_exactly_the_visible_elements(Lq, Lk, Hkv, Bq, Bk, sink, near):
    win = W.for_length(Lk, Hkv, sink, near, 0)
    lists = oracle.tile_lists(Lq, Lk, Hkv, Bq, Bk, win)
    for h in range(Hkv):
        m = oracle.full_mask(Lq, Lk, h, win)
        cover = np.zeros_like(m)
        for qb, ent in enumerate(lists[h]):
            kbs = [kb for kb, _ in ent]
            assert kbs == sorted(kbs)
            for kb, full in ent:
                t = m[qb * Bq:(qb + 1) * Bq, kb * Bk:(kb + 1) * Bk]
                assert t.any()
                assert full == (t.all() and t.shape == (Bq, Bk))
                cover[qb * Bq:(qb + 1) * Bq, kb * Bk:(kb + 1) * Bk] = True
        assert not (m & ~cover).any()  # nothing visible outside the listed tiles


def test_config1_tile_counts():
    # 1024 tokens, 2 KV heads, sink 64, near 128, 64x64 tiles: 121 + 79 visible tiles,
    # 57 of them partial (also derivable by hand from the band edges)
    win = W.for_length(1024, 2, 64, 128, 0)
    lists = oracle.tile_lists(1024, 1024, 2, 64, 64, win)
    per_head = [sum(len(e) for e in lists[h]) for h in range(2)]
    partial = sum(1 for h in range(2) for e in lists[h] for _, f in e if not f)
    assert per_head == [121, 79] and partial == 57


# ----------------------------------------------------------------------------- MALA

def _mala_inputs(Lq, Hq, Hkv, D, seed):
    return _rand((1, Lq, Hq, D), seed), _rand((1, Lq, Hkv, D), seed + 1), _rand((1, Lq, Hkv, D), seed + 2)


@pytest.mark.parametrize("mode", [oracle.DENSE, oracle.COMPLEMENTARY])
def test_mala_tau_zero_is_exact_attention(mode):
    """tau = 0 keeps every tile: MALA is then the textbook masked attention (torch SDPA in
    float64 with the explicit mask)."""
    L, Hq, Hkv, D = 70, 6, 2, 8
    win = W.for_length(L, Hkv, 3, 9, 0, mode=mode)
    q, k, v = _mala_inputs(L, Hq, Hkv, D, 70)
    O, LSE, kept = oracle.mala_fwd(q, k, v, win, 0.3, 0.0, 8, 16)
    assert kept.all()
    ref = _sdpa(q, k, v, _masks(L, L, Hq, Hkv, win), 0.3)
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-12)


def test_mala_tau_above_one_skips_every_tile():
    """A row's mass in a tile never exceeds 1, so tau > 1 skips every tile: O = 0, and LSE
    is still the logsumexp of the full scoring."""
    L, Hq, Hkv, D = 50, 4, 2, 8
    win = W.for_length(L, Hkv, 2, 6, 0, mode=oracle.DENSE)
    q, k, v = _mala_inputs(L, Hq, Hkv, D, 80)
    O, LSE, kept = oracle.mala_fwd(q, k, v, win, 0.25, 1.0001, 8, 8)
    assert not kept.any()
    assert np.all(O == 0)
    s = torch.einsum("bihd,bjhd->bhij", q, k.repeat_interleave(Hq // Hkv, dim=2)) * 0.25
    s = s.masked_fill(~torch.as_tensor(_masks(L, L, Hq, Hkv, win))[None], float("-inf"))
    np.testing.assert_allclose(LSE, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


def test_mala_brute_force_tiles_and_output():
    """Scalar loops over every tile, row and key: each row's probability (exp of the
    scaled score over the sum of exps of its visible keys), the tile's largest row mass,
    the keep decision at tau, and O as the sum over kept tiles of P v."""
    L, Hq, Hkv, D, Bq, Bk = 20, 4, 2, 4, 4, 4
    win = W.for_length(L, Hkv, 2, 5, 0, mode=oracle.DENSE)
    q, k, v = _mala_inputs(L, Hq, Hkv, D, 90)
    scale, tau = 0.6, 0.08
    G = Hq // Hkv
    qn, kn, vn = q.numpy(), k.numpy(), v.numpy()
    prob = np.zeros((Hq, L, L))
    for qh in range(Hq):
        h = qh // G
        for i in range(L):
            vis = [j for j in range(L) if j <= i]  # dense: causal
            ex = {j: math.exp(scale * sum(qn[0, i, qh, d] * kn[0, j, h, d] for d in range(D))) for j in vis}
            tot = sum(ex.values())
            for j in vis:
                prob[qh, i, j] = ex[j] / tot
    mass = oracle.mala_tile_mass(q, k, win, scale, Bq, Bk)
    O, _, kept = oracle.mala_fwd(q, k, v, win, scale, tau, Bq, Bk)
    want_O = np.zeros((L, Hq, D))
    for h in range(Hkv):
        for qb in range(L // Bq):
            for kb in range(L // Bk):
                rm = [sum(prob[qh, i, j] for j in range(kb * Bk, kb * Bk + Bk))
                      for qh in range(h * G, h * G + G) for i in range(qb * Bq, qb * Bq + Bq)]
                assert mass[h, qb, kb] == pytest.approx(max(rm), abs=1e-12)
                assert kept[h, qb, kb] == (max(rm) >= tau)
                if max(rm) >= tau:
                    for qh in range(h * G, h * G + G):
                        for i in range(qb * Bq, qb * Bq + Bq):
                            for j in range(kb * Bk, kb * Bk + Bk):
                                want_O[i, qh] += prob[qh, i, j] * vn[0, j, h]
    assert 0 < kept.sum() < kept.size
    np.testing.assert_allclose(O[0], want_O, atol=1e-12)


def test_mala_row_masses_sum_to_one_and_error_bound():
    """With one row per tile (a q-block of one token, one query head per KV head) the
    tile masses of a row are its probability split over the k-blocks: they sum to 1.  A
    row loses at most its dropped mass times max |v| per dimension."""
    L, H, D = 64, 2, 8
    win = W.for_length(L, H, 4, 8, 0)
    q, k, v = _mala_inputs(L, H, H, D, 100)
    mass = oracle.mala_tile_mass(q, k, win, 0.4, 1, 8)
    np.testing.assert_allclose(mass.sum(axis=2), 1.0, atol=1e-12)
    O, _, kept = oracle.mala_fwd(q, k, v, win, 0.4, 0.05, 1, 8)
    Oe, _ = oracle.attn_fwd(q, k, v, win, 0.4)
    dropped = (mass * ~kept).sum(axis=2)               # [H, L]
    err = np.abs(O - Oe).max(axis=3)[0]                 # [L, H]
    assert np.all(err <= dropped.T * np.abs(v.numpy()).max() + 1e-12)
    assert dropped.max() > 0


def test_mala_bwd_tau_zero_is_the_attention_backward():
    """With every tile kept the MALA gradients are those of masked attention (autograd of
    torch SDPA in float64)."""
    L, Hq, Hkv, D = 40, 4, 2, 8
    win = W.for_length(L, Hkv, 3, 6, 0, mode=oracle.DENSE)
    q, k, v = _mala_inputs(L, Hq, Hkv, D, 110)
    do = _rand((1, L, Hq, D), 113)
    kept = np.ones((Hkv, L // 8, L // 8), dtype=bool)
    dq, dk, dv = oracle.mala_bwd(q, k, v, do, win, 0.3, 8, 8, kept)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    (_sdpa(qa, ka, va, _masks(L, L, Hq, Hkv, win), 0.3) * do).sum().backward()
    np.testing.assert_allclose(dq, qa.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, ka.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, va.grad.numpy(), atol=1e-12)


def test_mala_bwd_finite_differences_with_fixed_decisions():
    """Central finite differences of sum(O * dO) for the MALA forward with its decisions
    held fixed (taken once at tau = 0.12, several tiles skipped)."""
    L, Hq, Hkv, D, Bq, Bk = 16, 2, 1, 4, 4, 4
    win = W.for_length(L, Hkv, 1, 3, 0, mode=oracle.DENSE)
    q, k, v = _mala_inputs(L, Hq, Hkv, D, 120)
    do = _rand((1, L, Hq, D), 123)
    scale = 0.8
    _, _, kept = oracle.mala_fwd(q, k, v, win, scale, 0.12, Bq, Bk)
    assert 0 < (~kept).sum()
    dq, dk, dv = oracle.mala_bwd(q, k, v, do, win, scale, Bq, Bk, kept)

    def loss(q_, k_, v_):
        O, _, _ = oracle.mala_fwd(q_, k_, v_, win, scale, 0.12, Bq, Bk, kept=kept)
        return float((O * do.numpy()).sum())

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros(x.shape)
        flat = x.reshape(-1)
        for idx in range(flat.numel()):
            old = float(flat[idx])
            flat[idx] = old + eps
            fp = loss(q, k, v)
            flat[idx] = old - eps
            fm = loss(q, k, v)
            flat[idx] = old
            num.reshape(-1)[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=2e-8, err_msg=name)


@pytest.mark.parametrize("mode", [oracle.COMPLEMENTARY, oracle.DENSE])
def test_mala_bwd_row_and_column_subsets_match_the_full_backward(mode):
    """The sampled MALA gradients (dQ on rows, dK/dV on key columns) equal the rows and
    columns of the full mala_bwd, under decisions that skip tiles (taken at tau = 0.1)
    and under an arbitrary keep pattern; chunked and threaded column gathers agree."""
    L, Hq, Hkv, D, Bq, Bk = 48, 4, 2, 8, 6, 8
    win = W.for_length(L, Hkv, 3, 9, 0, mode=mode)
    q, k, v = _mala_inputs(L, Hq, Hkv, D, 130)
    do = _rand((1, L, Hq, D), 133)
    scale = 0.5
    _, _, kept_tau = oracle.mala_fwd(q, k, v, win, scale, 0.1, Bq, Bk)
    assert 0 < (~kept_tau).sum() and kept_tau.sum() > 0
    rng = np.random.default_rng(7)
    for kept in (kept_tau, rng.random(kept_tau.shape) < 0.5):
        dq, dk, dv = oracle.mala_bwd(q, k, v, do, win, scale, Bq, Bk, kept)
        rows = [0, 1, 5, 6, 17, 30, 47]
        cols = [0, 2, 3, 8, 20, 39, 46, 47]
        np.testing.assert_allclose(oracle.mala_bwd_dq_rows(q, k, v, do, win, scale, Bq, Bk, kept, rows),
                                   dq[:, rows], atol=1e-12)
        for chunk, workers in ((256, 1), (5, 3)):
            rk, rv = oracle.mala_bwd_dkdv_cols(q, k, v, do, win, scale, Bq, Bk, kept, cols,
                                               row_chunk=chunk, workers=workers)
            np.testing.assert_allclose(rk, dk[:, cols], atol=1e-12)
            np.testing.assert_allclose(rv, dv[:, cols], atol=1e-12)
