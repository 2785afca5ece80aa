"""Plain CPU oracle of CoWindow Attention (CoWA) — TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The GPU library never calls it, and this module
imports nothing from the GPU library: the two share no code, no headers and no
constants.  Everything here is plain NumPy in float64, written from the pages'
description of the method, step by step, with no blocking or fusion beyond what the
definition states.

What the method computes (the pages' description, restated):

* CoWindow Attention: Full Causal Coverage Is a Collective Property — abstract (as
  carried on the crimsonlingua.com and humanity-list.pdj.dev pages) and the
  slinene.github.io ai-papers-daily page, section "method key points" (方法关键点):
  every KV head keeps a near-diagonal window of recent context and a prefix-sink window
  at the start of the sequence, both shared by all heads; the history left beyond the
  near window is split at breakpoints into equal-width long-range windows, one per KV
  head, so each head is dense nearby and sparse far away while the union over heads
  covers the whole causal prefix.
* Same page, method key point 2: one bottom-right-aligned causal distance defines
  training, prefill and decoding; a window is the quadruple
  (sink width, near width, gap, long-range width).
* Same page, method key point 3: windows follow the global KV-head index; the
  traversal skips KV blocks that are invisible.

The attention itself is exact masked softmax attention under that fixed mask (the
method saves work by skipping masked keys, not by approximating), so the oracle is the
plain definition: build the mask element by element, then softmax(scale q k^T) v over
the visible keys in float64.

Readings where the pages are silent:
  distance       d = i + (Lk - Lq) - j  (bottom-right alignment); causal iff d >= 0
  sink           absolute key index j < sink, shared by all heads, still causal
  near           0 <= d < near (half-open, includes the diagonal)
  gap            distances [near, near + gap) belong to no band
  bands          head h owns distances [near + gap + h*lr, near + gap + (h+1)*lr),
                 lr = ceil((Lmax - near - gap) / Hkv); "duplicated" gives every head
                 band 0; "dense" widens every band to all larger distances
  overlaps       the mask is the OR of the three windows (a key counts once)
  GQA            query head q reads KV head q // (Hq // Hkv)
  LSE            natural log of sum over visible keys of exp(scale * q.k)
  empty row      O = 0, LSE = -inf (only possible when near = 0)

Every function here is pinned by tests that do not re-use its formulas: textbook
dense attention (torch SDPA in float64) for the dense special case, brute-force loops on
tiny inputs, finite differences for the gradients, coverage / disjointness / width
invariants of the mask, and edge counts from an independent interval-arithmetic count.
"""

import math

import numpy as np

COMPLEMENTARY = "complementary"
DUPLICATED = "duplicated"
DENSE = "dense"
MODES = (COMPLEMENTARY, DUPLICATED, DENSE)


# --------------------------------------------------------------------------- window

def complementary_width(Lmax, Hkv, near, gap):
    """Width of each long-range band: the history beyond near (+gap) up to the longest
    distance Lmax split into Hkv equal widths (method key point 1, "equal widths";
    ceiling so that the Hkv bands reach Lmax)."""
    rest = Lmax - near - gap
    if rest <= 0:
        return 0
    return -(-rest // Hkv)


class Window:
    """The quadruple (sink, near, gap, lr) of method key point 2, plus the band mode."""

    def __init__(self, sink, near, gap, lr, mode=COMPLEMENTARY):
        assert mode in MODES
        assert min(sink, near, gap, lr) >= 0
        self.sink, self.near, self.gap, self.lr, self.mode = sink, near, gap, lr, mode

    @classmethod
    def for_length(cls, Lmax, Hkv, sink, near, gap=0, mode=COMPLEMENTARY):
        return cls(sink, near, gap, complementary_width(Lmax, Hkv, near, gap), mode)

    def band(self, h):
        """Distances [lo, hi) of KV head h's long-range window (hi = None: unbounded)."""
        start = self.near + self.gap
        if self.mode == DENSE:
            return start, None
        slot = h if self.mode == COMPLEMENTARY else 0
        lo = start + slot * self.lr
        return lo, lo + self.lr

    def __repr__(self):
        return (f"Window(sink={self.sink}, near={self.near}, gap={self.gap}, "
                f"lr={self.lr}, mode={self.mode})")


def mask_rows(rows, Lq, Lk, h, win, keys=None):
    """Boolean mask [len(rows), len(keys)]: key j visible to query row i under KV head h
    (keys default to all Lk keys).

    Evaluated element by element on the (i, j) grid from the definition — no interval
    arithmetic — so it stays independent of any block planner."""
    # int32 holds every index and distance of sequences up to 2^30 tokens
    it = np.int32 if Lq + Lk < 2 ** 30 else np.int64
    i = np.asarray(rows, dtype=it)[:, None]
    j = (np.arange(Lk, dtype=it) if keys is None else np.asarray(keys, dtype=it))[None, :]
    d = (i + it(Lk - Lq)) - j
    causal = d >= 0
    in_sink = j < win.sink
    in_near = d < win.near
    lo, hi = win.band(h)
    in_band = d >= lo
    if hi is not None:
        in_band = in_band & (d < hi)
    return causal & (in_sink | in_near | in_band)


def full_mask(Lq, Lk, h, win):
    return mask_rows(np.arange(Lq), Lq, Lk, h, win)


# --------------------------------------------------------------------------- forward

def _f64(x):
    """Upcast (exactly) to float64 NumPy; accepts NumPy arrays or torch CPU tensors."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # only for the dtype conversion of torch inputs
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _take_rows(x, rows):
    """x[:, rows] for a NumPy array or a torch tensor (no arithmetic)."""
    if hasattr(x, "detach"):
        import torch
        return x[:, torch.as_tensor(rows, dtype=torch.long)]
    return np.asarray(x)[:, rows]


def _masked_softmax_row_stats(s, m):
    """Probabilities and logsumexp of the rows of a masked score matrix s [R, K] (s is
    overwritten with the probabilities): hidden entries are set to -inf, the row max is
    subtracted, exp (exactly 0 at -inf), divided by the row sum.  A row with no visible
    entry gets P = 0 and LSE = -inf."""
    np.copyto(s, -np.inf, where=~m)
    mx = s.max(axis=1, keepdims=True)
    empty = ~np.isfinite(mx)
    mx[empty] = 0.0
    s -= mx
    np.exp(s, out=s)
    den = s.sum(axis=1, keepdims=True)
    safe = np.where(den > 0, den, 1.0)
    s /= safe
    lse = np.where(den > 0, mx + np.log(safe), -np.inf)
    return s, lse[:, 0]


def attn_fwd(q, k, v, win, scale, rows=None):
    """Masked-softmax attention forward on query rows `rows` (default: all).

    q [B, Lq, Hq, D], k/v [B, Lk, Hkv, D]  ->  O [B, R, Hq, D], LSE [B, Hq, R]
    For query head qh (KV head h = qh // G): s_ij = scale q_i.k_j, masked to the
    visible keys; O_i = sum_j softmax(s)_ij v_j; LSE_i = log sum_j exp(s_ij)."""
    B, Lq, Hq, D = q.shape
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    q = _f64(_take_rows(q, rows))  # only the requested rows are upcast
    k, v = _f64(k), _f64(v)
    _, Lk, Hkv, _ = k.shape
    G = Hq // Hkv
    O = np.zeros((B, len(rows), Hq, D))
    LSE = np.zeros((B, Hq, len(rows)))
    for h in range(Hkv):
        m = mask_rows(rows, Lq, Lk, h, win)
        for b in range(B):
            for qh in range(h * G, (h + 1) * G):
                s = scale * (q[b, :, qh, :] @ k[b, :, h, :].T)
                p, lse = _masked_softmax_row_stats(s, m)
                O[b, :, qh, :] = p @ v[b, :, h, :]
                LSE[b, qh, :] = lse
    return O, LSE


# --------------------------------------------------------------------------- backward

def attn_bwd(q, k, v, do, win, scale):
    """Full gradients of L = sum(O * dO) for the forward above (all rows).

    P = softmax of the masked scores; Delta_i = dO_i . O_i; dP_ij = dO_i . v_j;
    dS_ij = P_ij (dP_ij - Delta_i); dQ_i = scale sum_j dS_ij k_j;
    dK_j = scale sum over the KV head's query heads and rows of dS_ij q_i;
    dV_j = sum over the same of P_ij dO_i.
    Returns (dQ [B,Lq,Hq,D], dK [B,Lk,Hkv,D], dV [B,Lk,Hkv,D])."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Lq, Hq, D = q.shape
    _, Lk, Hkv, _ = k.shape
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(Hkv):
        m = full_mask(Lq, Lk, h, win)
        for b in range(B):
            for qh in range(h * G, (h + 1) * G):
                s = scale * (q[b, :, qh, :] @ k[b, :, h, :].T)
                p, _ = _masked_softmax_row_stats(s, m)
                o = p @ v[b, :, h, :]
                delta = (do[b, :, qh, :] * o).sum(axis=1, keepdims=True)
                dp = do[b, :, qh, :] @ v[b, :, h, :].T
                ds = p * (dp - delta)
                dq[b, :, qh, :] = scale * (ds @ k[b, :, h, :])
                dk[b, :, h, :] += scale * (ds.T @ q[b, :, qh, :])
                dv[b, :, h, :] += p.T @ do[b, :, qh, :]
    return dq, dk, dv


def attn_bwd_dq_rows(q, k, v, do, win, scale, rows):
    """dQ on the query rows `rows` only: needs just those rows' own softmax and
    Delta_i = dO_i . O_i with O_i from the rows' own forward.  -> [B, R, Hq, D]"""
    B, Lq, Hq, D = q.shape
    rows = np.asarray(rows, dtype=np.int64)
    q, do = _f64(_take_rows(q, rows)), _f64(_take_rows(do, rows))
    k, v = _f64(k), _f64(v)
    _, Lk, Hkv, _ = k.shape
    G = Hq // Hkv
    dq = np.zeros((B, len(rows), Hq, D))
    for h in range(Hkv):
        m = mask_rows(rows, Lq, Lk, h, win)
        for b in range(B):
            for qh in range(h * G, (h + 1) * G):
                s = scale * (q[b, :, qh, :] @ k[b, :, h, :].T)
                p, _ = _masked_softmax_row_stats(s, m)
                o = p @ v[b, :, h, :]
                delta = (do[b, :, qh, :] * o).sum(axis=1, keepdims=True)
                dp = do[b, :, qh, :] @ v[b, :, h, :].T
                ds = p * (dp - delta)
                dq[b, :, qh, :] = scale * (ds @ k[b, :, h, :])
    return dq


def attn_bwd_dkdv_cols(q, k, v, do, win, scale, cols, row_chunk=256, workers=1):
    """dK and dV on the key columns `cols` only.

    A column j receives from every query row that sees it, so those rows are found from
    the explicit mask evaluated at the requested columns, and each such row's full
    softmax (over all of its visible keys) is computed before its contribution to the
    requested columns is summed.  Per chunk of rows the products run over the keys that
    some row of the chunk sees (the mask on the full key range says which); every other
    key has probability exactly 0 for every row of the chunk and adds nothing.
    Chunks are independent; with workers > 1 they run in threads and their results are
    summed in chunk order.  -> dK [B, C, Hkv, D], dV [B, C, Hkv, D]"""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Lq, Hq, D = q.shape
    _, Lk, Hkv, _ = k.shape
    G = Hq // Hkv
    cols = np.asarray(cols, dtype=np.int64)

    def chunk_part(h, rows):
        dk = np.zeros((B, len(cols), D))
        dv = np.zeros((B, len(cols), D))
        m = mask_rows(rows, Lq, Lk, h, win)
        keys = np.nonzero(m.any(axis=0))[0]
        m = m[:, keys]
        at = np.searchsorted(keys, cols)  # requested columns inside `keys`
        seen = (at < len(keys)) & (keys[np.minimum(at, len(keys) - 1)] == cols)
        for b in range(B):
            kk, vv = k[b, keys, h, :], v[b, keys, h, :]
            for qh in range(h * G, (h + 1) * G):
                s = scale * (q[b, rows, qh, :] @ kk.T)
                p, _ = _masked_softmax_row_stats(s, m)
                o = p @ vv
                delta = (do[b, rows, qh, :] * o).sum(axis=1, keepdims=True)
                pc = np.where(seen[None, :], p[:, np.minimum(at, len(keys) - 1)], 0.0)
                dpc = do[b, rows, qh, :] @ v[b, cols, h, :].T
                dsc = pc * (dpc - delta)
                dk[b] += scale * (dsc.T @ q[b, rows, qh, :])
                dv[b] += pc.T @ do[b, rows, qh, :]
        return h, dk, dv

    tasks = []
    for h in range(Hkv):
        # rows that see at least one requested column
        need = mask_rows(np.arange(Lq), Lq, Lk, h, win, keys=cols).any(axis=1)
        rows_all = np.nonzero(need)[0]
        for start in range(0, len(rows_all), row_chunk):
            tasks.append((h, rows_all[start:start + row_chunk]))
    if workers > 1:
        # one BLAS thread per worker: the workers already fill the cores
        from concurrent.futures import ThreadPoolExecutor
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
            parts = list(ex.map(lambda t: chunk_part(*t), tasks))
    else:
        parts = [chunk_part(*t) for t in tasks]
    dk = np.zeros((B, len(cols), Hkv, D))
    dv = np.zeros((B, len(cols), Hkv, D))
    for h, pk, pv in parts:
        dk[:, :, h, :] += pk
        dv[:, :, h, :] += pv
    return dk, dv


# --------------------------------------------------------------------------- decode

def decode(q, k_cache, v_cache, win, scale):
    """One new query token per sequence over a cache of Lk positions holding the new
    token; the query is at position Lk - 1, i.e. the forward with Lq = 1 under the same
    bottom-right distance (method key point 2).  q [B, 1, Hq, D] -> O [B, 1, Hq, D],
    LSE [B, Hq, 1]."""
    return attn_fwd(q, k_cache, v_cache, win, scale, rows=[0])


# --------------------------------------------------------------------------- MALA

# MassAlloc Attention, the companion operator the pages describe alongside CoWA
# (beyondmarketintelligence.com post, second paragraph and takeaway; crimsonlingua.com
# news item, fifth paragraph): it keeps the full QK scoring of causal attention and uses
# the softmax's own statistics to decide whether the rest of a tile's computation is
# done, skipping it in low-contribution regions.  Readings taken here (the pages give no
# formula): the statistics are the exact row statistics of the full scoring (the softmax
# over every visible key); the contribution of a tile (KV head h, q-block of Bq tokens
# times the G query heads of h, k-block of Bk keys) to a row is the row's probability
# mass in the tile's keys; the tile is skipped when that mass is below tau for every row
# of the tile, and a skipped tile adds nothing to O while the denominator stays the full
# one (O_i = sum over kept tiles of P_ij v_j, P the full softmax).  tau = 0 keeps every
# tile: exact attention.

def _mala_rows(q, k, win, scale, h, rows, G, Lq):
    """Full-softmax probabilities P [G, R, Lk] of the given rows under KV head h."""
    m = mask_rows(rows, Lq, k.shape[1], h, win)
    P = []
    for qh in range(h * G, (h + 1) * G):
        s = scale * (q[0, rows, qh, :] @ k[0, :, h, :].T)
        p, _ = _masked_softmax_row_stats(s, m)
        P.append(p)
    return np.stack(P)


def mala_tile_mass(q, k, win, scale, Bq, Bk, qblocks=None):
    """Largest row mass of every tile: mass[h, qb, kb] = max over the tile's rows (its Bq
    tokens and G query heads) of sum over the tile's keys of P_ij.  B must be 1.  With
    `qblocks`, only those q-blocks are filled (the others stay 0)."""
    q, k = _f64(q), _f64(k)
    B, Lq, Hq, D = q.shape
    _, Lk, Hkv, _ = k.shape
    assert B == 1
    G = Hq // Hkv
    nqb, nkb = -(-Lq // Bq), -(-Lk // Bk)
    mass = np.zeros((Hkv, nqb, nkb))
    for h in range(Hkv):
        for qb in (range(nqb) if qblocks is None else qblocks):
            rows = np.arange(qb * Bq, min(Lq, (qb + 1) * Bq))
            P = _mala_rows(q, k, win, scale, h, rows, G, Lq)
            for kb in range(nkb):
                mass[h, qb, kb] = P[:, :, kb * Bk:(kb + 1) * Bk].sum(axis=2).max()
    return mass


def mala_fwd(q, k, v, win, scale, tau, Bq, Bk, kept=None, qblocks=None):
    """MALA forward: O [1, Lq, Hq, D] and the full LSE [1, Hq, Lq]; kept[h, qb, kb]
    (bool) is taken from the tile masses (mass >= tau) unless given.  With `qblocks`, only
    the rows of those q-blocks are computed (O and LSE stay 0 elsewhere).
    -> O, LSE, kept"""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Lq, Hq, D = q.shape
    _, Lk, Hkv, _ = k.shape
    assert B == 1
    G = Hq // Hkv
    nqb = -(-Lq // Bq)
    qbs = list(range(nqb)) if qblocks is None else list(qblocks)
    if kept is None:
        kept = mala_tile_mass(q, k, win, scale, Bq, Bk, qblocks=qblocks) >= tau
    rows_all = np.concatenate([np.arange(qb * Bq, min(Lq, (qb + 1) * Bq)) for qb in qbs])
    LSE = np.zeros((1, Hq, Lq))
    LSE[:, :, rows_all] = attn_fwd(q, k, v, win, scale, rows=rows_all)[1]
    O = np.zeros((1, Lq, Hq, D))
    for h in range(Hkv):
        for qb in qbs:
            rows = np.arange(qb * Bq, min(Lq, (qb + 1) * Bq))
            P = _mala_rows(q, k, win, scale, h, rows, G, Lq)
            keep_keys = np.repeat(np.asarray(kept[h, qb], dtype=bool), Bk)[:Lk]
            for gi, qh in enumerate(range(h * G, (h + 1) * G)):
                O[0, rows, qh, :] = (P[gi] * keep_keys[None, :]) @ v[0, :, h, :]
    return O, LSE, kept


def mala_bwd(q, k, v, do, win, scale, Bq, Bk, kept):
    """Gradients of L = sum(O * dO) for the MALA forward with the tile decisions `kept`
    held fixed (the function is smooth for fixed decisions): with P the full softmax and
    K_ij = 1 where key j lies in a kept tile of row i,
      dP_ij = K_ij dO_i . v_j,  Delta_i = sum_j P_ij dP_ij (= dO_i . O_i),
      dS_ij = P_ij (dP_ij - Delta_i),  dV_j = sum_i K_ij P_ij dO_i,
      dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i
    (a skipped tile still passes -P Delta to dQ and dK through the full denominator).
    B must be 1.  -> (dQ, dK, dV)"""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Lq, Hq, D = q.shape
    _, Lk, Hkv, _ = k.shape
    assert B == 1
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    nqb = -(-Lq // Bq)
    for h in range(Hkv):
        for qb in range(nqb):
            rows = np.arange(qb * Bq, min(Lq, (qb + 1) * Bq))
            P = _mala_rows(q, k, win, scale, h, rows, G, Lq)
            keep_keys = np.repeat(np.asarray(kept[h, qb], dtype=np.float64), Bk)[:Lk]
            for gi, qh in enumerate(range(h * G, (h + 1) * G)):
                p = P[gi]
                dp = (do[0, rows, qh, :] @ v[0, :, h, :].T) * keep_keys[None, :]
                delta = (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - delta)
                dq[0, rows, qh, :] = scale * (ds @ k[0, :, h, :])
                dk[0, :, h, :] += scale * (ds.T @ q[0, rows, qh, :])
                dv[0, :, h, :] += (p * keep_keys[None, :]).T @ do[0, rows, qh, :]
    return dq, dk, dv


def _kept_keys(kept, h, rows, Bq, Bk, keys):
    """K_ij of the MALA backward for the given rows and keys: 1.0 where key j lies in a
    kept tile (KV head h, forward q-block i // Bq, key block j // Bk), else 0.0."""
    return np.asarray(kept[h][np.ix_(np.asarray(rows) // Bq, np.asarray(keys) // Bk)], dtype=np.float64)


def mala_bwd_dq_rows(q, k, v, do, win, scale, Bq, Bk, kept, rows):
    """dQ of mala_bwd on the query rows `rows` only: each row needs just its own full
    softmax, its kept keys and Delta_i = sum_j P_ij dP_ij.  B must be 1.  -> [1, R, Hq, D]"""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Lq, Hq, D = q.shape
    _, Lk, Hkv, _ = k.shape
    assert B == 1
    G = Hq // Hkv
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.arange(Lk)
    dq = np.zeros((1, len(rows), Hq, D))
    for h in range(Hkv):
        P = _mala_rows(q, k, win, scale, h, rows, G, Lq)
        kk = _kept_keys(kept, h, rows, Bq, Bk, keys)
        for gi, qh in enumerate(range(h * G, (h + 1) * G)):
            p = P[gi]
            dp = (do[0, rows, qh, :] @ v[0, :, h, :].T) * kk
            delta = (p * dp).sum(axis=1, keepdims=True)
            dq[0, :, qh, :] = scale * ((p * (dp - delta)) @ k[0, :, h, :])
    return dq


def mala_bwd_dkdv_cols(q, k, v, do, win, scale, Bq, Bk, kept, cols, row_chunk=256, workers=1):
    """dK and dV of mala_bwd on the key columns `cols` only, the way attn_bwd_dkdv_cols
    gathers them: the rows that see a requested column are found from the mask, and per
    chunk of such rows their full softmax over the keys the chunk sees, their kept keys
    K_ij and Delta_i = dO_i . O_i with O_i = sum_j K_ij P_ij v_j (the MALA output) give
      dS_ij = P_ij (K_ij dO_i . v_j - Delta_i),  dV_j = sum_i K_ij P_ij dO_i.
    B must be 1.  -> dK [1, C, Hkv, D], dV [1, C, Hkv, D]"""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Lq, Hq, D = q.shape
    _, Lk, Hkv, _ = k.shape
    assert B == 1
    G = Hq // Hkv
    cols = np.asarray(cols, dtype=np.int64)

    def chunk_part(h, rows):
        dk = np.zeros((len(cols), D))
        dv = np.zeros((len(cols), D))
        m = mask_rows(rows, Lq, Lk, h, win)
        keys = np.nonzero(m.any(axis=0))[0]
        m = m[:, keys]
        at = np.searchsorted(keys, cols)
        seen = (at < len(keys)) & (keys[np.minimum(at, len(keys) - 1)] == cols)
        kk = _kept_keys(kept, h, rows, Bq, Bk, keys)
        kc = _kept_keys(kept, h, rows, Bq, Bk, cols)
        ks, vs = k[0, keys, h, :], v[0, keys, h, :]
        for qh in range(h * G, (h + 1) * G):
            s = scale * (q[0, rows, qh, :] @ ks.T)
            p, _ = _masked_softmax_row_stats(s, m)
            o = (p * kk) @ vs
            delta = (do[0, rows, qh, :] * o).sum(axis=1, keepdims=True)
            pc = np.where(seen[None, :], p[:, np.minimum(at, len(keys) - 1)], 0.0)
            dpc = (do[0, rows, qh, :] @ v[0, cols, h, :].T) * kc
            dsc = pc * (dpc - delta)
            dk += scale * (dsc.T @ q[0, rows, qh, :])
            dv += (pc * kc).T @ do[0, rows, qh, :]
        return h, dk, dv

    tasks = []
    for h in range(Hkv):
        need = mask_rows(np.arange(Lq), Lq, Lk, h, win, keys=cols).any(axis=1)
        rows_all = np.nonzero(need)[0]
        for start in range(0, len(rows_all), row_chunk):
            tasks.append((h, rows_all[start:start + row_chunk]))
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
            parts = list(ex.map(lambda t: chunk_part(*t), tasks))
    else:
        parts = [chunk_part(*t) for t in tasks]
    dk = np.zeros((1, len(cols), Hkv, D))
    dv = np.zeros((1, len(cols), Hkv, D))
    for h, pk, pv in parts:
        dk[0, :, h, :] += pk
        dv[0, :, h, :] += pv
    return dk, dv


# --------------------------------------------------------------------------- tiles

def tile_lists(Lq, Lk, Hkv, Bq, Bk, win):
    """Per KV head and q-block, the visible k-blocks with their FULL flag, read off
    the explicit mask: a tile is listed iff ANY of its elements is visible, and FULL
    iff every one of its Bq x Bk elements is in range and visible (method key point 3:
    only visible blocks are traversed).  -> lists[h][qb] = [(kb, full), ...] ascending."""
    nqb = -(-Lq // Bq)
    nkb = -(-Lk // Bk)
    out = []
    for h in range(Hkv):
        per_h = []
        for qb in range(nqb):
            rows = np.arange(qb * Bq, min(Lq, (qb + 1) * Bq))
            m = mask_rows(rows, Lq, Lk, h, win)
            ent = []
            for kb in range(nkb):
                t = m[:, kb * Bk:min(Lk, (kb + 1) * Bk)]
                if t.any():
                    full = bool(t.all()) and t.shape == (Bq, Bk)
                    ent.append((kb, full))
            per_h.append(ent)
        out.append(per_h)
    return out


def edge_counts(Lq, Lk, Hkv, win, row_chunk=256):
    """Visible (query row, key) pairs per KV head, counted on the explicit mask."""
    counts = []
    for h in range(Hkv):
        c = 0
        for start in range(0, Lq, row_chunk):
            r = np.arange(start, min(Lq, start + row_chunk))
            c += int(mask_rows(r, Lq, Lk, h, win).sum())
        counts.append(c)
    return counts


def default_scale(D):
    return 1.0 / math.sqrt(D)
