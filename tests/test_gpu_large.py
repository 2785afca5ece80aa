"""GPU parity at the 32K- and 128K-token workloads, in the launch configuration the
benchmark times: seeded stratified row samples against the CPU oracle, plus identities
that hold at any size (column sums of dK and dV, decode == last forward row).

Inputs are drawn on the device with the same recipe as the small tests (seeded randn in
float32, cast to bf16) and copied to the host for the oracle."""

import os
import sys
import time

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))
import oracle  # noqa: E402
from gpu_helpers import assert_bf16_close, sample_rows  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from structured_sparse_attention_plan_amd import api, inputs  # noqa: E402

DEV = "cuda:0"
HQ, HKV, D = 40, 8, 128
SCALE = D ** -0.5


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _setup(L, sink, near, mode="complementary", seed=0, with_dout=False):
    ow = oracle.Window.for_length(L, HKV, sink, near, 0, mode=mode)
    win = api.window(ow.sink, ow.near, ow.gap, ow.lr, mode)
    t = inputs.attention_inputs(1, L, L, HQ, HKV, D, seed=seed, device=DEV, with_dout=with_dout)
    return ow, win, t


@pytest.mark.parametrize("mode", ["complementary", "duplicated", "dense"])
def test_fwd_32k_sampled_rows(mode):
    _case(f"fwd 32K {mode}, 256 sampled rows")
    L, sink, near = 32768, 128, 2048
    ow, win, (q, k, v) = _setup(L, sink, near, mode, seed=10)
    o, lse = api.fwd(q, k, v, win)
    torch.cuda.synchronize()
    rows = sample_rows(L, sink, near, ow.lr, HKV, 256 // 5, 256, seed=100)
    Oo, Lo = oracle.attn_fwd(q.cpu(), k.cpu(), v.cpu(), ow, SCALE, rows=rows)
    idx = torch.as_tensor(rows, device=DEV)
    assert_bf16_close("O", o[:, idx], Oo)
    assert_bf16_close("LSE", lse[:, :, idx], Lo)


def _rounding_sigma(x):
    """Standard deviation, per (KV head, dim), of the sum over keys of the bf16 rounding
    errors of x [1, L, Hkv, D]: an element in [2^e, 2^(e+1)) has ulp 2^(e-7)."""
    a = x.double().abs()[0]
    e = torch.floor(torch.log2(torch.where(a > 0, a, torch.ones_like(a))))
    ulp = torch.where(a > 0, torch.pow(2.0, e - 7), torch.zeros_like(a))
    return (ulp.pow(2).sum(dim=0) / 12).sqrt()


def _workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _cols_check(name, dk, dv, cols, want_k, want_v):
    idx = torch.as_tensor(np.asarray(cols), device=dk.device)
    assert_bf16_close(f"dK[{name} columns]", dk[:, idx], want_k, gradient=True)
    assert_bf16_close(f"dV[{name} columns]", dv[:, idx], want_v, gradient=True)


# 32K key columns: the prefix sink (every row sees it, so its check needs the softmax of
# every row; all other columns then come at no extra cost), k-block edges of the backward
# (128 keys), columns whose last row sits at a band edge of heads 1, 4 and 7
# (L - 1 - (near + h lr) and its neighbours), the near edge and the last keys.
def _cols_32k(L, near, lr, mode):
    edge = [L - 1 - (near + h * lr) + e for h in (1, 4, 7) for e in (-1, 0, 1)]
    tail = [L - 1 - near - 1, L - 1 - near, L - 1 - near + 1, L - 129, L - 128, L - 2, L - 1]
    if mode == "dense":
        # in dense mode the sink column is seen by every row over its whole causal
        # history (about 2e10 (row, key, head) triples, minutes on the host); columns in
        # the last near window need only the rows at and after them
        return sorted(set(tail))
    return sorted(set([0, 1, 63, 64, 127, 128, 129, 255, 256, 5000, 12345, 20000] + edge + tail))


@pytest.mark.parametrize("mode", ["complementary", "duplicated", "dense"])
def test_bwd_32k_key_columns_and_rows(mode):
    """The 32K forward + backward the coverage ablation times: dK/dV on seeded key
    columns and dQ on 256 stratified rows, element by element against the oracle."""
    L, sink, near = 32768, 128, 2048
    _case(f"bwd 32K {mode}: dK/dV key columns, dQ sampled rows")
    ow, win, (q, k, v, do) = _setup(L, sink, near, mode, seed=60, with_dout=True)
    o, lse, dq, dk, dv = api.fwd_bwd(q, k, v, do, win)
    torch.cuda.synchronize()
    qc, kc, vc, doc = q.cpu(), k.cpu(), v.cpu(), do.cpu()
    cols = _cols_32k(L, near, ow.lr, mode)
    t0 = time.time()
    rk, rv = oracle.attn_bwd_dkdv_cols(qc, kc, vc, doc, ow, SCALE, cols, workers=_workers())
    print(f"  oracle: {len(cols)} key columns in {time.time() - t0:.1f} s ({_workers()} threads)",
          flush=True)
    _cols_check("32K", dk, dv, cols, rk, rv)
    rows = sample_rows(L, sink, near, ow.lr, HKV, 128 // 5, 256, seed=100)
    dqo = oracle.attn_bwd_dq_rows(qc, kc, vc, doc, ow, SCALE, rows)
    assert_bf16_close("dQ[sampled rows]", dq[:, torch.as_tensor(rows, device=DEV)], dqo, gradient=True)


def _mala_kept_array(fplan, kept, L, Bk=64):
    """The MALA forward's per-entry decisions as the oracle's [Hkv, nqb, nkb] array
    (tiles outside the lists hold no visible key; their value does not matter)."""
    rp = np.asarray(fplan.host.arrays["row_ptr"])
    ent = np.asarray(fplan.host.arrays["row_ent"])
    nqb = fplan.info.nqb
    items = np.repeat(np.arange(len(rp) - 1), np.diff(rp))
    kg = kept.cpu().numpy()[:len(items)]
    assert set(np.unique(kg)) <= {0, 1}, "every listed tile gets a decision"
    out = np.ones((HKV, nqb, -(-L // Bk)), dtype=bool)
    out[items // nqb, items % nqb, ent[:len(items)] >> 1] = kg.astype(bool)
    return out, int(kg.sum()), len(items)


@pytest.mark.parametrize("mode,tau", [("complementary", 0.02), ("dense", 0.004)])
def test_mala_bwd_32k_key_columns_and_rows(mode, tau):
    """The MALA backward at 32K tokens under the kernel's own decisions: dK/dV on seeded
    key columns and dQ on 256 stratified rows against the oracle."""
    L, sink, near = 32768, 128, 2048
    _case(f"MALA bwd 32K {mode} tau={tau}: dK/dV key columns, dQ sampled rows")
    ow, win, (q, k, v, do) = _setup(L, sink, near, mode, seed=70, with_dout=True)
    prob = api.problem(1, L, L, HQ, HKV, D, torch.bfloat16, SCALE, win)
    fplan = api.build_plan("fwd", prob, DEV)
    kept = torch.full((max(1, fplan.info.nnz),), -1, dtype=torch.int32, device=DEV)
    o_lo = torch.empty_like(q)
    o, lse = api.mala_fwd(q, k, v, win, tau, plan=fplan, kept=kept, o_lo=o_lo)
    dq, dk, dv = api.mala_bwd(q, k, v, o, lse, do, kept, fplan, win, o_lo=o_lo)
    torch.cuda.synchronize()
    kept_np, n_kept, n_tiles = _mala_kept_array(fplan, kept, L)
    print(f"  {n_kept} of {n_tiles} tiles kept", flush=True)
    assert 0 < n_kept < n_tiles
    qc, kc, vc, doc = q.cpu(), k.cpu(), v.cpu(), do.cpu()
    Bq = fplan.info.Bq
    cols = _cols_32k(L, near, ow.lr, mode)
    t0 = time.time()
    rk, rv = oracle.mala_bwd_dkdv_cols(qc, kc, vc, doc, ow, SCALE, Bq, 64, kept_np, cols,
                                       workers=_workers())
    print(f"  oracle: {len(cols)} key columns in {time.time() - t0:.1f} s", flush=True)
    _cols_check("MALA 32K", dk, dv, cols, rk, rv)
    rows = sample_rows(L, sink, near, ow.lr, HKV, 128 // 5, 256, seed=101)
    dqo = oracle.mala_bwd_dq_rows(qc, kc, vc, doc, ow, SCALE, Bq, 64, kept_np, rows)
    assert_bf16_close("dQ[sampled rows]", dq[:, torch.as_tensor(rows, device=DEV)], dqo, gradient=True)


@pytest.fixture(scope="module")
def run_128k():
    """One forward + backward of the 131072-token workload, results copied to the host."""
    L, sink, near = 131072, 128, 4096
    ow, win, (q, k, v, do) = _setup(L, sink, near, seed=20, with_dout=True)
    o, lse, dq, dk, dv = api.fwd_bwd(q, k, v, do, win)
    torch.cuda.synchronize()
    print("  128K GPU pass done", flush=True)
    r = dict(L=L, sink=sink, near=near, ow=ow, q=q.cpu(), k=k.cpu(), v=v.cpu(), do=do.cpu(),
             o=o.cpu(), lse=lse.cpu(), dq=dq.cpu(), dk=dk.cpu(), dv=dv.cpu())
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return r


def test_fwd_bwd_128k_sampled_rows_and_identities(run_128k):
    _case("fwd+bwd 128K, 128 sampled rows + column-sum identities")
    r = run_128k
    L, ow = r["L"], r["ow"]
    dk, dv, do = r["dk"], r["dv"], r["do"]
    # exact identities: sum_j dK_j = 0 and sum_j dV_j = sum over the KV head's query heads
    # and rows of dO (both per KV head and dim)
    sk = dk.double().sum(dim=1)[0]                      # [Hkv, D]
    sv = dv.double().sum(dim=1)[0]
    sdo = do.double().sum(dim=1)[0].view(HKV, HQ // HKV, D).sum(dim=1)
    # tolerance: each stored element carries its own bf16 rounding, uniform in half an ulp
    # either side (variance ulp^2 / 12), independent from element to element; six standard
    # deviations of their sum per (head, dim) over the 1024 sums (the kernels' fp32 sums
    # and fp16 operands add far less), plus 1e-3 of the dO sum for dV
    sig_k = _rounding_sigma(dk)
    sig_v = _rounding_sigma(dv)
    ex_k = (sk.abs() / sig_k).max().item()
    ex_v = ((sv - sdo).abs() / (sig_v + 1e-3 / 6 * sdo.abs())).max().item()
    print(f"  max|sum dK|={sk.abs().max().item():.3e} ({ex_k:.2f} sigma); "
          f"max|sum dV - sum dO|={(sv - sdo).abs().max().item():.3e} ({ex_v:.2f} sigma)", flush=True)
    assert ex_k <= 6.0
    assert ex_v <= 6.0
    rows = sample_rows(L, r["sink"], r["near"], ow.lr, HKV, 128 // 5, 128, seed=100)
    Oo, Lo = oracle.attn_fwd(r["q"], r["k"], r["v"], ow, SCALE, rows=rows)
    idx = torch.as_tensor(rows)
    assert_bf16_close("O", r["o"][:, idx], Oo)
    assert_bf16_close("LSE", r["lse"][:, :, idx], Lo)
    dqo = oracle.attn_bwd_dq_rows(r["q"], r["k"], r["v"], do, ow, SCALE, rows)
    assert_bf16_close("dQ", r["dq"][:, idx], dqo, gradient=True)


@pytest.mark.parametrize("cluster", ["near_end", "band3_edge", "band456_edges", "band7_edge",
                                     "sink"])
def test_bwd_128k_key_columns(run_128k, cluster):
    """dK/dV on key columns of the 131072-token backward, element by element.
    near_end: the last keys, the last k-block edges, the near edge and the column at
    distance near from the last row (band 0's first distance): about 4096 rows see them.
    band<h>_edge(s): columns whose last row sits at the lower edge of KV head h's band
    (L - 1 - (near + h lr)) and their neighbours, seen through the near window (all 40
    query heads) and, for the 5 query heads of each KV head below h, through that head's
    whole band (15872 rows): 0.4 to 0.7 million (row, head) pairs, each needing its
    softmax over about 20000 keys.
    sink: the prefix sink's first and last columns and the first two past it; every row
    and head sees the sink (5.2 million pairs)."""
    r = run_128k
    L, near, ow = r["L"], r["near"], r["ow"]
    if cluster == "near_end":
        cols = [L - 1 - near - 1, L - 1 - near, L - near, L - 129, L - 128, L - 65, L - 64, L - 2, L - 1]
    elif cluster == "sink":
        cols = [0, 1, r["sink"] - 1, r["sink"], r["sink"] + 1]
    elif cluster == "band456_edges":
        cols = sorted(L - 1 - (near + hb * ow.lr) + e for hb in (4, 5, 6) for e in (0, 1))
    else:
        hb = 3 if cluster == "band3_edge" else 7
        j = L - 1 - (near + hb * ow.lr)
        cols = [j - 1, j, j + 1]
    _case(f"bwd 128K dK/dV key columns ({cluster}): {cols}")
    t0 = time.time()
    rk, rv = oracle.attn_bwd_dkdv_cols(r["q"], r["k"], r["v"], r["do"], ow, SCALE, cols,
                                       workers=_workers())
    print(f"  oracle: {len(cols)} key columns in {time.time() - t0:.1f} s ({_workers()} threads)",
          flush=True)
    _cols_check("128K " + cluster, r["dk"], r["dv"], cols, rk, rv)


def test_prefill_chunk_4096_of_128k():
    """A chunked-prefill training step at full length: the last 4096 query tokens against
    the 131072-token keys (Lq < Lk, bottom-right distance d = i + Lk - Lq - j), forward and
    backward.  O, LSE and dQ on 128 sampled rows, dK and dV on key columns in the sink,
    in the bands of several heads, at the chunk's near edge and inside the chunk, each
    element against the oracle; and the column-sum identities over all keys."""
    Lq, Lk, sink, near = 4096, 131072, 128, 4096
    _case(f"prefill chunk fwd+bwd Lq={Lq} Lk={Lk}")
    ow = oracle.Window.for_length(Lk, HKV, sink, near, 0)
    win = api.window(ow.sink, ow.near, ow.gap, ow.lr)
    q, k, v, do = inputs.attention_inputs(1, Lq, Lk, HQ, HKV, D, seed=70, device=DEV, with_dout=True)
    o, lse, dq, dk, dv = api.fwd_bwd(q, k, v, do, win)
    torch.cuda.synchronize()
    qc, kc, vc, doc = q.cpu(), k.cpu(), v.cpu(), do.cpu()
    sk = dk.double().sum(dim=1)[0]
    sv = dv.double().sum(dim=1)[0]
    sdo = do.double().sum(dim=1)[0].view(HKV, HQ // HKV, D).sum(dim=1)
    ex_k = (sk.abs() / _rounding_sigma(dk)).max().item()
    ex_v = ((sv - sdo).abs() / (_rounding_sigma(dv) + 1e-3 / 6 * sdo.abs())).max().item()
    print(f"  column sums: dK {ex_k:.2f} sigma, dV - dO {ex_v:.2f} sigma", flush=True)
    assert ex_k <= 6.0 and ex_v <= 6.0
    rng = np.random.default_rng(170)
    must = {0, 1, 24, 25, 50, 51, 52, 255, 256, Lq - 2, Lq - 1}
    rows = np.array(sorted(must | set(int(x) for x in rng.choice(Lq, 128 - len(must), replace=False))))
    Oo, Lo = oracle.attn_fwd(qc, kc, vc, ow, SCALE, rows=rows)
    idx = torch.as_tensor(rows, device=DEV)
    assert_bf16_close("O", o[:, idx], Oo)
    assert_bf16_close("LSE", lse[:, :, idx], Lo)
    dqo = oracle.attn_bwd_dq_rows(qc, kc, vc, doc, ow, SCALE, rows)
    assert_bf16_close("dQ", dq[:, idx], dqo, gradient=True)
    off = Lk - Lq
    cols = sorted({0, sink - 1, sink, 5000, Lk - 1 - (near + 3 * ow.lr), Lk - 1 - (near + 6 * ow.lr),
                   off - near, off - near + 1, off - 1, off, off + 1, off + 777, Lk - 2, Lk - 1})
    t0 = time.time()
    rk, rv = oracle.attn_bwd_dkdv_cols(qc, kc, vc, doc, ow, SCALE, cols, workers=_workers())
    print(f"  oracle: {len(cols)} key columns in {time.time() - t0:.1f} s", flush=True)
    _cols_check("prefill chunk", dk, dv, cols, rk, rv)


def test_dense_128k_sampled():
    """Dense causal attention at 131072 tokens through the same kernels (the window that
    the CoWA-against-dense ratios are measured with): O, LSE and dQ on 128 sampled rows,
    dK and dV on the last key columns, and a two-sequence decode, against the oracle."""
    L, sink, near = 131072, 128, 4096
    _case("dense 128K fwd+bwd sampled rows, last key columns, decode")
    ow, win, (q, k, v, do) = _setup(L, sink, near, "dense", seed=80, with_dout=True)
    o, lse, dq, dk, dv = api.fwd_bwd(q, k, v, do, win)
    torch.cuda.synchronize()
    qc, kc, vc, doc = q.cpu(), k.cpu(), v.cpu(), do.cpu()
    rows = sample_rows(L, sink, near, ow.lr, HKV, 128 // 5, 128, seed=180)
    t0 = time.time()
    Oo, Lo = oracle.attn_fwd(qc, kc, vc, ow, SCALE, rows=rows)
    idx = torch.as_tensor(rows, device=DEV)
    assert_bf16_close("O", o[:, idx], Oo)
    assert_bf16_close("LSE", lse[:, :, idx], Lo)
    dqo = oracle.attn_bwd_dq_rows(qc, kc, vc, doc, ow, SCALE, rows)
    assert_bf16_close("dQ", dq[:, idx], dqo, gradient=True)
    cols = [L - 129, L - 128, L - 65, L - 64, L - 2, L - 1]
    rk, rv = oracle.attn_bwd_dkdv_cols(qc, kc, vc, doc, ow, SCALE, cols, workers=_workers())
    print(f"  oracle: rows and {len(cols)} key columns in {time.time() - t0:.1f} s", flush=True)
    _cols_check("dense 128K", dk, dv, cols, rk, rv)
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    qd, kd, vd = inputs.attention_inputs(2, 1, L, HQ, HKV, D, seed=81, device=DEV)
    od, lsed = api.decode(qd, kd, vd, win)
    torch.cuda.synchronize()
    for b in range(2):
        Oo, Lo = oracle.decode(qd[b:b + 1].cpu(), kd[b:b + 1].cpu(), vd[b:b + 1].cpu(), ow, SCALE)
        assert_bf16_close(f"decode O[b={b}]", od[b:b + 1], Oo)
        assert_bf16_close(f"decode LSE[b={b}]", lsed[b:b + 1], Lo[:, :, 0])


def test_bwd_4096_full_dk_dv():
    _case("bwd 4096 full dQ/dK/dV (the mid-size check of every key column)")
    L, sink, near = 4096, 128, 512
    ow, win, (q, k, v, do) = _setup(L, sink, near, seed=30, with_dout=True)
    o, lse, dq, dk, dv = api.fwd_bwd(q, k, v, do, win)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q.cpu(), k.cpu(), v.cpu(), do.cpu(), ow, SCALE)
    assert_bf16_close("dQ", dq, rq, gradient=True)
    assert_bf16_close("dK", dk, rk, gradient=True)
    assert_bf16_close("dV", dv, rv, gradient=True)


def test_decode_128k_batch16():
    _case("decode 16 x 131072 cache, oracle on sequences 0, 7, 15")
    B, L, sink, near = 16, 131072, 128, 4096
    ow = oracle.Window.for_length(L, HKV, sink, near, 0)
    win = api.window(ow.sink, ow.near, ow.gap, ow.lr)
    q, k, v = inputs.attention_inputs(B, 1, L, HQ, HKV, D, seed=40, device=DEV)
    o, lse = api.decode(q, k, v, win)
    torch.cuda.synchronize()
    for b in (0, 7, 15):
        Oo, Lo = oracle.decode(q[b:b + 1].cpu(), k[b:b + 1].cpu(), v[b:b + 1].cpu(), ow, SCALE)
        assert_bf16_close(f"O[b={b}]", o[b:b + 1], Oo)
        assert_bf16_close(f"LSE[b={b}]", lse[b:b + 1], Lo[:, :, 0])


def test_decode_matches_forward_last_row_128k():
    _case("decode of the last token == forward row L-1 at 128K")
    L, sink, near = 131072, 128, 4096
    ow, win, (q, k, v) = _setup(L, sink, near, seed=50)
    o, lse = api.fwd(q, k, v, win)
    od, lsed = api.decode(q[:, -1:].contiguous(), k, v, win)
    torch.cuda.synchronize()
    d = (od.float() - o[:, -1:].float()).abs().max().item()
    dl = (lsed - lse[:, :, -1]).abs().max().item()
    print(f"  max|O_dec - O_fwd[-1]|={d:.3e} max|dLSE|={dl:.3e}", flush=True)
    assert d <= 1e-2 and dl <= 1e-3


def test_decode_varlen_and_window_cache_16x128k():
    """The variable-length and window-cache decodes in the setting the benchmark times:
    16 caches of 131072 positions, sequence b of length 65536 + 4096 b (varlen) and of the
    full length (window caches filled from the full caches by one append each).  Varlen
    against the oracle on sequences 0, 9 and 15; the window-cache decode equal to the
    planned decode bit for bit, and against the oracle on sequences 3 and 15."""
    B, L, sink, near = 16, 131072, 128, 4096
    _case("decode varlen and window caches, 16 x 131072")
    ow = oracle.Window.for_length(L, HKV, sink, near, 0)
    win = api.window(ow.sink, ow.near, ow.gap, ow.lr)
    q, k, v = inputs.attention_inputs(B, 1, L, HQ, HKV, D, seed=45, device=DEV)
    lens = [65536 + 4096 * b for b in range(B)]
    ov, lv = api.decode_varlen(q, k, v, torch.tensor(lens, dtype=torch.int32, device=DEV), win)
    wc = api.WindowCache(B, HKV, D, L, win, DEV)
    wc.append(k, v, torch.zeros(B, dtype=torch.int32, device=DEV))
    ow_, lw_ = wc.decode(q, torch.full((B,), L, dtype=torch.int32, device=DEV))
    op, lp = api.decode(q, k, v, win)
    torch.cuda.synchronize()
    n_o, n_l = int((ow_ != op).sum().item()), int((lw_ != lp).sum().item())
    print(f"  window cache vs planned decode: O differs at {n_o}, LSE at {n_l}", flush=True)
    assert n_o == 0 and n_l == 0
    for b in (0, 9, 15):
        n = lens[b]
        Oo, Lo = oracle.decode(q[b:b + 1].cpu(), k[b:b + 1, :n].cpu(), v[b:b + 1, :n].cpu(), ow, SCALE)
        assert_bf16_close(f"varlen O[b={b}] (len {n})", ov[b:b + 1], Oo)
        assert_bf16_close(f"varlen LSE[b={b}]", lv[b:b + 1], Lo[:, :, 0])
    for b in (3, 15):
        Oo, Lo = oracle.decode(q[b:b + 1].cpu(), k[b:b + 1].cpu(), v[b:b + 1].cpu(), ow, SCALE)
        assert_bf16_close(f"window cache O[b={b}]", ow_[b:b + 1], Oo)
        assert_bf16_close(f"window cache LSE[b={b}]", lw_[b:b + 1], Lo[:, :, 0])
