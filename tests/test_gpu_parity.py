"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small and mid sizes are compared element by element in full; the 32K and 128K workloads
on seeded stratified row samples plus exact identities that hold at any size."""

import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))
import oracle  # noqa: E402
from gpu_helpers import (F32_MAX_ABS, assert_bf16_close, errors, sample_rows)  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from structured_sparse_attention_plan_amd import api, inputs  # noqa: E402

DEV = "cuda:0"


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _windows(L, Hkv, sink, near, gap=0, mode="complementary"):
    ow = oracle.Window.for_length(L, Hkv, sink, near, gap, mode=mode)
    return ow, api.window(ow.sink, ow.near, ow.gap, ow.lr, mode)


# ----------------------------------------------------------------------------- forward

def test_fwd_f32_config1():
    _case("fwd f32 L=1024 Hq=4 Hkv=2 D=64 sink=64 near=128")
    L, Hq, Hkv, D = 1024, 4, 2, 64
    ow, win = _windows(L, Hkv, 64, 128)
    q, k, v = inputs.attention_inputs(1, L, L, Hq, Hkv, D, dtype=torch.float32, seed=0)
    o, lse = api.fwd(q.to(DEV), k.to(DEV), v.to(DEV), win, scale=1 / 8)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attn_fwd(q, k, v, ow, 1 / 8)
    e_o, _ = errors(o, Oo)
    e_l, _ = errors(lse, Lo)
    print(f"  O max_abs={e_o:.3e} LSE max_abs={e_l:.3e}", flush=True)
    assert e_o <= F32_MAX_ABS and e_l <= F32_MAX_ABS


@pytest.mark.parametrize("B,Lq,Lk,Hq,Hkv,sink,near,mode", [
    (2, 300, 300, 4, 1, 8, 40, "complementary"),    # G = 4: 256 threads per group
    (1, 200, 500, 2, 2, 16, 64, "duplicated"),      # G = 1, prefill chunk (Lq < Lk)
    (1, 400, 250, 4, 2, 8, 40, "complementary"),    # Lq > Lk: the first 150 rows see nothing
    (1, 333, 333, 4, 2, 0, 0, "complementary"),     # near = 0, no sink: empty rows
    (1, 517, 517, 4, 2, 5, 20, "dense"),
    (1, 450, 450, 6, 2, 16, 64, "complementary"),   # G = 3: 24 of the 32 product columns
    (2, 129, 129, 2, 2, 1, 1, "complementary"),     # G = 1, one key per row besides the sink
])
def test_fwd_f32_small(B, Lq, Lk, Hq, Hkv, sink, near, mode):
    _case(f"fwd f32 B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} sink={sink} near={near} {mode}")
    ow, win = _windows(Lk, Hkv, sink, near, mode=mode)
    q, k, v = inputs.attention_inputs(B, Lq, Lk, Hq, Hkv, 64, dtype=torch.float32, seed=3)
    o, lse = api.fwd(q.to(DEV), k.to(DEV), v.to(DEV), win, scale=1 / 8)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attn_fwd(q, k, v, ow, 1 / 8)
    e_o, _ = errors(o, Oo)
    e_l, _ = errors(lse, Lo)
    print(f"  O max_abs={e_o:.3e} LSE max_abs={e_l:.3e}", flush=True)
    assert e_o <= F32_MAX_ABS and e_l <= F32_MAX_ABS


@pytest.mark.parametrize("B,Lq,Lk,Hq,Hkv,sink,near,mode", [
    (1, 1000, 1000, 40, 8, 16, 100, "complementary"),
    (2, 700, 700, 40, 8, 0, 64, "duplicated"),
    (1, 600, 600, 40, 8, 3, 50, "dense"),
    (1, 300, 1100, 40, 8, 20, 90, "complementary"),   # prefill chunk, Lq < Lk
    (1, 520, 520, 8, 2, 64, 128, "complementary"),    # G = 4
    (1, 333, 333, 8, 8, 5, 40, "complementary"),      # G = 1
])
def test_fwd_bf16_small_full(B, Lq, Lk, Hq, Hkv, sink, near, mode):
    _case(f"fwd bf16 B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} sink={sink} near={near} {mode}")
    ow, win = _windows(Lk, Hkv, sink, near, mode=mode)
    q, k, v = inputs.attention_inputs(B, Lq, Lk, Hq, Hkv, 128, seed=1)
    o, lse = api.fwd(q.to(DEV), k.to(DEV), v.to(DEV), win)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attn_fwd(q, k, v, ow, 128 ** -0.5)
    assert_bf16_close("O", o, Oo)
    assert_bf16_close("LSE", lse, Lo)


@pytest.mark.parametrize("case", ["rises", "first_mass_low"])
def test_fwd_bf16_reference_moves(case):
    """Inputs that take the forward's rare path, where a column's softmax reference moves:
    "rises", later keys score far above the first tile's maximum (tile sums above 2^32);
    "first_mass_low", no prefix sink, so some columns see no key in their item's first
    tile, and every score lies far below 0 (their first visible tile sums to less than
    2^-32).  The result does not depend on the reference, so the oracle's plain softmax
    is the bar."""
    L, Hq, Hkv = 700, 8, 2
    sink, near = (16, 100) if case == "rises" else (0, 64)
    _case(f"fwd bf16 L={L} Hq={Hq} Hkv={Hkv} sink={sink} near={near}, reference {case}")
    ow, win = _windows(L, Hkv, sink, near)
    q, k, v = inputs.attention_inputs(1, L, L, Hq, Hkv, 128, seed=21)
    q = q.abs()
    if case == "rises":
        k[:, 200:330] = 4.0   # q.k scale about +36 against about +3 in the first tile
    else:
        k[:] = -4.0           # every score about -36
    o, lse = api.fwd(q.to(DEV), k.to(DEV), v.to(DEV), win)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attn_fwd(q, k, v, ow, 128 ** -0.5)
    assert_bf16_close("O", o, Oo)
    assert_bf16_close("LSE", lse, Lo)


@pytest.mark.parametrize("Hq,Hkv", [(16, 8), (24, 8), (16, 2), (6, 2)])
def test_fwd_bf16_group_sizes(Hq, Hkv):
    """Group sizes G = 2, 3, 8 (and 3 with two KV heads): the q-block holds 256 / G tokens
    (85 for G = 3, so one row of the 256 is unused)."""
    L = 700
    _case(f"fwd bf16 L={L} Hq={Hq} Hkv={Hkv} (G={Hq // Hkv})")
    ow, win = _windows(L, Hkv, 16, 64)
    q, k, v = inputs.attention_inputs(1, L, L, Hq, Hkv, 128, seed=13)
    o, lse = api.fwd(q.to(DEV), k.to(DEV), v.to(DEV), win)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attn_fwd(q, k, v, ow, 128 ** -0.5)
    assert_bf16_close("O", o, Oo)
    assert_bf16_close("LSE", lse, Lo)


@pytest.mark.parametrize("Lq,Lk", [(500, 500), (700, 300)])
def test_fwd_bf16_empty_rows(Lq, Lk):
    """near = 0 and no prefix sink: under KV head h > 0 a query closer than the head's
    band to key 0 sees nothing (O = 0, LSE = -inf); with Lq > Lk, the first Lq - Lk rows
    lie before every key under the bottom-right distance and are empty under every head."""
    _case(f"fwd bf16 empty rows Lq={Lq} Lk={Lk} sink=0 near=0")
    Hq, Hkv = 16, 4
    ow, win = _windows(Lk, Hkv, 0, 0)
    q, k, v = inputs.attention_inputs(1, Lq, Lk, Hq, Hkv, 128, seed=14)
    o, lse = api.fwd(q.to(DEV), k.to(DEV), v.to(DEV), win)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attn_fwd(q, k, v, ow, 128 ** -0.5)
    n_empty = int(np.isinf(Lo).sum())
    print(f"  empty (row, head) pairs: {n_empty}", flush=True)
    assert n_empty > 0
    assert_bf16_close("O", o, Oo)
    assert_bf16_close("LSE", lse, Lo)
    assert torch.all(o.cpu()[torch.from_numpy(np.isinf(Lo).transpose(0, 2, 1).copy())] == 0)


@pytest.mark.parametrize("Lq,Lk,sink,near", [(400, 400, 16, 64), (500, 300, 8, 40)])
def test_fwd_bf16_more_queries_than_keys(Lq, Lk, sink, near):
    """Lq > Lk: query row i sits at key position i - (Lq - Lk); rows before key 0 are
    empty, the others see the usual window."""
    _case(f"fwd bf16 Lq={Lq} Lk={Lk} sink={sink} near={near}")
    ow, win = _windows(Lk, 8, sink, near)
    q, k, v = inputs.attention_inputs(1, Lq, Lk, 40, 8, 128, seed=15)
    o, lse = api.fwd(q.to(DEV), k.to(DEV), v.to(DEV), win)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attn_fwd(q, k, v, ow, 128 ** -0.5)
    assert_bf16_close("O", o, Oo)
    assert_bf16_close("LSE", lse, Lo)


def test_fwd_bf16_mid_4096_full():
    _case("fwd bf16 L=4096 Hq=40 Hkv=8 sink=128 near=512")
    L = 4096
    ow, win = _windows(L, 8, 128, 512)
    q, k, v = inputs.attention_inputs(1, L, L, 40, 8, 128, seed=2)
    o, lse = api.fwd(q.to(DEV), k.to(DEV), v.to(DEV), win)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attn_fwd(q, k, v, ow, 128 ** -0.5)
    assert_bf16_close("O", o, Oo)
    assert_bf16_close("LSE", lse, Lo)


def test_fwd_bitwise_repeatable():
    _case("fwd bf16 repeatability L=2048")
    L = 2048
    _, win = _windows(L, 8, 128, 256)
    q, k, v = (t.to(DEV) for t in inputs.attention_inputs(1, L, L, 40, 8, 128, seed=3))
    o1, l1 = api.fwd(q, k, v, win)
    o2, l2 = api.fwd(q, k, v, win)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ----------------------------------------------------------------------------- backward

@pytest.mark.parametrize("B,L,Hq,Hkv,sink,near,mode", [
    (1, 600, 40, 8, 16, 64, "complementary"),
    (2, 333, 40, 8, 0, 32, "duplicated"),
    (1, 300, 40, 8, 5, 20, "dense"),
    (1, 400, 8, 2, 16, 64, "complementary"),
    (1, 333, 8, 8, 5, 40, "complementary"),      # G = 1
])
def test_bwd_bf16_small_full(B, L, Hq, Hkv, sink, near, mode):
    _case(f"bwd bf16 B={B} L={L} Hq={Hq} Hkv={Hkv} sink={sink} near={near} {mode}")
    ow, win = _windows(L, Hkv, sink, near, mode=mode)
    q, k, v, do = inputs.attention_inputs(B, L, L, Hq, Hkv, 128, seed=4, with_dout=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse, dq, dk, dv = api.fwd_bwd(qd, kd, vd, dod, win)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, ow, 128 ** -0.5)
    assert_bf16_close("dQ", dq, rq, gradient=True)
    assert_bf16_close("dK", dk, rk, gradient=True)
    assert_bf16_close("dV", dv, rv, gradient=True)


@pytest.mark.parametrize("B,Lq,Lk,Hq,Hkv,sink,near", [
    (1, 500, 500, 16, 8, 16, 64),    # G = 2
    (1, 500, 500, 24, 8, 16, 64),    # G = 3: 42 tokens per q-block, two rows unused
    (1, 500, 500, 16, 2, 16, 64),    # G = 8
    (1, 400, 400, 16, 4, 0, 0),      # near = 0, no sink: empty rows under heads 1-3
    (1, 500, 300, 40, 8, 8, 40),     # Lq > Lk: the first 200 rows are empty
])
def test_bwd_bf16_group_sizes_and_empty_rows(B, Lq, Lk, Hq, Hkv, sink, near):
    _case(f"bwd bf16 B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} sink={sink} near={near}")
    ow, win = _windows(Lk, Hkv, sink, near)
    q, k, v, do = inputs.attention_inputs(B, Lq, Lk, Hq, Hkv, 128, seed=16, with_dout=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse, dq, dk, dv = api.fwd_bwd(qd, kd, vd, dod, win)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, ow, 128 ** -0.5)
    assert_bf16_close("dQ", dq, rq, gradient=True)
    assert_bf16_close("dK", dk, rk, gradient=True)
    assert_bf16_close("dV", dv, rv, gradient=True)


@pytest.mark.parametrize("Lq,Lk", [(1, 1), (1, 70), (3, 3), (2, 65), (65, 65)])
def test_tiny_sizes(Lq, Lk):
    """Degenerate sizes: one query and one key, a single query over a tile and a bit, keys
    one past a tile; forward and backward in bf16, the fp32 forward, and the decode of the
    last key position."""
    _case(f"tiny Lq={Lq} Lk={Lk}")
    Hq, Hkv = 8, 2
    ow, win = _windows(Lk, Hkv, 4, 16)
    q, k, v, do = inputs.attention_inputs(1, Lq, Lk, Hq, Hkv, 128, seed=21, with_dout=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse, dq, dk, dv = api.fwd_bwd(qd, kd, vd, dod, win)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attn_fwd(q, k, v, ow, 128 ** -0.5)
    assert_bf16_close("O", o, Oo)
    assert_bf16_close("LSE", lse, Lo)
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, ow, 128 ** -0.5)
    assert_bf16_close("dQ", dq, rq, gradient=True)
    assert_bf16_close("dK", dk, rk, gradient=True)
    assert_bf16_close("dV", dv, rv, gradient=True)
    qf, kf, vf = inputs.attention_inputs(1, Lq, Lk, Hq, Hkv, 64, dtype=torch.float32, seed=22)
    of, lf = api.fwd(qf.to(DEV), kf.to(DEV), vf.to(DEV), win, scale=1 / 8)
    torch.cuda.synchronize()
    Of, Lf = oracle.attn_fwd(qf, kf, vf, ow, 1 / 8)
    assert errors(of, Of)[0] <= F32_MAX_ABS and errors(lf, Lf)[0] <= F32_MAX_ABS
    qd1, kc, vc = inputs.attention_inputs(2, 1, Lk, Hq, Hkv, 128, seed=23)
    od, ld = api.decode(qd1.to(DEV), kc.to(DEV), vc.to(DEV), win)
    torch.cuda.synchronize()
    Od, Ld = oracle.decode(qd1, kc, vc, ow, 128 ** -0.5)
    assert_bf16_close("decode O", od, Od)
    assert_bf16_close("decode LSE", ld, Ld[:, :, 0])


@pytest.mark.parametrize("do_exp,v_exp", [(12, 0), (-24, 0), (0, 6), (8, 5)])
def test_bwd_bf16_gradient_ranges(do_exp, v_exp):
    """dO multiplied by 2^do_exp (a loss-scaled or a tiny upstream gradient) and V by
    2^v_exp: dS scales with both, and the fp16 dK product must neither overflow nor lose
    its precision to subnormals.  Compared in the units of the unscaled problem, where
    the bars are set (dQ and dK scale by 2^(do_exp + v_exp), dV by 2^do_exp)."""
    L = 600
    _case(f"bwd bf16 L={L} dO * 2^{do_exp}, V * 2^{v_exp}")
    ow, win = _windows(L, 8, 16, 64)
    q, k, v, do = inputs.attention_inputs(1, L, L, 40, 8, 128, seed=17, with_dout=True)
    do = (do.float() * 2.0 ** do_exp).to(torch.bfloat16)
    v = (v.float() * 2.0 ** v_exp).to(torch.bfloat16)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse, dq, dk, dv = api.fwd_bwd(qd, kd, vd, dod, win)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, ow, 128 ** -0.5)
    sg, sv = 2.0 ** -(do_exp + v_exp), 2.0 ** -do_exp
    for name, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert torch.isfinite(t).all(), f"{name} has non-finite entries"
    assert_bf16_close("dQ (rescaled)", dq.double() * sg, rq * sg, gradient=True)
    assert_bf16_close("dK (rescaled)", dk.double() * sg, rk * sg, gradient=True)
    assert_bf16_close("dV (rescaled)", dv.double() * sv, rv * sv, gradient=True)


def test_bwd_bf16_mid_2048_full():
    """The backward without O's rounding residual (Delta from the bf16 O alone)."""
    _case("bwd bf16 L=2048 Hq=40 Hkv=8 sink=128 near=512, no residual of O")
    L = 2048
    ow, win = _windows(L, 8, 128, 512)
    q, k, v, do = inputs.attention_inputs(1, L, L, 40, 8, 128, seed=5, with_dout=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = api.fwd(qd, kd, vd, win)
    dq, dk, dv = api.bwd(qd, kd, vd, o, lse, dod, win)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, ow, 128 ** -0.5)
    assert_bf16_close("dQ", dq, rq, gradient=True)
    assert_bf16_close("dK", dk, rk, gradient=True)
    assert_bf16_close("dV", dv, rv, gradient=True)


@pytest.mark.parametrize("B,Lq,Lk,Hq,Hkv,sink,near,mode", [
    (1, 300, 1100, 40, 8, 20, 90, "complementary"),   # prefill chunk: rows at the end of Lk
    (2, 130, 700, 40, 8, 7, 64, "duplicated"),
])
def test_bwd_bf16_prefill_chunk(B, Lq, Lk, Hq, Hkv, sink, near, mode):
    """Backward of a chunk of Lq query rows at positions Lk - Lq .. Lk - 1 (bottom-right
    distance d = i + Lk - Lq - j)."""
    _case(f"bwd bf16 B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} sink={sink} near={near} {mode}")
    ow, win = _windows(Lk, Hkv, sink, near, mode=mode)
    q, k, v, do = inputs.attention_inputs(B, Lq, Lk, Hq, Hkv, 128, seed=8, with_dout=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse, dq, dk, dv = api.fwd_bwd(qd, kd, vd, dod, win)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, ow, 128 ** -0.5)
    assert_bf16_close("dQ", dq, rq, gradient=True)
    assert_bf16_close("dK", dk, rk, gradient=True)
    assert_bf16_close("dV", dv, rv, gradient=True)


@pytest.mark.parametrize("qexp", [9, -9])
def test_bwd_bf16_scaled_q(qexp):
    """Q multiplied by 2^qexp and K by 2^-qexp (exact in bf16; the scores do not change):
    the fp16 dK product's per-row and per-item power-of-two scales move away from 1, dK
    scales by 2^qexp and dQ by 2^-qexp."""
    L = 600
    _case(f"bwd bf16 L={L} Q * 2^{qexp}, K * 2^{-qexp}")
    ow, win = _windows(L, 8, 16, 64)
    q, k, v, do = inputs.attention_inputs(1, L, L, 40, 8, 128, seed=12, with_dout=True)
    q = (q.float() * 2.0 ** qexp).to(torch.bfloat16)
    k = (k.float() * 2.0 ** -qexp).to(torch.bfloat16)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse, dq, dk, dv = api.fwd_bwd(qd, kd, vd, dod, win)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, ow, 128 ** -0.5)
    # compare in the units of the unscaled problem, where the bars are set
    assert_bf16_close("dQ * 2^qexp", dq.float() * 2.0 ** qexp, rq * 2.0 ** qexp, gradient=True)
    assert_bf16_close("dK * 2^-qexp", dk.float() * 2.0 ** -qexp, rk * 2.0 ** -qexp, gradient=True)
    assert_bf16_close("dV", dv, rv, gradient=True)


def test_chunked_prefill_matches_full_forward():
    """Chunked prefill: the forward of rows [c0, c1) against keys [0, c1) (Lq < Lk, the
    same window) equals rows c0..c1-1 of the forward over the whole sequence, bit for bit.
    Each row's result depends only on its own visible keys taken in ascending tile order,
    and with sink >= 1 every row's first tile (keys 0..63) is visible to it, so the
    softmax reference is the same however rows are grouped into q-blocks.  The decode of
    each chunk's last token then agrees with the full forward's row within bf16."""
    L = 2000
    _case(f"chunked prefill L={L} chunks 0-700-1300-2000 + decode at each chunk end")
    _, win = _windows(L, 8, 32, 256)
    q, k, v = (t.to(DEV) for t in inputs.attention_inputs(1, L, L, 40, 8, 128, seed=9))
    o, lse = api.fwd(q, k, v, win)
    for c0, c1 in ((0, 700), (700, 1300), (1300, 2000)):
        oc, lsec = api.fwd(q[:, c0:c1].contiguous(), k[:, :c1].contiguous(), v[:, :c1].contiguous(), win)
        od, lsed = api.decode(q[:, c1 - 1:c1].contiguous(), k[:, :c1].contiguous(), v[:, :c1].contiguous(), win)
        torch.cuda.synchronize()
        n_o = int((oc != o[:, c0:c1]).sum().item())
        n_l = int((lsec != lse[:, :, c0:c1]).sum().item())
        d = (od.float() - o[:, c1 - 1:c1].float()).abs().max().item()
        dl = (lsed - lse[:, :, c1 - 1]).abs().max().item()
        print(f"  chunk [{c0}, {c1}): O differs at {n_o}, LSE at {n_l}; decode max|dO|={d:.3e} "
              f"max|dLSE|={dl:.3e}", flush=True)
        assert n_o == 0 and n_l == 0
        assert d <= 1e-2 and dl <= 1e-3


# ----------------------------------------------------------------------------- decode

@pytest.mark.parametrize("B,Lk,Hq,Hkv,sink,near,mode", [
    (3, 5000, 40, 8, 128, 256, "complementary"),
    (2, 4099, 40, 8, 0, 100, "duplicated"),
    (1, 3000, 16, 4, 10, 64, "complementary"),   # G = 4
    (2, 777, 40, 8, 7, 33, "dense"),
    (2, 2000, 8, 8, 16, 64, "complementary"),    # G = 1
    (1, 1500, 16, 8, 16, 64, "duplicated"),      # G = 2
    (2, 2500, 16, 2, 32, 128, "complementary"),  # G = 8
    (2, 1800, 24, 8, 16, 64, "complementary"),   # G = 3
    (1, 2100, 12, 2, 8, 50, "duplicated"),       # G = 6
    (2, 1300, 14, 2, 16, 64, "dense"),           # G = 7
])
def test_decode_small(B, Lk, Hq, Hkv, sink, near, mode):
    _case(f"decode B={B} Lk={Lk} Hq={Hq} Hkv={Hkv} sink={sink} near={near} {mode}")
    ow, win = _windows(Lk, Hkv, sink, near, mode=mode)
    q, k, v = inputs.attention_inputs(B, 1, Lk, Hq, Hkv, 128, seed=6)
    o, lse = api.decode(q.to(DEV), k.to(DEV), v.to(DEV), win)
    torch.cuda.synchronize()
    Oo, Lo = oracle.decode(q, k, v, ow, 128 ** -0.5)
    assert_bf16_close("O", o, Oo)
    assert_bf16_close("LSE", lse, Lo[:, :, 0])


def test_decode_empty_rows():
    """near = 0, no sink: the query at position Lk - 1 sees only its head's band, and KV
    heads whose band starts beyond it see nothing (O = 0, LSE = -inf)."""
    B, Lk, Hq, Hkv = 2, 900, 16, 4
    _case(f"decode empty rows B={B} Lk={Lk} Hq={Hq} Hkv={Hkv} sink=0 near=0")
    ow = oracle.Window(0, 0, 0, 400)
    win = api.window(0, 0, 0, 400)
    q, k, v = inputs.attention_inputs(B, 1, Lk, Hq, Hkv, 128, seed=18)
    o, lse = api.decode(q.to(DEV), k.to(DEV), v.to(DEV), win)
    torch.cuda.synchronize()
    Oo, Lo = oracle.decode(q, k, v, ow, 128 ** -0.5)
    assert np.isinf(Lo).sum() > 0
    assert_bf16_close("O", o, Oo)
    assert_bf16_close("LSE", lse, Lo[:, :, 0])


def test_decode_varlen():
    """Decode of sequences of different lengths in one batch (capacity 3000): each
    sequence b against the oracle's decode over its first seqlens[b] keys, with the
    window of the capacity; length 0 gives O = 0 and LSE = -inf."""
    Lk, B = 3000, 6
    lens = [3000, 1, 77, 1500, 2999, 0]
    _case(f"decode varlen capacity {Lk} lengths {lens}")
    ow, win = _windows(Lk, 8, 128, 256)
    q, k, v = inputs.attention_inputs(B, 1, Lk, 40, 8, 128, seed=10)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, lse = api.decode_varlen(q.to(DEV), k.to(DEV), v.to(DEV), seq, win)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.all(o[b] == 0) and torch.all(lse[b] == -float("inf")), "empty sequence"
            continue
        Oo, Lo = oracle.decode(q[b:b + 1], k[b:b + 1, :n], v[b:b + 1, :n], ow, 128 ** -0.5)
        assert_bf16_close(f"O[{b}] (len {n})", o[b:b + 1], Oo)
        assert_bf16_close(f"LSE[{b}]", lse[b:b + 1], Lo[:, :, 0])


def test_decode_varlen_full_lengths_equal_decode():
    """With every length equal to the capacity the varlen decode visits the same blocks in
    the same order as the planned decode: bit-equal outputs."""
    B, Lk = 4, 5000
    _case(f"decode varlen B={B} all lengths {Lk} vs planned decode")
    _, win = _windows(Lk, 8, 128, 256)
    q, k, v = (t.to(DEV) for t in inputs.attention_inputs(B, 1, Lk, 40, 8, 128, seed=11))
    o, lse = api.decode(q, k, v, win)
    ov, lsev = api.decode_varlen(q, k, v, torch.full((B,), Lk, dtype=torch.int32, device=DEV), win)
    torch.cuda.synchronize()
    n_o = int((o != ov).sum().item())
    n_l = int((lse != lsev).sum().item())
    print(f"  O differs at {n_o}, LSE at {n_l}", flush=True)
    assert n_o == 0 and n_l == 0


@pytest.mark.parametrize("mode,sink,near", [("complementary", 16, 64), ("duplicated", 16, 64),
                                            ("dense", 8, 32), ("complementary", 0, 100)])
def test_wcache_appends_then_decode(mode, sink, near):
    """Window-only caches filled by appends of uneven chunks (5, 1000, three single tokens,
    769, 1223), some sequences skipped by positions past Lmax, so the three sequences end
    at lengths 3000, 1777 and 5.  Decoding over them equals the variable-length decode over
    full caches holding the same rows bit for bit (same blocks, same order), and the oracle
    decode of each truncated sequence; checked after the middle append too."""
    B, Lmax, Hq, Hkv = 3, 3000, 40, 8
    _case(f"window cache appends + decode {mode} sink={sink} near={near}")
    ow, win = _windows(Lmax, Hkv, sink, near, mode=mode)
    q, k, v = inputs.attention_inputs(B, 1, Lmax, Hq, Hkv, 128, seed=30)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    cache = api.WindowCache(B, Hkv, 128, Lmax, win, DEV)
    print(f"  slots per sequence {cache.slots} (full cache {Hkv * Lmax})", flush=True)
    skip = Lmax + 7  # a position past the cache: the sequence takes no token
    lens = [0, 0, 0]

    def append(T, take):
        pos0 = [lens[b] if take[b] else skip for b in range(B)]
        kn = torch.zeros((B, T, Hkv, 128), dtype=torch.bfloat16, device=DEV)
        vn = torch.zeros_like(kn)
        for b in range(B):
            if take[b]:
                kn[b] = kd[b, lens[b]:lens[b] + T]
                vn[b] = vd[b, lens[b]:lens[b] + T]
                lens[b] += T
        cache.append(kn, vn, torch.tensor(pos0, dtype=torch.int32, device=DEV))

    def check(tag):
        seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
        ow_, lw_ = cache.decode(qd, seq)
        of, lf = api.decode_varlen(qd, kd, vd, seq, win)
        torch.cuda.synchronize()
        n_o, n_l = int((ow_ != of).sum().item()), int((lw_ != lf).sum().item())
        print(f"  {tag} lengths {lens}: differs from full-cache varlen at O {n_o}, LSE {n_l}", flush=True)
        assert n_o == 0 and n_l == 0
        for b, n in enumerate(lens):
            Oo, Lo = oracle.decode(q[b:b + 1], k[b:b + 1, :n], v[b:b + 1, :n], ow, 128 ** -0.5)
            assert_bf16_close(f"O[{b}] (len {n})", ow_[b:b + 1], Oo)
            assert_bf16_close(f"LSE[{b}]", lw_[b:b + 1], Lo[:, :, 0])

    append(5, [1, 1, 1])
    append(1000, [1, 1, 0])
    check("after 1005")
    for _ in range(3):
        append(1, [1, 1, 0])
    append(769, [1, 1, 0])
    append(1223, [1, 0, 0])
    check("final")


def test_wcache_whole_prefill_in_one_append():
    """A whole 5000-token prefill appended in one call (the chunk exceeds every head's
    ring: only the positions each head can still see are written), then 8 single-token
    appends, each followed by a decode equal bit for bit to the planned decode over the
    full cache of that length."""
    B, Lmax, Hq, Hkv = 2, 5008, 40, 8
    _case(f"window cache: one {Lmax - 8}-token append, then 8 decode steps")
    ow, win = _windows(Lmax, Hkv, 128, 256)
    q, k, v = (t.to(DEV) for t in inputs.attention_inputs(B, 9, Lmax, Hq, Hkv, 128, seed=31))
    cache = api.WindowCache(B, Hkv, 128, Lmax, win, DEV)
    n = Lmax - 8
    cache.append(k[:, :n].contiguous(), v[:, :n].contiguous(), torch.zeros(B, dtype=torch.int32, device=DEV))
    for step in range(9):
        L = n + step
        qs = q[:, step:step + 1].contiguous()
        ow_, lw_ = cache.decode(qs, torch.full((B,), L, dtype=torch.int32, device=DEV))
        # the planned decode of a length-L sequence, with the window of the capacity
        of, lf = api.decode_varlen(qs, k, v, torch.full((B,), L, dtype=torch.int32, device=DEV), win)
        torch.cuda.synchronize()
        assert torch.equal(ow_, of) and torch.equal(lw_, lf), f"step {step}"
        if step < 8:
            cache.append(k[:, L:L + 1].contiguous(), v[:, L:L + 1].contiguous(),
                         torch.full((B,), L, dtype=torch.int32, device=DEV))
    Oo, Lo = oracle.decode(q[:, 8:9].cpu(), k.cpu(), v.cpu(), ow, 128 ** -0.5)
    assert_bf16_close("O (last step)", ow_, Oo)


def test_decode_equals_forward_last_row():
    _case("decode vs forward last row L=3000")
    L = 3000
    _, win = _windows(L, 8, 64, 256)
    q, k, v = (t.to(DEV) for t in inputs.attention_inputs(1, L, L, 40, 8, 128, seed=7))
    o, lse = api.fwd(q, k, v, win)
    od, lsed = api.decode(q[:, -1:].contiguous(), k, v, win)
    torch.cuda.synchronize()
    d = (od.float() - o[:, -1:].float()).abs().max().item()
    dl = (lsed - lse[:, :, -1]).abs().max().item()
    print(f"  max|O_dec - O_fwd[-1]|={d:.3e} max|dLSE|={dl:.3e}", flush=True)
    assert d <= 1e-2 and dl <= 1e-3


def test_fwd_residual_is_what_bf16_rounding_drops():
    """The forward's optional residual: O and LSE are bit-identical with and without it,
    and O + residual is closer to the oracle than O (the residual is the rounding error
    of the bf16 O, itself rounded to bf16)."""
    L = 900
    _case(f"fwd residual of O, L={L}")
    ow, win = _windows(L, 8, 16, 64)
    q, k, v = inputs.attention_inputs(1, L, L, 40, 8, 128, seed=19)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o1, l1 = api.fwd(qd, kd, vd, win)
    o_lo = torch.empty_like(qd)
    o2, l2 = api.fwd(qd, kd, vd, win, o_lo=o_lo)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    Oo, _ = oracle.attn_fwd(q, k, v, ow, 128 ** -0.5)
    e_hi, _ = errors(o2, Oo)
    e_sum, _ = errors(o2.double() + o_lo.double(), Oo)
    print(f"  max|O - oracle|={e_hi:.3e}  max|O + residual - oracle|={e_sum:.3e}", flush=True)
    # the residual never exceeds half an ulp of O's bf16 value (2^-9 relative)
    lo, hi = o_lo.double().abs(), o2.double().abs()
    assert bool((lo <= hi * 2.0 ** -8 + 1e-30).all())
    assert e_sum < e_hi


# ----------------------------------------------------------------------------- MALA

def _plan_tiles(plan):
    """(h, qb, kb) of every entry of a device plan's row lists, in entry order."""
    rp = plan.host.arrays["row_ptr"]
    ent = plan.host.arrays["row_ent"]
    nqb = plan.info.nqb
    out = []
    for item in range(len(rp) - 1):
        h, qb = divmod(item, nqb)
        for e in range(rp[item], rp[item + 1]):
            out.append((h, qb, int(ent[e]) >> 1))
    return out


def mala_check(q, k, v, ow, win, tau, qblocks=None, Bk=64):
    """Run the MALA forward and compare: the keep decisions with the oracle's (bit for bit
    except for tiles whose oracle mass lies within 1e-4 of tau, where the fp32 and fp64
    sums may fall either side), O with the oracle evaluated with the kernel's decisions,
    and LSE with the full scoring."""
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    prob = api.problem(B, L, L, Hq, Hkv, D, torch.bfloat16, D ** -0.5, win)
    plan = api.build_plan("fwd", prob, DEV)
    Bq = plan.info.Bq
    kept = torch.full((max(1, plan.info.nnz),), -1, dtype=torch.int32, device=DEV)
    o, lse = api.mala_fwd(qd, kd, vd, win, tau, plan=plan, kept=kept)
    torch.cuda.synchronize()
    tiles = _plan_tiles(plan)
    kg = kept.cpu().numpy()[:len(tiles)]
    assert set(np.unique(kg)) <= {0, 1}, "every listed tile gets a decision"
    mass = oracle.mala_tile_mass(q, k, ow, D ** -0.5, Bq, Bk, qblocks=qblocks)
    nqb = plan.info.nqb
    kept_gpu = np.ones((Hkv, nqb, -(-L // Bk)), dtype=bool)  # unlisted tiles see nothing
    n_cmp = n_amb = 0
    for (h, qb, kb), g in zip(tiles, kg):
        kept_gpu[h, qb, kb] = bool(g)
        if qblocks is not None and qb not in qblocks:
            continue
        if abs(mass[h, qb, kb] - tau) <= 1e-4:
            n_amb += 1
            continue
        n_cmp += 1
        assert bool(g) == (mass[h, qb, kb] >= tau), (h, qb, kb, mass[h, qb, kb], g)
    n_kept = int(kg.sum())
    print(f"  tau={tau}: {n_kept} of {len(tiles)} tiles kept; {n_cmp} decisions compared, "
          f"{n_amb} within 1e-4 of tau", flush=True)
    Oo, Lo, _ = oracle.mala_fwd(q, k, v, ow, D ** -0.5, tau, Bq, Bk, kept=kept_gpu, qblocks=qblocks)
    if qblocks is None:
        assert_bf16_close("O", o, Oo)
        assert_bf16_close("LSE", lse, Lo)
    else:
        rows = np.concatenate([np.arange(qb * Bq, min(L, (qb + 1) * Bq)) for qb in qblocks])
        idx = torch.as_tensor(rows, device=DEV)
        assert_bf16_close("O[sampled q-blocks]", o[:, idx], Oo[:, rows])
        assert_bf16_close("LSE[sampled q-blocks]", lse[:, :, idx], Lo[:, :, rows])
    return o, lse, n_kept, len(tiles)


@pytest.mark.parametrize("L,Hq,Hkv,mode,tau", [
    (700, 40, 8, "dense", 0.0),
    (700, 40, 8, "dense", 0.02),
    (700, 40, 8, "dense", 0.1),
    (700, 40, 8, "dense", 1.5),
    (900, 16, 2, "dense", 0.05),
    (1000, 40, 8, "complementary", 0.05),
])
def test_mala_fwd(L, Hq, Hkv, mode, tau):
    _case(f"MALA fwd L={L} Hq={Hq} Hkv={Hkv} {mode} tau={tau}")
    ow, win = _windows(L, Hkv, 16, 64, mode=mode)
    q, k, v = inputs.attention_inputs(1, L, L, Hq, Hkv, 128, seed=40)
    o, lse, n_kept, n_tiles = mala_check(q, k, v, ow, win, tau)
    if tau == 0.0:
        assert n_kept == n_tiles
    if tau > 1.0:
        assert n_kept == 0 and bool((o == 0).all())
    else:
        assert 0 < n_kept


def test_mala_fwd_empty_rows_and_items():
    """near = 0 and no sink: the early rows under heads 1-3 see no key, and whole work
    items have empty lists (no scoring sums, no kept entries): O = 0 and LSE = -inf there,
    the rest against the oracle."""
    L, Hq, Hkv, tau = 600, 16, 4, 0.05
    _case(f"MALA fwd L={L} sink=0 near=0 tau={tau}: empty rows and items")
    ow, win = _windows(L, Hkv, 0, 0)
    q, k, v = inputs.attention_inputs(1, L, L, Hq, Hkv, 128, seed=47)
    o, lse, n_kept, n_tiles = mala_check(q, k, v, ow, win, tau)
    assert bool(torch.isinf(lse).any()), "some rows see no key"
    assert 0 < n_kept < n_tiles


def test_mala_fwd_two_sequences_equal_one_at_a_time():
    """B = 2 (the workspace holds each sequence's row sums and kept lists): each sequence's
    O and LSE equal a B = 1 call on that sequence bit for bit, and the first against the
    oracle under the decisions of its own call."""
    L, Hq, Hkv, tau = 800, 40, 8, 0.1
    _case(f"MALA fwd B=2 L={L} dense tau={tau} == two B=1 calls")
    ow, win = _windows(L, Hkv, 16, 64, mode="dense")
    q, k, v = inputs.attention_inputs(2, L, L, Hq, Hkv, 128, seed=46, device=DEV)
    o2, l2 = api.mala_fwd(q, k, v, win, tau)
    for bi in range(2):
        qb, kb, vb = (t[bi:bi + 1].contiguous() for t in (q, k, v))
        o1, l1 = api.mala_fwd(qb, kb, vb, win, tau)
        torch.cuda.synchronize()
        assert torch.equal(o2[bi:bi + 1], o1) and torch.equal(l2[bi:bi + 1], l1), bi
    mala_check(q[0:1].cpu(), k[0:1].cpu(), v[0:1].cpu(), ow, win, tau)


def test_mala_fwd_32k_dense_sampled_qblocks():
    """Full causal MALA at 32K tokens: decisions of 16 sampled q-blocks (all heads, every
    key block) and their rows' O and LSE against the oracle."""
    L, Hq, Hkv = 32768, 40, 8
    _case(f"MALA fwd L={L} dense tau=0.004, sampled q-blocks")
    ow = oracle.Window.for_length(L, Hkv, 128, 2048, 0, mode="dense")
    win = api.window(ow.sink, ow.near, ow.gap, ow.lr, "dense")
    q, k, v = inputs.attention_inputs(1, L, L, Hq, Hkv, 128, seed=41, device=DEV)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    Bq = 256 // (Hq // Hkv)
    nqb = -(-L // Bq)
    rng = np.random.default_rng(141)
    qblocks = sorted({0, 1, nqb - 1} | set(int(x) for x in rng.choice(nqb, 13, replace=False)))
    mala_check(qc, kc, vc, ow, win, 0.004, qblocks=qblocks)


# ------------------------------------------------------------------- MALA backward

def _mala_forward_for_bwd(q, k, v, win, tau):
    """The MALA forward on the device with its keep flags and O's rounding residual."""
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    prob = api.problem(B, L, L, Hq, Hkv, D, torch.bfloat16, D ** -0.5, win)
    fplan = api.build_plan("fwd", prob, DEV)
    kept = torch.full((max(1, fplan.info.nnz),), -1, dtype=torch.int32, device=DEV)
    o_lo = torch.empty_like(q)
    o, lse = api.mala_fwd(q, k, v, win, tau, plan=fplan, kept=kept, o_lo=o_lo)
    return fplan, kept, o, lse, o_lo


def _kept_array(fplan, kept, Hkv, L, Bk=64):
    """The device's decisions as the oracle's [Hkv, nqb, nkb] array (unlisted tiles hold
    no visible key; their value does not matter)."""
    tiles = _plan_tiles(fplan)
    kg = kept.cpu().numpy()[:len(tiles)]
    assert set(np.unique(kg)) <= {0, 1}
    out = np.ones((Hkv, fplan.info.nqb, -(-L // Bk)), dtype=bool)
    for (h, qb, kb), g in zip(tiles, kg):
        out[h, qb, kb] = bool(g)
    return out, int(kg.sum()), len(tiles)


@pytest.mark.parametrize("L,Hq,Hkv,mode,tau,expect_skip", [
    (700, 40, 8, "dense", 0.02, False),
    (700, 40, 8, "dense", 0.2, True),      # about half the tiles skipped
    (1000, 40, 8, "complementary", 0.3, True),
    (900, 16, 2, "dense", 0.15, True),     # G = 8
    (600, 24, 8, "dense", 0.2, True),      # G = 3: two rows of each q-block unused
    (500, 40, 8, "dense", 1.5, True),      # nothing kept: dV = 0, dS = -P Delta everywhere
])
def test_mala_bwd(L, Hq, Hkv, mode, tau, expect_skip):
    """The MALA backward with the kernel's own tile decisions against the oracle's
    gradients under those decisions."""
    _case(f"MALA bwd L={L} Hq={Hq} Hkv={Hkv} {mode} tau={tau}")
    ow, win = _windows(L, Hkv, 16, 64, mode=mode)
    q, k, v, do = inputs.attention_inputs(1, L, L, Hq, Hkv, 128, seed=43, with_dout=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    fplan, kept, o, lse, o_lo = _mala_forward_for_bwd(qd, kd, vd, win, tau)
    dq, dk, dv = api.mala_bwd(qd, kd, vd, o, lse, dod, kept, fplan, win, o_lo=o_lo)
    torch.cuda.synchronize()
    kept_np, n_kept, n_tiles = _kept_array(fplan, kept, Hkv, L)
    print(f"  {n_kept} of {n_tiles} tiles kept", flush=True)
    if expect_skip:
        assert n_kept < n_tiles
    rq, rk, rv = oracle.mala_bwd(q, k, v, do, ow, 128 ** -0.5, fplan.info.Bq, 64, kept_np)
    assert_bf16_close("dQ", dq, rq, gradient=True)
    assert_bf16_close("dK", dk, rk, gradient=True)
    assert_bf16_close("dV", dv, rv, gradient=True)
    if n_kept == 0:
        assert bool((dv == 0).all())


@pytest.mark.parametrize("mode", ["dense", "complementary"])
def test_mala_bwd_tau_zero_is_the_backward(mode):
    """tau = 0 keeps every tile: the MALA backward of the same O and LSE is the CoWA
    backward bit for bit (the mask factors are all 1)."""
    L, Hq, Hkv = 800, 40, 8
    _case(f"MALA bwd tau=0 == bwd, L={L} {mode}")
    ow, win = _windows(L, Hkv, 16, 64, mode=mode)
    q, k, v, do = inputs.attention_inputs(1, L, L, Hq, Hkv, 128, seed=44, with_dout=True,
                                          device=DEV)
    fplan, kept, o, lse, o_lo = _mala_forward_for_bwd(q, k, v, win, 0.0)
    m = api.mala_bwd(q, k, v, o, lse, do, kept, fplan, win, o_lo=o_lo)
    c = api.bwd(q, k, v, o, lse, do, win, o_lo=o_lo)
    torch.cuda.synchronize()
    assert int(kept.sum()) == fplan.info.nnz
    for name, a, b in zip(("dQ", "dK", "dV"), m, c):
        assert torch.equal(a, b), name


def test_mala_bwd_4096_dense():
    """Full causal MALA at 4096 tokens (64 key blocks per row list), a threshold that
    skips a good part of the tiles: every gradient element against the oracle."""
    L, Hq, Hkv, tau = 4096, 40, 8, 0.03
    _case(f"MALA bwd L={L} dense tau={tau}")
    ow = oracle.Window.for_length(L, Hkv, 128, 512, 0, mode="dense")
    win = api.window(ow.sink, ow.near, ow.gap, ow.lr, "dense")
    q, k, v, do = inputs.attention_inputs(1, L, L, Hq, Hkv, 128, seed=45, with_dout=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    fplan, kept, o, lse, o_lo = _mala_forward_for_bwd(qd, kd, vd, win, tau)
    dq, dk, dv = api.mala_bwd(qd, kd, vd, o, lse, dod, kept, fplan, win, o_lo=o_lo)
    torch.cuda.synchronize()
    kept_np, n_kept, n_tiles = _kept_array(fplan, kept, Hkv, L)
    print(f"  {n_kept} of {n_tiles} tiles kept", flush=True)
    assert n_kept < 0.9 * n_tiles
    rq, rk, rv = oracle.mala_bwd(q, k, v, do, ow, 128 ** -0.5, fplan.info.Bq, 64, kept_np)
    assert_bf16_close("dQ", dq, rq, gradient=True)
    assert_bf16_close("dK", dk, rk, gradient=True)
    assert_bf16_close("dV", dv, rv, gradient=True)
