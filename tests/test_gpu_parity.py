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
    o, lse = api.fwd(qd, kd, vd, win)
    dq, dk, dv = api.bwd(qd, kd, vd, o, lse, dod, win)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, ow, 128 ** -0.5)
    assert_bf16_close("dQ", dq, rq, value_scaled=True)
    assert_bf16_close("dK", dk, rk, value_scaled=True)
    assert_bf16_close("dV", dv, rv, value_scaled=True)


def test_bwd_bf16_mid_2048_full():
    _case("bwd bf16 L=2048 Hq=40 Hkv=8 sink=128 near=512")
    L = 2048
    ow, win = _windows(L, 8, 128, 512)
    q, k, v, do = inputs.attention_inputs(1, L, L, 40, 8, 128, seed=5, with_dout=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = api.fwd(qd, kd, vd, win)
    dq, dk, dv = api.bwd(qd, kd, vd, o, lse, dod, win)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, ow, 128 ** -0.5)
    assert_bf16_close("dQ", dq, rq, value_scaled=True)
    assert_bf16_close("dK", dk, rk, value_scaled=True)
    assert_bf16_close("dV", dv, rv, value_scaled=True)


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
    o, lse = api.fwd(qd, kd, vd, win)
    dq, dk, dv = api.bwd(qd, kd, vd, o, lse, dod, win)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, ow, 128 ** -0.5)
    assert_bf16_close("dQ", dq, rq, value_scaled=True)
    assert_bf16_close("dK", dk, rk, value_scaled=True)
    assert_bf16_close("dV", dv, rv, value_scaled=True)


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
    o, lse = api.fwd(qd, kd, vd, win)
    dq, dk, dv = api.bwd(qd, kd, vd, o, lse, dod, win)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, ow, 128 ** -0.5)
    # compare in the units of the unscaled problem, where the bars are set
    assert_bf16_close("dQ * 2^qexp", dq.float() * 2.0 ** qexp, rq * 2.0 ** qexp, value_scaled=True)
    assert_bf16_close("dK * 2^-qexp", dk.float() * 2.0 ** -qexp, rk * 2.0 ** -qexp, value_scaled=True)
    assert_bf16_close("dV", dv, rv, value_scaled=True)


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
