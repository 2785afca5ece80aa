"""The C ABI: libcowa.so loads, exports every function include/cowa.h declares, and
rejects bad arguments before launching anything (no GPU needed for these paths)."""

import ctypes
import os
import re

import pytest

api = pytest.importorskip("structured_sparse_attention_plan_amd.api")
from structured_sparse_attention_plan_amd import _cowa as C  # noqa: E402

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "cowa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(cowa_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(C.EXPORTS), names
    for n in names:
        assert hasattr(C.lib, n), n


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert C.status_string(s) and C.status_string(s) != "unknown status"
    assert C.status_string(7) == "unknown status"


def _prob(**kw):
    d = dict(B=1, Lq=256, Lk=256, Hq=40, Hkv=8, D=128, dtype=C.COWA_DTYPE_BF16, scale=0.088,
             win=api.make_window(256, 8, 4, 16))
    d.update(kw)
    return C.cowa_problem(d["B"], d["Lq"], d["Lk"], d["Hq"], d["Hkv"], d["D"], d["dtype"], d["scale"],
                          d["win"])


def test_tile_sizes_and_workspace():
    p = _prob()
    assert api.tile_sizes("fwd", p) == (256 // 5, 64)
    assert api.tile_sizes("bwd", p) == (128 // 5, 128)
    assert api.workspace_size("fwd", p) == 0
    # Delta and the row scales of Q (fp32 each), then the fp16 copy of Q
    assert api.workspace_size("bwd", p) == 2 * 40 * 256 * 4 + 256 * 40 * 128 * 2
    pd = _prob(Lq=1, Lk=4096)
    assert api.tile_sizes("decode", pd) == (1, 64)
    assert api.workspace_size("decode", pd) > 0
    f = _prob(dtype=C.COWA_DTYPE_F32, D=64, Hq=4, Hkv=2)
    assert api.tile_sizes("fwd", f) == (64, 64)


@pytest.mark.parametrize("op,kw,status", [
    ("fwd", dict(Hq=41), C.COWA_ERR_UNSUPPORTED),          # Hq % Hkv != 0
    ("fwd", dict(D=96), C.COWA_ERR_UNSUPPORTED),           # bf16 needs D = 128
    ("fwd", dict(dtype=C.COWA_DTYPE_F32), C.COWA_ERR_UNSUPPORTED),  # f32 needs D = 64
    ("bwd", dict(dtype=C.COWA_DTYPE_F32, D=64), C.COWA_ERR_UNSUPPORTED),
    ("decode", dict(Lq=2), C.COWA_ERR_UNSUPPORTED),        # decode is one query row
    ("decode", dict(Lq=1, Hq=24, Hkv=8), C.COWA_ERR_UNSUPPORTED),   # G = 3 not built
    ("fwd", dict(B=0), C.COWA_ERR_INVALID_ARG),
    ("fwd", dict(scale=0.0), C.COWA_ERR_INVALID_ARG),
])
def test_unsupported_and_invalid_problems(op, kw, status):
    p = _prob(**kw)
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    assert C.lib.cowa_tile_sizes(api.OPS[op], ctypes.byref(p), ctypes.byref(bq),
                                 ctypes.byref(bk)) == status


def _fake_plan(p, op, **override):
    bq, bk = api.tile_sizes(op, p)
    info = api.plan_info(p.Lq, p.Lk, p.Hkv, bq, bk, p.win)
    for k, v in override.items():
        setattr(info, k, v)
    one = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation
    return C.cowa_plan_dev(info, p.win, one, one, one, one, one, one)


def test_entry_points_validate_before_launch():
    p = _prob()
    plan = _fake_plan(p, "fwd")
    x = ctypes.c_void_p(256)
    # null output
    assert C.lib.cowa_fwd(ctypes.byref(p), ctypes.byref(plan), x, x, x, None, x, None, 0,
                          None) == C.COWA_ERR_INVALID_ARG
    # plan built for another length / tiling / window
    for bad in (dict(Lq=128), dict(Bq=32)):
        pl = _fake_plan(p, "fwd", **bad)
        assert C.lib.cowa_fwd(ctypes.byref(p), ctypes.byref(pl), x, x, x, x, x, None, 0,
                              None) == C.COWA_ERR_PLAN_MISMATCH
    pl = _fake_plan(p, "fwd")
    pl.win = api.make_window(256, 8, 5, 16)
    assert C.lib.cowa_fwd(ctypes.byref(p), ctypes.byref(pl), x, x, x, x, x, None, 0,
                          None) == C.COWA_ERR_PLAN_MISMATCH
    # backward: workspace too small / misaligned
    pb = _fake_plan(p, "bwd")
    assert C.lib.cowa_bwd(ctypes.byref(p), ctypes.byref(pb), x, x, x, x, x, x, x, x, x, 7, x, 16,
                          None) == C.COWA_ERR_WORKSPACE_TOO_SMALL
    assert C.lib.cowa_bwd(ctypes.byref(p), ctypes.byref(pb), x, x, x, x, x, x, x, x, x, 7,
                          ctypes.c_void_p(260), 1 << 23, None) == C.COWA_ERR_INVALID_ARG
    for bad_stages in (0, 8):
        assert C.lib.cowa_bwd(ctypes.byref(p), ctypes.byref(pb), x, x, x, x, x, x, x, x, x,
                              bad_stages, ctypes.c_void_p(256), 1 << 20,
                              None) == C.COWA_ERR_INVALID_ARG
    # decode: workspace too small
    pd = _prob(Lq=1, Lk=4096, win=api.make_window(4096, 8, 4, 16))
    pld = _fake_plan(pd, "decode")
    assert C.lib.cowa_decode(ctypes.byref(pd), ctypes.byref(pld), x, x, x, x, None, x, 8,
                             None) == C.COWA_ERR_WORKSPACE_TOO_SMALL
    # varlen decode: NULL lengths, workspace too small, more than one query row
    assert C.lib.cowa_decode_varlen(ctypes.byref(pd), x, x, x, None, x, None, x, 1 << 30,
                                    None) == C.COWA_ERR_INVALID_ARG
    assert C.lib.cowa_decode_varlen(ctypes.byref(pd), x, x, x, x, x, None, x, 8,
                                    None) == C.COWA_ERR_WORKSPACE_TOO_SMALL
    p2 = _prob(Lq=2, Lk=4096, win=api.make_window(4096, 8, 4, 16))
    assert C.lib.cowa_decode_varlen(ctypes.byref(p2), x, x, x, x, x, None, x, 1 << 30,
                                    None) == C.COWA_ERR_UNSUPPORTED
