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
    assert api.workspace_size("fwd", p) == 256  # the optional per-XCD work queue heads
    # Delta and the power-of-two scales of Q and dO (fp32 each), 256 bytes of launch-wide
    # maxima, the fp16 copies of Q and dO, then that of K
    assert api.workspace_size("bwd", p) == 3 * 40 * 256 * 4 + 256 + 2 * 256 * 40 * 128 * 2 + 256 * 8 * 128 * 2
    # MALA backward: the backward's tiling and workspace, then one byte per forward tile
    # (8 KV heads x ceil(256 / 51) q-blocks x 4 64-key blocks, rounded up to 256)
    assert api.tile_sizes("mala_bwd", p) == api.tile_sizes("bwd", p)
    assert api.workspace_size("mala_bwd", p) == api.workspace_size("bwd", p) + 256
    pl = _prob(Lq=4096, Lk=4096)
    assert (api.workspace_size("mala_bwd", pl) - api.workspace_size("bwd", pl)
            == -(-(8 * -(-4096 // 51) * 64) // 256) * 256)
    # MALA forward: 1 KB of row sums and 4 bytes of kept list per visible forward tile,
    # 4 bytes per item, each part rounded up to 256
    bq, bk = api.tile_sizes("fwd", pl)
    info = api.plan_info(4096, 4096, 8, bq, bk, pl.win)
    r256 = lambda x: -(-x // 256) * 256  # noqa: E731
    assert api.workspace_size("mala_fwd", pl) == (r256(info.nnz * 1024) + r256(info.nnz * 4)
                                                  + r256(8 * info.nqb * 4))
    pd = _prob(Lq=1, Lk=4096)
    assert api.tile_sizes("decode", pd) == (1, 64)
    assert api.workspace_size("decode", pd) > 0
    f = _prob(dtype=C.COWA_DTYPE_F32, D=64, Hq=4, Hkv=2)
    assert api.tile_sizes("fwd", f) == (8, 64)


@pytest.mark.parametrize("op,kw,status", [
    ("fwd", dict(Hq=41), C.COWA_ERR_UNSUPPORTED),          # Hq % Hkv != 0
    ("fwd", dict(D=96), C.COWA_ERR_UNSUPPORTED),           # bf16 needs D = 128
    ("fwd", dict(dtype=C.COWA_DTYPE_F32), C.COWA_ERR_UNSUPPORTED),  # f32 needs D = 64
    ("bwd", dict(dtype=C.COWA_DTYPE_F32, D=64), C.COWA_ERR_UNSUPPORTED),
    ("decode", dict(Lq=2), C.COWA_ERR_UNSUPPORTED),        # decode is one query row
    ("decode", dict(Lq=1, Hq=72, Hkv=8), C.COWA_ERR_UNSUPPORTED),   # G = 9 not built
    ("mala_bwd", dict(B=2), C.COWA_ERR_UNSUPPORTED),       # one sequence only
    ("mala_bwd", dict(dtype=C.COWA_DTYPE_F32, D=64), C.COWA_ERR_UNSUPPORTED),
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
    assert C.lib.cowa_fwd(ctypes.byref(p), ctypes.byref(plan), x, x, x, None, x, None, None, 0,
                          None) == C.COWA_ERR_INVALID_ARG
    # a rounding residual of O is bf16 only
    pf = _prob(dtype=C.COWA_DTYPE_F32, D=64, Hq=4, Hkv=2)
    plf = _fake_plan(pf, "fwd")
    assert C.lib.cowa_fwd(ctypes.byref(pf), ctypes.byref(plf), x, x, x, x, x, x, None, 0,
                          None) == C.COWA_ERR_INVALID_ARG
    # plan built for another length / tiling / window
    for bad in (dict(Lq=128), dict(Bq=32)):
        pl = _fake_plan(p, "fwd", **bad)
        assert C.lib.cowa_fwd(ctypes.byref(p), ctypes.byref(pl), x, x, x, x, x, None, None, 0,
                              None) == C.COWA_ERR_PLAN_MISMATCH
    pl = _fake_plan(p, "fwd")
    pl.win = api.make_window(256, 8, 5, 16)
    assert C.lib.cowa_fwd(ctypes.byref(p), ctypes.byref(pl), x, x, x, x, x, None, None, 0,
                          None) == C.COWA_ERR_PLAN_MISMATCH
    # backward: workspace too small / misaligned
    pb = _fake_plan(p, "bwd")
    assert C.lib.cowa_bwd(ctypes.byref(p), ctypes.byref(pb), x, x, x, x, None, x, x, x, x, x, 7, x,
                          16, None) == C.COWA_ERR_WORKSPACE_TOO_SMALL
    assert C.lib.cowa_bwd(ctypes.byref(p), ctypes.byref(pb), x, x, x, x, x, x, x, x, x, x, 7,
                          ctypes.c_void_p(260), 1 << 24, None) == C.COWA_ERR_INVALID_ARG
    for bad_stages in (0, 8):
        assert C.lib.cowa_bwd(ctypes.byref(p), ctypes.byref(pb), x, x, x, x, None, x, x, x, x, x,
                              bad_stages, ctypes.c_void_p(256), 1 << 24,
                              None) == C.COWA_ERR_INVALID_ARG
    # MALA backward: NULL keep flags, plans swapped (a backward plan is no forward plan),
    # workspace too small for the mask after the backward's arrays
    pf = _fake_plan(p, "fwd")
    pm = _fake_plan(p, "mala_bwd")
    big = 1 << 30
    assert C.lib.cowa_mala_bwd(ctypes.byref(p), ctypes.byref(pf), ctypes.byref(pm), None, x, x, x, x,
                               None, x, x, x, x, x, ctypes.c_void_p(256), big,
                               None) == C.COWA_ERR_INVALID_ARG
    assert C.lib.cowa_mala_bwd(ctypes.byref(p), ctypes.byref(pm), ctypes.byref(pm), x, x, x, x, x,
                               None, x, x, x, x, x, ctypes.c_void_p(256), big,
                               None) == C.COWA_ERR_PLAN_MISMATCH
    assert C.lib.cowa_mala_bwd(ctypes.byref(p), ctypes.byref(pf), ctypes.byref(pf), x, x, x, x, x,
                               None, x, x, x, x, x, ctypes.c_void_p(256), big,
                               None) == C.COWA_ERR_PLAN_MISMATCH
    assert C.lib.cowa_mala_bwd(ctypes.byref(p), ctypes.byref(pf), ctypes.byref(pm), x, x, x, x, x,
                               None, x, x, x, x, x, ctypes.c_void_p(256), api.workspace_size("bwd", p),
                               None) == C.COWA_ERR_WORKSPACE_TOO_SMALL
    # MALA forward: negative tau, keep flags with B > 1, workspace too small
    assert C.lib.cowa_mala_fwd(ctypes.byref(p), ctypes.byref(pf), -0.5, x, x, x, x, x, None, None,
                               ctypes.c_void_p(256), big, None) == C.COWA_ERR_INVALID_ARG
    p2b = _prob(B=2)
    pf2 = _fake_plan(p2b, "fwd")
    assert C.lib.cowa_mala_fwd(ctypes.byref(p2b), ctypes.byref(pf2), 0.1, x, x, x, x, x, None, x,
                               ctypes.c_void_p(256), big, None) == C.COWA_ERR_INVALID_ARG
    assert C.lib.cowa_mala_fwd(ctypes.byref(p), ctypes.byref(pf), 0.1, x, x, x, x, x, None, None,
                               ctypes.c_void_p(256), 16, None) == C.COWA_ERR_WORKSPACE_TOO_SMALL
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
    # window-only caches: a head whose slots pass 2^31 bytes (dense: every position kept)
    for Lmax, status in ((1 << 23, C.COWA_ERR_UNSUPPORTED), ((1 << 23) - 1, C.COWA_ERR_WORKSPACE_TOO_SMALL)):
        wd = api.window(4, 16, 0, 0, "dense")
        pw = _prob(Lq=1, Lk=Lmax, win=wd)
        cw = C.cowa_wcache(1, pw.Hkv, 128, Lmax, wd, x, x)
        assert C.lib.cowa_wcache_decode(ctypes.byref(pw), ctypes.byref(cw), x, x, x, None, x, 8,
                                        None) == status


def test_python_layer_rejects_host_and_misshapen_tensors():
    """The Python layer checks every tensor it passes (inputs, caller-supplied outputs,
    gradients, workspace) before calling into the library: host tensors, wrong shapes
    and dtypes raise ValueError, so nothing reaches a kernel."""
    import torch
    win = api.make_window(64, 2, 4, 16)
    q = torch.zeros((1, 64, 4, 128), dtype=torch.bfloat16)
    k = torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        api.fwd(q, k, k, win)
    with pytest.raises(ValueError):
        api._check_tensor("lse", torch.zeros((1, 4, 63)), (1, 4, 64), torch.float32)
    with pytest.raises(ValueError):
        api._workspace("workspace", torch.zeros(16, dtype=torch.uint8), 32, torch.device("cpu"))


def test_decode_noalloc_rejects_problems_beyond_its_array():
    """cowa_decode_noalloc checks the problem's partials against its fixed device array
    before touching the device: a batch whose partials exceed COWA_DECODE_SCRATCH_BYTES
    gets WORKSPACE_TOO_SMALL (the plan's pointers are never read)."""
    pd = _prob(B=2048, Lq=1, Lk=4096, win=api.make_window(4096, 8, 4, 16))
    need = api.workspace_size("decode", pd)
    assert need > C.COWA_DECODE_SCRATCH_BYTES
    pld = _fake_plan(pd, "decode")
    x = ctypes.c_void_p(256)
    assert C.lib.cowa_decode_noalloc(ctypes.byref(pd), ctypes.byref(pld), x, x, x, x, None,
                                     None) == C.COWA_ERR_WORKSPACE_TOO_SMALL
    # and it validates like cowa_decode (null output)
    ps = _prob(B=2, Lq=1, Lk=4096, win=api.make_window(4096, 8, 4, 16))
    pls = _fake_plan(ps, "decode")
    assert C.lib.cowa_decode_noalloc(ctypes.byref(ps), ctypes.byref(pls), x, x, x, None, None,
                                     None) == C.COWA_ERR_INVALID_ARG
