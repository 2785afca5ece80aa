"""Thin Python layer over the C ABI: builds plans, moves them to the device and calls
cowa_fwd / cowa_bwd / cowa_decode with torch-owned buffers.

Marshalling only — every step of the attention runs in libcowa's HIP kernels; torch
supplies device memory and the current stream.
"""

import ctypes

import numpy as np
import torch

from . import _cowa as C

MODES = {"complementary": C.COWA_BAND_COMPLEMENTARY, "duplicated": C.COWA_BAND_DUPLICATED,
         "dense": C.COWA_BAND_DENSE}
OPS = {"fwd": C.COWA_OP_FWD, "bwd": C.COWA_OP_BWD, "decode": C.COWA_OP_DECODE,
       "mala_bwd": C.COWA_OP_MALA_BWD, "mala_fwd": C.COWA_OP_MALA_FWD}


def make_window(Lmax, Hkv, sink, near, gap=0, mode="complementary"):
    """cowa_window_make: bands of width ceil((Lmax - near - gap) / Hkv)."""
    w = C.cowa_window()
    C.check("cowa_window_make", C.lib.cowa_window_make(Lmax, Hkv, sink, near, gap, MODES[mode],
                                                      ctypes.byref(w)))
    return w


def window(sink, near, gap, lr, mode="complementary"):
    return C.cowa_window(sink, near, gap, lr, MODES[mode])


def problem(B, Lq, Lk, Hq, Hkv, D, dtype, scale, win):
    dt = {torch.bfloat16: C.COWA_DTYPE_BF16, torch.float32: C.COWA_DTYPE_F32}[dtype]
    return C.cowa_problem(B, Lq, Lk, Hq, Hkv, D, dt, float(scale), win)


def tile_sizes(op, prob):
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    C.check("cowa_tile_sizes", C.lib.cowa_tile_sizes(OPS[op], ctypes.byref(prob), ctypes.byref(bq),
                                                    ctypes.byref(bk)))
    return bq.value, bk.value


_WS_SIZES = {}


def workspace_size(op, prob):
    """cowa_workspace_size, remembered per (op, problem): for the MALA forward the library
    counts the visible tiles with the planner, which takes milliseconds at 32K tokens."""
    w = prob.win
    key = (op, prob.B, prob.Lq, prob.Lk, prob.Hq, prob.Hkv, prob.D, prob.dtype,
           w.sink, w.near_w, w.gap, w.lr, w.band_mode)
    if key not in _WS_SIZES:
        n = ctypes.c_size_t()
        C.check("cowa_workspace_size", C.lib.cowa_workspace_size(OPS[op], ctypes.byref(prob),
                                                                ctypes.byref(n)))
        _WS_SIZES[key] = n.value
    return _WS_SIZES[key]


class HostPlan:
    """Output of cowa_plan_blocks: the info struct and (optionally) the CSR arrays."""

    def __init__(self, info, win, arrays):
        self.info = info
        self.win = win
        self.arrays = arrays  # dict of int32 numpy arrays, or None


def plan_info(Lq, Lk, Hkv, Bq, Bk, win):
    info = C.cowa_plan_info()
    C.check("cowa_plan_blocks", C.lib.cowa_plan_blocks(Lq, Lk, Hkv, Bq, Bk, ctypes.byref(win),
                                                      ctypes.byref(info), None, None, None, None,
                                                      None, None))
    return info


def plan_blocks(Lq, Lk, Hkv, Bq, Bk, win):
    info = plan_info(Lq, Lk, Hkv, Bq, Bk, win)
    arr = {
        "row_ptr": np.zeros(Hkv * info.nqb + 1, np.int32),
        "row_ent": np.zeros(max(1, info.nnz), np.int32),
        "col_ptr": np.zeros(Hkv * info.nkb + 1, np.int32),
        "col_ent": np.zeros(max(1, info.nnz), np.int32),
        "row_order": np.zeros(Hkv * info.nqb, np.int32),
        "col_order": np.zeros(Hkv * info.nkb, np.int32),
    }
    ptr = {k: v.ctypes.data_as(C._pi32) for k, v in arr.items()}
    info2 = C.cowa_plan_info()
    C.check("cowa_plan_blocks", C.lib.cowa_plan_blocks(
        Lq, Lk, Hkv, Bq, Bk, ctypes.byref(win), ctypes.byref(info2), ptr["row_ptr"],
        ptr["row_ent"], ptr["col_ptr"], ptr["col_ent"], ptr["row_order"], ptr["col_order"]))
    return HostPlan(info2, win, arr)


class DevicePlan:
    """A HostPlan copied to device memory, with the cowa_plan_dev struct pointing at it."""

    def __init__(self, host, device):
        self.host = host
        self.tensors = {k: torch.from_numpy(v).to(device) for k, v in host.arrays.items()}
        t = self.tensors
        self.struct = C.cowa_plan_dev(host.info, host.win, t["row_ptr"].data_ptr(),
                                      t["row_ent"].data_ptr(), t["col_ptr"].data_ptr(),
                                      t["col_ent"].data_ptr(), t["row_order"].data_ptr(),
                                      t["col_order"].data_ptr())

    @property
    def info(self):
        return self.host.info


def build_plan(op, prob, device):
    bq, bk = tile_sizes(op, prob)
    return DevicePlan(plan_blocks(prob.Lq, prob.Lk, prob.Hkv, bq, bk, prob.win), device)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tensor(name, t, shape, dtype, device=None):
    if (tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda
            or (device is not None and t.device != device)):
        raise ValueError(f"{name}: expected contiguous {dtype} device tensor of shape {tuple(shape)}"
                         f"{'' if device is None else ' on ' + str(device)}, got {t.dtype} "
                         f"{tuple(t.shape)} contiguous={t.is_contiguous()} device={t.device}")


def _workspace(name, ws, nbytes, device):
    """A caller's workspace: a contiguous uint8 tensor of at least nbytes on the device
    (the library checks the size and the 256-byte alignment again)."""
    if ws is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device != device or ws.numel() < nbytes:
        raise ValueError(f"{name}: expected a contiguous uint8 tensor of at least {nbytes} bytes on "
                         f"{device}, got {ws.dtype} of {ws.numel()} elements on {ws.device}")
    return ws


def fwd(q, k, v, win, scale=None, plan=None, out=None, lse=None, o_lo=None, workspace=None):
    """Forward: q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D] -> (o like q, lse [B,Hq,Lq] fp32).
    o_lo (a tensor like q, bf16 only): filled with O's bf16 rounding residual, for bwd.
    workspace (uint8, workspace_size("fwd") bytes; allocated when None): holds the launch's
    work queues (bf16, one sequence)."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    scale = D ** -0.5 if scale is None else scale
    prob = problem(B, Lq, Lk, Hq, Hkv, D, q.dtype, scale, win)
    _check_tensor("q", q, (B, Lq, Hq, D), q.dtype)
    _check_tensor("k", k, (B, Lk, Hkv, D), q.dtype, q.device)
    _check_tensor("v", v, (B, Lk, Hkv, D), q.dtype, q.device)
    plan = build_plan("fwd", prob, q.device) if plan is None else plan
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor("out", out, (B, Lq, Hq, D), q.dtype, q.device)
    _check_tensor("lse", lse, (B, Hq, Lq), torch.float32, q.device)
    if o_lo is not None:
        _check_tensor("o_lo", o_lo, (B, Lq, Hq, D), q.dtype, q.device)
    nbytes = workspace_size("fwd", prob)
    ws = _workspace("workspace", workspace, nbytes, q.device) if nbytes else None
    C.check("cowa_fwd", C.lib.cowa_fwd(ctypes.byref(prob), ctypes.byref(plan.struct), q.data_ptr(),
                                       k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                       None if o_lo is None else o_lo.data_ptr(),
                                       None if ws is None else ws.data_ptr(), nbytes,
                                       _stream(q.device)))
    return out, lse


def mala_fwd(q, k, v, win, tau, scale=None, plan=None, out=None, lse=None, kept=None, o_lo=None,
             workspace=None):
    """MALA forward (cowa_mala_fwd): -> (o like q, lse [B,Hq,Lq] fp32).  kept: optional
    int32 tensor of the plan's nnz entries, filled with the per-tile keep decisions;
    o_lo: optional tensor like q for O's rounding residual (for mala_bwd); workspace:
    optional uint8 tensor of workspace_size("mala_fwd") bytes."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    scale = D ** -0.5 if scale is None else scale
    prob = problem(B, Lq, Lk, Hq, Hkv, D, q.dtype, scale, win)
    _check_tensor("q", q, (B, Lq, Hq, D), q.dtype)
    _check_tensor("k", k, (B, Lk, Hkv, D), q.dtype, q.device)
    _check_tensor("v", v, (B, Lk, Hkv, D), q.dtype, q.device)
    plan = build_plan("fwd", prob, q.device) if plan is None else plan
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor("out", out, (B, Lq, Hq, D), q.dtype, q.device)
    _check_tensor("lse", lse, (B, Hq, Lq), torch.float32, q.device)
    if kept is not None:
        _check_tensor("kept", kept, (max(1, plan.info.nnz),), torch.int32, q.device)
    if o_lo is not None:
        _check_tensor("o_lo", o_lo, (B, Lq, Hq, D), q.dtype, q.device)
    workspace = _workspace("workspace", workspace, workspace_size("mala_fwd", prob), q.device)
    C.check("cowa_mala_fwd", C.lib.cowa_mala_fwd(
        ctypes.byref(prob), ctypes.byref(plan.struct), float(tau), q.data_ptr(), k.data_ptr(),
        v.data_ptr(), out.data_ptr(), lse.data_ptr(), None if o_lo is None else o_lo.data_ptr(),
        None if kept is None else kept.data_ptr(), workspace.data_ptr(), workspace.numel(),
        _stream(q.device)))
    return out, lse


def bwd(q, k, v, o, lse, dout, win, scale=None, plan=None, grads=None, workspace=None,
        stages=C.COWA_BWD_ALL, o_lo=None):
    """Backward: -> (dq like q, dk like k, dv like v).  `stages` as in cowa_bwd; o_lo is
    the residual fwd wrote (optional)."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    scale = D ** -0.5 if scale is None else scale
    prob = problem(B, Lq, Lk, Hq, Hkv, D, q.dtype, scale, win)
    for name, t, shp in (("q", q, (B, Lq, Hq, D)), ("k", k, (B, Lk, Hkv, D)), ("v", v, (B, Lk, Hkv, D)),
                         ("o", o, (B, Lq, Hq, D)), ("dout", dout, (B, Lq, Hq, D))):
        _check_tensor(name, t, shp, q.dtype, q.device)
    _check_tensor("lse", lse, (B, Hq, Lq), torch.float32, q.device)
    if o_lo is not None:
        _check_tensor("o_lo", o_lo, (B, Lq, Hq, D), q.dtype, q.device)
    plan = build_plan("bwd", prob, q.device) if plan is None else plan
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    _check_tensor("dq", dq, (B, Lq, Hq, D), q.dtype, q.device)
    _check_tensor("dk", dk, (B, Lk, Hkv, D), q.dtype, q.device)
    _check_tensor("dv", dv, (B, Lk, Hkv, D), q.dtype, q.device)
    workspace = _workspace("workspace", workspace, workspace_size("bwd", prob), q.device)
    C.check("cowa_bwd", C.lib.cowa_bwd(ctypes.byref(prob), ctypes.byref(plan.struct), q.data_ptr(),
                                       k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       None if o_lo is None else o_lo.data_ptr(), lse.data_ptr(),
                                       dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                       int(stages), workspace.data_ptr(), workspace.numel(),
                                       _stream(q.device)))
    return dq, dk, dv


def mala_bwd(q, k, v, o, lse, dout, kept, fwd_plan, win, scale=None, plan=None, grads=None,
             workspace=None, o_lo=None):
    """MALA backward (cowa_mala_bwd) with the forward's tile decisions held fixed: kept is
    the int32 tensor mala_fwd filled for fwd_plan; -> (dq like q, dk like k, dv like v)."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    scale = D ** -0.5 if scale is None else scale
    prob = problem(B, Lq, Lk, Hq, Hkv, D, q.dtype, scale, win)
    for name, t, shp in (("q", q, (B, Lq, Hq, D)), ("k", k, (B, Lk, Hkv, D)), ("v", v, (B, Lk, Hkv, D)),
                         ("o", o, (B, Lq, Hq, D)), ("dout", dout, (B, Lq, Hq, D))):
        _check_tensor(name, t, shp, q.dtype, q.device)
    _check_tensor("lse", lse, (B, Hq, Lq), torch.float32, q.device)
    _check_tensor("kept", kept, (max(1, fwd_plan.info.nnz),), torch.int32, q.device)
    if o_lo is not None:
        _check_tensor("o_lo", o_lo, (B, Lq, Hq, D), q.dtype, q.device)
    plan = build_plan("mala_bwd", prob, q.device) if plan is None else plan
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    _check_tensor("dq", dq, (B, Lq, Hq, D), q.dtype, q.device)
    _check_tensor("dk", dk, (B, Lk, Hkv, D), q.dtype, q.device)
    _check_tensor("dv", dv, (B, Lk, Hkv, D), q.dtype, q.device)
    workspace = _workspace("workspace", workspace, workspace_size("mala_bwd", prob), q.device)
    C.check("cowa_mala_bwd", C.lib.cowa_mala_bwd(
        ctypes.byref(prob), ctypes.byref(fwd_plan.struct), ctypes.byref(plan.struct), kept.data_ptr(),
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), None if o_lo is None else o_lo.data_ptr(),
        lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
        workspace.data_ptr(), workspace.numel(), _stream(q.device)))
    return dq, dk, dv


def decode(q, k_cache, v_cache, win, scale=None, plan=None, out=None, lse=None, workspace=None):
    """Decode: q [B,1,Hq,D] at position Lk-1 over caches [B,Lk,Hkv,D] -> (o, lse [B,Hq])."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k_cache.shape[1], k_cache.shape[2]
    scale = D ** -0.5 if scale is None else scale
    prob = problem(B, Lq, Lk, Hq, Hkv, D, q.dtype, scale, win)
    _check_tensor("q", q, (B, 1, Hq, D), q.dtype)
    _check_tensor("k_cache", k_cache, (B, Lk, Hkv, D), q.dtype, q.device)
    _check_tensor("v_cache", v_cache, (B, Lk, Hkv, D), q.dtype, q.device)
    plan = build_plan("decode", prob, q.device) if plan is None else plan
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor("out", out, (B, 1, Hq, D), q.dtype, q.device)
    _check_tensor("lse", lse, (B, Hq), torch.float32, q.device)
    workspace = _workspace("workspace", workspace, workspace_size("decode", prob), q.device)
    C.check("cowa_decode", C.lib.cowa_decode(ctypes.byref(prob), ctypes.byref(plan.struct),
                                             q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                             out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                                             workspace.numel(), _stream(q.device)))
    return out, lse


def decode_varlen(q, k_cache, v_cache, seqlens, win, scale=None, out=None, lse=None, workspace=None):
    """Decode of B sequences of their own lengths: q [B,1,Hq,D]; caches [B,Lk,Hkv,D] hold
    Lk positions, sequence b uses the first seqlens[b] (int32 [B] on the device) and its
    query sits at position seqlens[b]-1 -> (o, lse [B,Hq])."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k_cache.shape[1], k_cache.shape[2]
    scale = D ** -0.5 if scale is None else scale
    prob = problem(B, Lq, Lk, Hq, Hkv, D, q.dtype, scale, win)
    _check_tensor("q", q, (B, 1, Hq, D), q.dtype)
    _check_tensor("k_cache", k_cache, (B, Lk, Hkv, D), q.dtype, q.device)
    _check_tensor("v_cache", v_cache, (B, Lk, Hkv, D), q.dtype, q.device)
    _check_tensor("seqlens", seqlens, (B,), torch.int32, q.device)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor("out", out, (B, 1, Hq, D), q.dtype, q.device)
    _check_tensor("lse", lse, (B, Hq), torch.float32, q.device)
    workspace = _workspace("workspace", workspace, workspace_size("decode", prob), q.device)
    C.check("cowa_decode_varlen",
            C.lib.cowa_decode_varlen(ctypes.byref(prob), q.data_ptr(), k_cache.data_ptr(),
                                     v_cache.data_ptr(), seqlens.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                     _stream(q.device)))
    return out, lse


def fwd_bwd(q, k, v, dout, win, scale=None):
    """Training step of the operator: forward keeping O's rounding residual, then the
    backward from it -> (o, lse, dq, dk, dv)."""
    o_lo = torch.empty_like(q)
    o, lse = fwd(q, k, v, win, scale, o_lo=o_lo)
    dq, dk, dv = bwd(q, k, v, o, lse, dout, win, scale, o_lo=o_lo)
    return o, lse, dq, dk, dv


def wcache_layout(win, Hkv, Lmax):
    """cowa_wcache_layout -> (slots per sequence, first slot of each head [Hkv + 1])."""
    offs = (ctypes.c_int64 * (Hkv + 1))()
    slots = ctypes.c_int64()
    C.check("cowa_wcache_layout", C.lib.cowa_wcache_layout(ctypes.byref(win), Hkv, Lmax, offs,
                                                          ctypes.byref(slots)))
    return slots.value, list(offs)


class WindowCache:
    """Window-only KV caches of B sequences (cowa_wcache): per KV head the prefix sink and
    the ring of positions the head can still see, K and V [B, slots, D] bf16 on `device`."""

    def __init__(self, B, Hkv, D, Lmax, win, device, dtype=torch.bfloat16):
        self.slots, self.head_offset = wcache_layout(win, Hkv, Lmax)
        self.B, self.Hkv, self.D, self.Lmax, self.win = B, Hkv, D, Lmax, win
        self.k = torch.zeros((B, self.slots, D), dtype=dtype, device=device)
        self.v = torch.zeros_like(self.k)
        self.struct = C.cowa_wcache(B, Hkv, D, Lmax, win, self.k.data_ptr(), self.v.data_ptr())

    def nbytes(self):
        return 2 * self.k.numel() * self.k.element_size()

    def append(self, k_new, v_new, pos0):
        """Append T tokens per sequence: k_new/v_new [B, T, Hkv, D] at positions
        pos0[b] .. pos0[b] + T - 1 (pos0: int32 [B] on the device)."""
        B, T = k_new.shape[0], k_new.shape[1]
        _check_tensor("k_new", k_new, (self.B, T, self.Hkv, self.D), self.k.dtype, self.k.device)
        _check_tensor("v_new", v_new, (self.B, T, self.Hkv, self.D), self.k.dtype, self.k.device)
        _check_tensor("pos0", pos0, (self.B,), torch.int32, self.k.device)
        C.check("cowa_wcache_append",
                C.lib.cowa_wcache_append(ctypes.byref(self.struct), k_new.data_ptr(), v_new.data_ptr(), T,
                                         pos0.data_ptr(), _stream(self.k.device)))

    def decode(self, q, seqlens, scale=None, out=None, lse=None, workspace=None):
        """Decode of q [B,1,Hq,D]: sequence b has length seqlens[b] (int32 [B] on the
        device), its query at position seqlens[b] - 1 -> (o, lse [B,Hq])."""
        B, Lq, Hq, D = q.shape
        scale = D ** -0.5 if scale is None else scale
        prob = problem(B, 1, self.Lmax, Hq, self.Hkv, D, q.dtype, scale, self.win)
        _check_tensor("q", q, (self.B, 1, Hq, self.D), self.k.dtype, self.k.device)
        _check_tensor("seqlens", seqlens, (self.B,), torch.int32, self.k.device)
        out = torch.empty_like(q) if out is None else out
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
        _check_tensor("out", out, (B, 1, Hq, D), q.dtype, q.device)
        _check_tensor("lse", lse, (B, Hq), torch.float32, q.device)
        workspace = _workspace("workspace", workspace, workspace_size("decode", prob), q.device)
        C.check("cowa_wcache_decode",
                C.lib.cowa_wcache_decode(ctypes.byref(prob), ctypes.byref(self.struct), q.data_ptr(),
                                         seqlens.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                         workspace.data_ptr(), workspace.numel(), _stream(q.device)))
        return out, lse
