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
OPS = {"fwd": C.COWA_OP_FWD, "bwd": C.COWA_OP_BWD, "decode": C.COWA_OP_DECODE}


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


def workspace_size(op, prob):
    n = ctypes.c_size_t()
    C.check("cowa_workspace_size", C.lib.cowa_workspace_size(OPS[op], ctypes.byref(prob),
                                                            ctypes.byref(n)))
    return n.value


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


def _check_tensor(name, t, shape, dtype):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} device tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()} "
                         f"device={t.device}")


def fwd(q, k, v, win, scale=None, plan=None, out=None, lse=None):
    """Forward: q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D] -> (o like q, lse [B,Hq,Lq] fp32)."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    scale = D ** -0.5 if scale is None else scale
    prob = problem(B, Lq, Lk, Hq, Hkv, D, q.dtype, scale, win)
    _check_tensor("q", q, (B, Lq, Hq, D), q.dtype)
    _check_tensor("k", k, (B, Lk, Hkv, D), q.dtype)
    _check_tensor("v", v, (B, Lk, Hkv, D), q.dtype)
    plan = build_plan("fwd", prob, q.device) if plan is None else plan
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device) if lse is None else lse
    C.check("cowa_fwd", C.lib.cowa_fwd(ctypes.byref(prob), ctypes.byref(plan.struct), q.data_ptr(),
                                       k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                       None, 0, _stream(q.device)))
    return out, lse


def bwd(q, k, v, o, lse, dout, win, scale=None, plan=None, grads=None, workspace=None,
        stages=C.COWA_BWD_ALL):
    """Backward: -> (dq like q, dk like k, dv like v).  `stages` as in cowa_bwd."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    scale = D ** -0.5 if scale is None else scale
    prob = problem(B, Lq, Lk, Hq, Hkv, D, q.dtype, scale, win)
    for name, t, shp in (("q", q, (B, Lq, Hq, D)), ("k", k, (B, Lk, Hkv, D)), ("v", v, (B, Lk, Hkv, D)),
                         ("o", o, (B, Lq, Hq, D)), ("dout", dout, (B, Lq, Hq, D))):
        _check_tensor(name, t, shp, q.dtype)
    _check_tensor("lse", lse, (B, Hq, Lq), torch.float32)
    plan = build_plan("bwd", prob, q.device) if plan is None else plan
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    nbytes = workspace_size("bwd", prob)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    C.check("cowa_bwd", C.lib.cowa_bwd(ctypes.byref(prob), ctypes.byref(plan.struct), q.data_ptr(),
                                       k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                       dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                       int(stages), workspace.data_ptr(), workspace.numel(),
                                       _stream(q.device)))
    return dq, dk, dv


def decode(q, k_cache, v_cache, win, scale=None, plan=None, out=None, lse=None, workspace=None):
    """Decode: q [B,1,Hq,D] at position Lk-1 over caches [B,Lk,Hkv,D] -> (o, lse [B,Hq])."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k_cache.shape[1], k_cache.shape[2]
    scale = D ** -0.5 if scale is None else scale
    prob = problem(B, Lq, Lk, Hq, Hkv, D, q.dtype, scale, win)
    _check_tensor("q", q, (B, 1, Hq, D), q.dtype)
    _check_tensor("k_cache", k_cache, (B, Lk, Hkv, D), q.dtype)
    _check_tensor("v_cache", v_cache, (B, Lk, Hkv, D), q.dtype)
    plan = build_plan("decode", prob, q.device) if plan is None else plan
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    nbytes = workspace_size("decode", prob)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
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
    _check_tensor("k_cache", k_cache, (B, Lk, Hkv, D), q.dtype)
    _check_tensor("v_cache", v_cache, (B, Lk, Hkv, D), q.dtype)
    _check_tensor("seqlens", seqlens, (B,), torch.int32)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    nbytes = workspace_size("decode", prob)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    C.check("cowa_decode_varlen",
            C.lib.cowa_decode_varlen(ctypes.byref(prob), q.data_ptr(), k_cache.data_ptr(),
                                     v_cache.data_ptr(), seqlens.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                     _stream(q.device)))
    return out, lse
