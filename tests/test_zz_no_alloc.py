"""cowa_decode_noalloc through the C ABI: the decode whose split partials live in the
library's fixed device array gives the same bits as cowa_decode with a caller workspace,
on two calls in a row (the second smaller, after the array holds the first call's
partials)."""

import ctypes
import os
import sys

import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))
import oracle  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from structured_sparse_attention_plan_amd import api, inputs  # noqa: E402
from structured_sparse_attention_plan_amd import _cowa as C  # noqa: E402

DEV = "cuda:0"


def _noalloc(q, k, v, win):
    B, _, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    prob = api.problem(B, 1, Lk, Hq, Hkv, D, q.dtype, D ** -0.5, win)
    plan = api.build_plan("decode", prob, q.device)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=q.device)
    st = C.lib.cowa_decode_noalloc(ctypes.byref(prob), ctypes.byref(plan.struct), q.data_ptr(),
                                   k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    C.check("cowa_decode_noalloc", st)
    return o, lse, plan


@pytest.mark.parametrize("B,Lk,Hq,Hkv,sink,near", [
    (16, 6000, 40, 8, 128, 512),   # first call
    (3, 2000, 16, 4, 16, 64),      # second call, smaller
])
def test_decode_noalloc_matches_decode(B, Lk, Hq, Hkv, sink, near):
    print(f"\n[case] decode_noalloc B={B} Lk={Lk} Hq={Hq} Hkv={Hkv}", flush=True)
    ow = oracle.Window.for_length(Lk, Hkv, sink, near, 0)
    win = api.window(ow.sink, ow.near, ow.gap, ow.lr)
    q, k, v = (t.to(DEV) for t in inputs.attention_inputs(B, 1, Lk, Hq, Hkv, 128, seed=70 + B))
    o1, l1, plan = _noalloc(q, k, v, win)
    o2, l2 = api.decode(q, k, v, win, plan=plan)
    torch.cuda.synchronize()
    n_o = int((o1 != o2).sum().item())
    n_l = int((l1 != l2).sum().item())
    print(f"  O differs at {n_o}, LSE at {n_l}", flush=True)
    assert n_o == 0 and n_l == 0
