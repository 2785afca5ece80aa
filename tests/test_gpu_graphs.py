"""The library's launches captured in HIP graphs (torch.cuda.CUDAGraph over the current
stream): nothing in them allocates, copies from the host or clears memory with a memset
(the clears are fill kernels), so a captured decode step and a captured training step
replay correctly.  Each graph is replayed several times with new inputs copied in,
eager work and synchronisations between the replays, and every replay is compared bit
for bit with the eager call on the same inputs."""

import os
import sys

import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from structured_sparse_attention_plan_amd import api, inputs  # noqa: E402

DEV = "cuda:0"


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def test_decode_step_in_a_graph():
    B, Lk, Hq, Hkv, D = 4, 6000, 40, 8, 128
    _case(f"decode B={B} Lk={Lk} captured in a graph, 4 replays")
    win = api.make_window(Lk, Hkv, 64, 512)
    prob = api.problem(B, 1, Lk, Hq, Hkv, D, torch.bfloat16, D ** -0.5, win)
    plan = api.build_plan("decode", prob, DEV)
    _, k, v = inputs.attention_inputs(B, 1, Lk, Hq, Hkv, D, seed=80, device=DEV)
    q = torch.empty((B, 1, Hq, D), dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    ws = torch.empty(api.workspace_size("decode", prob), dtype=torch.uint8, device=DEV)
    q.copy_(inputs.attention_inputs(B, 1, Lk, Hq, Hkv, D, seed=81, device=DEV)[0])
    api.decode(q, k, v, win, plan=plan, out=o, lse=lse, workspace=ws)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.decode(q, k, v, win, plan=plan, out=o, lse=lse, workspace=ws)
    for r in range(4):
        q.copy_(inputs.attention_inputs(B, 1, Lk, Hq, Hkv, D, seed=90 + r, device=DEV)[0])
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = o.clone(), lse.clone()
        want_o, want_l = api.decode(q, k, v, win, plan=plan)
        torch.cuda.synchronize()
        assert torch.equal(got_o, want_o) and torch.equal(got_l, want_l), f"replay {r}"


def test_training_step_in_a_graph():
    B, L, Hq, Hkv, D = 1, 1500, 40, 8, 128
    _case(f"forward + backward L={L} captured in a graph, 3 replays")
    win = api.make_window(L, Hkv, 16, 128)
    prob = api.problem(B, L, L, Hq, Hkv, D, torch.bfloat16, D ** -0.5, win)
    fplan = api.build_plan("fwd", prob, DEV)
    bplan = api.build_plan("bwd", prob, DEV)
    q, k, v, do = (torch.empty_like(t) for t in inputs.attention_inputs(B, L, L, Hq, Hkv, D, seed=82,
                                                                         device=DEV, with_dout=True))
    o, o_lo = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = torch.empty(api.workspace_size("bwd", prob), dtype=torch.uint8, device=DEV)

    def step():
        api.fwd(q, k, v, win, plan=fplan, out=o, lse=lse, o_lo=o_lo)
        api.bwd(q, k, v, o, lse, do, win, plan=bplan, grads=grads, workspace=ws, o_lo=o_lo)

    def load(seed):
        for dst, src in zip((q, k, v, do), inputs.attention_inputs(B, L, L, Hq, Hkv, D, seed=seed,
                                                                    device=DEV, with_dout=True)):
            dst.copy_(src)

    load(83)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        load(100 + r)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, *grads)]
        step()
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), got, (o, lse, *grads)):
            assert torch.equal(a, b), f"replay {r}: {name}"
