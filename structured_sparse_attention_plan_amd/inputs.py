"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it only draws standard-normal tensors.
Recipe: ``torch.Generator(device).manual_seed(seed)``, ``randn`` in float32, then a
round-to-nearest-even cast to the storage dtype (bf16 for the bf16 paths).  Per-tensor
seeds are base + {0: Q, 1: K, 2: V, 3: dO}.  The CPU generator is used for every size
the oracle checks in full; the 128K-token workloads may be drawn on the device (same
recipe, the device's Philox stream) and copied to the host for the sampled oracle
checks, because drawing 1.6e9 normals on one host core takes minutes.
"""

import torch

SEED_Q, SEED_K, SEED_V, SEED_DO = 0, 1, 2, 3


def randn(shape, seed, dtype=torch.bfloat16, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    return x.to(dtype)


def attention_inputs(B, Lq, Lk, Hq, Hkv, D, dtype=torch.bfloat16, seed=0, device="cpu",
                     with_dout=False):
    """Q [B, Lq, Hq, D], K/V [B, Lk, Hkv, D] (and dO like Q), contiguous BSHD."""
    q = randn((B, Lq, Hq, D), seed + SEED_Q, dtype, device)
    k = randn((B, Lk, Hkv, D), seed + SEED_K, dtype, device)
    v = randn((B, Lk, Hkv, D), seed + SEED_V, dtype, device)
    if not with_dout:
        return q, k, v
    do = randn((B, Lq, Hq, D), seed + SEED_DO, dtype, device)
    return q, k, v, do
