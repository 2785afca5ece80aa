"""Helpers for the GPU parity tests: error metrics and stratified row samples."""

import numpy as np
import torch

BF16_MAX_ABS = 2e-2   # bf16 outputs and gradients: max-abs and relative-L2 bars
BF16_REL_L2 = 1e-2
F32_MAX_ABS = 1e-4    # fp32 forward


def errors(got, want):
    g = got.detach().to("cpu", torch.float64).numpy() if hasattr(got, "detach") else np.asarray(got, np.float64)
    w = np.asarray(want, dtype=np.float64)
    assert g.shape == w.shape, (g.shape, w.shape)
    fin = np.isfinite(w)
    assert np.array_equal(fin, np.isfinite(g)), "non-finite pattern differs"
    d = np.abs(g[fin] - w[fin])
    max_abs = float(d.max()) if d.size else 0.0
    nrm = float(np.linalg.norm(w[fin]))
    rel = float(np.linalg.norm(g[fin] - w[fin]) / nrm) if nrm > 0 else 0.0
    return max_abs, rel


def assert_bf16_close(name, got, want, value_scaled=False):
    """max-abs <= 2e-2 and relative-L2 <= 1e-2 against the float64 oracle.

    value_scaled=True applies the max-abs bar per element as max(2e-2, 2^-7 |want|):
    bf16 spaces values in [4, 8) 2^-5 apart, so rounding the output alone can cost 2^-6,
    and the bf16 rounding of P / dS before the products adds about as much again; the
    bar then allows two bf16 half-ulps at the value.  Only gradients of small test
    shapes (few visible keys, so entries of magnitude 2-8) reach that range."""
    max_abs, rel = errors(got, want)
    g = got.detach().to("cpu", torch.float64).numpy() if hasattr(got, "detach") else np.asarray(got)
    w = np.asarray(want, dtype=np.float64)
    fin = np.isfinite(w)
    excess = np.abs(g[fin] - w[fin]) - np.maximum(BF16_MAX_ABS, np.abs(w[fin]) * 2.0 ** -7)
    n_over_abs = int((np.abs(g[fin] - w[fin]) > BF16_MAX_ABS).sum())
    print(f"  {name}: max_abs={max_abs:.3e} rel_l2={rel:.3e} max|want|={np.abs(w[fin]).max():.3e} "
          f"n(|err|>2e-2)={n_over_abs}", flush=True)
    if value_scaled:
        assert excess.max(initial=-1.0) <= 0, f"{name}: value-scaled max-abs exceeded by {excess.max()}"
    else:
        assert max_abs <= BF16_MAX_ABS, f"{name}: max_abs {max_abs}"
    assert rel <= BF16_REL_L2, f"{name}: rel_l2 {rel}"


def sample_rows(L, sink, near, lr, Hkv, Bq, n, seed):
    """Mandatory boundary rows (tile, sink, near and band edges, first/last) plus seeded
    random rows, sorted and unique."""
    must = {0, 1, Bq - 1, Bq, sink - 1, sink, near - 1, near, L - 1}
    for h in range(1, Hkv):
        must |= {near + h * lr - 1, near + h * lr}
    must = {r for r in must if 0 <= r < L}
    rng = np.random.default_rng(seed)
    extra = rng.choice(L, size=max(0, n - len(must)), replace=False)
    return np.array(sorted(must | set(int(x) for x in extra)), dtype=np.int64)
