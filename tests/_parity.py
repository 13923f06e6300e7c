"""Shared helpers of the GPU parity tests: tolerances and element-wise comparison.

Tolerances (fixed for this path): fp32 forward max-abs <= 1e-5; bf16 outputs and gradients
max-abs <= 2e-2 and mean-abs <= 2e-3; LSE max-abs <= 1e-3.  The reference is always the fp64
oracle on the very same (bf16- or fp32-rounded) inputs.
"""
import numpy as np

TOL_F32 = 1e-5
TOL_BF16_MAX = 2e-2
TOL_BF16_MEAN = 2e-3
TOL_LSE = 1e-3


def np64(t):
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def check_close(name, got, ref, max_tol, mean_tol=None, mask=None):
    """Element-wise |got - ref|: max <= max_tol (and mean <= mean_tol).  -inf must match -inf."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), f"{name}: -inf pattern differs"
    got, ref = got[~inf_ref], ref[~inf_ref]
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if got.size == 0:
        return 0.0, 0.0
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= max_tol, f"{name}: max-abs {mx:.3g} > {max_tol}"
    if mean_tol is not None:
        assert mean <= mean_tol, f"{name}: mean-abs {mean:.3g} > {mean_tol}"
    return mx, mean
