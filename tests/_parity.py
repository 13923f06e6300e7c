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


class Agg:
    """|got - ref| element by element over several pieces of one tensor (e.g. its heads, checked
    one at a time): the maximum and the mean over every checked element, and the -inf pattern."""

    def __init__(self, name, max_tol, mean_tol=None):
        self.name, self.max_tol, self.mean_tol = name, max_tol, mean_tol
        self.max, self.sum, self.n = 0.0, 0.0, 0

    def add(self, got, ref):
        got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        assert got.shape == ref.shape, (self.name, got.shape, ref.shape)
        inf_ref = np.isneginf(ref)
        assert np.array_equal(np.isneginf(got), inf_ref), f"{self.name}: -inf pattern differs"
        got, ref = got[~inf_ref], ref[~inf_ref]
        assert np.all(np.isfinite(got)), f"{self.name}: non-finite values"
        if got.size:
            err = np.abs(got - ref)
            self.max = max(self.max, float(err.max()))
            self.sum += float(err.sum())
            self.n += err.size

    def check(self):
        mean = self.sum / max(self.n, 1)
        assert self.max <= self.max_tol, f"{self.name}: max-abs {self.max:.3g} > {self.max_tol}"
        if self.mean_tol is not None:
            assert mean <= self.mean_tol, f"{self.name}: mean-abs {mean:.3g} > {self.mean_tol}"
        return self.max, mean


def oracle_map(fn, jobs):
    """fn(job) for every job on a pool of threads, results in job order.  numpy releases the
    interpreter lock inside its array kernels and BLAS, so whole heads of the fp64 oracle run in
    parallel on the host's cores."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(jobs)))
    with ThreadPoolExecutor(workers) as ex:
        yield from ex.map(fn, jobs)
