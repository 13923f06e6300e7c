"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Each mutant replaces one helper of ``oracle.naive`` with a plausible bug (a dropped term, a wrong
index, a wrong base, a missing shift, a wrong head map); the pins are then run as plain
functions and at least one must raise.  This shows the pins can tell the oracle apart from its
near misses; nothing is ever planted in the HIP path.
"""
import contextlib

import numpy as np
import pytest

import oracle.naive as nv
from tests import test_oracle_grad as G
from tests import test_oracle_pins as P

PINS = [
    P.test_worked_example_row0_closed_form,
    P.test_worked_example_all_rows_closed_form,
    P.test_worked_example_causal,
    lambda: P.test_identity_values_expose_P(True),
    P.test_zero_queries_average_values.__wrapped__ if hasattr(
        P.test_zero_queries_average_values, "__wrapped__") else
    (lambda: P.test_zero_queries_average_values(True)),
    P.test_single_token,
    P.test_extreme_scores_stay_finite,
    lambda: P.test_matches_torch_sdpa_float64(True, [31, 20], 4, 1),
    lambda: P.test_matches_torch_sdpa_float64(False, [31, 16], 4, 2),
    lambda: G.test_grads_match_finite_differences(True, [6, 2], 4, 2),
]

_orig_softmax = nv._softmax_rows


def _no_shift(s, vis):
    e = np.where(vis, np.exp(np.where(vis, s, 0.0)), 0.0)
    l = e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        P = e / l[:, None]
    m = np.where(vis, s, -np.inf).max(axis=1)
    return np.nan_to_num(P), np.zeros_like(m), l


def _sum_over_hidden(s, vis):
    P, m, l = _orig_softmax(s, vis)
    e = np.exp(s - np.where(np.isfinite(m), m, 0)[:, None])
    l2 = e.sum(axis=1)
    return P * (l / l2)[:, None], m, l2


MUTANTS = {
    "scale dropped": ("score_rows", lambda q, K, scale: q @ K.T),
    "scale squared": ("score_rows", lambda q, K, scale: scale * scale * (q @ K.T)),
    "causal off by one": ("visible_mask", lambda rows, L, causal: (
        np.arange(L)[None, :] < np.asarray(rows)[:, None]) | (not causal)),
    "causal bottom-right": ("visible_mask", lambda rows, L, causal: (
        np.arange(L)[None, :] <= np.asarray(rows)[:, None] + 1) | (not causal)),
    "gqa strided map": ("kv_head_of", lambda h, Hq, Hkv: h % Hkv),
    "no max shift": ("_softmax_rows", _no_shift),
    "denominator over hidden keys": ("_softmax_rows", _sum_over_hidden),
}


@contextlib.contextmanager
def planted(attr, fn):
    keep = getattr(nv, attr)
    setattr(nv, attr, fn)
    try:
        yield
    finally:
        setattr(nv, attr, keep)


def test_pins_pass_unmutated():
    for pin in PINS:
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_each_mutant_fails_a_pin(name):
    attr, fn = MUTANTS[name]
    caught = []
    with planted(attr, fn), np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except Exception as e:          # AssertionError, or a crash the bug causes
                caught.append((getattr(pin, "__name__", "pin"), type(e).__name__))
    assert caught, f"mutant '{name}' passed every pin"
