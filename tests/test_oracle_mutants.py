"""Planted mistakes in the oracle must each fail a pin of every path they touch (CPU only).

Each mutant replaces one function of ``oracle.naive`` with a plausible bug (a dropped or doubled
factor, an off-by-one edge, a wrong index, a missing term or sum) that keeps the original's
signature.  It is planted in every loaded module that holds the original under that name, so
tests that imported the function directly see it too.  The pins (the ``-m "not gpu"`` tests of
``tests/test_oracle_*.py``, with all their parameters) of each path the mutant touches are then
run as plain functions; only an ``AssertionError`` raised by a pin counts as catching it, never a
crash the bug happens to cause.  Nothing is ever planted in the HIP path.

Paths: ``fwd`` (the plain forward), ``window``, ``sparse`` (block bitmap), ``decode``, ``bwd``
(the full backward) and ``dq_rows`` (per-row dQ).
"""
import contextlib
import itertools
import sys

import numpy as np
import pytest

import oracle.naive as nv
from tests import test_oracle_blocksparse as TS
from tests import test_oracle_decode as TD
from tests import test_oracle_grad as TG
from tests import test_oracle_pins as TP
from tests import test_oracle_window as TW


def _calls(fn):
    """Every parameter combination of a pytest test function, as zero-argument calls."""
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    if not marks:
        return [((), fn)]
    axes = []
    for m in marks:
        names, values = m.args[0], m.args[1]
        names = [n.strip() for n in names.split(",")] if isinstance(names, str) else list(names)
        axes.append([dict(zip(names, v if len(names) > 1 else (v,))) for v in values])
    out = []
    for combo in itertools.product(*axes):
        kw = {k: v for part in combo for k, v in part.items()}
        out.append((tuple(sorted(kw.items(), key=lambda kv: kv[0])),
                    (lambda f=fn, kw=kw: f(**kw))))
    return out


def _pins(module, path_of):
    pins = []
    for name in sorted(dir(module)):
        fn = getattr(module, name)
        if name.startswith("test_") and callable(fn):
            for params, call in _calls(fn):
                pins.append((path_of(name), f"{name}{list(params) if params else ''}", call))
    return pins


PINS = (_pins(TP, lambda n: "fwd") + _pins(TW, lambda n: "window")
        + _pins(TS, lambda n: "sparse") + _pins(TD, lambda n: "decode")
        + _pins(TG, lambda n: "dq_rows" if n.startswith("test_dq_rows") else "bwd"))

_orig = {name: getattr(nv, name) for name in
         ("score_rows", "visible_mask", "kv_head_of", "_softmax_rows", "_lens", "_softmax_vjp",
          "attn_decode", "attn_bwd", "attn_dq_rows")}


# ------------------------------------------------------------------ the mutants

def _no_shift(s, vis):
    """Softmax without subtracting the row max (overflows for large scores)."""
    e = np.where(vis, np.exp(np.where(vis, s, 0.0)), 0.0)
    l = e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        P = e / l[:, None]
    m = np.where(vis, s, -np.inf).max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    return np.nan_to_num(P), np.zeros_like(m), l


def _sum_over_hidden(s, vis):
    """Denominator summed over every key, hidden ones included."""
    P, m, l = _orig["_softmax_rows"](s, vis)
    e = np.exp(s - np.where(np.isfinite(m), m, 0)[:, None])
    l2 = e.sum(axis=1)
    return P * (l / l2)[:, None], m, l2


def _mask(rows, L, causal, window=None, block_mask=None, *, causal_rel=None, win=None, blk=None):
    """visible_mask with one rule replaced: causal_rel(i, j), win(i, j, left, right) or
    blk(bm, i, j, bq, bk) stand in for the causal, window or block rule."""
    j = np.arange(L)[None, :]
    i = np.asarray(rows)[:, None]
    vis = np.ones((len(rows), L), dtype=bool)
    if causal:
        vis &= (j <= i) if causal_rel is None else causal_rel(i, j)
    if window is not None:
        left, right = window
        if win is not None:
            vis &= win(i, j, left, right)
        else:
            if left >= 0:
                vis &= j >= i - left
            if right >= 0:
                vis &= j <= i + right
    if block_mask is not None:
        bm, bq, bk = block_mask
        bm = np.asarray(bm) != 0
        vis &= bm[i // bq, j // bk] if blk is None else blk(bm, i, j, bq, bk)
    return vis


def _win_left_exclusive(i, j, left, right):
    ok = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if left >= 0:
        ok &= j > i - left
    if right >= 0:
        ok &= j <= i + right
    return ok


def _win_swapped(i, j, left, right):
    ok = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if right >= 0:
        ok &= j >= i - right
    if left >= 0:
        ok &= j <= i + left
    return ok


def _bwd_no_group_sum(orig):
    """dK and dV of a kv-head taken from one q-head of its group instead of the group's sum."""
    def f(q, k, v, do, scale, causal=False, key_lens=None, kv_heads=None, chunk=1024):
        dQ, dK, dV = orig(q, k, v, do, scale, causal, key_lens, kv_heads, chunk)
        G = np.shape(q)[1] // np.shape(k)[1]
        _, dK1, dV1 = orig(nv.to64(q)[:, ::G], k, v, nv.to64(do)[:, ::G], scale, causal,
                           key_lens, kv_heads, chunk)
        return dQ, dK1, dV1
    return f


def _bwd_dk_unscaled(orig):
    def f(q, k, v, do, scale, causal=False, key_lens=None, kv_heads=None, chunk=1024):
        dQ, dK, dV = orig(q, k, v, do, scale, causal, key_lens, kv_heads, chunk)
        return dQ, dK / scale, dV
    return f


def _dq_rows_unscaled(orig):
    def f(q, k, v, do, scale, causal, key_lens, picks):
        return orig(q, k, v, do, scale, causal, key_lens, picks) / scale
    return f


def _decode_no_lens(orig):
    def f(q, k, v, scale, key_lens=None):
        return orig(q, k, v, scale, None)
    return f


def _lens_one_more(orig):
    def f(key_lens, B, N):
        return [min(l + 1, N) for l in orig(key_lens, B, N)]
    return f


ALL = ("fwd", "window", "sparse", "decode", "bwd", "dq_rows")

# name -> (function replaced, factory(original) -> mutant, paths whose pins must catch it)
MUTANTS = {
    "scale dropped": ("score_rows", lambda o: (lambda q, K, scale: q @ K.T), ALL),
    "scale squared": ("score_rows", lambda o: (lambda q, K, scale: scale * scale * (q @ K.T)),
                      ALL),
    "causal off by one": ("visible_mask", lambda o: (
        lambda *a, **k: _mask(*a, **k, causal_rel=lambda i, j: j < i)),
        ("fwd", "window", "sparse", "bwd", "dq_rows")),
    "causal bottom-right": ("visible_mask", lambda o: (
        lambda *a, **k: _mask(*a, **k, causal_rel=lambda i, j: j <= i + 1)),
        ("fwd", "window", "sparse", "bwd", "dq_rows")),
    "window left edge exclusive": ("visible_mask", lambda o: (
        lambda *a, **k: _mask(*a, **k, win=_win_left_exclusive)), ("window",)),
    "window sides swapped": ("visible_mask", lambda o: (
        lambda *a, **k: _mask(*a, **k, win=_win_swapped)), ("window",)),
    "block index of keys by the query block size": ("visible_mask", lambda o: (
        lambda *a, **k: _mask(*a, **k, blk=lambda bm, i, j, bq, bk: bm[i // bq, j // bq])),
        ("sparse",)),
    "gqa strided head map": ("kv_head_of", lambda o: (lambda h, Hq, Hkv: h % Hkv),
                             ("fwd", "decode", "bwd", "dq_rows")),
    "no max shift": ("_softmax_rows", lambda o: _no_shift, ("fwd",)),
    # (decode slices the keys to the key length and has no other mask: nothing is hidden there)
    "denominator over hidden keys": ("_softmax_rows", lambda o: _sum_over_hidden,
                                     ("fwd", "window", "sparse", "bwd", "dq_rows")),
    "key length one too long": ("_lens", _lens_one_more,
                                ("fwd", "window", "decode", "bwd", "dq_rows")),
    "decode ignores key lengths": ("attn_decode", _decode_no_lens, ("decode",)),
    "dS without the D term": ("_softmax_vjp", lambda o: (lambda P, dP: P * dP),
                              ("bwd", "dq_rows")),
    "dS with D over the wrong sign": ("_softmax_vjp", lambda o: (
        lambda P, dP: P * (dP + (P * dP).sum(axis=1)[:, None])), ("bwd", "dq_rows")),
    "backward misses the grouped-head sum": ("attn_bwd", _bwd_no_group_sum, ("bwd",)),
    "dK without the scale": ("attn_bwd", _bwd_dk_unscaled, ("bwd",)),
    "per-row dQ without the scale": ("attn_dq_rows", _dq_rows_unscaled, ("dq_rows",)),
}


@contextlib.contextmanager
def planted(attr, fn):
    """Replace oracle.naive.<attr> by fn in every loaded module that holds the original."""
    orig = _orig[attr]
    holders = [m for m in list(sys.modules.values())
               if m is not None and getattr(m, "__dict__", {}).get(attr) is orig]
    assert nv in holders
    for m in holders:
        setattr(m, attr, fn)
    try:
        yield
    finally:
        for m in holders:
            setattr(m, attr, orig)


def run_pins(paths):
    """Run the pins of the given paths; returns {path: [(pin, exception type name)]}."""
    out = {p: [] for p in paths}
    with np.errstate(all="ignore"):
        for path, name, call in PINS:
            if path not in out:
                continue
            try:
                call()
            except Exception as e:      # recorded by type; only AssertionError counts as a catch
                out[path].append((name, type(e).__name__))
    return out


def test_every_path_has_pins():
    assert {p for p, _, _ in PINS} == set(ALL)
    assert len(PINS) >= 70


def test_pins_pass_unmutated():
    failed = run_pins(ALL)
    assert all(not v for v in failed.values()), failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_each_mutant_fails_a_pin_of_every_path_it_touches(name):
    attr, factory, paths = MUTANTS[name]
    with planted(attr, factory(_orig[attr])):
        failed = run_pins(paths)
    for path in paths:
        caught = [pin for pin, kind in failed[path] if kind == "AssertionError"]
        assert caught, (f"mutant '{name}' passed every pin of path '{path}' "
                        f"(other failures: {failed[path]})")
