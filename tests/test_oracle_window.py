"""Pins of the oracle's local-window mask and windowed forward (tutorial page, "Other Efficient
Attention Variants", worked example "Local Attention Window").

Each pin ties the windowed path to something other than itself: the mask the page prints for
N = 6, w = 3; torch float64 scaled_dot_product_attention with that boolean mask; the closed form
of a zero-width window; and the unwindowed and causal forwards the window contains as cases.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import attn_fwd, visible_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "local_window_n6_w3.json")


def test_printed_mask_n6_w3():
    g = json.load(open(GOLDEN))
    half = (g["w"] - 1) // 2
    vis = visible_mask(np.arange(g["N"]), g["N"], False, (half, half))
    np.testing.assert_array_equal(vis.astype(int), np.array(g["mask"]))


def _sdpa_masked(q, k, v, scale, vis):
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(
        *t, attn_mask=torch.from_numpy(vis), scale=scale).numpy()


@pytest.mark.parametrize("window,causal,L", [((1, 1), False, 40), ((5, 2), False, 33),
                                              ((7, -1), False, 40), ((-1, 3), False, 29),
                                              ((6, 0), True, 40), ((4, 9), True, 35)])
def test_matches_torch_sdpa_with_the_mask(window, causal, L):
    r = np.random.default_rng(sum(window) + L)
    N, d = 40, 8
    q, k, v = r.normal(size=(1, 1, N, d)), r.normal(size=(1, 1, N, d)), r.normal(size=(1, 1, N, d))
    O, _ = attn_fwd(q, k, v, 0.3, causal, [L], window=window, chunk=11)
    # explicit boolean mask, written out from the definition i - left <= j <= i + right
    i, j = np.arange(N)[:, None], np.arange(N)[None, :]
    vis = (j < L) & ((j >= i - window[0]) if window[0] >= 0 else True) & \
        ((j <= i + window[1]) if window[1] >= 0 else True) & ((j <= i) if causal else True)
    ref = _sdpa_masked(q, k, v, 0.3, vis[None, None])
    rows = vis.any(axis=1)
    np.testing.assert_allclose(O[0, 0, rows], ref[0, 0, rows], rtol=0, atol=1e-13)
    assert np.all(O[0, 0, ~rows] == 0)


def test_zero_width_window_returns_own_value():
    r = np.random.default_rng(1)
    q, k, v = r.normal(size=(2, 2, 9, 4)), r.normal(size=(2, 1, 9, 4)), r.normal(size=(2, 1, 9, 4))
    O, LSE = attn_fwd(q, k, v, 0.5, False, window=(0, 0))
    np.testing.assert_allclose(O, np.repeat(v, 2, axis=1), atol=1e-14)
    np.testing.assert_allclose(LSE, 0.5 * np.einsum("bhid,bhid->bhi", q, np.repeat(k, 2, axis=1)),
                               atol=1e-13)


def test_wide_windows_are_the_plain_and_causal_forwards():
    r = np.random.default_rng(2)
    q, k, v = r.normal(size=(1, 2, 17, 4)), r.normal(size=(1, 2, 17, 4)), r.normal(size=(1, 2, 17, 4))
    full = attn_fwd(q, k, v, 0.4, False)
    causal = attn_fwd(q, k, v, 0.4, True)
    for a, b in zip(attn_fwd(q, k, v, 0.4, False, window=(16, 16)), full):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(attn_fwd(q, k, v, 0.4, False, window=(-1, 0)), causal):
        np.testing.assert_array_equal(a, b)


def test_rows_past_the_key_length_can_see_nothing():
    r = np.random.default_rng(3)
    q, k, v = r.normal(size=(1, 1, 12, 4)), r.normal(size=(1, 1, 12, 4)), r.normal(size=(1, 1, 12, 4))
    O, LSE = attn_fwd(q, k, v, 1.0, False, [5], window=(1, 1))
    assert np.all(O[0, 0, 7:] == 0) and np.all(np.isneginf(LSE[0, 0, 7:]))
    assert np.all(np.isfinite(LSE[0, 0, :6]))
