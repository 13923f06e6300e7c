"""Pins of the oracle's block-sparse mask (a tile-level bitmap over (query block, key block)
pairs; the study-note page names block-sparse attention as an extension without defining it).

Each pin ties the block-sparse path to something other than itself: torch float64
scaled_dot_product_attention with the element mask expanded by repetition (np.kron), an all-ones
bitmap equal to the plain forward, a block-lower-triangular bitmap combined with causal equal to
causal, and the closed form of zero queries over one active block.
"""
import numpy as np
import pytest
import torch

from oracle import attn_fwd, visible_mask


def _expand(bm, bq, bk, N):
    """Element mask from the bitmap by Kronecker product with all-ones blocks (a different route
    from the oracle's index arithmetic), cut to N x N."""
    return np.kron(np.asarray(bm) != 0, np.ones((bq, bk), dtype=bool))[:N, :N]


@pytest.mark.parametrize("N,bq,bk,density,causal", [(37, 8, 4, 0.4, False), (64, 16, 8, 0.3, True),
                                                     (50, 4, 8, 0.6, False)])
def test_matches_torch_sdpa_with_expanded_mask(N, bq, bk, density, causal):
    r = np.random.default_rng(N)
    bm = (r.random((-(-N // bq), -(-N // bk))) < density).astype(np.uint8)
    q, k, v = r.normal(size=(1, 1, N, 8)), r.normal(size=(1, 1, N, 8)), r.normal(size=(1, 1, N, 8))
    O, LSE = attn_fwd(q, k, v, 0.3, causal, block_mask=(bm, bq, bk), chunk=13)
    vis = _expand(bm, bq, bk, N)
    if causal:
        vis &= np.tri(N, dtype=bool)
    rows = vis.any(axis=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), attn_mask=torch.from_numpy(vis[None, None]),
        scale=0.3).numpy()
    np.testing.assert_allclose(O[0, 0, rows], ref[0, 0, rows], rtol=0, atol=1e-13)
    assert np.all(O[0, 0, ~rows] == 0) and np.all(np.isneginf(LSE[0, 0, ~rows]))


def test_all_ones_is_the_plain_forward():
    r = np.random.default_rng(1)
    q, k, v = r.normal(size=(2, 2, 30, 4)), r.normal(size=(2, 1, 30, 4)), r.normal(size=(2, 1, 30, 4))
    bm = np.ones((4, 8), dtype=np.uint8)
    for causal in (False, True):
        a = attn_fwd(q, k, v, 0.5, causal, [30, 17], block_mask=(bm, 8, 4))
        b = attn_fwd(q, k, v, 0.5, causal, [30, 17])
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


def test_block_lower_triangle_with_causal_is_causal():
    r = np.random.default_rng(2)
    q, k, v = r.normal(size=(1, 1, 40, 4)), r.normal(size=(1, 1, 40, 4)), r.normal(size=(1, 1, 40, 4))
    bm = np.tril(np.ones((5, 5), dtype=np.uint8))
    for x, y in zip(attn_fwd(q, k, v, 0.5, True, block_mask=(bm, 8, 8)), attn_fwd(q, k, v, 0.5, True)):
        np.testing.assert_array_equal(x, y)


def test_zero_queries_average_the_one_active_block():
    r = np.random.default_rng(3)
    k, v = r.normal(size=(1, 1, 24, 4)), r.normal(size=(1, 1, 24, 4))
    q = np.zeros((1, 1, 24, 4))
    bm = np.zeros((3, 6), dtype=np.uint8)
    bm[0, 2] = bm[1, 5] = 1          # rows 0..7 see keys 8..11; rows 8..15 keys 20..23; 16..23 none
    O, LSE = attn_fwd(q, k, v, 1.0, False, block_mask=(bm, 8, 4))
    np.testing.assert_allclose(O[0, 0, :8], np.broadcast_to(v[0, 0, 8:12].mean(0), (8, 4)), atol=1e-14)
    np.testing.assert_allclose(O[0, 0, 8:16], np.broadcast_to(v[0, 0, 20:24].mean(0), (8, 4)), atol=1e-14)
    np.testing.assert_allclose(LSE[0, 0, :16], np.log(4.0), atol=1e-14)
    assert np.all(O[0, 0, 16:] == 0) and np.all(np.isneginf(LSE[0, 0, 16:]))


def test_mask_is_constant_on_blocks():
    bm = np.array([[1, 0, 1], [0, 1, 0]], dtype=np.uint8)
    vis = visible_mask(np.arange(8), 12, False, block_mask=(bm, 4, 4))
    np.testing.assert_array_equal(vis, _expand(bm, 4, 4, 12)[:8])
