"""Pins of the oracle's decode-shaped forward (Nq query rows against Nk keys, no causal mask).

Each pin ties ``attn_decode`` to something other than itself: torch's float64
scaled_dot_product_attention and logsumexp with Nq != Nk, closed forms (zero queries, one key,
no key), and agreement with the pinned square forward when Nq = Nk.
"""
import numpy as np
import pytest
import torch

from oracle import attn_decode, attn_fwd


def _ref(q, k, v, scale, lens, Hq, Hkv):
    """torch float64 SDPA with kv heads repeated per group, a boolean key mask, and the natural-log
    logsumexp of the masked scaled scores."""
    G = Hq // Hkv
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    k, v = k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1)
    B, _, Nq, _ = q.shape
    Nk = k.shape[2]
    L = torch.tensor(lens if lens is not None else [Nk] * B)
    mask = (torch.arange(Nk)[None, :] < L[:, None])[:, None, None, :].expand(B, 1, Nq, Nk)
    O = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    s = torch.where(mask, scale * q @ k.transpose(-1, -2), torch.tensor(-torch.inf, dtype=q.dtype))
    return O.numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("Nq,Nk,Hq,Hkv,lens", [
    (1, 37, 4, 1, None), (1, 64, 8, 2, [64, 9]), (3, 50, 4, 4, [50, 1]), (5, 33, 6, 2, [17, 33])])
def test_matches_torch_float64(Nq, Nk, Hq, Hkv, lens):
    r = np.random.default_rng(Nq * 100 + Nk)
    d = 8
    q = r.normal(size=(2, Hq, Nq, d))
    k, v = r.normal(size=(2, Hkv, Nk, d)), r.normal(size=(2, Hkv, Nk, d))
    O, LSE = attn_decode(q, k, v, 0.4, lens)
    Or, Lr = _ref(q, k, v, 0.4, lens, Hq, Hkv)
    np.testing.assert_allclose(O, Or, rtol=0, atol=1e-13)
    np.testing.assert_allclose(LSE, Lr, rtol=0, atol=1e-12)


def test_zero_queries_average_the_visible_values():
    r = np.random.default_rng(3)
    k, v = r.normal(size=(2, 2, 40, 4)), r.normal(size=(2, 2, 40, 4))
    q = np.zeros((2, 4, 3, 4))
    O, LSE = attn_decode(q, k, v, 1.0, [40, 7])
    for b, L in enumerate([40, 7]):
        for h in range(4):
            np.testing.assert_allclose(O[b, h], np.broadcast_to(v[b, h // 2, :L].mean(0), (3, 4)),
                                       atol=1e-14)
            np.testing.assert_allclose(LSE[b, h], np.log(L), atol=1e-14)


def test_one_key_and_no_key():
    r = np.random.default_rng(4)
    q = r.normal(size=(2, 2, 2, 4))
    k, v = r.normal(size=(2, 1, 5, 4)), r.normal(size=(2, 1, 5, 4))
    O, LSE = attn_decode(q, k, v, 0.5, [1, 0])
    np.testing.assert_allclose(O[0], np.broadcast_to(v[0, 0, 0], (2, 2, 4)), atol=1e-15)
    np.testing.assert_allclose(LSE[0], 0.5 * q[0] @ k[0, 0, 0], atol=1e-14)
    assert np.all(O[1] == 0) and np.all(np.isneginf(LSE[1]))


def test_square_case_is_the_noncausal_forward():
    r = np.random.default_rng(5)
    q, k, v = r.normal(size=(1, 4, 19, 8)), r.normal(size=(1, 2, 19, 8)), r.normal(size=(1, 2, 19, 8))
    O, LSE = attn_decode(q, k, v, 0.3, [11])
    O2, LSE2 = attn_fwd(q, k, v, 0.3, False, [11])
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(LSE, LSE2)


def test_padding_keys_never_reach_outputs():
    r = np.random.default_rng(6)
    q, k, v = r.normal(size=(1, 2, 2, 4)), r.normal(size=(1, 2, 30, 4)), r.normal(size=(1, 2, 30, 4))
    O, LSE = attn_decode(q, k, v, 0.7, [12])
    k[:, :, 12:] = np.nan
    v[:, :, 12:] = np.nan
    O2, LSE2 = attn_decode(q, k, v, 0.7, [12])
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(LSE, LSE2)
