"""Pins of the oracle backward (CPU only): brute-force central differences, torch float64
autograd through its SDPA math path, and algebraic invariants of the softmax VJP."""
import numpy as np
import pytest
import torch

from oracle import attn_bwd, attn_bwd_heads, attn_dq_rows, attn_fwd
from oracle.fd import numeric_grads


def _rand(seed, B, Hq, Hkv, N, d):
    r = np.random.default_rng(seed)
    return (r.normal(size=(B, Hq, N, d)), r.normal(size=(B, Hkv, N, d)),
            r.normal(size=(B, Hkv, N, d)), r.normal(size=(B, Hq, N, d)))


@pytest.mark.parametrize("causal,lens,Hq,Hkv", [
    (False, None, 1, 1), (True, None, 1, 1), (True, [5, 3], 2, 2),
    (False, [6, 4], 4, 2), (True, [6, 2], 4, 2)])
def test_grads_match_finite_differences(causal, lens, Hq, Hkv):
    q, k, v, do = _rand(11, 2, Hq, Hkv, 6, 3)
    dQ, dK, dV = attn_bwd(q, k, v, do, 0.8, causal, lens)
    nQ, nK, nV = numeric_grads(q, k, v, do, 0.8, causal, lens)
    for a, n in ((dQ, nQ), (dK, nK), (dV, nV)):
        np.testing.assert_allclose(a, n, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal,lens,Hq,Hkv", [
    (False, None, 2, 2), (True, None, 4, 2), (True, [19, 40], 4, 1)])
def test_grads_match_torch_autograd_float64(causal, lens, Hq, Hkv):
    q, k, v, do = _rand(12, 2, Hq, Hkv, 40, 16)
    dQ, dK, dV = attn_bwd(q, k, v, do, 0.25, causal, lens, chunk=13)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    G = Hq // Hkv
    mask = torch.ones(2, 1, 40, 40, dtype=torch.bool)
    if causal:
        mask &= torch.ones(40, 40, dtype=torch.bool).tril()
    if lens is not None:
        mask &= (torch.arange(40)[None, :] < torch.tensor(lens)[:, None])[:, None, None, :]
    O = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1), attn_mask=mask, scale=0.25)
    O.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dQ, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), atol=1e-12)


def test_grad_invariants():
    """Rows of dS sum to 0 -> sum_j dK_j = 0; rows of P sum to 1 -> sum_j dV_j = sum_i dO_i over
    rows with a visible key; padded keys get zero gradient."""
    q, k, v, do = _rand(13, 2, 4, 2, 30, 8)
    lens = [30, 11]
    dQ, dK, dV = attn_bwd(q, k, v, do, 0.5, True, lens)
    for b in range(2):
        for g in range(2):
            np.testing.assert_allclose(dK[b, g].sum(0), 0, atol=1e-12)
            np.testing.assert_allclose(dV[b, g].sum(0), do[b, 2 * g:2 * g + 2].sum((0, 1)),
                                       atol=1e-12)
    assert np.all(dK[1, :, 11:] == 0) and np.all(dV[1, :, 11:] == 0)


def test_equal_value_rows_give_zero_qk_grads():
    """All V rows equal -> O does not depend on Q or K -> dQ = dK = 0."""
    q, k, v, do = _rand(14, 1, 2, 2, 20, 5)
    v[:] = v[:, :, :1]
    dQ, dK, _ = attn_bwd(q, k, v, do, 0.7, True)
    np.testing.assert_allclose(dQ, 0, atol=1e-13)
    np.testing.assert_allclose(dK, 0, atol=1e-13)


def test_empty_rows_have_zero_grads():
    q, k, v, do = _rand(15, 2, 2, 1, 8, 4)
    dQ, dK, dV = attn_bwd(q, k, v, do, 1.0, False, [0, 8])
    assert np.all(dQ[0] == 0) and np.all(dK[0] == 0) and np.all(dV[0] == 0)
    O, LSE = attn_fwd(q, k, v, 1.0, False, [0, 8])
    assert np.all(O[0] == 0) and np.all(np.isneginf(LSE[0]))


def test_heads_api_matches_full():
    q, k, v, do = _rand(16, 2, 4, 2, 24, 4)
    lens = [24, 13]
    dQ, dK, dV = attn_bwd(q, k, v, do, 0.6, True, lens)
    got = attn_bwd_heads(q, k, v, do, 0.6, True, lens, [(1, 1), (0, 0)])
    for (b, g), (gq, gk, gv) in got.items():
        np.testing.assert_allclose(gq, dQ[b, 2 * g:2 * g + 2], atol=1e-15)
        np.testing.assert_allclose(gk, dK[b, g], atol=1e-15)
        np.testing.assert_allclose(gv, dV[b, g], atol=1e-15)


@pytest.mark.parametrize("causal,lens,Hq,Hkv", [
    (False, None, 2, 2), (True, None, 4, 2), (True, [19, 33], 4, 1)])
def test_dq_rows_match_torch_autograd_float64(causal, lens, Hq, Hkv):
    """The per-row dQ against torch float64 autograd through its SDPA math path."""
    q, k, v, do = _rand(13, 2, Hq, Hkv, 40, 16)
    tq = torch.from_numpy(q).requires_grad_()
    G = Hq // Hkv
    mask = torch.ones(2, 1, 40, 40, dtype=torch.bool)
    if causal:
        mask &= torch.ones(40, 40, dtype=torch.bool).tril()
    if lens is not None:
        mask &= (torch.arange(40)[None, :] < torch.tensor(lens)[:, None])[:, None, None, :]
    O = torch.nn.functional.scaled_dot_product_attention(
        tq, torch.from_numpy(k).repeat_interleave(G, 1), torch.from_numpy(v).repeat_interleave(G, 1),
        attn_mask=mask, scale=0.25)
    O.backward(torch.from_numpy(do))
    picks = [(b, h, i) for b in range(2) for h in range(Hq) for i in (0, 1, 18, 19, 32, 39)]
    got = attn_dq_rows(q, k, v, do, 0.25, causal, lens, picks)
    ref = np.stack([tq.grad.numpy()[b, h, i] for b, h, i in picks])
    np.testing.assert_allclose(got, ref, atol=1e-12)


@pytest.mark.parametrize("causal,lens", [(False, None), (True, [5, 3])])
def test_dq_rows_match_finite_differences(causal, lens):
    q, k, v, do = _rand(14, 2, 4, 2, 6, 3)
    nQ, _, _ = numeric_grads(q, k, v, do, 0.8, causal, lens)
    picks = [(b, h, i) for b in range(2) for h in range(4) for i in range(6)]
    got = attn_dq_rows(q, k, v, do, 0.8, causal, lens, picks)
    np.testing.assert_allclose(got, np.stack([nQ[b, h, i] for b, h, i in picks]),
                               rtol=1e-6, atol=1e-8)


def test_dq_rows_of_a_batch_with_no_keys_are_zero():
    q, k, v, do = _rand(15, 2, 2, 2, 8, 4)
    got = attn_dq_rows(q, k, v, do, 0.5, True, [0, 8], [(0, 1, 3), (1, 0, 5)])
    assert np.all(got[0] == 0) and np.any(got[1] != 0)
