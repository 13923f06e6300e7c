"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a number the tutorial page prints in its worked
example (tests/golden/worked_example.json), a closed form derived from the definition, an
invariant of softmax attention, or an independent library routine (torch's float64
scaled_dot_product_attention math path, scipy's logsumexp).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attn_fwd, attn_fwd_rows, kv_head_of
from oracle.blocked import blocked_row, merge

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")
S2 = math.sqrt(0.5)                    # the page divides by sqrt(2): exact fp64 value here
A = math.exp(-S2)                      # e^{-1/sqrt(2)} = 0.4930687...


def _example():
    g = json.load(open(GOLD))
    Q = np.array(g["Q"], float)[None, None]
    K = np.array(g["K"], float)[None, None]
    V = np.array(g["V"], float)[None, None]
    return g, Q, K, V


# ---------------------------------------------------------------- worked example (page values)

def test_worked_example_printed_intermediates():
    """Every intermediate the tutorial page prints for row 0, block size 2."""
    g, Q, K, V = _example()
    p, tol = g["printed"], g["tolerance"]
    O, lse, stats, (m, l, Ot) = blocked_row(Q[0, 0, 0], K[0, 0], V[0, 0], S2, [2])
    b1, b2 = stats
    close = lambda x, y: np.testing.assert_allclose(x, y, rtol=0, atol=tol)
    close(b1.scores, p["block1_scores"]); close(b1.m, p["block1_max"])
    close(b1.exps, p["block1_exps"]); close(b1.l, p["block1_sum"])
    close(b1.Otilde, p["block1_Otilde"])
    close(b2.scores, p["block2_scores"]); close(b2.m, p["block2_max"])
    close(b2.exps, p["block2_exps"]); close(b2.l, p["block2_sum"])
    close(b2.Otilde, p["block2_Otilde"])
    close(m, p["merged_max"]); close(l, p["merged_sum"]); close(Ot, p["merged_numerator"])
    close(O, p["row0_output"])


def test_worked_example_row0_closed_form():
    """Row 0 = [1+3a, 3+a] / (2+2a) with a = e^{-1/sqrt 2}, from the definition, both forms."""
    _, Q, K, V = _example()
    want = np.array([1 + 3 * A, 3 + A]) / (2 + 2 * A)
    np.testing.assert_allclose(want, [0.8302385, 1.1697615], atol=5e-8)
    O, LSE = attn_fwd(Q, K, V, S2)
    np.testing.assert_allclose(O[0, 0, 0], want, rtol=0, atol=1e-14)
    Ob, lse_b, _, _ = blocked_row(Q[0, 0, 0], K[0, 0], V[0, 0], S2, [2])
    np.testing.assert_allclose(Ob, want, rtol=0, atol=1e-14)
    assert abs(LSE[0, 0, 0] - (S2 + math.log(2 + 2 * A))) < 1e-14
    assert abs(lse_b - LSE[0, 0, 0]) < 1e-14


def test_worked_example_all_rows_closed_form():
    """Rows 1..3 of the example, derived by hand from the definition (not printed on the page)."""
    _, Q, K, V = _example()
    O, LSE = attn_fwd(Q, K, V, S2)
    rows = np.array([
        [1 + 3 * A, 3 + A],                             # row 0 (over 2 + 2a)
        [2 + 2 * A, 2 + 2 * A],                         # row 1 (over 2 + 2a) -> [1, 1]
        [3 * A + A * A, 2 + A + A * A],                 # row 2 (over (1 + a)^2)
        [1.0, 1.0],                                     # row 3: uniform weights, mean of V
    ]) / np.array([2 + 2 * A, 2 + 2 * A, (1 + A) ** 2, 1.0])[:, None]
    np.testing.assert_allclose(O[0, 0], rows, rtol=0, atol=1e-14)
    np.testing.assert_allclose(O[0, 0].sum(1), 2.0, atol=1e-14)   # V rows sum to 2, O convex
    np.testing.assert_allclose(
        LSE[0, 0], [S2 + math.log(2 + 2 * A)] * 2 + [2 * S2 + 2 * math.log(1 + A), math.log(4)],
        atol=1e-14)


def test_worked_example_rescale_factor():
    """Page: with block maxima 1/sqrt2 and sqrt2 the block-1 factor is e^{1/sqrt2 - sqrt2} ~ 0.493.
    Query row 2 = [1, 1] produces exactly those block maxima."""
    g, Q, K, V = _example()
    _, _, stats, _ = blocked_row(Q[0, 0, 2], K[0, 0], V[0, 0], S2, [2])
    assert abs(stats[0].m - S2) < 1e-15 and abs(stats[1].m - 2 * S2) < 1e-15
    m, l, _ = merge((stats[0].m, 1.0, np.zeros(2)), (stats[1].m, 0.0, np.zeros(2)))
    assert abs(l - g["printed"]["rescale_factor_if_second_max_is_sqrt2"]) < g["tolerance"]
    assert abs(l - A) < 1e-15


def test_worked_example_causal():
    """Causal (top-left) reading: row 0 sees only key 0 -> O = V_0, LSE = s_00; row 1 closed form."""
    _, Q, K, V = _example()
    O, LSE = attn_fwd(Q, K, V, S2, causal=True)
    np.testing.assert_allclose(O[0, 0, 0], V[0, 0, 0], atol=0)
    assert abs(LSE[0, 0, 0] - S2) < 1e-15
    np.testing.assert_allclose(O[0, 0, 1], np.array([2 + A, A]) / (1 + A), atol=1e-14)
    np.testing.assert_allclose(O[0, 0, 1], [1.6697615, 0.3302385], atol=5e-8)


# ---------------------------------------------------------------- merge identity

@pytest.mark.parametrize("seed", range(6))
def test_merge_identity_random_splits(seed):
    """Merging per-block (m, l, Otilde) reproduces the two-pass row for any split (>= 2 blocks)."""
    r = np.random.default_rng(seed)
    N, d = int(r.integers(3, 70)), int(r.integers(1, 9))
    q = r.normal(size=(1, 1, N, d)) * 2
    k, v = r.normal(size=(1, 1, N, d)) * 2, r.normal(size=(1, 1, N, d))
    O, LSE = attn_fwd(q, k, v, 0.7)
    for i in range(N):
        nb = int(r.integers(2, min(N, 6) + 1))
        cuts = sorted(r.choice(np.arange(1, N), size=nb - 1, replace=False))
        Ob, lse_b, stats, _ = blocked_row(q[0, 0, i], k[0, 0], v[0, 0], 0.7, cuts)
        assert len(stats) == nb
        np.testing.assert_allclose(Ob, O[0, 0, i], rtol=0, atol=1e-12)
        assert abs(lse_b - LSE[0, 0, i]) < 1e-12


# ---------------------------------------------------------------- softmax invariants

@pytest.mark.parametrize("causal", [False, True])
def test_identity_values_expose_P(causal):
    """With V = I (d = N), O is P itself: P >= 0, rows sum to 1, P_ij / P_ik = e^{s_ij - s_ik},
    zero above the diagonal when causal and zero on padded keys."""
    r = np.random.default_rng(1)
    N, dk = 12, 5
    q, k = r.normal(size=(2, 1, N, dk)), r.normal(size=(2, 1, N, dk))
    v = np.broadcast_to(np.eye(N), (2, 1, N, N)).copy()
    lens = [N, 7]
    P, LSE = attn_fwd(q, k, v, 0.9, causal, lens)
    for b, L in enumerate(lens):
        s = 0.9 * q[b, 0] @ k[b, 0].T
        for i in range(N):
            vis = [j for j in range(L) if (not causal or j <= i)]
            hid = [j for j in range(N) if j not in vis]
            assert np.all(P[b, 0, i] >= 0)
            assert abs(P[b, 0, i].sum() - 1) < 1e-13
            assert np.all(P[b, 0, i, hid] == 0)
            j0 = vis[0]
            np.testing.assert_allclose(P[b, 0, i, vis] / P[b, 0, i, j0],
                                       np.exp(s[i, vis] - s[i, j0]), rtol=1e-12)
            # LSE is the log-sum-exp of the visible scores (scipy, independent routine)
            assert abs(LSE[b, 0, i] - logsumexp(s[i, vis])) < 1e-12


def test_key_permutation_invariance():
    """Non-causal, unpadded: permuting K and V rows together leaves O and LSE unchanged."""
    r = np.random.default_rng(2)
    q, k, v = (r.normal(size=(2, 3, 40, 8)) for _ in range(3))
    O, LSE = attn_fwd(q, k, v, 0.3)
    perm = r.permutation(40)
    O2, LSE2 = attn_fwd(q, k[:, :, perm], v[:, :, perm], 0.3)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(LSE2, LSE, atol=1e-13)


def test_value_shift_equivariance():
    """O is a convex combination of V rows: O(V + 1 c^T) = O(V) + 1 c^T."""
    r = np.random.default_rng(3)
    q, k, v = (r.normal(size=(1, 2, 33, 6)) for _ in range(3))
    c = r.normal(size=6)
    for causal in (False, True):
        O, _ = attn_fwd(q, k, v, 0.5, causal, [20])
        O2, _ = attn_fwd(q, k, v + c, 0.5, causal, [20])
        np.testing.assert_allclose(O2, O + c, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_average_values(causal):
    """Q = 0: every visible key has score 0, so O_i is the mean of the visible V rows and
    LSE_i = ln(number of visible keys)."""
    r = np.random.default_rng(4)
    N, d = 17, 4
    k, v = r.normal(size=(2, 1, N, d)), r.normal(size=(2, 1, N, d))
    lens = [N, 9]
    O, LSE = attn_fwd(np.zeros((2, 1, N, d)), k, v, 1.0, causal, lens)
    for b, L in enumerate(lens):
        for i in range(N):
            n = min(L, i + 1) if causal else L
            np.testing.assert_allclose(O[b, 0, i], v[b, 0, :n].mean(0), atol=1e-14)
            assert abs(LSE[b, 0, i] - math.log(n)) < 1e-14


def test_single_token():
    """N = 1: O = V, LSE = the single score."""
    r = np.random.default_rng(5)
    q, k, v = (r.normal(size=(1, 2, 1, 3)) for _ in range(3))
    for causal in (False, True):
        O, LSE = attn_fwd(q, k, v, 0.25, causal)
        np.testing.assert_allclose(O, v, atol=0)
        np.testing.assert_allclose(LSE[..., 0], 0.25 * (q * k).sum(-1)[..., 0], atol=1e-15)


def test_empty_rows_and_nan_padding():
    """L_b = 0: O = 0 and LSE = -inf; keys beyond L_b may hold NaN without reaching any output."""
    r = np.random.default_rng(6)
    q, k, v = (r.normal(size=(2, 1, 10, 4)) for _ in range(3))
    k[1, :, 6:] = np.nan
    v[1, :, 6:] = np.nan
    O, LSE = attn_fwd(q, k, v, 1.0, False, [0, 6])
    assert np.all(O[0] == 0) and np.all(LSE[0] == -np.inf)
    assert np.all(np.isfinite(O[1])) and np.all(np.isfinite(LSE[1]))
    O6, LSE6 = attn_fwd(q[1:, :, :6], k[1:, :, :6], v[1:, :, :6], 1.0)   # N = 6, same keys
    np.testing.assert_allclose(O[1, :, :6], O6[0, :, :6], atol=0)


# ---------------------------------------------------------------- independent library routine

def _sdpa64(q, k, v, scale, causal, lens, Hq, Hkv):
    """torch float64 SDPA (math path) with kv heads repeated per group and a boolean key mask."""
    G = Hq // Hkv
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    k, v = k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1)
    B, _, N, _ = q.shape
    mask = torch.ones(B, 1, N, N, dtype=torch.bool)
    if causal:
        mask &= torch.ones(N, N, dtype=torch.bool).tril()
    if lens is not None:
        mask &= (torch.arange(N)[None, :] < torch.tensor(lens)[:, None])[:, None, None, :]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)


@pytest.mark.parametrize("causal,lens,Hq,Hkv", [
    (False, None, 2, 2), (True, None, 2, 2), (False, [31, 16], 4, 2),
    (True, [31, 20], 4, 1), (True, [25, 31], 6, 3)])
def test_matches_torch_sdpa_float64(causal, lens, Hq, Hkv):
    r = np.random.default_rng(7)
    N, d = 31, 8
    q = r.normal(size=(2, Hq, N, d))
    k, v = r.normal(size=(2, Hkv, N, d)), r.normal(size=(2, Hkv, N, d))
    O, _ = attn_fwd(q, k, v, 0.35, causal, lens, chunk=7)   # chunking exercised too
    ref = _sdpa64(q, k, v, 0.35, causal, lens, Hq, Hkv).numpy()
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-13)


def test_gqa_head_map_contiguous():
    assert [kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [kv_head_of(h, 6, 3) for h in range(6)] == [0, 0, 1, 1, 2, 2]
    assert [kv_head_of(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]


def test_rows_api_matches_full():
    r = np.random.default_rng(8)
    q = torch.from_numpy(r.normal(size=(2, 4, 50, 8))).to(torch.bfloat16)
    k = torch.from_numpy(r.normal(size=(2, 2, 50, 8))).to(torch.bfloat16)
    v = torch.from_numpy(r.normal(size=(2, 2, 50, 8))).to(torch.bfloat16)
    lens = torch.tensor([50, 23], dtype=torch.int32)
    O, LSE = attn_fwd(q, k, v, 0.4, True, lens)
    picks = [(0, 0, 0), (1, 3, 49), (1, 2, 22), (0, 1, 17), (1, 0, 23)]
    Or, Lr = attn_fwd_rows(q, k, v, 0.4, True, lens, picks)
    for n, (b, h, i) in enumerate(picks):
        np.testing.assert_allclose(Or[n], O[b, h, i], atol=1e-15)
        assert abs(Lr[n] - LSE[b, h, i]) < 1e-15


def test_extreme_scores_stay_finite():
    """Safe softmax: scores near +-1000 would overflow exp without the max shift.  The row
    reduces to the arg-max key's value (ties share the weight equally)."""
    q = np.array([[[[30.0, 0.0], [0.0, -30.0]]]])
    k = np.array([[[[30.0, 1.0], [29.0, 0.0], [0.0, 31.0]]]])
    q = np.concatenate([q, np.zeros((1, 1, 1, 2))], axis=2)           # N = 3 rows
    v = np.array([[[[1.0, 0.0], [0.0, 1.0], [5.0, 5.0]]]])
    O, LSE = attn_fwd(q, k, v, 1.0)
    np.testing.assert_allclose(O[0, 0, 0], [1.0, 0.0], atol=1e-12)   # scores 900, 870, 0
    np.testing.assert_allclose(O[0, 0, 1], [0.0, 1.0], atol=1e-12)   # scores -30, 0, -930
    assert abs(LSE[0, 0, 0] - 900.0) < 1e-9
    np.testing.assert_allclose(O[0, 0, 2], v[0, 0].mean(0), atol=1e-14)
