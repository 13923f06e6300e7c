"""GPU parity of fa_fwd (through the C ABI) against the fp64 oracle on the same inputs."""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_68_amd as fa
import fa_inputs as fi
from oracle import attn_fwd, attn_fwd_rows
from tests._parity import (TOL_BF16_MAX, TOL_BF16_MEAN, TOL_F32, TOL_LSE, check_close, np64)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_fwd(x, causal, want_lse=True):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    kl = None if x.get("key_lens") is None else x["key_lens"].to(DEV)
    o, lse = fa.fa_fwd(q, k, v, scale=x["scale"], causal=causal, key_lens=kl, want_lse=want_lse)
    torch.cuda.synchronize()
    return o, lse


def gen(B, Hq, Hkv, N, d, dtype, seed, padded=False, std=1.0):
    w = fi.Workload("t", B, Hq, Hkv, N, d, dtype, False, padded, False, std, seed)
    return fi.make(w)


# ------------------------------------------------------------------ fp32 instance

def test_worked_example_fp32():
    ex = fi.worked_example()
    ex["scale"] = 1 / math.sqrt(2)
    for causal in (False, True):
        o, lse = run_fwd(ex, causal)
        O, LSE = attn_fwd(ex["q"], ex["k"], ex["v"], ex["scale"], causal)
        check_close("O", np64(o), O, TOL_F32)
        check_close("LSE", np64(lse), LSE, TOL_F32)
    o, _ = run_fwd(ex, False)
    np.testing.assert_allclose(np64(o)[0, 0, 0], [0.8302385, 1.1697615], atol=1e-6)


def test_c1_fp32_full():
    x = fi.make(fi.WORKLOADS["c1"])
    o, lse = run_fwd(x, False, want_lse=False)
    assert lse is None
    O, _ = attn_fwd(x["q"], x["k"], x["v"], x["scale"])
    check_close("O", np64(o), O, TOL_F32)


@pytest.mark.parametrize("d", [1, 37, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_ragged(d, causal):
    x = gen(2, 4, 2, 150, d, "f32", 100 + d, padded=True)
    o, lse = run_fwd(x, causal)
    O, LSE = attn_fwd(x["q"], x["k"], x["v"], x["scale"], causal, x["key_lens"])
    check_close("O", np64(o), O, TOL_F32)
    check_close("LSE", np64(lse), LSE, TOL_F32)


# ------------------------------------------------------------------ bf16 instances

CASES = [  # (B, Hq, Hkv, N, d, causal, padded)
    (2, 2, 2, 300, 64, False, False),
    (2, 2, 2, 300, 128, False, False),
    (2, 2, 2, 300, 64, True, False),
    (2, 2, 2, 300, 128, True, False),
    (2, 4, 2, 300, 128, True, True),
    (3, 4, 1, 257, 64, True, True),
    (2, 6, 3, 200, 128, False, True),
    (1, 2, 2, 1, 128, True, False),
    (1, 2, 2, 63, 64, False, False),
    (1, 2, 1, 129, 128, True, False),
    (1, 1, 1, 640, 128, True, False),
    # causal grids whose per-XCD share takes each branch of the workgroup order: three heads
    # (ranked over all), two heads whose K and V fit in the L2 (ranked together), one head, a
    # share that is not whole heads, and grouped-query heads; shares ranked in pairs of heads
    # (K and V past the L2) are the full-size c3, c4 and c5 tests
    (1, 24, 24, 384, 128, True, False),
    (2, 8, 8, 512, 64, True, True),
    (1, 8, 8, 640, 128, True, False),
    (1, 4, 4, 768, 128, True, False),
    (1, 16, 4, 512, 128, True, True),
    # the non-causal d = 64 instance takes 256-row workgroups: several of them with a ragged
    # last one, grouped-query heads and key lengths
    (2, 6, 2, 700, 64, False, True),
    (1, 3, 3, 513, 64, False, False),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,padded", CASES)
def test_bf16_parity_small(B, Hq, Hkv, N, d, causal, padded):
    x = gen(B, Hq, Hkv, N, d, "bf16", 1000 + N + d + 7 * Hq, padded)
    print(f"\nfwd bf16 B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}", flush=True)
    o, lse = run_fwd(x, causal)
    O, LSE = attn_fwd(x["q"], x["k"], x["v"], x["scale"], causal, x["key_lens"])
    check_close("O", np64(o), O, TOL_BF16_MAX, TOL_BF16_MEAN)
    check_close("LSE", np64(lse), LSE, TOL_LSE)


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_key_lengths_edge_values(d):
    """key_lens of 0 (row has no key: O = 0, LSE = -inf), 1, a tile edge and N."""
    x = gen(4, 2, 1, 200, d, "bf16", 7)
    x["key_lens"] = torch.tensor([0, 1, 64, 200], dtype=torch.int32)
    for causal in (False, True):
        o, lse = run_fwd(x, causal)
        O, LSE = attn_fwd(x["q"], x["k"], x["v"], x["scale"], causal, x["key_lens"])
        check_close("O", np64(o), O, TOL_BF16_MAX, TOL_BF16_MEAN)
        check_close("LSE", np64(lse), LSE, TOL_LSE)
        assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_nan_padding_never_reaches_outputs():
    x = gen(2, 2, 2, 256, 64, "bf16", 8)
    x["key_lens"] = torch.tensor([100, 193], dtype=torch.int32)
    refs = [run_fwd(x, causal) for causal in (False, True)]
    for b, L in enumerate([100, 193]):
        x["k"][b, :, L:] = float("nan")
        x["v"][b, :, L:] = float("nan")
    for causal, (o_ref, l_ref) in zip((False, True), refs):
        o, lse = run_fwd(x, causal)
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


@pytest.mark.parametrize("d,causal", [(128, True), (64, False)])
def test_every_output_written_and_canaries_intact(d, causal):
    x = gen(2, 2, 1, 190, d, "bf16", 9)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    n_o, n_l = q.numel(), 2 * 2 * 190
    ob = torch.full((n_o + 2048,), float("nan"), dtype=torch.bfloat16, device=DEV)
    lb = torch.full((n_l + 2048,), float("nan"), dtype=torch.float32, device=DEV)
    o = ob[1024:1024 + n_o].view(q.shape)
    lse = lb[1024:1024 + n_l].view(2, 2, 190)
    fa.fa_fwd(q, k, v, scale=x["scale"], causal=causal, o=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert torch.isnan(ob[:1024]).all() and torch.isnan(ob[1024 + n_o:]).all()
    assert torch.isnan(lb[:1024]).all() and torch.isnan(lb[1024 + n_l:]).all()


def test_bf16_lse_null_gives_the_same_o():
    """lse = NULL (O only) changes nothing in O, and no LSE is written."""
    x = gen(2, 4, 2, 333, 128, "bf16", 12, padded=True)
    o1, l1 = run_fwd(x, True)
    o2, l2 = run_fwd(x, True, want_lse=False)
    assert l2 is None and l1 is not None
    assert torch.equal(o1, o2)


def test_forward_is_bitwise_deterministic():
    x = gen(2, 4, 2, 333, 128, "bf16", 10, padded=True)
    o1, l1 = run_fwd(x, True)
    o2, l2 = run_fwd(x, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_scores_rising_and_falling_along_keys(causal, d):
    """Head 0: scores rise by about 140-200 (log2 units) from the first keys to the last, so
    exponentials taken against the first keys' maximum would overflow fp32 and the kernel's
    reference point has to move many times.  Head 1: scores fall just as far, so the later
    exponentials underflow to zero."""
    B, N = 1, 700
    print(f"\nfwd rising/falling scores d={d} causal={causal}", flush=True)
    g = torch.Generator().manual_seed(77 + d)
    q = 1.0 + 0.1 * torch.randn(B, 2, N, d, generator=g)
    ramp = torch.linspace(0.0, 12.0, N).view(1, 1, N, 1)
    k = torch.cat([ramp, 12.0 - ramp], dim=1) + 0.1 * torch.randn(B, 2, N, d, generator=g)
    v = torch.randn(B, 2, N, d, generator=g)
    x = {"q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16), "v": v.to(torch.bfloat16),
         "scale": float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32)), "key_lens": None}
    o, lse = run_fwd(x, causal)
    O, LSE = attn_fwd(x["q"], x["k"], x["v"], x["scale"], causal)
    assert np.max(LSE[:, 0]) > 90.0   # the rise really is past the fp32 exponent range
    check_close("O", np64(o), O, TOL_BF16_MAX, TOL_BF16_MEAN)
    check_close("LSE", np64(lse), LSE, TOL_LSE)


# ------------------------------------------------------------------ full-size workloads

def _sample_rows(w, n_rand, seed, key_lens=None):
    """Tile and sequence edges of every (batch, q-head) (the rows around each batch's key length
    included), more edges of the first and last q-head, and n_rand random rows."""
    r = np.random.default_rng(seed)
    picks = set()
    for b in range(w.B):
        L = w.N if key_lens is None else int(key_lens[b])
        edges = {0, 127, 128, L - 1, L, L + 1, w.N - 1}
        for h in range(w.Hq):
            picks.update((b, h, i) for i in edges if 0 <= i < w.N)
        for h in (0, w.Hq - 1):
            picks.update((b, h, i) for i in (1, 63, 64, w.N // 2, w.N - 2))
    n0 = len(picks)
    while len(picks) < n0 + n_rand:
        picks.add((int(r.integers(w.B)), int(r.integers(w.Hq)), int(r.integers(w.N))))
    return sorted(picks)


@pytest.mark.parametrize("name", ["c4"])
def test_full_size_workload_sampled_rows(name):
    """Rows of every q-head of the largest workload, beyond the head subset that
    tests/test_gpu_full_parity.py checks in full: the oracle recomputes sampled rows one by one
    (first, last, tile edges and the rows around each batch's key length of every q-head, plus
    random rows) and every row is checked for finiteness."""
    w = fi.WORKLOADS[name]
    print(f"\nfull-size {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d}", flush=True)
    x = fi.make(w)
    o, lse = run_fwd(x, w.causal)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    picks = _sample_rows(w, 96, w.seed, x["key_lens"])
    assert {(b, h) for b, h, _ in picks} == {(b, h) for b in range(w.B) for h in range(w.Hq)}
    O, LSE = attn_fwd_rows(x["q"], x["k"], x["v"], x["scale"], w.causal, x["key_lens"], picks)
    idx = tuple(torch.tensor(a) for a in zip(*picks))
    check_close("O", np64(o[idx]), O, TOL_BF16_MAX, TOL_BF16_MEAN)
    check_close("LSE", np64(lse[idx]), LSE, TOL_LSE)


def test_tensors_past_2_31_elements():
    """Q and O of more than 2^31 elements (4.8 GB each): the kernel's addressing is 64-bit.  Rows
    of the first and of the last batch and head (element offsets past 2^31) are recomputed by the
    oracle one by one; every output is checked for finiteness.  Grouped heads and key lengths as
    in the largest workload."""
    w = fi.Workload("big", 9, 64, 8, 32768, 128, "bf16", True, True, False, 1.0, 11)
    assert w.B * w.Hq * w.N * w.d > 2**31
    print(f"\n> 2^31 elements: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d}", flush=True)
    x = fi.make_on_device(w, DEV)
    o, lse = fa.fa_fwd(x["q"], x["k"], x["v"], scale=x["scale"], causal=True,
                       key_lens=x["key_lens"])
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    picks = sorted({(b, h, i) for b in (0, w.B - 1) for h in (0, w.Hq - 1)
                    for i in (0, 1, 127, 128, w.N // 2, w.N - 2, w.N - 1)}
                   | {(w.B - 1, int(h), int(i)) for h, i in
                      zip(np.random.default_rng(11).integers(w.Hq, size=8),
                          np.random.default_rng(12).integers(w.N, size=8))})
    kl = x["key_lens"].cpu()
    O, LSE = attn_fwd_rows(x["q"], x["k"], x["v"], x["scale"], True, kl, picks)
    idx = tuple(torch.tensor(a) for a in zip(*picks))
    check_close("O", np64(o[idx]), O, TOL_BF16_MAX, TOL_BF16_MEAN)
    check_close("LSE", np64(lse[idx]), LSE, TOL_LSE)
    del x, o, lse
    torch.cuda.empty_cache()
