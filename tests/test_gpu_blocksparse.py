"""GPU parity of fa_fwd_blocksparse (through the C ABI) against the oracle's block-sparse forward."""
import numpy as np
import pytest
import torch

import exact_io_aware_68_amd as fa
import fa_inputs as fi
from oracle import attn_fwd, attn_fwd_rows
from tests._parity import TOL_BF16_MAX, TOL_BF16_MEAN, TOL_LSE, check_close, np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gen(B, Hq, Hkv, N, d, seed, padded=False):
    return fi.make(fi.Workload("t", B, Hq, Hkv, N, d, "bf16", False, padded, False, 1.0, seed))


def run(x, bm, causal):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    kl = None if x.get("key_lens") is None else x["key_lens"].to(DEV)
    o, lse = fa.fa_fwd_blocksparse(q, k, v, bm.to(DEV), scale=x["scale"], causal=causal,
                                   key_lens=kl)
    torch.cuda.synchronize()
    return o, lse


def check(x, bm, causal, o, lse):
    O, LSE = attn_fwd(x["q"], x["k"], x["v"], x["scale"], causal, x["key_lens"],
                      block_mask=(bm.numpy(), fa.BLOCK_Q, fa.BLOCK_K))
    rows = np.isfinite(LSE)
    check_close("O", np64(o), O, TOL_BF16_MAX, TOL_BF16_MEAN)
    check_close("LSE", np64(lse)[rows], LSE[rows], TOL_LSE)
    assert np.all(np.isneginf(np64(lse)[~rows])) and np.all(np64(o)[~rows] == 0)


CASES = [  # (B, Hq, Hkv, N, d, density, causal, padded)
    (2, 2, 2, 512, 128, 0.3, False, False),
    (2, 4, 2, 700, 128, 0.5, True, True),
    (1, 2, 1, 1000, 64, 0.2, False, True),
    (2, 2, 2, 300, 64, 0.7, True, False),
    (1, 2, 2, 129, 128, 0.4, False, False),
    (1, 4, 4, 1500, 128, 0.1, True, False),
    (2, 8, 4, 512, 128, 0.3, True, False),   # causal: each XCD ranks two heads together
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,density,causal,padded", CASES)
def test_blocksparse_parity(B, Hq, Hkv, N, d, density, causal, padded):
    print(f"\nblocksparse B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} density={density} causal={causal}",
          flush=True)
    x = gen(B, Hq, Hkv, N, d, 800 + N + d, padded)
    g = torch.Generator().manual_seed(N)
    bm = (torch.rand(-(-N // 128), -(-N // 64), generator=g) < density).to(torch.uint8)
    o, lse = run(x, bm, causal)
    check(x, bm, causal, o, lse)


def test_all_on_equals_the_dense_forward():
    x = gen(2, 2, 1, 600, 128, 41, padded=True)
    bm = torch.ones(5, 10, dtype=torch.uint8)
    for causal in (False, True):
        o, lse = run(x, bm, causal)
        check(x, bm, causal, o, lse)
        q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
        o2, l2 = fa.fa_fwd(q, k, v, scale=x["scale"], causal=causal, key_lens=x["key_lens"].to(DEV))
        torch.cuda.synchronize()
        assert (o.float() - o2.float()).abs().max().item() <= 2 * TOL_BF16_MAX
        assert (lse - l2).abs().max().item() <= 2 * TOL_LSE


def test_rows_with_every_block_off_and_empty_bitmap():
    x = gen(1, 2, 2, 384, 64, 42)
    bm = torch.zeros(3, 6, dtype=torch.uint8)
    bm[1, 3] = 1                   # rows 128..255 see keys 192..255 only
    o, lse = run(x, bm, False)
    check(x, bm, False, o, lse)
    assert torch.all(o[:, :, :128] == 0) and torch.all(torch.isneginf(lse[:, :, 256:]))
    o, lse = run(x, torch.zeros(3, 6, dtype=torch.uint8), False)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_nan_in_skipped_blocks_and_padding_never_reaches_outputs():
    x = gen(1, 2, 2, 512, 128, 43)
    x["key_lens"] = torch.tensor([450], dtype=torch.int32)
    bm = torch.ones(4, 8, dtype=torch.uint8)
    bm[:, 2] = 0
    o_ref, l_ref = run(x, bm, False)
    x["k"][:, :, 128:192] = float("nan")     # key block 2: off for every row
    x["v"][:, :, 128:192] = float("nan")
    x["k"][:, :, 450:] = float("nan")
    x["v"][:, :, 450:] = float("nan")
    o, lse = run(x, bm, False)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_sparse_workload_sampled_rows():
    w, density = fi.SPARSE_WORKLOADS["sparse"]
    print(f"\nsparse workload B={w.B} H={w.Hq} N={w.N} d={w.d} density={density}", flush=True)
    x = fi.make(w)
    bm = fi.block_bitmap(w.N, density, w.seed)
    o, lse = run(x, bm, w.causal)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    r = np.random.default_rng(w.seed)
    picks = sorted({(b, h, i) for b in range(w.B) for h in (0, w.Hq - 1)
                    for i in (0, 127, 128, 4095, w.N - 1)} |
                   {(int(r.integers(w.B)), int(r.integers(w.Hq)), int(r.integers(w.N)))
                    for _ in range(48)})
    O, LSE = attn_fwd_rows(x["q"], x["k"], x["v"], x["scale"], w.causal, None, picks,
                           block_mask=(bm.numpy(), fa.BLOCK_Q, fa.BLOCK_K))
    idx = tuple(torch.tensor(a) for a in zip(*picks))
    check_close("O", np64(o[idx]), O, TOL_BF16_MAX, TOL_BF16_MEAN)
    check_close("LSE", np64(lse[idx]), LSE, TOL_LSE)


def test_sparse_past_2_31_elements():
    """Q and O of more than 2^31 elements under a block bitmap (causal, grouped heads, key
    lengths): the sparse kernel's addressing is 64-bit.  Rows of the first and of the last batch
    and head against the oracle; every output finite."""
    w = fi.Workload("bigs", 9, 64, 8, 32768, 128, "bf16", True, True, False, 1.0, 19)
    assert w.B * w.Hq * w.N * w.d > 2**31
    print(f"\n> 2^31 elements, block-sparse: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d}",
          flush=True)
    x = fi.make_on_device(w, DEV)
    bm = fi.block_bitmap(w.N, 0.1, 19)
    kl = x["key_lens"]
    o, lse = fa.fa_fwd_blocksparse(x["q"], x["k"], x["v"], bm.to(DEV), scale=x["scale"],
                                   causal=True, key_lens=kl)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    picks = sorted({(b, h, i) for b in (0, w.B - 1) for h in (0, w.Hq - 1)
                    for i in (0, 1, 127, 128, w.N // 2, w.N - 2, w.N - 1)})
    O, LSE = attn_fwd_rows(x["q"], x["k"], x["v"], x["scale"], True, kl.cpu(), picks,
                           block_mask=(bm.numpy(), fa.BLOCK_Q, fa.BLOCK_K))
    idx = tuple(torch.tensor(a) for a in zip(*picks))
    check_close("O", np64(o[idx]), O, TOL_BF16_MAX, TOL_BF16_MEAN)
    check_close("LSE", np64(lse[idx]), LSE, TOL_LSE)
    del x, o, lse
    torch.cuda.empty_cache()


def test_causal_rows_whose_only_block_lies_past_them():
    """Causal, one active block on the diagonal: the first half of that row block's rows sees no
    key at all (O = 0, LSE = -inf) and its waves skip every step; the rest see part of it."""
    x = gen(1, 2, 2, 384, 128, 43)
    bm = torch.zeros(3, 6, dtype=torch.uint8)
    bm[1, 3] = 1                   # rows 128..255: keys 192..255, visible to rows >= 192 only
    bm[2, 2] = 1                   # rows 256..383: keys 128..191, visible to all of them
    o, lse = run(x, bm, True)
    check(x, bm, True, o, lse)
    assert torch.all(o[:, :, 128:192] == 0) and torch.all(torch.isneginf(lse[:, :, 128:192]))


@pytest.mark.parametrize("causal", [False, True])
def test_very_negative_logits(causal):
    """Every scaled logit near -150 in log2 units (K close to -Q), with sparse rows whose first
    active block is far from key 0: exponentials taken against any reference point other than a
    visible score's would underflow fp32."""
    B, Hq, Hkv, N, d = 1, 2, 1, 640, 128
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    a = (150.0 / (scale * 1.4426950408889634 * d)) ** 0.5
    g = torch.Generator().manual_seed(97 + causal)
    q = (a + 0.1 * a * torch.randn(B, Hq, N, d, generator=g)).to(torch.bfloat16)
    k = (-a + 0.1 * a * torch.randn(B, Hkv, N, d, generator=g)).to(torch.bfloat16)
    v = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16)
    x = {"q": q, "k": k, "v": v, "scale": scale, "key_lens": None}
    bm = (torch.rand(5, 10, generator=g) < 0.4).to(torch.uint8)
    bm[:, :3] = 0                  # no row block sees keys 0..191
    bm[1:, 3] = 1
    o, lse = run(x, bm, causal)
    O, LSE = attn_fwd(q, k, v, scale, causal, None, block_mask=(bm.numpy(), fa.BLOCK_Q, fa.BLOCK_K))
    rows = np.isfinite(LSE)
    assert np.median(LSE[rows]) < -90.0
    check(x, bm, causal, o, lse)
