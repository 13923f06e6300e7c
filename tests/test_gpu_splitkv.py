"""GPU parity of fa_fwd_splitkv (through the C ABI) against the oracle's decode-shaped forward."""
import numpy as np
import pytest
import torch

import exact_io_aware_68_amd as fa
import fa_inputs as fi
from oracle import attn_decode
from tests._parity import TOL_BF16_MAX, TOL_BF16_MEAN, TOL_LSE, check_close, np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gen(B, Hq, Hkv, Nq, Nk, d, seed, lens=None, std=1.0):
    w = fi.DecodeWorkload("t", B, Hq, Hkv, Nq, Nk, d, False, std, seed)
    x = fi.make_decode(w)
    if lens is not None:
        x["key_lens"] = torch.tensor(lens, dtype=torch.int32)
    return x


def run(x, num_splits=0):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    kl = None if x["key_lens"] is None else x["key_lens"].to(DEV)
    o, lse = fa.fa_fwd_splitkv(q, k, v, scale=x["scale"], key_lens=kl, num_splits=num_splits)
    torch.cuda.synchronize()
    return o, lse


CASES = [  # (B, Hq, Hkv, Nq, Nk, d, lens, num_splits)
    (2, 8, 2, 1, 1000, 128, None, 0),
    (2, 8, 2, 1, 1000, 128, [1000, 333], 0),
    (3, 4, 4, 3, 257, 64, [0, 1, 257], 0),
    (1, 32, 8, 2, 4096, 128, [4000], 5),
    (2, 16, 2, 4, 700, 64, [700, 64], 1),
    (1, 12, 1, 4, 300, 128, None, 0),          # 48 rows per kv-head: two row tiles
    (2, 4, 1, 1, 31, 128, [31, 5], 0),         # fewer keys than one step
    (1, 2, 2, 7, 129, 64, None, 2),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,lens,splits", CASES)
def test_splitkv_parity(B, Hq, Hkv, Nq, Nk, d, lens, splits):
    print(f"\nsplitkv B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} lens={lens} splits={splits}",
          flush=True)
    x = gen(B, Hq, Hkv, Nq, Nk, d, 600 + Nk + Nq, lens)
    o, lse = run(x, splits)
    O, LSE = attn_decode(x["q"], x["k"], x["v"], x["scale"], x["key_lens"])
    check_close("O", np64(o), O, TOL_BF16_MAX, TOL_BF16_MEAN)
    check_close("LSE", np64(lse), LSE, TOL_LSE)
    if lens is not None:
        for b, L in enumerate(lens):
            if L == 0:
                assert torch.all(o[b] == 0) and torch.all(torch.isneginf(lse[b]))


def test_no_keys_at_all():
    x = gen(1, 4, 2, 2, 0, 128, 9)
    o, lse = run(x)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_nan_padding_never_reaches_outputs():
    x = gen(2, 8, 2, 1, 900, 128, 11, [900, 401])
    o_ref, l_ref = run(x)
    x["k"][1, :, 401:] = float("nan")
    x["v"][1, :, 401:] = float("nan")
    o, lse = run(x)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_split_counts_agree():
    """Any number of key ranges computes the same attention (merge identity)."""
    x = gen(2, 8, 2, 2, 2000, 128, 12, [2000, 1500])
    O, LSE = attn_decode(x["q"], x["k"], x["v"], x["scale"], x["key_lens"])
    for s in (1, 3, 0):
        o, lse = run(x, s)
        check_close(f"O splits={s}", np64(o), O, TOL_BF16_MAX, TOL_BF16_MEAN)
        check_close(f"LSE splits={s}", np64(lse), LSE, TOL_LSE)


def test_matches_square_forward_when_noncausal():
    """With Nq = Nk and no causal mask the decode path computes the same attention as fa_fwd."""
    x = gen(1, 4, 2, 256, 256, 64, 13, [200])
    o1, l1 = run(x)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o2, l2 = fa.fa_fwd(q, k, v, scale=x["scale"], causal=False, key_lens=x["key_lens"].to(DEV))
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2 * TOL_BF16_MAX
    assert (l1 - l2).abs().max().item() <= 2 * TOL_LSE


def test_decode_workload_full():
    """The decode workload in the launch configuration the bench times, every row checked."""
    w = fi.DECODE_WORKLOADS["decode"]
    print(f"\ndecode workload B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d}", flush=True)
    x = fi.make_decode(w)
    o, lse = run(x)
    O, LSE = attn_decode(x["q"], x["k"], x["v"], x["scale"], x["key_lens"])
    check_close("O", np64(o), O, TOL_BF16_MAX, TOL_BF16_MEAN)
    check_close("LSE", np64(lse), LSE, TOL_LSE)


def test_cache_past_2_31_elements():
    """K and V caches of more than 2^31 elements each (72 sequences of 32768 keys, 4.8 GB each):
    the range kernel's and the merge's addressing is 64-bit.  The first and the last sequence
    (cache offsets past 2^31) are checked in full against the oracle; every row is finite."""
    w = fi.DecodeWorkload("bigd", 72, 32, 8, 1, 32768, 128, True, 1.0, 17)
    assert w.B * w.Hkv * w.Nk * w.d > 2**31
    print(f"\n> 2^31-element cache: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d}",
          flush=True)
    x = fi.make_decode_on_device(w, DEV)
    kl = x["key_lens"]
    o, lse = fa.fa_fwd_splitkv(x["q"], x["k"], x["v"], scale=x["scale"], key_lens=kl)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    for b in (0, w.B - 1):
        sl = slice(b, b + 1)
        O, LSE = attn_decode(x["q"][sl], x["k"][sl], x["v"][sl], x["scale"], kl[sl].cpu())
        check_close("O", np64(o[sl]), O, TOL_BF16_MAX, TOL_BF16_MEAN)
        check_close("LSE", np64(lse[sl]), LSE, TOL_LSE)
    del x, o, lse
    torch.cuda.empty_cache()
