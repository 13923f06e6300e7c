"""GPU parity of fa_bwd (through the C ABI) against the fp64 oracle's gradients."""
import numpy as np
import pytest
import torch

import exact_io_aware_68_amd as fa
import fa_inputs as fi
from oracle import attn_bwd, attn_dq_rows, attn_fwd
from tests._parity import TOL_BF16_MAX, TOL_BF16_MEAN, check_close, np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gen(B, Hq, Hkv, N, d, seed, padded=False, std=1.0):
    w = fi.Workload("t", B, Hq, Hkv, N, d, "bf16", False, padded, True, std, seed)
    return fi.make(w)


def dev(x):
    out = {n: (t.to(DEV) if torch.is_tensor(t) else t) for n, t in x.items()}
    return out


def run_fwd_bwd(x, causal, o_lse=None):
    g = dev(x)
    if o_lse is None:
        o, lse = fa.fa_fwd(g["q"], g["k"], g["v"], scale=x["scale"], causal=causal,
                           key_lens=g["key_lens"])
    else:
        o, lse = (t.to(DEV) for t in o_lse)
    dq, dk, dv = fa.fa_bwd(g["q"], g["k"], g["v"], o, g["do"], lse, scale=x["scale"],
                           causal=causal, key_lens=g["key_lens"])
    torch.cuda.synchronize()
    return dq, dk, dv


def check_grads(got, ref):
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        check_close(name, np64(a), b, TOL_BF16_MAX, TOL_BF16_MEAN)


CASES = [  # (B, Hq, Hkv, N, d, causal, padded)
    (2, 2, 2, 300, 128, True, False),
    (2, 2, 2, 300, 128, False, False),
    (2, 2, 2, 300, 64, True, False),
    (2, 2, 2, 300, 64, False, False),
    (2, 4, 2, 300, 128, True, True),
    (2, 4, 1, 200, 64, False, True),
    (1, 2, 2, 1, 128, True, False),
    (1, 2, 2, 65, 128, True, False),
    (1, 1, 1, 513, 128, True, False),
    # grouped heads with several query tiles per q-head: the diagonal tiles of every q-head
    # come first, then the rest, with odd and even run lengths
    (1, 8, 2, 700, 128, True, True),
    (1, 4, 1, 450, 64, True, False),
    # causal grids whose per-XCD share takes each branch of the workgroup order (dK/dV and dQ):
    # three heads, two heads ranked together, and grouped-query heads whose dK/dV share is not
    # whole heads (pairs of heads: the full-size c5 test)
    (1, 24, 24, 384, 128, True, False),
    (2, 8, 8, 512, 64, True, False),
    (1, 16, 4, 512, 128, True, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,padded", CASES)
def test_bwd_parity_small(B, Hq, Hkv, N, d, causal, padded):
    x = gen(B, Hq, Hkv, N, d, 2000 + N + d + Hq, padded)
    print(f"\nbwd bf16 B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}", flush=True)
    got = run_fwd_bwd(x, causal)
    ref = attn_bwd(x["q"], x["k"], x["v"], x["do"], x["scale"], causal, x["key_lens"])
    check_grads(got, ref)


def test_bwd_with_oracle_forward_state():
    """Isolate the backward: feed it the oracle's O (rounded to bf16) and LSE."""
    x = gen(2, 4, 2, 260, 128, 77, padded=True)
    O, LSE = attn_fwd(x["q"], x["k"], x["v"], x["scale"], True, x["key_lens"])
    o = torch.from_numpy(O).to(torch.bfloat16)
    lse = torch.from_numpy(LSE).to(torch.float32)
    got = run_fwd_bwd(x, True, (o, lse))
    ref = attn_bwd(x["q"], x["k"], x["v"], x["do"], x["scale"], True, x["key_lens"])
    check_grads(got, ref)


def test_bwd_key_length_zero_and_nan_padding():
    x = gen(3, 2, 1, 160, 128, 78)
    x["key_lens"] = torch.tensor([0, 1, 97], dtype=torch.int32)
    clean = run_fwd_bwd(x, True)
    ref = attn_bwd(x["q"], x["k"], x["v"], x["do"], x["scale"], True, x["key_lens"])
    check_grads(clean, ref)
    assert all(torch.all(t[0] == 0) for t in clean)
    for b, L in enumerate([0, 1, 97]):
        x["k"][b, :, L:] = float("nan")
        x["v"][b, :, L:] = float("nan")
    dirty = run_fwd_bwd(x, True)
    for a, b in zip(clean[1:], dirty[1:]):
        assert torch.equal(a, b)
    check_close("dQ", np64(dirty[0]), ref[0], TOL_BF16_MAX, TOL_BF16_MEAN)


def test_gradients_bitwise_deterministic():
    """Every gradient element is written once by one lane (no atomics): bitwise reproducible."""
    x = gen(1, 4, 2, 300, 128, 79)
    a = run_fwd_bwd(x, True)
    b = run_fwd_bwd(x, True)
    assert all(torch.equal(u, v) for u, v in zip(a, b))


def test_stages_match_fa_bwd():
    """fa_bwd_prep + fa_bwd_dkdv + fa_bwd_dq (the timed stages) equal fa_bwd bit for bit."""
    x = dev(gen(2, 4, 2, 260, 128, 80, padded=True))
    o, lse = fa.fa_fwd(x["q"], x["k"], x["v"], scale=x["scale"], causal=True,
                       key_lens=x["key_lens"])
    whole = fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, scale=x["scale"], causal=True,
                      key_lens=x["key_lens"])
    ws = torch.empty(fa.fa_bwd_workspace_size(2, 4, 260), dtype=torch.uint8, device=DEV)
    dq, dk, dv = (torch.empty_like(t) for t in whole)
    fa.fa_bwd_prep(o, x["do"], lse, ws)
    fa.fa_bwd_dkdv(x["q"], x["k"], x["v"], x["do"], dk, dv, ws, scale=x["scale"], causal=True,
                   key_lens=x["key_lens"])
    fa.fa_bwd_dq(x["q"], x["k"], x["v"], x["do"], dq, ws, scale=x["scale"], causal=True,
                 key_lens=x["key_lens"])
    torch.cuda.synchronize()
    assert all(torch.equal(u, v) for u, v in zip(whole, (dq, dk, dv)))


def test_side_stream_gives_the_same_results():
    """Work enqueued on another stream (passed explicitly, or current inside a stream context)
    gives bitwise the results of the default stream: the stream argument is honoured and the
    library keeps no state between calls."""
    x = gen(2, 4, 2, 333, 128, 7, padded=True)
    ref = run_fwd_bwd(x, True)
    g = dev(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, lse = fa.fa_fwd(g["q"], g["k"], g["v"], scale=x["scale"], causal=True,
                       key_lens=g["key_lens"], stream=side)
    got1 = fa.fa_bwd(g["q"], g["k"], g["v"], o, g["do"], lse, scale=x["scale"], causal=True,
                     key_lens=g["key_lens"], stream=side)
    with torch.cuda.stream(side):
        o2, lse2 = fa.fa_fwd(g["q"], g["k"], g["v"], scale=x["scale"], causal=True,
                             key_lens=g["key_lens"])
        got2 = fa.fa_bwd(g["q"], g["k"], g["v"], o2, g["do"], lse2, scale=x["scale"],
                         causal=True, key_lens=g["key_lens"])
    side.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b, c in zip(ref, got1, got2):
        assert torch.equal(a, b) and torch.equal(a, c)


def test_backward_tensors_past_2_31_elements():
    """Backward on Q, O, dO and an fp32 dQ of more than 2^31 elements (dQ 9.7 GB): the kernels'
    addressing is 64-bit.  dQ rows of the first and of the last batch and head (offsets past
    2^31) against the oracle's per-row dQ; every gradient finite; for every kv-head,
    sum_j dV_j equals the sum of dO over its query heads' rows (rows of P sum to one)."""
    w = fi.Workload("bigb", 9, 64, 8, 32768, 128, "bf16", True, True, True, 1.0, 13)
    assert w.B * w.Hq * w.N * w.d > 2**31
    print(f"\n> 2^31 elements, backward: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d}", flush=True)
    x = fi.make_on_device(w, DEV)
    kl = x["key_lens"]
    o, lse = fa.fa_fwd(x["q"], x["k"], x["v"], scale=x["scale"], causal=True, key_lens=kl)
    dq, dk, dv = fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, scale=x["scale"], causal=True,
                           key_lens=kl)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    del o, lse
    picks = sorted({(b, h, i) for b in (0, w.B - 1) for h in (0, w.Hq - 1)
                    for i in (0, 1, 127, 128, w.N // 2, w.N - 2, w.N - 1)})
    ref = attn_dq_rows(x["q"], x["k"], x["v"], x["do"], x["scale"], True, kl.cpu(), picks)
    idx = tuple(torch.tensor(a) for a in zip(*picks))
    check_close("dQ", np64(dq[idx]), ref, TOL_BF16_MAX, TOL_BF16_MEAN)
    G = w.Hq // w.Hkv
    sdv = dv.double().sum(2)                                            # [B, Hkv, d]
    sdo = x["do"].double().sum(2).view(w.B, w.Hkv, G, w.d).sum(2)       # [B, Hkv, d]
    assert (sdv - sdo).abs().max().item() < 1.0
    del x, dq, dk, dv
    torch.cuda.empty_cache()
