"""GPU parity of fa_fwd_window (through the C ABI) against the oracle's windowed forward."""
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


def run(x, window):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    kl = None if x.get("key_lens") is None else x["key_lens"].to(DEV)
    o, lse = fa.fa_fwd_window(q, k, v, window=window, scale=x["scale"], key_lens=kl)
    torch.cuda.synchronize()
    return o, lse


CASES = [  # (B, Hq, Hkv, N, d, window, padded)
    (1, 2, 2, 6, 64, (1, 1), False),          # the tutorial's N = 6, w = 3 example shape
    (2, 2, 2, 300, 128, (1, 1), False),
    (2, 4, 2, 700, 128, (64, 64), True),
    (2, 2, 1, 513, 64, (127, 0), False),       # causal local window
    (1, 4, 4, 900, 128, (300, 20), True),
    (1, 2, 2, 400, 128, (-1, 5), False),
    (2, 2, 2, 400, 64, (5, -1), True),
    (1, 2, 2, 333, 128, (0, 0), False),
    (1, 2, 1, 260, 128, (10000, 10000), True),  # wider than N: plain attention
    (1, 2, 2, 1000, 128, (-1, 0), False),       # unbounded left, right 0: causal
    # long enough that each wave has masked steps at both window edges and a run of unmasked
    # steps between them
    (1, 4, 2, 2000, 128, (700, 300), True),
    (2, 2, 2, 1500, 64, (257, 33), False),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,window,padded", CASES)
def test_window_parity(B, Hq, Hkv, N, d, window, padded):
    print(f"\nwindow B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} window={window} padded={padded}", flush=True)
    x = gen(B, Hq, Hkv, N, d, 700 + N + d, padded)
    o, lse = run(x, window)
    O, LSE = attn_fwd(x["q"], x["k"], x["v"], x["scale"], False, x["key_lens"], window=window)
    rows = np.isfinite(LSE)
    check_close("O", np64(o), O, TOL_BF16_MAX, TOL_BF16_MEAN)
    check_close("LSE", np64(lse)[rows], LSE[rows], TOL_LSE)
    assert np.all(np.isneginf(np64(lse)[~rows])) and np.all(np64(o)[~rows] == 0)


def test_key_length_shorter_than_some_windows():
    """Rows whose window lies entirely beyond key_lens[b] see nothing: O = 0, LSE = -inf."""
    x = gen(2, 2, 1, 500, 128, 31)
    x["key_lens"] = torch.tensor([100, 500], dtype=torch.int32)
    o, lse = run(x, (20, 20))
    O, LSE = attn_fwd(x["q"], x["k"], x["v"], x["scale"], False, x["key_lens"], window=(20, 20))
    assert torch.all(torch.isneginf(lse[0, :, 121:])) and torch.all(o[0, :, 121:] == 0)
    rows = np.isfinite(LSE)
    check_close("O", np64(o), O, TOL_BF16_MAX, TOL_BF16_MEAN)
    check_close("LSE", np64(lse)[rows], LSE[rows], TOL_LSE)


def test_nan_padding_never_reaches_outputs():
    x = gen(2, 2, 2, 384, 64, 32)
    x["key_lens"] = torch.tensor([200, 331], dtype=torch.int32)
    o_ref, l_ref = run(x, (50, 50))
    for b, L in enumerate([200, 331]):
        x["k"][b, :, L:] = float("nan")
        x["v"][b, :, L:] = float("nan")
    o, lse = run(x, (50, 50))
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_window_workload_sampled_rows():
    """The windowed workload in the launch configuration the bench times, sampled rows."""
    w, window = fi.WINDOW_WORKLOADS["window"]
    print(f"\nwindow workload B={w.B} H={w.Hq} N={w.N} d={w.d} window={window}", flush=True)
    x = fi.make(w)
    o, lse = run(x, window)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    r = np.random.default_rng(w.seed)
    picks = sorted({(b, h, i) for b in range(w.B) for h in (0, w.Hq - 1)
                    for i in (0, 1, 511, 512, 513, 4095, w.N - 513, w.N - 1)} |
                   {(int(r.integers(w.B)), int(r.integers(w.Hq)), int(r.integers(w.N)))
                    for _ in range(64)})
    O, LSE = attn_fwd_rows(x["q"], x["k"], x["v"], x["scale"], False, None, picks, window=window)
    idx = tuple(torch.tensor(a) for a in zip(*picks))
    check_close("O", np64(o[idx]), O, TOL_BF16_MAX, TOL_BF16_MEAN)
    check_close("LSE", np64(lse[idx]), LSE, TOL_LSE)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window,padded", [((3, 3), False), ((40, 5), True), ((0, 70), False)])
def test_very_negative_logits(d, window, padded):
    """Every scaled logit near -150 in log2 units (K close to -Q): exponentials taken against
    any reference point other than a visible score's would underflow fp32.  With a small left
    window most rows see no key in their workgroup's first steps, so the kernel must set each
    row's reference point from the first key that row actually sees."""
    B, Hq, Hkv, N = 2, 2, 1, 700
    print(f"\nwindow very negative logits d={d} window={window} padded={padded}", flush=True)
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    a = (150.0 / (scale * 1.4426950408889634 * d)) ** 0.5
    g = torch.Generator().manual_seed(91 + d + window[0])
    q = (a + 0.1 * a * torch.randn(B, Hq, N, d, generator=g)).to(torch.bfloat16)
    k = (-a + 0.1 * a * torch.randn(B, Hkv, N, d, generator=g)).to(torch.bfloat16)
    v = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16)
    kl = torch.tensor([N, 451], dtype=torch.int32) if padded else None
    x = {"q": q, "k": k, "v": v, "scale": scale, "key_lens": kl}
    o, lse = run(x, window)
    O, LSE = attn_fwd(q, k, v, scale, False, kl, window=window)
    rows = np.isfinite(LSE)
    assert np.median(LSE[rows]) < -90.0   # natural log: the logits really sit near -150 log2 units
    check_close("O", np64(o), O, TOL_BF16_MAX, TOL_BF16_MEAN)
    check_close("LSE", np64(lse)[rows], LSE[rows], TOL_LSE)
    assert np.all(np.isneginf(np64(lse)[~rows])) and np.all(np64(o)[~rows] == 0)
