"""Every output of every entry point is written, and nothing around it: outputs and workspaces
are views into larger buffers filled with NaN (or 0xFF bytes); after the call the outputs are
finite and the guard regions are untouched.  Ragged shapes, grouped heads and key lengths, so
the tail tiles and the masked paths all run."""
import pytest
import torch

import exact_io_aware_68_amd as fa
import fa_inputs as fi

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
G = 1024   # guard elements on each side


def guarded(shape, dtype):
    n = 1
    for s in shape:
        n *= s
    buf = torch.full((n + 2 * G,), float("nan"), dtype=dtype, device=DEV)
    return buf, buf[G:G + n].view(*shape)


def guards_intact(buf):
    return bool(torch.isnan(buf[:G]).all() and torch.isnan(buf[-G:]).all())


def inputs(B, Hq, Hkv, N, d, seed, lens):
    w = fi.Workload("t", B, Hq, Hkv, N, d, "bf16", True, False, True, 1.0, seed)
    x = fi.make(w)
    g = {n: x[n].to(DEV) for n in ("q", "k", "v", "do")}
    g["key_lens"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
    g["scale"] = x["scale"]
    return g


def test_backward_outputs_and_workspace():
    B, Hq, Hkv, N, d = 2, 4, 2, 190, 128
    x = inputs(B, Hq, Hkv, N, d, 21, [190, 77])
    o, lse = fa.fa_fwd(x["q"], x["k"], x["v"], scale=x["scale"], causal=True,
                       key_lens=x["key_lens"])
    qb, dq = guarded((B, Hq, N, d), torch.float32)
    kb, dk = guarded((B, Hkv, N, d), torch.float32)
    vb, dv = guarded((B, Hkv, N, d), torch.float32)
    nws = fa.fa_bwd_workspace_size(B, Hq, N)
    wsb = torch.full((nws + 2 * G,), 0xFF, dtype=torch.uint8, device=DEV)
    ws = wsb[G:G + nws]
    fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, scale=x["scale"], causal=True,
              key_lens=x["key_lens"], dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    assert (dk[1, :, 77:] == 0).all() and (dv[1, :, 77:] == 0).all()   # keys past the length
    for b in (qb, kb, vb):
        assert guards_intact(b)
    assert (wsb[:G] == 0xFF).all() and (wsb[-G:] == 0xFF).all()


def test_window_outputs():
    B, Hq, Hkv, N, d = 2, 4, 2, 333, 128
    x = inputs(B, Hq, Hkv, N, d, 22, [333, 150])
    ob, o = guarded((B, Hq, N, d), torch.bfloat16)
    lb, lse = guarded((B, Hq, N), torch.float32)
    fa.fa_fwd_window(x["q"], x["k"], x["v"], window=(70, 5), scale=x["scale"],
                     key_lens=x["key_lens"], o=o, lse=lse)
    torch.cuda.synchronize()
    # rows past the key length plus the left width see no key: O = 0 and LSE = -inf there
    assert torch.isfinite(o).all() and not torch.isnan(lse).any()
    assert torch.isneginf(lse[1, :, 150 + 70:]).all() and (o[1, :, 150 + 70:] == 0).all()
    assert guards_intact(ob) and guards_intact(lb)


def test_blocksparse_outputs():
    B, Hq, Hkv, N, d = 2, 4, 2, 333, 128
    x = inputs(B, Hq, Hkv, N, d, 23, [333, 200])
    bm = fi.block_bitmap(N, 0.3, 23).to(DEV)
    ob, o = guarded((B, Hq, N, d), torch.bfloat16)
    lb, lse = guarded((B, Hq, N), torch.float32)
    fa.fa_fwd_blocksparse(x["q"], x["k"], x["v"], bm, scale=x["scale"], causal=True,
                          key_lens=x["key_lens"], o=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and not torch.isnan(lse).any()
    assert guards_intact(ob) and guards_intact(lb)


def test_splitkv_outputs_and_workspace():
    w = fi.DecodeWorkload("t", 3, 8, 2, 3, 1000, 128, False, 1.0, 24)
    x = fi.make_decode(w)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    kl = torch.tensor([1000, 333, 1], dtype=torch.int32, device=DEV)
    ob, o = guarded((w.B, w.Hq, w.Nq, w.d), torch.bfloat16)
    lb, lse = guarded((w.B, w.Hq, w.Nq), torch.float32)
    nws = fa.fa_fwd_splitkv_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)
    wsb = torch.full((nws + 2 * G,), 0xFF, dtype=torch.uint8, device=DEV)
    fa.fa_fwd_splitkv(q, k, v, scale=x["scale"], key_lens=kl, o=o, lse=lse,
                      workspace=wsb[G:G + nws])
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert guards_intact(ob) and guards_intact(lb)
    assert (wsb[:G] == 0xFF).all() and (wsb[-G:] == 0xFF).all()


def test_variants_are_bitwise_deterministic():
    """No atomics anywhere: repeated calls give identical bits (window, block-sparse, split-KV
    with several ranges)."""
    x = inputs(2, 4, 2, 333, 128, 25, [333, 201])
    bm = fi.block_bitmap(333, 0.3, 25).to(DEV)
    runs = []
    for _ in range(2):
        a = fa.fa_fwd_window(x["q"], x["k"], x["v"], window=(40, 40), scale=x["scale"],
                             key_lens=x["key_lens"])
        b = fa.fa_fwd_blocksparse(x["q"], x["k"], x["v"], bm, scale=x["scale"], causal=True,
                                  key_lens=x["key_lens"])
        c = fa.fa_fwd_splitkv(x["q"][:, :, :3].contiguous(), x["k"], x["v"], scale=x["scale"],
                              key_lens=x["key_lens"], num_splits=3)
        torch.cuda.synchronize()
        runs.append([t.clone() for t in (*a, *b, *c)])
    for t1, t2 in zip(*runs):
        assert torch.equal(t1, t2)
