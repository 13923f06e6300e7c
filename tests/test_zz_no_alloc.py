"""fa_bwd_noalloc (the backward that allocates nothing, its per-row statistics in the library's
fixed device scratch) against fa_bwd on the same inputs, through the C ABI.

Both run the same three kernels on the same inputs, so the gradients must be bitwise equal
(stricter than the bf16 tolerance against the oracle).  Calls come in a row on one GPU with
different sizes, the second smaller than the first, so the scratch always holds the previous
call's statistics when a call starts.
"""
import pytest
import torch

import exact_io_aware_68_amd as fa
import fa_inputs as fi

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _pair(w):
    x = fi.make(w)
    g = {n: x[n].to(DEV) for n in ("q", "k", "v", "do")}
    kl = None if x["key_lens"] is None else x["key_lens"].to(DEV)
    o, lse = fa.fa_fwd(g["q"], g["k"], g["v"], scale=x["scale"], causal=w.causal, key_lens=kl)
    ref = fa.fa_bwd(g["q"], g["k"], g["v"], o, g["do"], lse, scale=x["scale"], causal=w.causal,
                    key_lens=kl)
    torch.cuda.synchronize()
    got = tuple(torch.full(t.shape, float("nan"), dtype=torch.float32, device=DEV) for t in ref)
    return g, kl, o, lse, x["scale"], ref, got


def _noalloc(w):
    g, kl, o, lse, scale, ref, (dq, dk, dv) = _pair(w)
    print(f"\nfa_bwd_noalloc B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal={w.causal} "
          f"key_lens={None if kl is None else kl.tolist()}", flush=True)
    fa.fa_bwd_noalloc(g["q"], g["k"], g["v"], o, g["do"], lse, dq, dk, dv, scale=scale,
                      causal=w.causal, key_lens=kl)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert torch.isfinite(a).all(), name
        assert torch.equal(a, b), f"{name} differs from fa_bwd"


def test_noalloc_matches_fa_bwd_on_calls_of_decreasing_size():
    big = fi.Workload("na1", 2, 8, 2, 1100, 128, "bf16", True, True, True, 1.0, 301)
    small = fi.Workload("na2", 1, 2, 1, 190, 64, "bf16", False, True, True, 1.0, 302)
    tiny = fi.Workload("na3", 1, 1, 1, 33, 128, "bf16", True, False, True, 1.0, 303)
    _noalloc(big)
    _noalloc(small)     # smaller than the call before: the scratch still holds big's rows
    _noalloc(tiny)
    _noalloc(big)       # and larger again


def test_noalloc_rejects_more_rows_than_the_scratch():
    q = torch.zeros(1, 64, 65537, 64, dtype=torch.bfloat16, device=DEV)   # 4194368 rows
    k = torch.zeros(1, 1, 65537, 64, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(1, 64, 65537, dtype=torch.float32, device=DEV)
    dq = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    dk = torch.empty(k.shape, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FAError) as e:
        fa.fa_bwd_noalloc(q, k, k, q, q, lse, dq, dk, dk.clone(), causal=True)
    assert e.value.status == 11
    assert fa.NOALLOC_MAX_ROWS < 64 * 65537
