"""The seeded input generator: determinism, shapes, dtypes, key-length range (CPU only)."""
import torch

import fa_inputs as fi


def test_small_workload_shapes_and_determinism():
    w = fi.WORKLOADS["c1"]
    a, b = fi.make(w), fi.make(w)
    assert a["q"].shape == (1, 1, 256, 64) and a["q"].dtype == torch.float32
    assert torch.equal(a["q"], b["q"]) and torch.equal(a["v"], b["v"])
    assert a["do"] is None and a["key_lens"] is None
    assert a["scale"] == 0.125


def test_padded_gqa_workload_small_copy():
    w = fi.WORKLOADS["c4"].with_(N=64, B=16)
    x = fi.make(w)
    assert x["q"].shape == (16, 32, 64, 128) and x["k"].shape == (16, 8, 64, 128)
    assert x["q"].dtype == torch.bfloat16
    kl = x["key_lens"]
    assert kl.dtype == torch.int32 and int(kl.min()) >= 32 and int(kl.max()) <= 64


def test_backward_draws_do_and_std():
    w = fi.WORKLOADS["c5"].with_(N=128, B=1, Hq=2, Hkv=2)
    x = fi.make(w)
    assert x["do"].shape == x["q"].shape
    w3 = fi.WORKLOADS["c3"].with_(N=512, B=1)
    s = fi.make(w3)["q"].float().std().item()
    assert 0.45 < s < 0.55                           # N(0, 1) * 0.5


def test_worked_example_shape():
    ex = fi.worked_example()
    assert ex["q"].shape == (1, 1, 4, 2) and torch.equal(ex["q"], ex["k"])
