"""Seeded synthetic inputs for the attention workloads.

This module is shared by the tests, the bench and the smoke check, and by both sides of every
parity comparison (the HIP path and the CPU oracle).  It draws random numbers and casts them;
it holds none of the attention arithmetic.

Recipe (the same for every workload): a CPU ``torch.Generator`` seeded with the workload's seed
draws, in this order, Q, K, V, then dO (backward workloads), then the per-batch key lengths
(padded workloads).  Q, K, V and dO are iid N(0, 1) in fp32, multiplied by the workload's
standard deviation, then rounded to the workload dtype (bf16: round to nearest even).  Key
lengths are integers drawn uniformly from [N // 2, N] inclusive.  The softmax scale is the fp32
value of 1 / sqrt(d).  No public dataset is involved: the pages measure nothing on one, and these
shapes are the attention workloads themselves.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    padded: bool        # per-batch key lengths drawn from [N // 2, N]
    backward: bool      # dO drawn, gradients checked
    std: float
    seed: int

    @property
    def scale(self) -> float:
        """fp32 value of 1/sqrt(d), returned as a Python float."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # single head, fp32, forward O only
    "c1": Workload("c1", 1, 1, 1, 256, 64, "f32", False, False, False, 1.0, 1),
    # bf16 forward, non-causal
    "c2": Workload("c2", 4, 16, 16, 2048, 64, "bf16", False, False, False, 1.0, 2),
    # bf16 causal forward at N = 8192, d = 128 (the timed shape; the backward is timed on it too)
    "c3": Workload("c3", 2, 16, 16, 8192, 128, "bf16", True, False, False, 0.5, 3),
    # grouped-query causal forward with per-batch key padding
    "c4": Workload("c4", 4, 32, 8, 16384, 128, "bf16", True, True, False, 1.0, 4),
    # causal backward with recomputation
    "c5": Workload("c5", 2, 16, 16, 4096, 128, "bf16", True, False, True, 1.0, 5),
}

# Local-window workloads: the timed causal shape (c3) with a window instead of the causal mask.
# window = (left, right): row i sees keys i - left .. i + right.
WINDOW_WORKLOADS = {
    "window": (Workload("window", 2, 16, 16, 8192, 128, "bf16", False, False, False, 0.5, 7),
               (512, 512)),
}

# Block-sparse workloads: a shape and the recipe of its bitmap (see ``block_bitmap``).
SPARSE_WORKLOADS = {
    "sparse": (Workload("sparse", 2, 16, 16, 8192, 128, "bf16", False, False, False, 0.5, 8),
               0.2),
}


def block_bitmap(N: int, density: float, seed: int, band: int = 2, bq: int = 128,
                 bk: int = 64) -> torch.Tensor:
    """uint8 [ceil(N/bq), ceil(N/bk)] bitmap: the key blocks within ``band`` blocks of each query
    block's diagonal, plus every other block independently with probability ``density`` (CPU
    generator seeded with ``seed``)."""
    nq, nk = -(-N // bq), -(-N // bk)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    bm = (torch.rand(nq, nk, generator=g) < density)
    qb = torch.arange(nq)[:, None] * (bq // bk)
    kb = torch.arange(nk)[None, :]
    bm |= (kb >= qb - band) & (kb <= qb + (bq // bk) - 1 + band)
    return bm.to(torch.uint8)


_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def make(w: Workload, want_do: bool | None = None) -> dict:
    """Generate the workload's tensors on the CPU.

    Returns a dict with q [B,Hq,N,d], k, v [B,Hkv,N,d] in the workload dtype, ``do`` (like q,
    when the workload has a backward or ``want_do``), ``key_lens`` (int32 [B] or None) and
    ``scale`` (float).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    dt = _TORCH_DTYPE[w.dtype]

    def draw(*shape):
        return (torch.randn(*shape, generator=g, dtype=torch.float32) * w.std).to(dt)

    out = {
        "q": draw(w.B, w.Hq, w.N, w.d),
        "k": draw(w.B, w.Hkv, w.N, w.d),
        "v": draw(w.B, w.Hkv, w.N, w.d),
        "do": None,
        "key_lens": None,
        "scale": w.scale,
    }
    if w.backward if want_do is None else want_do:
        out["do"] = draw(w.B, w.Hq, w.N, w.d)
    if w.padded:
        out["key_lens"] = torch.randint(w.N // 2, w.N + 1, (w.B,), generator=g,
                                        dtype=torch.int32)
    return out


def make_on_device(w: Workload, device) -> dict:
    """The same recipe drawn by a seeded generator on ``device``, for workloads too large to
    draw on the host (tensors of more than 2^31 elements).  The values differ from ``make``'s for
    the same seed (another generator), but are drawn the same way: Q, K, V iid N(0, 1) times the
    workload's standard deviation, rounded to its dtype, then the key lengths (padded workloads)."""
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    dt = _TORCH_DTYPE[w.dtype]

    def draw(*shape):
        t = torch.empty(*shape, dtype=dt, device=device)
        for i in range(shape[0]):   # one batch at a time: the fp32 draw is 2x the bf16 tensor
            t[i] = (torch.randn(*shape[1:], generator=g, dtype=torch.float32, device=device)
                    * w.std).to(dt)
        return t

    out = {"q": draw(w.B, w.Hq, w.N, w.d), "k": draw(w.B, w.Hkv, w.N, w.d),
           "v": draw(w.B, w.Hkv, w.N, w.d), "do": None, "key_lens": None, "scale": w.scale}
    if w.backward:
        out["do"] = draw(w.B, w.Hq, w.N, w.d)
    if w.padded:
        out["key_lens"] = torch.randint(w.N // 2, w.N + 1, (w.B,), generator=g, dtype=torch.int32,
                                        device=device)
    return out


@dataclass(frozen=True)
class DecodeWorkload:
    """Decode shape: Nq query rows per q-head against Nk cached keys per kv-head."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    padded: bool        # per-batch key lengths drawn from [Nk // 2, Nk]
    std: float
    seed: int

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))


DECODE_WORKLOADS = {
    # one new token per sequence against a 16k-key cache, with the grouped heads and key padding of
    # the grouped-query forward workload (c4)
    "decode": DecodeWorkload("decode", 4, 32, 8, 1, 16384, 128, True, 1.0, 6),
}


def make_decode(w: DecodeWorkload) -> dict:
    """Same recipe as ``make``: Q [B,Hq,Nq,d], then K, V [B,Hkv,Nk,d] (bf16), then key lengths
    uniform in [Nk // 2, Nk] when padded."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)

    def draw(*shape):
        return (torch.randn(*shape, generator=g, dtype=torch.float32) * w.std).to(torch.bfloat16)

    out = {"q": draw(w.B, w.Hq, w.Nq, w.d), "k": draw(w.B, w.Hkv, w.Nk, w.d),
           "v": draw(w.B, w.Hkv, w.Nk, w.d), "key_lens": None, "scale": w.scale}
    if w.padded:
        out["key_lens"] = torch.randint(w.Nk // 2, w.Nk + 1, (w.B,), generator=g,
                                        dtype=torch.int32)
    return out


def make_decode_on_device(w: DecodeWorkload, device) -> dict:
    """``make_decode``'s recipe drawn by a seeded generator on ``device`` (for caches of more than
    2^31 elements); the values differ from ``make_decode``'s for the same seed."""
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)

    def draw(*shape):
        t = torch.empty(*shape, dtype=torch.bfloat16, device=device)
        for i in range(shape[0]):
            t[i] = (torch.randn(*shape[1:], generator=g, dtype=torch.float32, device=device)
                    * w.std).to(torch.bfloat16)
        return t

    out = {"q": draw(w.B, w.Hq, w.Nq, w.d), "k": draw(w.B, w.Hkv, w.Nk, w.d),
           "v": draw(w.B, w.Hkv, w.Nk, w.d), "key_lens": None, "scale": w.scale}
    if w.padded:
        out["key_lens"] = torch.randint(w.Nk // 2, w.Nk + 1, (w.B,), generator=g,
                                        dtype=torch.int32, device=device)
    return out


def worked_example() -> dict:
    """The tutorial page's worked example (N = 4, d = 2): Q = K, V as printed, scale 1/sqrt(2)."""
    q = torch.tensor([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [0.0, 0.0]])
    v = torch.tensor([[1.0, 1.0], [2.0, 0.0], [0.0, 2.0], [1.0, 1.0]])
    return {"q": q.reshape(1, 1, 4, 2), "k": q.clone().reshape(1, 1, 4, 2),
            "v": v.reshape(1, 1, 4, 2), "scale": float(torch.tensor(1 / math.sqrt(2.0)))}
