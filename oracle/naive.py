"""Plain fp64 CPU oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY. This module defines what the attention path must compute; it is
imported by the tests, by ``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py``,
and by nothing else. The HIP library never imports, links or calls it, and it shares no code,
table or constant with the HIP path.

What it computes (sources are the three pages on FlashAttention):

* Standard attention ("The Standard Attention Problem", tutorial page): scores S = Q K^T,
  probabilities P = softmax of the scaled scores, output O = P V.  The caller's ``scale``
  multiplies the dot product (the page divides by sqrt(d_k); the configs pass 1/sqrt(d)).
* Safe softmax (tutorial page, "Derivation: Incremental Softmax", step 1): subtract the row
  maximum before exponentiating.  This module is the plain two-pass form of that definition:
  pass 1 takes the row max over the valid keys, pass 2 sums the shifted exponentials.  The
  online/blocked form is NOT used here; ``oracle.blocked`` models it separately so that tests can
  compare the two.
* Masks: the guide page ("Tiling through SRAM") lists causal masks, padding and grouped-query
  attention as tiling details that leave the result definition unchanged; the tutorial page adds
  a local attention window ("Other Efficient Attention Variants").  Readings taken where the
  pages are silent:
    - causal is top-left aligned: query i sees keys j <= i;
    - padding is a per-batch key length L_b: keys j >= L_b are invisible to every query of batch b,
      query rows are still computed;
    - grouped-query heads use contiguous groups: q-head h reads kv-head h * Hkv // Hq;
    - a row with no visible key has O = 0 and LSE = -inf, and contributes no gradient;
    - a local window (left, right) lets row i see keys i - left .. i + right; the page's window
      w (odd) is left = right = (w - 1) / 2.
* Saved metadata (guide page, "Tiling through SRAM": a little softmax metadata is written in
  training): read as the natural-log log-sum-exp of each row's scaled, masked scores,
  LSE_i = m_i + ln(sum_j exp(s_ij - m_i)).
* Backward (tutorial page, "Backward Pass: Recomputation"; the pages give no formulas): the
  vector-Jacobian product of O with respect to Q, K, V contracted with dO, written out from the
  softmax derivative:
      dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P * (dP - D),
      dQ = scale * dS K,  dK = scale * dS^T Q,
  and, with grouped-query heads, dK and dV of a kv-head are summed over its q-heads.

Inputs are widened exactly to float64 (bf16 and fp32 values are exactly representable), so the
oracle sees the same numbers as the GPU.  Keys beyond L_b are sliced away before any arithmetic,
so padding rows may hold anything (NaN included).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "to64", "kv_head_of", "visible_mask", "attn_fwd", "attn_fwd_rows",
    "attn_bwd", "attn_bwd_heads", "attn_dq_rows", "score_rows", "attn_decode",
]


def to64(x) -> np.ndarray:
    """Widen a numpy array or a torch tensor (any float dtype, any device) to float64 exactly."""
    if hasattr(x, "detach"):  # torch tensor; imported lazily so numpy-only callers need no torch
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """Contiguous grouped-query map: q-heads [g*G, (g+1)*G) read kv-head g, with G = Hq // Hkv."""
    return (h * Hkv) // Hq


def visible_mask(rows: np.ndarray, L: int, causal: bool, window=None,
                 block_mask=None) -> np.ndarray:
    """Boolean [len(rows), L]: key j is visible to query row i iff j < L and (not causal or j <= i)
    and, with window = (left, right), i - left <= j <= i + right (a negative side is unbounded).

    The window is the tutorial page's local attention window ("Other Efficient Attention
    Variants", worked example: w = 3 lets each token see itself and one neighbour on each side,
    i.e. left = right = (w - 1) / 2).

    With block_mask = (bm, bq, bk), key j is visible to row i only if bm[i // bq][j // bk] is
    nonzero: a tile-level bitmap over (query block, key block) pairs.  The study-note page
    ("FlashAttention paper", What it does not claim) names block-sparse attention as a separate
    extension and defines nothing more; the reading here is the plainest one, an element mask
    that is constant on blocks, combined with the other masks."""
    j = np.arange(L)[None, :]
    i = np.asarray(rows)[:, None]
    vis = np.ones((len(rows), L), dtype=bool)
    if causal:
        vis &= j <= i
    if window is not None:
        left, right = window
        if left >= 0:
            vis &= j >= i - left
        if right >= 0:
            vis &= j <= i + right
    if block_mask is not None:
        bm, bq, bk = block_mask
        bm = np.asarray(bm) != 0
        vis &= bm[np.asarray(rows)[:, None] // bq, j // bk]
    return vis


def _softmax_vjp(P: np.ndarray, dP: np.ndarray) -> np.ndarray:
    """Softmax derivative contracted row by row: dS = P * (dP - D) with D_i = sum_j P_ij dP_ij
    (rows of P over the visible keys; invisible entries have P = 0 and get dS = 0)."""
    D = (P * dP).sum(axis=1)
    return P * (dP - D[:, None])


def _lens(key_lens, B: int, N: int) -> list[int]:
    if key_lens is None:
        return [N] * B
    kl = [int(x) for x in (key_lens.tolist() if hasattr(key_lens, "tolist") else key_lens)]
    if len(kl) != B or any(l < 0 or l > N for l in kl):
        raise ValueError("key_lens must hold B integers in [0, N]")
    return kl


def score_rows(q_rows: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Scaled scores s_ij = scale * <q_i, k_j> for a block of query rows (fp64 matmul)."""
    return float(scale) * (q_rows @ K.T)


def _softmax_rows(s: np.ndarray, vis: np.ndarray):
    """Two-pass safe softmax over the visible entries of each row.

    Returns (P, m, l) where P has zeros at invisible entries; rows with no visible key get
    P = 0, m = -inf, l = 0.
    """
    masked = np.where(vis, s, -np.inf)
    m = masked.max(axis=1) if masked.shape[1] else np.full(masked.shape[0], -np.inf)
    has = np.isfinite(m)
    shift = np.where(has, m, 0.0)
    e = np.where(vis, np.exp(np.where(vis, s, 0.0) - shift[:, None]), 0.0)   # pass 2
    l = e.sum(axis=1)
    P = np.zeros_like(e)
    P[has] = e[has] / l[has, None]
    return P, m, l


def attn_fwd(q, k, v, scale: float, causal: bool = False, key_lens=None,
             heads=None, chunk: int = 1024, window=None, block_mask=None):
    """Exact attention forward.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (any float type, widened to fp64).
    Returns (O [B, Hq, N, d] fp64, LSE [B, Hq, N] fp64, natural log).
    ``heads``: optional iterable of (b, h) pairs to compute; other entries stay O = 0, LSE = nan.
    ``chunk``: query rows per block; chunking over query rows does not change any row's math.
    ``window``: optional (left, right) local window, see ``visible_mask``.
    ``block_mask``: optional (bm, bq, bk) tile-level bitmap, see ``visible_mask``.
    """
    q, k, v = to64(q), to64(k), to64(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    lens = _lens(key_lens, B, N)
    O = np.zeros((B, Hq, N, v.shape[-1]))     # value width may differ from the key width
    LSE = np.full((B, Hq, N), np.nan)
    todo = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    for b, h in todo:
        g = kv_head_of(h, Hq, Hkv)
        L = lens[b]
        K, V = k[b, g, :L], v[b, g, :L]
        for r0 in range(0, N, chunk):
            rows = np.arange(r0, min(N, r0 + chunk))
            s = score_rows(q[b, h, rows], K, scale)
            P, m, l = _softmax_rows(s, visible_mask(rows, L, causal, window, block_mask))
            O[b, h, rows] = P @ V
            with np.errstate(divide="ignore"):
                LSE[b, h, rows] = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)),
                                           -np.inf)
    return O, LSE


def attn_decode(q, k, v, scale: float, key_lens=None):
    """Decode-shaped forward: Nq query rows per head against Nk keys, Nq and Nk independent.

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d].  Every query row of batch b sees the keys j < L_b
    (L_b = key_lens[b], default Nk) and no causal mask applies: the rows stand for new tokens
    attending to a cache of L_b keys.  The guide page ("FlashAttention", Key takeaways) says
    decode wants another mapping of the same math; the mask reading is this module's.
    Returns (O [B, Hq, Nq, d], LSE [B, Hq, Nq]), fp64.
    """
    q, k, v = to64(q), to64(k), to64(v)
    B, Hq, Nq, _ = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    lens = _lens(key_lens, B, Nk)
    O = np.zeros((B, Hq, Nq, v.shape[-1]))
    LSE = np.zeros((B, Hq, Nq))
    rows = np.arange(Nq)
    for b in range(B):
        L = lens[b]
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            K, V = k[b, g, :L], v[b, g, :L]
            s = score_rows(q[b, h], K, scale)
            P, m, l = _softmax_rows(s, visible_mask(rows, L, False))
            O[b, h] = P @ V
            with np.errstate(divide="ignore"):
                LSE[b, h] = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return O, LSE


def attn_fwd_rows(q, k, v, scale: float, causal: bool, key_lens, picks, window=None,
                  block_mask=None):
    """Forward for individual rows: ``picks`` is a list of (b, h, i).

    Returns (O_rows [len(picks), d], LSE_rows [len(picks)]).  Each row is computed on its own from
    the definition, so this scales to full-size workloads where only sampled rows are checked.
    Inputs may be torch tensors; only the needed rows are widened.
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    lens = _lens(key_lens, B, N)
    O = np.zeros((len(picks), v.shape[-1]))
    LSE = np.zeros(len(picks))
    cache = {}
    for n, (b, h, i) in enumerate(picks):
        g = kv_head_of(h, Hq, Hkv)
        L = lens[b]
        if (b, g) not in cache:
            cache[(b, g)] = (to64(k[b, g, :L]), to64(v[b, g, :L]))
        K, V = cache[(b, g)]
        s = score_rows(to64(q[b, h, i:i + 1]), K, scale)
        P, m, l = _softmax_rows(s, visible_mask(np.array([i]), L, causal, window, block_mask))
        O[n] = (P @ V)[0]
        LSE[n] = m[0] + np.log(l[0]) if np.isfinite(m[0]) else -np.inf
    return O, LSE


def attn_dq_rows(q, k, v, do, scale: float, causal: bool, key_lens, picks):
    """dQ of individual query rows: ``picks`` is a list of (b, h, i); returns [len(picks), d].

    dQ_i needs only row i of P and of dP (the softmax derivative is row-wise): with
    P_i = softmax(scale q_i K^T) over the visible keys, dP_i = dO_i V^T and D_i = sum_j P_ij dP_ij,
    dQ_i = scale * sum_j P_ij (dP_ij - D_i) K_j.  Each row costs O(N d), so full-size workloads
    can be checked on sampled rows.  A row with no visible key gets dQ_i = 0.
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    lens = _lens(key_lens, B, N)
    out = np.zeros((len(picks), d))
    cache = {}
    for n, (b, h, i) in enumerate(picks):
        g = kv_head_of(h, Hq, Hkv)
        L = lens[b]
        if (b, g) not in cache:
            cache[(b, g)] = (to64(k[b, g, :L]), to64(v[b, g, :L]))
        K, V = cache[(b, g)]
        s = score_rows(to64(q[b, h, i:i + 1]), K, scale)
        P, m, _ = _softmax_rows(s, visible_mask(np.array([i]), L, causal))
        if not np.isfinite(m[0]):
            continue
        dP = to64(do[b, h, i:i + 1]) @ V.T
        out[n] = float(scale) * (_softmax_vjp(P, dP) @ K)[0]
    return out


def attn_bwd(q, k, v, do, scale: float, causal: bool = False, key_lens=None,
             kv_heads=None, chunk: int = 1024):
    """Exact attention backward (softmax VJP), recomputing P from Q, K, V.

    Returns (dQ [B,Hq,N,d], dK [B,Hkv,N,d], dV [B,Hkv,N,d]) in fp64.  Keys beyond L_b get zero
    gradient.  ``kv_heads``: optional iterable of (b, g) kv-head pairs to compute (all q-heads of
    each group are included); other entries stay 0.
    """
    q, k, v, do = to64(q), to64(k), to64(v), to64(do)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    lens = _lens(key_lens, B, N)
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    todo = [(b, g) for b in range(B) for g in range(Hkv)] if kv_heads is None else list(kv_heads)
    for b, g in todo:
        L = lens[b]
        K, V = k[b, g, :L], v[b, g, :L]
        for h in range(g * G, (g + 1) * G):
            for r0 in range(0, N, chunk):
                rows = np.arange(r0, min(N, r0 + chunk))
                s = score_rows(q[b, h, rows], K, scale)
                P, _, _ = _softmax_rows(s, visible_mask(rows, L, causal))
                dO = do[b, h, rows]
                dP = dO @ V.T
                dS = _softmax_vjp(P, dP)
                dQ[b, h, rows] = scale * (dS @ K)
                dK[b, g, :L] += scale * (dS.T @ q[b, h, rows])
                dV[b, g, :L] += P.T @ dO
    return dQ, dK, dV


def attn_bwd_heads(q, k, v, do, scale: float, causal: bool, key_lens, kv_picks):
    """Backward restricted to the kv-heads in ``kv_picks`` [(b, g), ...], widening only those
    slices (for sampled checks of full-size workloads).

    Returns a dict {(b, g): (dQ [G, N, d] for the group's q-heads, dK [N, d], dV [N, d])}.
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = {}
    for b, g in kv_picks:
        kl = None if key_lens is None else [int(key_lens[b])]
        sl = slice(g * G, (g + 1) * G)
        dQ, dK, dV = attn_bwd(q[b:b + 1, sl], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                              do[b:b + 1, sl], scale, causal, kl)
        out[(b, g)] = (dQ[0], dK[0, 0], dV[0, 0])
    return out
