"""Central finite differences of the oracle forward, fp64, for tiny gradient checks.

TEST INFRASTRUCTURE ONLY.  The scalar loss is L = sum(O * dO); its gradient with respect to each
input element is estimated by (L(x + h) - L(x - h)) / (2h), straight from the definition of the
derivative, so it pins ``oracle.naive.attn_bwd`` without sharing any of its algebra.
"""
from __future__ import annotations

import numpy as np

from .naive import attn_fwd, to64


def numeric_grads(q, k, v, do, scale: float, causal: bool = False, key_lens=None,
                  h: float = 1e-6):
    """Return (dQ, dK, dV) estimated by central differences of sum(attn_fwd(...)[0] * do)."""
    q, k, v, do = (to64(t).copy() for t in (q, k, v, do))

    def loss():
        O, _ = attn_fwd(q, k, v, scale, causal, key_lens)
        return float((O * do).sum())

    grads = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        flat, gflat = x.reshape(-1), g.reshape(-1)
        for n in range(flat.size):
            keep = flat[n]
            flat[n] = keep + h
            up = loss()
            flat[n] = keep - h
            dn = loss()
            flat[n] = keep
            gflat[n] = (up - dn) / (2 * h)
        grads.append(g)
    return tuple(grads)
