"""CPU model of the blocked (incremental) softmax merge, fp64.

TEST INFRASTRUCTURE ONLY, and never the source of truth: ``oracle.naive`` is the definition.
This module follows the tutorial page's "Derivation: Incremental Softmax" (steps 1-3) and its
"Worked example" so that tests can pin the page's printed intermediates and check that merging
per-block statistics reproduces the two-pass definition for any split of the keys.

For one query row q and keys split into blocks, each block b yields
    m_b = max of the block's scaled scores,
    l_b = sum over the block of exp(x_j - m_b),
    Otilde_b = sum over the block of exp(x_j - m_b) v_j          (unnormalised block output),
and two summaries merge with m = max(m_1, m_2), l = e^(m_1 - m) l_1 + e^(m_2 - m) l_2,
Otilde = e^(m_1 - m) Otilde_1 + e^(m_2 - m) Otilde_2; the final row is Otilde / l.
The page states the merge for two blocks and that it extends to any number of blocks; here
blocks are folded in left to right.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .naive import to64


@dataclass
class BlockStats:
    scores: np.ndarray      # the block's scaled scores
    m: float                # block max
    exps: np.ndarray        # exp(x - m) per key of the block
    l: float                # block sum
    Otilde: np.ndarray      # unnormalised block output [d]


def block_stats(q_row, K_blk, V_blk, scale: float) -> BlockStats:
    """Statistics of one block of keys for one query row (step 2 and the block output)."""
    x = float(scale) * (to64(K_blk) @ to64(q_row))
    m = float(x.max())
    e = np.exp(x - m)
    return BlockStats(x, m, e, float(e.sum()), e @ to64(V_blk))


def merge(a: tuple, b: tuple) -> tuple:
    """Merge two (m, l, Otilde) summaries with the step-3 rescaling factors."""
    (m1, l1, o1), (m2, l2, o2) = a, b
    m = max(m1, m2)
    f1, f2 = np.exp(m1 - m), np.exp(m2 - m)
    return m, f1 * l1 + f2 * l2, f1 * o1 + f2 * o2


def blocked_row(q_row, K, V, scale: float, splits):
    """Attention for one query row with the keys cut at the indices in ``splits``.

    ``splits`` are the interior cut points (sorted, in (0, N)); returns
    (O_row, lse, [BlockStats per block], (m, l, Otilde) after the last merge).
    """
    K, V = to64(K), to64(V)
    edges = [0, *sorted(int(s) for s in splits), K.shape[0]]
    stats = [block_stats(q_row, K[a:b], V[a:b], scale) for a, b in zip(edges[:-1], edges[1:])
             if b > a]
    acc = (stats[0].m, stats[0].l, stats[0].Otilde)
    for st in stats[1:]:
        acc = merge(acc, (st.m, st.l, st.Otilde))
    m, l, Ot = acc
    return Ot / l, m + np.log(l), stats, acc
