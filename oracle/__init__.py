"""fp64 CPU oracle for exact softmax attention — TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The HIP library and its Python binding never do; the two share no code.

* ``naive``   — the definition: two-pass safe softmax attention, forward and backward.
* ``blocked`` — a CPU model of the pages' blocked merge, used only to pin the worked example's
                intermediates and the merge identity.  Never used as truth.
* ``fd``      — central finite differences of the forward, to pin the analytic backward.

Every function here is pinned by the ``-m "not gpu"`` tests against values the pages print,
closed forms, invariants, an independent library routine and brute force.
"""
from .naive import (attn_bwd, attn_bwd_heads, attn_decode, attn_dq_rows, attn_fwd,  # noqa: F401
                    attn_fwd_rows, kv_head_of, score_rows, to64, visible_mask)
