"""Pure-Python attention for tiny shapes — test infrastructure only.

Scalar loops with ``math.exp``, ``math.log`` and ``math.fsum`` (exactly
rounded summation), no numpy arithmetic.  Used to check the vectorised
oracle in ``oracle/attention.py`` on shapes with N <= 16, d <= 8.

Definition followed: the standard attention of [HFL "Standard Attention
Algorithm"] — every score of a row is formed first, then the row is
normalised, then the output is the weighted sum of value rows.  Masked
(invisible) keys are left out of the row entirely, which is what an additive
-inf mask does.  Page tags are defined in ``oracle/__init__.py``.
"""

from __future__ import annotations

import math


def visible(i, j, causal, key_len, block_mask, block_size):
    if causal and j > i:
        return False
    if key_len is not None and j >= key_len:
        return False
    if block_mask is not None and not block_mask[i // block_size][j // block_size]:
        return False
    return True


def attention_head(q, k, v, scale, causal=False, key_len=None, block_mask=None,
                   block_size=128):
    """One head: q, k, v are lists of rows (lists of floats).

    Returns (O rows, lse list).  Empty rows: O = zeros, lse = -inf.
    """
    n = len(q)
    dv = len(v[0])
    out, lse = [], []
    for i in range(n):
        keys = [j for j in range(len(k))
                if visible(i, j, causal, key_len, block_mask, block_size)]
        if not keys:
            out.append([0.0] * dv)
            lse.append(-math.inf)
            continue
        s = {j: scale * math.fsum(q[i][c] * k[j][c] for c in range(len(q[i])))
             for j in keys}
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in keys}
        den = math.fsum(w.values())
        out.append([math.fsum(w[j] * v[j][c] for j in keys) / den
                    for c in range(dv)])
        lse.append(mx + math.log(den))
    return out, lse
