"""Attention at q = 0 in closed form, at any size — test infrastructure only.

With q = 0 every visible score is 0, so each row of P is uniform over the
n_i keys that query i sees (the softmax of a constant row), and attention
reduces to means (the definition written out in ``attention.py``; [DEC
"Decoding the Abstract", Sentence 4]: the method returns exactly that
result):

    O_i   = (1 / n_i) sum_{j visible} v_j
    lse_i = ln n_i
    dV_j  = sum_{i: j visible to i} dO_i / n_i
    dQ_i  = (scale / n_i) (dO_i^T A_i - (dO_i . O_i) ksum_i),
            A_i = sum_{j visible} v_j k_j^T,  ksum_i = sum_{j visible} k_j
    dK    = scale dS^T q = 0

(dQ is scale sum_j P_ij (dP_ij - D_i) k_j with dP_ij = dO_i . v_j and
D_i = dO_i . O_i.)  Causal and key-padding masks make the visible keys of
row i a prefix j <= min(i, L_b - 1), so running sums over j give every row
in O(N d^2); a block mask makes them a union of key blocks, so per-block
sums do.  Empty rows: O = 0, lse = -inf, no gradient.  This gives exact
references for the GPU at the full workload sizes, where the materialising
oracle can only be sampled.
"""

from __future__ import annotations

import numpy as np

__all__ = ["q_zero_attention"]


def _prefix_head(k, v, dO, scale, L, causal, chunk=512):
    N, d = k.shape
    O = np.zeros((N, d))
    lse = np.full(N, -np.inf)
    dq = np.zeros((N, d))
    dv = np.zeros((N, d))
    if L <= 0:
        return O, lse, dq, dv
    rows = np.arange(N)
    last = np.minimum(rows, L - 1) if causal else np.full(N, L - 1)  # last visible key
    n = (last + 1).astype(np.float64)
    vsum = np.cumsum(v, axis=0)
    ksum = np.cumsum(k, axis=0)
    O = vsum[last] / n[:, None]
    lse = np.log(n)
    D = (dO * O).sum(1)
    # t_i = dO_i^T A_i with A_i = sum_{j <= last_i} v_j k_j^T
    if not causal:
        t = dO @ (v[:L].T @ k[:L])
    else:  # one chunk of rows at a time; A holds the keys before the chunk
        t = np.zeros((N, d))
        A = np.zeros((d, d))
        for r0 in range(0, N, chunk):
            r1 = min(N, r0 + chunk)
            lo, hi = min(r0, L), min(r1, L)
            t[r0:r1] = dO[r0:r1] @ A
            if hi > lo:
                js = np.arange(lo, hi)
                W = (dO[r0:r1] @ v[lo:hi].T) * (js[None, :] <= last[r0:r1, None])
                t[r0:r1] += W @ k[lo:hi]
                A += v[lo:hi].T @ k[lo:hi]
    dq = (scale / n)[:, None] * (t - D[:, None] * ksum[last])
    # dV_j = sum_{i: last_i >= j} dO_i / n_i (every row i >= j sees key j < L)
    g = dO / n[:, None]
    if causal:
        rev = np.cumsum(g[::-1], axis=0)[::-1]
        dv[:L] = rev[:L]
    else:
        dv[:L] = g.sum(0)
    return O, lse, dq, dv


def _block_head(k, v, dO, scale, bm, bs):
    N, d = k.shape
    nb = (N + bs - 1) // bs
    bm = np.asarray(bm, dtype=bool)[:nb, :nb]
    size = np.array([min(bs, N - c * bs) for c in range(nb)], dtype=np.float64)
    vb = np.stack([v[c * bs:(c + 1) * bs].sum(0) for c in range(nb)])
    kb = np.stack([k[c * bs:(c + 1) * bs].sum(0) for c in range(nb)])
    Ab = np.stack([v[c * bs:(c + 1) * bs].T @ k[c * bs:(c + 1) * bs] for c in range(nb)])
    n_r = bm.astype(np.float64) @ size
    O = np.zeros((N, d))
    lse = np.full(N, -np.inf)
    dq = np.zeros((N, d))
    dv = np.zeros((N, d))
    G = np.zeros((nb, d))  # sum over the rows of block r of dO_i / n_r
    for r in range(nb):
        if n_r[r] == 0:
            continue
        sl = slice(r * bs, min(N, (r + 1) * bs))
        sel = np.nonzero(bm[r])[0]
        Or = vb[sel].sum(0) / n_r[r]
        O[sl] = Or
        lse[sl] = np.log(n_r[r])
        A = Ab[sel].sum(0)
        D = dO[sl] @ Or
        dq[sl] = (scale / n_r[r]) * (dO[sl] @ A - D[:, None] * kb[sel].sum(0)[None, :])
        G[r] = dO[sl].sum(0) / n_r[r]
    colg = bm.T.astype(np.float64) @ G  # [nb, d]: what each key block receives
    for c in range(nb):
        dv[c * bs:(c + 1) * bs] = colg[c]
    return O, lse, dq, dv


def q_zero_attention(k, v, dO, scale, causal=False, key_len=None, block_mask=None,
                     block_size=128):
    """(O, lse, dq, dk, dv) of attention with q = 0; k, v, dO [B, H, N, d].
    key_len: per-batch visible key count (keys j >= key_len[b] hidden);
    block_mask: [nb, nb] shared by every (b, h), not combined with the other
    masks."""
    k, v, dO = (np.asarray(t, dtype=np.float64) for t in (k, v, dO))
    B, H, N, d = k.shape
    O = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    dq = np.zeros((B, H, N, d))
    dv = np.zeros((B, H, N, d))
    for b in range(B):
        L = N if key_len is None else int(min(max(int(key_len[b]), 0), N))
        for h in range(H):
            if block_mask is not None:
                r = _block_head(k[b, h], v[b, h], dO[b, h], scale, block_mask, block_size)
            else:
                r = _prefix_head(k[b, h], v[b, h], dO[b, h], scale, L, causal)
            O[b, h], lse[b, h], dq[b, h], dv[b, h] = r
    return O, lse, dq, np.zeros_like(k), dv
