"""Attention with dropout on the probabilities — test infrastructure only.

Dropout is named on the pages, with masking and softmax, as one of the
elementwise passes that dominate the time of standard attention ([HFL]
"Standard Attention Algorithm", the GPT-2 operator timing).  The pages fix
neither where the random numbers come from nor the scaling; the reading
here is the usual one:

    P   = row softmax of the masked scores (as in ``attention.py``)
    M_ij ~ Bernoulli(1 - p), independent; P~ = P * M / (1 - p)
    O   = P~ v;   lse is that of P (dropout does not change it)

and the backward is the chain rule through it (D_i = sum_c dO_ic O_ic is
still sum_j P~_ij (dO v^T)_ij):

    dV = P~^T dO;  dP = (dO v^T) * M / (1 - p);  dS = P * (dP - D)
    dQ = scale dS k;  dK = scale dS^T q

M is a function of the indices only, drawn from the counter-based
generator Philox4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC 2011), written here from
its published definition: each of 10 rounds multiplies counter words 0 and 2
by 0xD2511F53 and 0xCD9E8D57 into 64-bit products and forms the new counter
(hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key is increased by
0x9E3779B9 and 0xBB67AE85 between rounds.  One call gives four 32-bit words,
read as eight 16-bit draws (half u of word w is draw 2 w + u, low half
first).  The keys are taken 16 at a time; inside a block of 16, the 8 keys
with bit 2 of j clear share one call and the 8 with it set another:

    call  g(j) = 2 (j div 16) + (j div 4) mod 2
    draw  t(j) = 4 ((j div 8) mod 2) + j mod 4

Element (b, h, i, j) takes draw t(j) of Philox(counter = (g(j), i, b H + h,
offset), key = (seed mod 2^32, seed div 2^32)) and is kept iff that draw is
>= floor(p 2^16), so the keep probability is 1 - p to within 2^-16.  (The
grouping follows the register layout of the kernels, where a lane holds
exactly those 8 keys of one query; the pages fix no generator.)
"""

from __future__ import annotations

import numpy as np

from .attention import _f64, _key_len_of, _row_softmax, _visible, allowed_mask

__all__ = ["philox4x32_10", "drop_threshold", "draw_index", "keep_mask",
           "attention_fwd_dropout", "attention_bwd_dropout"]

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)
_LO = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 on arrays of counter words (broadcast); returns the four
    32-bit output words as uint64 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _LO for x in (c0, c1, c2, c3)]
    c0, c1, c2, c3 = np.broadcast_arrays(*c)
    k0 = np.uint64(int(k0) & 0xFFFFFFFF)
    k1 = np.uint64(int(k1) & 0xFFFFFFFF)
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & _LO
            k1 = (k1 + _W1) & _LO
        p0 = _M0 * c0
        p1 = _M1 * c2
        c0, c1, c2, c3 = ((p1 >> _S32) ^ c1 ^ k0) & _LO, p1 & _LO, \
                         ((p0 >> _S32) ^ c3 ^ k1) & _LO, p0 & _LO
    return c0, c1, c2, c3


def drop_threshold(p: float) -> int:
    """Draws below this are dropped: floor(p 2^16), at most 2^16 - 1."""
    return min(int(np.floor(float(p) * 65536.0)), 65535)


def draw_index(j):
    """(call g, draw t) of key j (module docstring)."""
    j = np.asarray(j, dtype=np.int64)
    return 2 * (j // 16) + (j // 4) % 2, 4 * ((j // 8) % 2) + j % 4


def keep_mask(rows, n_keys, bh, p, seed, offset=0):
    """bool [len(rows), n_keys]: entry (r, j) kept for query rows[r], key j
    of head index bh = b H + h."""
    rows = np.asarray(rows, dtype=np.uint64)
    g, t = draw_index(np.arange(n_keys))
    calls = np.arange(int(g.max()) + 1 if n_keys else 0, dtype=np.uint64)
    words = philox4x32_10(calls[None, :], rows[:, None], bh, offset,
                          int(seed) & 0xFFFFFFFF, int(seed) >> 32)
    w = np.stack(words, axis=-1)                      # [rows, calls, 4]
    draws = np.stack([w & np.uint64(0xFFFF), w >> np.uint64(16)], axis=-1)
    draws = draws.reshape(rows.size, calls.size, 8)   # draw 2 w + u
    return draws[:, g, t] >= np.uint64(drop_threshold(p))


def attention_fwd_dropout(q, k, v, scale, p, seed, offset=0, causal=False, key_len=None,
                          row_chunk=512):
    """(O, lse) of attention with dropout (module docstring); [B, H, N, d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    O = np.zeros((B, H, N, v.shape[-1]))
    lse = np.full((B, H, N), -np.inf)
    inv = 1.0 / (1.0 - p)
    for b in range(B):
        L = _key_len_of(key_len, b)
        for r0 in range(0, N, row_chunk):
            rows = np.arange(r0, min(N, r0 + row_chunk))
            ok = allowed_mask(rows, Nk, causal, L)
            idx = _visible(ok)
            for h in range(H):
                S = scale * (q[b, h, rows] @ k[b, h, idx].T)
                P, lse_r, _ = _row_softmax(S, ok[:, idx])
                Mk = keep_mask(rows, Nk, b * H + h, p, seed, offset)[:, idx]
                O[b, h, rows] = (P * Mk * inv) @ v[b, h, idx]
                lse[b, h, rows] = lse_r
    return O, lse


def attention_bwd_dropout(q, k, v, dO, scale, p, seed, offset=0, causal=False, key_len=None,
                          row_chunk=512):
    """(dq, dk, dv) of sum(dO * O) for attention with dropout."""
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    inv = 1.0 / (1.0 - p)
    for b in range(B):
        L = _key_len_of(key_len, b)
        for r0 in range(0, N, row_chunk):
            rows = np.arange(r0, min(N, r0 + row_chunk))
            ok = allowed_mask(rows, Nk, causal, L)
            idx = _visible(ok)
            for h in range(H):
                S = scale * (q[b, h, rows] @ k[b, h, idx].T)
                P, _, _ = _row_softmax(S, ok[:, idx])
                Mk = keep_mask(rows, Nk, b * H + h, p, seed, offset)[:, idx] * inv
                Pd = P * Mk
                g = dO[b, h, rows]
                O = Pd @ v[b, h, idx]
                Drow = (g * O).sum(axis=1, keepdims=True)
                dv[b, h, idx] += Pd.T @ g
                dP = (g @ v[b, h, idx].T) * Mk
                dS = P * (dP - Drow)
                dq[b, h, rows] = scale * (dS @ k[b, h, idx])
                dk[b, h, idx] += scale * (dS.T @ q[b, h, rows])
    return dq, dk, dv
