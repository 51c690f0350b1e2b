"""Exact attention written out in numpy float64 — test infrastructure only.

This module is the oracle the HIP path is compared against.  It shares no
code with that path and imports nothing from it.  Page tags ([DEC], [HFL],
[ODP]) are defined in ``oracle/__init__.py``.

What it computes (for one batch element b and head h; tensors [B, H, N, d]):

    S   = scale * q k^T                       (materialised, [HFL "Standard
                                               Attention Algorithm"]: the
                                               standard algorithm writes S out)
    S_ij = -inf where key j is not visible to query i (the additive mask)
    P   = row softmax of S                    (each row normalised over the
                                               visible keys)
    O   = P v
    lse_i = log sum_j exp(S_ij)               (natural log; the per-row
                                               statistic the backward reuses)

The pages state that FlashAttention returns exactly this result ([DEC
"Decoding the Abstract", Sentence 4]; [ODP "The key idea"] and "Why it
mattered"), so the oracle is the plain definition, not the tiled method.

The backward is the chain rule through the row softmax (not printed on the
pages; it is what any correct backward of the definition must return): with
upstream gradient dO,

    dV = P^T dO
    dP = dO v^T
    dS_ij = P_ij * (dP_ij - sum_k P_ik dP_ik)       (softmax Jacobian)
    dQ = scale * dS k
    dK = scale * dS^T q

Rows with no visible key ("empty rows") are defined as O_i = 0,
lse_i = -inf, and they contribute nothing to any gradient.

Large sequence lengths are handled by materialising S for a chunk of query
rows at a time (each chunk holds whole rows, so the softmax is still the
plain two-pass definition, never an online update).  Sampled variants
compute the same quantities for chosen query rows or chosen key rows only.

``online_softmax_attention`` is different in kind: it is a CPU model of the
tiled method itself (running row max, running row sum, rescaling the partial
output as each key tile arrives — [ODP "The key idea"]; tiling into blocks
that fit on-chip — [DEC "Decoding the Abstract", Sentence 4]).  It exists so
that tests can check the pages' exactness claim on the CPU, independently of
any GPU code.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "allowed_mask",
    "attention_fwd",
    "attention_bwd",
    "attention_rows",
    "attention_key_grads",
    "online_softmax_attention",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def allowed_mask(rows, n_keys, causal=False, key_len=None, block_mask=None,
                 block_size=128):
    """Visibility of keys to queries for one batch element.

    Returns a bool array ``[len(rows), n_keys]``; entry (r, j) is True when
    key j is visible to query ``rows[r]``.  The mask is the additive
    {0, -inf} mask of softmax(q k^T * scale + mask):

    * causal: key j visible to query i only if j <= i (queries and keys have
      the same length, so top-left and bottom-right alignment coincide);
    * key padding: only the first ``key_len`` keys of the sequence are valid
      (``key_len`` is this batch element's valid length, or None);
    * block-sparse: attention is computed only on selected blocks of the
      score matrix ([DEC "Key Vocabulary", block-sparse attention]); block
      (i // block_size, j // block_size) of ``block_mask`` selects the pair.

    The conditions combine with AND.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(n_keys, dtype=np.int64)
    ok = np.ones((rows.size, n_keys), dtype=bool)
    if causal:
        ok &= cols[None, :] <= rows[:, None]
    if key_len is not None:
        ok &= cols[None, :] < int(key_len)
    if block_mask is not None:
        bm = np.asarray(block_mask).astype(bool)
        # expand each selected block row to block_size columns per block
        ok &= np.repeat(bm[rows // block_size], block_size, axis=1)[:, :n_keys]
    return ok


def _visible(ok):
    """Indices of the keys visible to at least one row of ``ok``.

    Leaving the other keys out of a materialised chunk changes nothing:
    their masked scores are -inf and their softmax weights exactly 0.
    """
    return np.nonzero(ok.any(axis=0))[0]


def _chunk(row_chunk, block_mask, block_size):
    # with a block mask, never mix block rows in one chunk, so that each
    # chunk only touches the key blocks its rows select
    return min(row_chunk, block_size) if block_mask is not None else row_chunk


def _row_softmax(S, ok):
    """Plain two-pass row softmax of S restricted to the visible entries.

    Returns (P, lse, nonempty).  Empty rows get P = 0 and lse = -inf.
    """
    S = np.where(ok, S, -np.inf)
    nonempty = ok.any(axis=1)
    m = np.where(nonempty, S.max(axis=1, initial=-np.inf), 0.0)
    E = np.where(ok, np.exp(S - m[:, None]), 0.0)
    den = E.sum(axis=1)
    P = np.where(nonempty[:, None], E / np.where(nonempty, den, 1.0)[:, None], 0.0)
    lse = np.where(nonempty, m + np.log(np.where(nonempty, den, 1.0)), -np.inf)
    return P, lse, nonempty


def _key_len_of(key_len, b):
    return None if key_len is None else int(np.asarray(key_len)[b])


def attention_fwd(q, k, v, scale, causal=False, key_len=None, block_mask=None,
                  block_size=128, row_chunk=1024):
    """O = softmax(scale * q k^T + mask) v and the natural-log row lse.

    ``q, k, v``: [B, H, N, d] (any float dtype; computed in float64).
    ``key_len``: None or int array [B].  Returns (O [B,H,N,d], lse [B,H,N]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    Nk = k.shape[2]                   # key count (equal to N except in tests)
    O = np.zeros((B, H, N, v.shape[-1]))
    lse = np.full((B, H, N), -np.inf)
    row_chunk = _chunk(row_chunk, block_mask, block_size)
    for b in range(B):
        L = _key_len_of(key_len, b)
        for r0 in range(0, N, row_chunk):
            rows = np.arange(r0, min(N, r0 + row_chunk))
            ok = allowed_mask(rows, Nk, causal, L, block_mask, block_size)
            idx = _visible(ok)
            for h in range(H):
                S = scale * (q[b, h, rows] @ k[b, h, idx].T)
                P, lse_r, _ = _row_softmax(S, ok[:, idx])
                O[b, h, rows] = P @ v[b, h, idx]
                lse[b, h, rows] = lse_r
    return O, lse


def attention_bwd(q, k, v, dO, scale, causal=False, key_len=None,
                  block_mask=None, block_size=128, row_chunk=1024):
    """Gradients of sum(dO * O) with respect to q, k and v.

    P is rebuilt from q and k here exactly as in the forward definition.
    Returns (dq, dk, dv), each [B, H, N, d].
    """
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    row_chunk = _chunk(row_chunk, block_mask, block_size)
    for b in range(B):
        L = _key_len_of(key_len, b)
        for r0 in range(0, N, row_chunk):
            rows = np.arange(r0, min(N, r0 + row_chunk))
            ok = allowed_mask(rows, Nk, causal, L, block_mask, block_size)
            idx = _visible(ok)
            for h in range(H):
                S = scale * (q[b, h, rows] @ k[b, h, idx].T)
                P, _, _ = _row_softmax(S, ok[:, idx])
                g = dO[b, h, rows]
                dv[b, h, idx] += P.T @ g
                dP = g @ v[b, h, idx].T
                dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                dq[b, h, rows] = scale * (dS @ k[b, h, idx])
                dk[b, h, idx] += scale * (dS.T @ q[b, h, rows])
    return dq, dk, dv


def attention_rows(q, k, v, scale, b, h, rows, dO=None, causal=False,
                   key_len=None, block_mask=None, block_size=128):
    """Forward (and dQ) for selected query rows of one (b, h).

    Each selected row is computed against all N keys, so the result equals
    the corresponding rows of :func:`attention_fwd` / :func:`attention_bwd`.
    Returns (O_rows, lse_rows, dq_rows or None).
    """
    q, k, v = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
    N = k.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    ok = allowed_mask(rows, N, causal, _key_len_of(key_len, b), block_mask,
                      block_size)
    idx = _visible(ok)
    S = scale * (q[rows] @ k[idx].T)
    P, lse_r, _ = _row_softmax(S, ok[:, idx])
    O_r = P @ v[idx]
    dq_r = None
    if dO is not None:
        g = _f64(dO[b, h])[rows]
        dP = g @ v[idx].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dq_r = scale * (dS @ k[idx])
    return O_r, lse_r, dq_r


def attention_key_grads(q, k, v, dO, scale, b, h, cols, causal=False,
                        key_len=None, block_mask=None, block_size=128,
                        row_chunk=1024):
    """dK and dV for selected key rows ``cols`` of one (b, h).

    dK_j and dV_j sum over every query row that sees key j, and each such
    row's softmax needs that row in full, so every query row that sees any
    selected key is materialised (in chunks of whole rows).  Rows that see
    none of the selected keys contribute zero and are skipped.
    Returns (dk_cols, dv_cols), each [len(cols), d].
    """
    q, k, v, g = (_f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]),
                  _f64(dO[b, h]))
    N = k.shape[0]
    cols = np.asarray(cols, dtype=np.int64)
    L = _key_len_of(key_len, b)
    dk_c = np.zeros((cols.size, k.shape[1]))
    dv_c = np.zeros((cols.size, v.shape[1]))
    row_chunk = _chunk(row_chunk, block_mask, block_size)
    for r0 in range(0, N, row_chunk):
        rows = np.arange(r0, min(N, r0 + row_chunk))
        sees = allowed_mask(rows, N, causal, L, block_mask, block_size)
        need = sees[:, cols].any(axis=1)      # rows that see a selected key
        if not need.any():
            continue
        rows, sees = rows[need], sees[need]
        idx = _visible(sees)                  # keys those rows see (full rows)
        S = scale * (q[rows] @ k[idx].T)
        P, _, _ = _row_softmax(S, sees[:, idx])
        dP = g[rows] @ v[idx].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        pos = np.searchsorted(idx, cols)
        hit = (pos < idx.size) & (idx[np.minimum(pos, idx.size - 1)] == cols)
        dk_c[hit] += scale * (dS[:, pos[hit]].T @ q[rows])
        dv_c[hit] += P[:, pos[hit]].T @ g[rows]
    return dk_c, dv_c


def online_softmax_attention(q, k, v, scale, causal=False, key_len=None,
                             block_mask=None, block_size=128, br=64, bc=64):
    """CPU float64 model of the tiled method (forward only).

    Queries are split into tiles of ``br`` rows and keys into tiles of ``bc``
    rows ([DEC "Decoding the Abstract", Sentence 4]: process blocks one at a
    time and merge the partial softmax results).  For each query tile the key
    tiles arrive in order; per query row a running maximum m and running sum
    l are kept, and the partial output is rescaled whenever m grows
    ([ODP "The key idea"]).  Nothing of size N x N exists at any time.

    Returns (O, lse) with the same conventions as :func:`attention_fwd`.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, v.shape[-1]))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        L = _key_len_of(key_len, b)
        for h in range(H):
            for i0 in range(0, N, br):
                rows = np.arange(i0, min(N, i0 + br))
                m = np.full(rows.size, -np.inf)      # running row max
                l = np.zeros(rows.size)              # running row sum
                acc = np.zeros((rows.size, v.shape[-1]))  # unnormalised O
                for j0 in range(0, N, bc):
                    cols = np.arange(j0, min(N, j0 + bc))
                    ok = allowed_mask(rows, N, causal, L, block_mask,
                                      block_size)[:, cols]
                    S = np.where(ok, scale * (q[b, h, rows] @ k[b, h, cols].T),
                                 -np.inf)
                    m_new = np.maximum(m, S.max(axis=1, initial=-np.inf))
                    # rows that have seen no visible key yet keep m = -inf;
                    # shift by 0 there so that no inf - inf is formed
                    shift = np.where(np.isfinite(m_new), m_new, 0.0)
                    alpha = np.exp(m - shift)        # exp(-inf) = 0 at start
                    Pt = np.where(ok, np.exp(S - shift[:, None]), 0.0)
                    l = alpha * l + Pt.sum(axis=1)
                    acc = alpha[:, None] * acc + Pt @ v[b, h, cols]
                    m = m_new
                seen = l > 0
                O[b, h, rows] = np.where(seen[:, None],
                                         acc / np.where(seen, l, 1.0)[:, None],
                                         0.0)
                lse[b, h, rows] = np.where(seen, m + np.log(np.where(seen, l, 1.0)),
                                           -np.inf)
    return O, lse
