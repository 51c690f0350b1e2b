"""Pins for the fp64 oracle (CPU only).

Each test fixes the oracle to something other than itself: a hand-derived
worked example, closed forms, invariants that any correct attention must
satisfy, special cases that reduce to textbook results, finite differences,
a library implementation (torch autograd in float64 on the CPU), and the
tiled online-softmax model of the method.  Page tags as in
``oracle/__init__.py``.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import bruteforce
from oracle.closed_forms import q_zero_attention
from oracle.attention import (allowed_mask, attention_bwd, attention_fwd,
                              attention_key_grads, attention_rows,
                              online_softmax_attention)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


MASKS = [
    dict(),
    dict(causal=True),
    dict(key_len=np.array([5, 11])),
    dict(causal=True, key_len=np.array([1, 7])),
]


# --------------------------------------------------------------------------
# hand-worked example (tests/golden/hand_worked.json)
# --------------------------------------------------------------------------

def test_hand_worked_example():
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        qf = case.get("q_factor", 1.0)
        q = np.array(g["q"])[None, None] * qf
        k = np.array(g["k"])[None, None]
        v = np.array(g["v"])[None, None]
        kl = None if case["key_len"] is None else np.array([case["key_len"]])
        O, lse = attention_fwd(q, k, v, case["scale"], causal=case["causal"], key_len=kl)
        np.testing.assert_allclose(O[0, 0], case["O"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, 0], case["lse"], rtol=0, atol=1e-14)
        if "dO" in case:
            dO = np.array(case["dO"])[None, None]
            dq, dk, dv = attention_bwd(q, k, v, dO, case["scale"], causal=case["causal"], key_len=kl)
            np.testing.assert_allclose(dq[0, 0], case["dq"], rtol=0, atol=1e-14)
            np.testing.assert_allclose(dk[0, 0], case["dk"], rtol=0, atol=1e-14)
            np.testing.assert_allclose(dv[0, 0], case["dv"], rtol=0, atol=1e-14)
        On, lsen = online_softmax_attention(q, k, v, case["scale"], causal=case["causal"],
                                            key_len=kl, br=2, bc=2)
        np.testing.assert_allclose(On[0, 0], case["O"], rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# P1 normalisation, P2 constant values, P3 argmax routing + mask correctness
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mask", MASKS)
def test_rows_of_P_sum_to_one(mask):
    # With v = identity (d = N), O is P itself.
    B, H, N = 2, 2, 13
    q, k = rnd((B, H, N, 8), 1), rnd((B, H, N, 8), 2)
    v = np.broadcast_to(np.eye(N), (B, H, N, N))
    O, _ = attention_fwd(q, k, v, 0.7, **mask)
    for b in range(B):
        ok = allowed_mask(np.arange(N), N, mask.get("causal", False),
                          None if "key_len" not in mask else mask["key_len"][b])
        for h in range(H):
            assert np.all(O[b, h][~ok] == 0.0)          # no weight through the mask
            s = O[b, h].sum(axis=1)
            np.testing.assert_allclose(s[ok.any(1)], 1.0, rtol=0, atol=1e-14 * N)
            assert np.all(O[b, h] >= 0)


@pytest.mark.parametrize("mask", MASKS)
def test_constant_value_rows(mask):
    B, H, N, d = 2, 3, 11, 5
    q, k = rnd((B, H, N, d), 3), rnd((B, H, N, d), 4)
    c = rnd((d,), 5)
    v = np.broadcast_to(c, (B, H, N, d)).copy()
    O, _ = attention_fwd(q, k, v, 0.5, **mask)
    np.testing.assert_allclose(O, np.broadcast_to(c, O.shape), rtol=0, atol=1e-14)


def test_dominant_key_routes_its_value_and_masks_block_it():
    N, d = 12, 4
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, N, d)) * 0.1
    k = rng.standard_normal((1, 1, N, d)) * 0.1
    v = rng.standard_normal((1, 1, N, d))
    i, jstar = 5, 3
    q[0, 0, i] = [10.0, 0, 0, 0]
    k[0, 0, jstar] = [10.0, 0, 0, 0]         # S_{i,j*} = 100 * scale, others ~ 0.1
    O, _ = attention_fwd(q, k, v, 1.0)
    np.testing.assert_allclose(O[0, 0, i], v[0, 0, jstar], rtol=0, atol=1e-30)  # other weights <= N e^-80
    # the same dominant key hidden by causality (j* > i) must have no effect:
    q2 = q.copy(); k2 = k.copy()
    i2, j2 = 2, 9
    q2[0, 0, i2] = [10.0, 0, 0, 0]
    k2[0, 0, j2] = [10.0, 0, 0, 0]
    Oc, _ = attention_fwd(q2, k2, v, 1.0, causal=True)
    # reference: row i2 computed over keys 0..i2 only by brute force
    ob, _ = bruteforce.attention_head(q2[0, 0].tolist(), k2[0, 0, :i2 + 1].tolist(),
                                      v[0, 0, :i2 + 1].tolist(), 1.0)
    np.testing.assert_allclose(Oc[0, 0, i2], ob[i2], rtol=0, atol=1e-14)
    assert np.abs(Oc[0, 0, i2] - v[0, 0, j2]).max() > 0.1
    # and hidden by key padding (j* >= key_len)
    Op, _ = attention_fwd(q2, k2, v, 1.0, key_len=np.array([j2]))
    ob2, _ = bruteforce.attention_head(q2[0, 0].tolist(), k2[0, 0, :j2].tolist(),
                                       v[0, 0, :j2].tolist(), 1.0)
    np.testing.assert_allclose(Op[0, 0], np.array(ob2), rtol=0, atol=1e-14)


def test_causal_row0_and_keylen1():
    B, H, N, d = 2, 2, 9, 6
    q, k, v = rnd((B, H, N, d), 7), rnd((B, H, N, d), 8), rnd((B, H, N, d), 9)
    s = 0.3
    O, lse = attention_fwd(q, k, v, s, causal=True)
    np.testing.assert_array_equal(O[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], s * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=0, atol=1e-15)
    O1, lse1 = attention_fwd(q, k, v, s, key_len=np.array([1, 1]))
    np.testing.assert_array_equal(O1, np.broadcast_to(v[:, :, :1], O1.shape))


# --------------------------------------------------------------------------
# P5 brute force on tiny shapes (all mask kinds)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N,d", [(1, 1), (2, 3), (7, 4), (16, 8)])
@pytest.mark.parametrize("kind", ["none", "causal", "pad", "causal_pad", "block"])
def test_bruteforce(N, d, kind):
    q, k, v = rnd((1, 1, N, d), 10), rnd((1, 1, N, d), 11), rnd((1, 1, N, d), 12)
    kw = {}
    if kind in ("causal", "causal_pad"):
        kw["causal"] = True
    if kind in ("pad", "causal_pad"):
        kw["key_len"] = np.array([max(1, N // 2)])
    bs = 4
    if kind == "block":
        nb = (N + bs - 1) // bs
        bm = (np.random.default_rng(13).random((nb, nb)) < 0.6).astype(np.uint8)
        bm[0, 0] = 1
        kw.update(block_mask=bm, block_size=bs)
    O, lse = attention_fwd(q, k, v, 0.9, **kw)
    ob, lb = bruteforce.attention_head(
        q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.9,
        causal=kw.get("causal", False),
        key_len=None if "key_len" not in kw else int(kw["key_len"][0]),
        block_mask=None if "block_mask" not in kw else kw["block_mask"].tolist(),
        block_size=bs)
    np.testing.assert_allclose(O[0, 0], np.array(ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.array(lb), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# P6 finite differences, P7 torch autograd (float64, CPU)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mask", MASKS[:3])
def test_backward_finite_differences(mask):
    B, H, N, d = 2, 1, 7, 3
    q, k, v, dO = (rnd((B, H, N, d), s) for s in (20, 21, 22, 23))
    s = 0.8
    dq, dk, dv = attention_bwd(q, k, v, dO, s, **mask)

    def loss(q_, k_, v_):
        O, _ = attention_fwd(q_, k_, v_, s, **mask)
        return float((O * dO).sum())

    eps = 1e-6
    for name, X, G in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = dict(q_=q, k_=k, v_=v)
            args_m = dict(q_=q, k_=k, v_=v)
            args_p[name + "_"] = Xp
            args_m[name + "_"] = Xm
            num[idx] = (loss(**args_p) - loss(**args_m)) / (2 * eps)
        np.testing.assert_allclose(G, num, rtol=1e-6, atol=1e-7, err_msg=name)


def _torch_ref(q, k, v, dO, scale, causal=False, key_len=None, block_mask=None, block_size=128):
    torch = pytest.importorskip("torch")
    B, H, N, d = q.shape
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    add = torch.zeros(B, 1, N, N, dtype=torch.float64)
    i = torch.arange(N)
    for b in range(B):
        m = torch.ones(N, N, dtype=torch.bool)
        if causal:
            m &= i[None, :] <= i[:, None]
        if key_len is not None:
            m &= i[None, :] < int(key_len[b])
        if block_mask is not None:
            bm = torch.tensor(np.asarray(block_mask).astype(bool))
            m &= bm[(i // block_size)[:, None], (i // block_size)[None, :]]
        add[b, 0][~m] = -math.inf
    S = scale * (tq @ tk.transpose(-1, -2)) + add
    P = torch.softmax(S, dim=-1)
    empty = torch.isinf(S).all(-1, keepdim=True)
    P = torch.where(empty, torch.zeros_like(P), P)
    O = P @ tv
    lse = torch.logsumexp(S, dim=-1)
    O.backward(torch.tensor(dO, dtype=torch.float64))
    return (O.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(),
            tv.grad.numpy())


@pytest.mark.parametrize("mask", MASKS + [dict(block_mask=np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], np.uint8),
                                               block_size=16)])
def test_against_torch_autograd_fp64(mask):
    B, H, N, d = 2, 3, 40, 16
    q, k, v, dO = (rnd((B, H, N, d), s) for s in (30, 31, 32, 33))
    s = 1 / math.sqrt(d)
    O, lse = attention_fwd(q, k, v, s, **mask)
    dq, dk, dv = attention_bwd(q, k, v, dO, s, **mask)
    tO, tl, tdq, tdk, tdv = _torch_ref(q, k, v, dO, s, **mask)
    for a, b_ in ((O, tO), (lse, tl), (dq, tdq), (dk, tdk), (dv, tdv)):
        fin = np.isfinite(b_)
        np.testing.assert_array_equal(np.isfinite(a), fin)
        np.testing.assert_allclose(a[fin], b_[fin], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P8 closed forms at q = 0 (any N, any mask)
# --------------------------------------------------------------------------

def q0_closed_forms(k, v, dO, scale, ok):
    """q = 0 -> every visible key has weight 1/n_i (textbook: softmax of a
    constant row is uniform)."""
    n = ok.sum(1).astype(np.float64)
    W = ok / np.where(n > 0, n, 1)[:, None]
    O = W @ v
    lse = np.where(n > 0, np.log(np.where(n > 0, n, 1)), -np.inf)
    dv = W.T @ dO
    D = (dO * O).sum(1)
    dP = dO @ v.T
    dq = scale * ((W * (dP - D[:, None])) @ k)
    return O, lse, dv, dq


@pytest.mark.parametrize("mask", MASKS + [dict(block_mask=np.eye(4, dtype=np.uint8), block_size=8)])
def test_q_zero_closed_forms(mask):
    B, H, N, d = 2, 2, 29, 6
    q = np.zeros((B, H, N, d))
    k, v, dO = rnd((B, H, N, d), 40), rnd((B, H, N, d), 41), rnd((B, H, N, d), 42)
    s = 0.37
    O, lse = attention_fwd(q, k, v, s, **mask)
    dq, dk, dv = attention_bwd(q, k, v, dO, s, **mask)
    np.testing.assert_array_equal(dk, 0.0)
    for b in range(B):
        ok = allowed_mask(np.arange(N), N, mask.get("causal", False),
                          None if "key_len" not in mask else mask["key_len"][b],
                          mask.get("block_mask"), mask.get("block_size", 128))
        for h in range(H):
            cO, cl, cdv, cdq = q0_closed_forms(k[b, h], v[b, h], dO[b, h], s, ok)
            np.testing.assert_allclose(O[b, h], cO, atol=1e-13)
            np.testing.assert_allclose(lse[b, h], cl, atol=1e-13)
            np.testing.assert_allclose(dv[b, h], cdv, atol=1e-13)
            np.testing.assert_allclose(dq[b, h], cdq, atol=1e-13)


def test_q_zero_causal_prefix_means():
    # causal + q = 0: O_i is the running mean of v_0..v_i, lse_i = ln(i + 1)
    N, d = 50, 3
    v = rnd((1, 1, N, d), 43)
    O, lse = attention_fwd(np.zeros((1, 1, N, d)), rnd((1, 1, N, d), 44), v, 1.0, causal=True)
    np.testing.assert_allclose(O[0, 0], np.cumsum(v[0, 0], 0) / np.arange(1, N + 1)[:, None],
                               atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, N + 1)), atol=1e-14)


# --------------------------------------------------------------------------
# P9 invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mask", MASKS)
def test_invariants(mask):
    B, H, N, d = 2, 2, 33, 8
    q, k, v, dO = (rnd((B, H, N, d), s) for s in (50, 51, 52, 53))
    q *= 2.0
    s = 0.6
    O, lse = attention_fwd(q, k, v, s, **mask)
    dq, dk, dv = attention_bwd(q, k, v, dO, s, **mask)
    for b in range(B):
        ok = allowed_mask(np.arange(N), N, mask.get("causal", False),
                          None if "key_len" not in mask else mask["key_len"][b])
        ne = ok.any(1)
        for h in range(H):
            # sum_j dK_j = 0 (rows of dS sum to zero); sum_j dV_j = sum of dO over non-empty rows
            np.testing.assert_allclose(dk[b, h].sum(0), 0.0, atol=1e-12)
            np.testing.assert_allclose(dv[b, h].sum(0), dO[b, h][ne].sum(0), atol=1e-12)
            # O in the box spanned by the visible value rows
            for i in np.nonzero(ne)[0]:
                vv = v[b, h][ok[i]]
                assert np.all(O[b, h, i] >= vv.min(0) - 1e-12)
                assert np.all(O[b, h, i] <= vv.max(0) + 1e-12)
            S = s * q[b, h] @ k[b, h].T
            Smax = np.where(ok, S, -np.inf).max(1)
            n = ok.sum(1)
            assert np.all(lse[b, h][ne] >= Smax[ne] - 1e-12)
            assert np.all(lse[b, h][ne] <= Smax[ne] + np.log(n[ne]) + 1e-12)
            assert np.all(np.isneginf(lse[b, h][~ne]))


# --------------------------------------------------------------------------
# P10 block-sparse semantics, P11 padding semantics, P12 permutations
# --------------------------------------------------------------------------

def test_block_sparse_semantics():
    B, H, N, d, bs = 1, 2, 40, 8, 8
    q, k, v, dO = (rnd((B, H, N, d), s) for s in (60, 61, 62, 63))
    nb = N // bs
    # same row chunks on both sides -> the same arithmetic, bit for bit
    dense_O, dense_l = attention_fwd(q, k, v, 0.4, row_chunk=bs)
    O1, l1 = attention_fwd(q, k, v, 0.4, block_mask=np.ones((nb, nb), np.uint8), block_size=bs)
    np.testing.assert_array_equal(O1, dense_O)
    np.testing.assert_array_equal(l1, dense_l)
    g_dense = attention_bwd(q, k, v, dO, 0.4, row_chunk=bs)
    g_ones = attention_bwd(q, k, v, dO, 0.4, block_mask=np.ones((nb, nb), np.uint8), block_size=bs)
    for a, b_ in zip(g_dense, g_ones):
        np.testing.assert_array_equal(a, b_)
    # identity block mask == independent attention inside each block
    Oi, li = attention_fwd(q, k, v, 0.4, block_mask=np.eye(nb, dtype=np.uint8), block_size=bs)
    for t in range(nb):
        sl = slice(t * bs, (t + 1) * bs)
        Ot, lt = attention_fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.4)
        np.testing.assert_allclose(Oi[:, :, sl], Ot, atol=1e-14)
        np.testing.assert_allclose(li[:, :, sl], lt, atol=1e-14)


def test_key_padding_semantics():
    B, H, N, d = 2, 2, 21, 5
    q, k, v, dO = (rnd((B, H, N, d), s) for s in (70, 71, 72, 73))
    Of, lf = attention_fwd(q, k, v, 0.5, key_len=np.array([N, N]))
    O0, l0 = attention_fwd(q, k, v, 0.5)
    np.testing.assert_array_equal(Of, O0)
    L = np.array([6, 13])
    Op, lp = attention_fwd(q, k, v, 0.5, key_len=L)
    gp = attention_bwd(q, k, v, dO, 0.5, key_len=L)
    for b in range(B):
        Ot, lt = attention_fwd(q[b:b + 1], k[b:b + 1, :, :L[b]], v[b:b + 1, :, :L[b]], 0.5)
        np.testing.assert_allclose(Op[b], Ot[0], atol=1e-14)
        gt = attention_bwd(q[b:b + 1], k[b:b + 1, :, :L[b]], v[b:b + 1, :, :L[b]], dO[b:b + 1], 0.5)
        np.testing.assert_allclose(gp[0][b], gt[0][0], atol=1e-13)
        np.testing.assert_allclose(gp[1][b, :, :L[b]], gt[1][0], atol=1e-13)
        np.testing.assert_array_equal(gp[1][b, :, L[b]:], 0.0)
        np.testing.assert_array_equal(gp[2][b, :, L[b]:], 0.0)


def test_permutation_structure():
    N, d = 17, 6
    q, k, v = rnd((1, 1, N, d), 80), rnd((1, 1, N, d), 81), rnd((1, 1, N, d), 82)
    O, l = attention_fwd(q, k, v, 0.45)
    pk = np.random.default_rng(83).permutation(N)
    Ok, lk = attention_fwd(q, k[:, :, pk], v[:, :, pk], 0.45)
    np.testing.assert_allclose(Ok, O, atol=1e-14)
    np.testing.assert_allclose(lk, l, atol=1e-14)
    pq = np.random.default_rng(84).permutation(N)
    Oq, lq = attention_fwd(q[:, :, pq], k, v, 0.45)
    np.testing.assert_allclose(Oq, O[:, :, pq], atol=1e-14)


# --------------------------------------------------------------------------
# P13 the tiled online-softmax method equals the definition
# --------------------------------------------------------------------------

@pytest.mark.parametrize("br,bc", [(1, 1), (3, 3), (16, 16), (128, 128), (16, 3), (5, 64)])
@pytest.mark.parametrize("mask", MASKS + [dict(block_mask=np.array([[0, 1, 0], [0, 0, 1], [1, 1, 1]], np.uint8),
                                               block_size=16)])
def test_online_softmax_model_is_exact(br, bc, mask):
    B, H, N, d = 2, 1, 45, 8           # ragged against every tile size
    q, k, v = rnd((B, H, N, d), 90) * 3, rnd((B, H, N, d), 91), rnd((B, H, N, d), 92)
    O, lse = attention_fwd(q, k, v, 0.5, **mask)
    Ot, lt = online_softmax_attention(q, k, v, 0.5, br=br, bc=bc, **mask)
    np.testing.assert_allclose(Ot, O, rtol=0, atol=1e-13)
    fin = np.isfinite(lse)
    np.testing.assert_array_equal(np.isfinite(lt), fin)
    np.testing.assert_allclose(lt[fin], lse[fin], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# sampled variants equal the full computation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mask", MASKS[:3] + [dict(block_mask=np.eye(3, dtype=np.uint8) | np.eye(3, k=1, dtype=np.uint8),
                                                   block_size=16)])
def test_sampled_rows_and_keys(mask):
    B, H, N, d = 2, 2, 45, 8
    q, k, v, dO = (rnd((B, H, N, d), s) for s in (100, 101, 102, 103))
    O, lse = attention_fwd(q, k, v, 0.3, **mask, row_chunk=7)
    dq, dk, dv = attention_bwd(q, k, v, dO, 0.3, **mask, row_chunk=11)
    O2, lse2 = attention_fwd(q, k, v, 0.3, **mask)
    np.testing.assert_allclose(O, O2, atol=1e-14)
    rows = [0, 4, 44, 17]
    cols = [0, 44, 9, 30]
    for b in range(B):
        for h in range(H):
            Or, lr, dqr = attention_rows(q, k, v, 0.3, b, h, rows, dO=dO, **mask)
            np.testing.assert_allclose(Or, O[b, h, rows], atol=1e-14)
            np.testing.assert_allclose(lr, lse[b, h, rows], atol=1e-14)
            np.testing.assert_allclose(dqr, dq[b, h, rows], atol=1e-13)
            dkc, dvc = attention_key_grads(q, k, v, dO, 0.3, b, h, cols, **mask, row_chunk=10)
            np.testing.assert_allclose(dkc, dk[b, h, cols], atol=1e-13)
            np.testing.assert_allclose(dvc, dv[b, h, cols], atol=1e-13)


def test_empty_rows_are_zero():
    # a block mask with an all-zero block row leaves those queries empty
    N, d, bs = 24, 4, 8
    q, k, v, dO = (rnd((1, 1, N, d), s) for s in (110, 111, 112, 113))
    bm = np.ones((3, 3), np.uint8)
    bm[1, :] = 0
    O, lse = attention_fwd(q, k, v, 1.0, block_mask=bm, block_size=bs)
    dq, dk, dv = attention_bwd(q, k, v, dO, 1.0, block_mask=bm, block_size=bs)
    assert np.all(O[0, 0, 8:16] == 0) and np.all(np.isneginf(lse[0, 0, 8:16]))
    assert np.all(dq[0, 0, 8:16] == 0)
    # the empty rows' dO must not leak into dV
    dO2 = dO.copy()
    dO2[0, 0, 8:16] = 1e3
    _, _, dv2 = attention_bwd(q, k, v, dO2, 1.0, block_mask=bm, block_size=bs)
    np.testing.assert_array_equal(dv2, dv)


def test_oracle_is_independent_of_the_product():
    # neither side imports the other (static check of the sources)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for f in os.listdir(os.path.join(root, "oracle")):
        if f.endswith(".py"):
            src = open(os.path.join(root, "oracle", f)).read()
            assert "io_aware_tiled_05_amd" not in src and "import torch" not in src
    pkg = os.path.join(root, "io_aware_tiled_05_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
    assert oracle.attention_fwd is attention_fwd


@pytest.mark.parametrize("key_len", [None, 5, 0])
def test_decode_shape_fewer_queries_than_keys(key_len):
    # Nq != Nk (decode: a few queries against a longer key sequence, no
    # causal order): the vectorised oracle equals pure-Python loops, and
    # equals the same rows of the square problem
    rng = np.random.default_rng(31)
    q = rng.standard_normal((1, 2, 13, 8))
    k = rng.standard_normal((1, 2, 13, 8))
    v = rng.standard_normal((1, 2, 13, 8))
    kl = None if key_len is None else np.array([key_len])
    rows = [0, 7, 12]
    O, lse = attention_fwd(q[:, :, rows], k, v, 0.35, key_len=kl)
    for h in range(2):
        ob, lb = bruteforce.attention_head(q[0, h, rows].tolist(), k[0, h].tolist(),
                                           v[0, h].tolist(), 0.35, key_len=key_len)
        np.testing.assert_allclose(O[0, h], np.array(ob), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], np.array(lb), rtol=0, atol=1e-12)
    Of, lf = attention_fwd(q, k, v, 0.35, key_len=kl)
    np.testing.assert_array_equal(O, Of[:, :, rows])
    np.testing.assert_array_equal(lse, lf[:, :, rows])


# --------------------------------------------------------------------------
# P8 at scale: the running-sum closed forms used for the full-size GPU checks
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mask", MASKS + [dict(causal=True, key_len=np.array([5, 0])),
                                          dict(block_mask=(np.eye(9, k=1, dtype=np.uint8)
                                                           + np.tri(9, k=-2, dtype=np.uint8))
                                               * (np.arange(9) != 4)[:, None].astype(np.uint8),
                                               block_size=128)])
def test_q_zero_running_sum_forms_equal_the_definition(mask):
    # the O(N d^2) forms in oracle/closed_forms.py (chunked running sums,
    # per-block sums) against the materialising definition at q = 0, on a
    # length with several chunks and a ragged last block
    B, H, N, d = 2, 2, 1100, 5
    k, v, dO = rnd((B, H, N, d), 60), rnd((B, H, N, d), 61), rnd((B, H, N, d), 62)
    q = np.zeros((B, H, N, d))
    kw = {key: val for key, val in mask.items() if key != "block_size"}
    if "key_len" in kw and len(kw["key_len"]) != B:
        kw["key_len"] = kw["key_len"][:B]
    O, lse = attention_fwd(q, k, v, 0.3, **mask)
    dq, dk, dv = attention_bwd(q, k, v, dO, 0.3, **mask)
    cO, cl, cdq, cdk, cdv = q_zero_attention(k, v, dO, 0.3, **kw)
    np.testing.assert_array_equal(np.isfinite(cl), np.isfinite(lse))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(cl[fin], lse[fin], atol=1e-12)
    for a, b_ in ((cO, O), (cdq, dq), (cdk, dk), (cdv, dv)):
        np.testing.assert_allclose(a, b_, atol=1e-11)
