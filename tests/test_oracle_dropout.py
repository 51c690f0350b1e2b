"""Pins of the dropout oracle (oracle/dropout.py) — CPU only.

* Philox4x32-10 reproduces the known-answer vectors published with the
  generator (Random123 distribution, Salmon et al., SC 2011).
* p = 0 keeps every probability: the dropout oracle equals the plain
  definition bit for bit.
* Gradients: central finite differences of sum(dO * O) with the mask held
  fixed, and torch.autograd in float64 over softmax(...) * M / (1 - p) @ v.
* The mask: kept fraction within binomial bounds of 1 - p, different
  seeds / offsets / heads give different masks, and averaging O over many
  masks approaches the dropout-free O (the 1/(1 - p) scaling).
* The draw map: every (call, draw) pair of a 16-key block is used exactly
  once, and the vectorised mask agrees element by element with a scalar
  reading of one generator call per element.
"""

import numpy as np
import pytest

from oracle import (attention_bwd, attention_bwd_dropout, attention_fwd, attention_fwd_dropout,
                    drop_threshold, keep_mask, philox4x32_10)
from oracle.dropout import draw_index


def test_philox_known_answers():
    # (counter, key) -> output, from the published known-answer vectors
    cases = [
        ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
        ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF),
         (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
        ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
         (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
    ]
    for ctr, key, want in cases:
        got = philox4x32_10(*ctr, *key)
        assert tuple(int(x) for x in got) == want


def inputs(N=9, d=4, B=1, H=2, seed=3):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)) for _ in range(4)]


@pytest.mark.parametrize("causal", [False, True])
def test_zero_rate_is_plain_attention(causal):
    q, k, v, dO = inputs(N=37, d=8)
    O, lse = attention_fwd_dropout(q, k, v, 0.3, 0.0, seed=5, causal=causal)
    O0, lse0 = attention_fwd(q, k, v, 0.3, causal=causal)
    np.testing.assert_array_equal(O, O0)
    np.testing.assert_array_equal(lse, lse0)
    g = attention_bwd_dropout(q, k, v, dO, 0.3, 0.0, seed=5, causal=causal)
    g0 = attention_bwd(q, k, v, dO, 0.3, causal=causal)
    for a, b in zip(g, g0):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_finite_differences(causal):
    q, k, v, dO = inputs()
    p, seed, off = 0.25, 1234567890123, 7
    dq, dk, dv = attention_bwd_dropout(q, k, v, dO, 0.5, p, seed, off, causal=causal)

    def loss(qq, kk, vv):
        O, _ = attention_fwd_dropout(qq, kk, vv, 0.5, p, seed, off, causal=causal)
        return float((O * dO).sum())

    eps = 1e-6
    for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[i] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_against_torch_autograd_fp64():
    import torch
    q, k, v, dO = inputs(N=33, d=8, B=2, H=2)
    p, seed = 0.4, 99
    B, H, N, _ = q.shape
    M = np.stack([np.stack([keep_mask(np.arange(N), N, b * H + h, p, seed)
                            for h in range(H)]) for b in range(B)])
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    causal = torch.ones(N, N, dtype=torch.bool).tril()
    S = (tq @ tk.transpose(-1, -2)) * 0.35
    S = S.masked_fill(~causal, float("-inf"))
    P = torch.softmax(S, dim=-1)
    O = (P * torch.tensor(M, dtype=torch.float64) / (1 - p)) @ tv
    O.backward(torch.tensor(dO))
    Oo, _ = attention_fwd_dropout(q, k, v, 0.35, p, seed, causal=True)
    np.testing.assert_allclose(Oo, O.detach().numpy(), rtol=0, atol=1e-12)
    g = attention_bwd_dropout(q, k, v, dO, 0.35, p, seed, causal=True)
    for a, t in zip(g, (tq, tk, tv)):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=0, atol=1e-11)


def test_mask_statistics_and_independence():
    p = 0.3
    m = keep_mask(np.arange(512), 512, 3, p, seed=2024)
    n = m.size
    kept = m.mean()
    assert abs(kept - (1 - p)) < 5 * np.sqrt(p * (1 - p) / n)
    assert drop_threshold(p) == int(np.floor(0.3 * 2 ** 16))
    assert drop_threshold(0.0) == 0 and drop_threshold(0.999999) == 65535
    # every other index changes the mask
    for other in (keep_mask(np.arange(512), 512, 3, p, seed=2025),
                  keep_mask(np.arange(512), 512, 3, p, seed=2024, offset=1),
                  keep_mask(np.arange(512), 512, 4, p, seed=2024)):
        assert 0.3 < (other != m).mean() < 0.5   # ~2 p (1 - p) = 0.42
    # neighbouring rows and key groups are not copies of each other
    assert (m[1:] != m[:-1]).mean() > 0.3 and (m[:, 4:] != m[:, :-4]).mean() > 0.3


def test_mean_over_masks_is_the_dropout_free_output():
    q, k, v, _ = inputs(N=6, d=3, B=1, H=1)
    p, n = 0.5, 3000
    acc = np.zeros((1, 1, 6, 3))
    for off in range(n):
        O, _ = attention_fwd_dropout(q, k, v, 0.5, p, seed=11, offset=off)
        acc += O
    O0, _ = attention_fwd(q, k, v, 0.5)
    # each entry is a mean of n draws with std <= max|v| / sqrt(n) * sqrt(p/(1-p))
    tol = 5 * np.abs(v).max() * np.sqrt(p / (1 - p) / n)
    np.testing.assert_allclose(acc / n, O0, rtol=0, atol=tol)


def test_draw_map_is_a_bijection_per_16_keys():
    g, t = draw_index(np.arange(16 * 7))
    pairs = set(zip(g.tolist(), t.tolist()))
    assert len(pairs) == 16 * 7                          # no (call, draw) used twice
    assert set(g.tolist()) == set(range(14)) and set(t.tolist()) == set(range(8))
    # the 8 keys of a call: one 16-key block, one value of bit 2
    for call in range(14):
        js = np.nonzero(g == call)[0]
        assert len(js) == 8 and len(set((js // 16).tolist())) == 1
        assert len(set(((js >> 2) & 1).tolist())) == 1


def test_mask_matches_one_call_per_element():
    p, seed, off, bh = 0.37, (0xDEADBEEF << 32) | 0x12345, 5, 6
    rows, nk = np.array([0, 3, 1000]), 45
    m = keep_mask(rows, nk, bh, p, seed, off)
    th = drop_threshold(p)
    for r, i in enumerate(rows):
        for j in range(nk):
            g, t = (int(x) for x in draw_index(j))
            w = philox4x32_10(g, int(i), bh, off, seed & 0xFFFFFFFF, seed >> 32)
            word = int(w[t // 2])
            draw = (word >> 16) if t % 2 else (word & 0xFFFF)
            assert m[r, j] == (draw >= th), (i, j)
