"""Dropout parity: fa_fwd_dropout / fa_bwd_dropout (through the C ABI) vs
the fp64 dropout oracle (oracle/dropout.py, pinned in
test_oracle_dropout.py), which draws the same Philox4x32-10 mask from the
element indices.  The mask is exact on both sides (integer words compared
with the same integer threshold), so any difference is rounding.

Tolerance: the plain path's (fp16 1e-2, bf16 2e-2) divided by 1 - p, on
|error| / max(1, |reference|).  The backward takes O as the forward stored
it, in the input dtype, and D = sum_c dO_c O_c inherits that rounding;
dropout multiplies O's kept terms, and with them the rounding error that D
and every dS carry, by 1 / (1 - p).  (A CPU emulation of only the bf16 O
entering D reaches 1.96e-2 on dK for p = 0.1, d = 128, N = 129, causal,
against 9.4e-3 without dropout; the fp16 rounding of dS adds 4e-3.)
Outputs above 1 are compared relative to their size.
"""

import numpy as np
import pytest

from helpers import TOL, to_dev, to_np
from oracle import attention_bwd_dropout, attention_fwd_dropout
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

SEED = (0x1234_5678 << 32) | 0x9ABC_DEF1   # both key words non-zero


def tol(dtype, p):
    return TOL[dtype] / (1.0 - p)


def assert_close(name, got, ref, tol):
    # max |error| / max(1, |ref|): outputs and gradients can exceed 8 at
    # p = 0.5, where a bf16 store alone errs by more than 2e-2
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), "non-finite pattern differs"
    e = float((np.abs(got[fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin]))).max()) \
        if fin.any() else 0.0
    print(f"  {name}: max|err|/max(1,|ref|) = {e:.3e} (tol {tol:g})", flush=True)
    assert e <= tol, f"{name}: {e:.3e} > {tol:g}"


@pytest.fixture(scope="module")
def fa():
    import io_aware_tiled_05_amd as fa
    fa.load()
    return fa


def inputs(dtype, N, d, B=2, H=3, seed=17):
    return make_inputs(Workload("drop", B, H, N, d, dtype, seed=seed))


def run(fa, x, dtype, p, seed, offset, causal=False, key_len=None):
    import torch
    q, k, v, dO = (to_dev(x[n], dtype) for n in ("q", "k", "v", "dO"))
    kl = None if key_len is None else torch.tensor(key_len, dtype=torch.int32, device="cuda:0")
    o, lse = fa.fa_fwd_dropout(q, k, v, p, seed, offset, scale=x["scale"], causal=causal,
                               key_len=kl)
    dq, dk, dv = fa.fa_bwd_dropout(q, k, v, o, lse, dO, p, seed, offset, scale=x["scale"],
                                   causal=causal, key_len=kl)
    torch.cuda.synchronize()
    return [to_np(t) for t in (o, lse, dq, dk, dv)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("N", [64, 129, 300])
@pytest.mark.parametrize("mask", ["none", "causal", "pad"])
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout_matches_oracle(fa, dtype, d, N, mask, p):
    x = inputs(dtype, N, d)
    causal = mask == "causal"
    key_len = np.array([N, N // 2 + 1]) if mask == "pad" else None
    off = 3
    o, lse, dq, dk, dv = run(fa, x, dtype, p, SEED, off, causal, key_len)
    ro, rl = attention_fwd_dropout(x["q"], x["k"], x["v"], x["scale"], p, SEED, off,
                                   causal=causal, key_len=key_len)
    rq, rk, rv = attention_bwd_dropout(x["q"], x["k"], x["v"], x["dO"], x["scale"], p, SEED,
                                       off, causal=causal, key_len=key_len)
    print(f"[dropout {dtype} d={d} N={N} {mask} p={p}]")
    assert_close("o", o, ro, tol(dtype, p))
    assert_close("lse", lse, rl, TOL[dtype])
    assert_close("dq", dq, rq, tol(dtype, p))
    assert_close("dk", dk, rk, tol(dtype, p))
    assert_close("dv", dv, rv, tol(dtype, p))


def test_zero_rate_is_the_plain_path(fa):
    import torch
    x = inputs("bf16", 300, 64)
    q, k, v, dO = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "dO"))
    o0, l0 = fa.fa_fwd(q, k, v, scale=x["scale"], causal=True)
    o1, l1 = fa.fa_fwd_dropout(q, k, v, 0.0, 5, scale=x["scale"], causal=True)
    g0 = fa.fa_bwd(q, k, v, o0, l0, dO, scale=x["scale"], causal=True)
    g1 = fa.fa_bwd_dropout(q, k, v, o1, l1, dO, 0.0, 5, scale=x["scale"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


def test_mask_follows_seed_and_offset(fa):
    import torch
    x = inputs("bf16", 256, 64, B=1, H=2)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    a, _ = fa.fa_fwd_dropout(q, k, v, 0.3, 11, 0, scale=x["scale"])
    b, _ = fa.fa_fwd_dropout(q, k, v, 0.3, 11, 0, scale=x["scale"])
    c, _ = fa.fa_fwd_dropout(q, k, v, 0.3, 11, 1, scale=x["scale"])
    e, _ = fa.fa_fwd_dropout(q, k, v, 0.3, 12, 0, scale=x["scale"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, c) and not torch.equal(a, e)


def test_autograd_dropout(fa):
    from io_aware_tiled_05_amd.autograd import attention
    x = inputs("bf16", 200, 64)
    q, k, v = (to_dev(x[n], "bf16").requires_grad_(True) for n in ("q", "k", "v"))
    o = attention(q, k, v, scale=x["scale"], causal=True, dropout_p=0.2, seed=SEED, offset=9)
    o.backward(to_dev(x["dO"], "bf16"))
    ro, _ = attention_fwd_dropout(x["q"], x["k"], x["v"], x["scale"], 0.2, SEED, 9, causal=True)
    rq, rk, rv = attention_bwd_dropout(x["q"], x["k"], x["v"], x["dO"], x["scale"], 0.2, SEED,
                                       9, causal=True)
    for name, got, ref in (("o", o.detach(), ro), ("dq", q.grad, rq), ("dk", k.grad, rk),
                           ("dv", v.grad, rv)):
        assert_close(name, to_np(got), ref, tol("bf16", 0.2))
