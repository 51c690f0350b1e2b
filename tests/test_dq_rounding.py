"""CPU emulation of how the 16-bit backward rounds dS before dQ = scale dS K.

The dQ product runs on fp16 operands, so dS = P * (dP - D) is rounded to
fp16 first.  fp16 holds magnitudes from about 6e-8 (subnormal) to 65504, so
the product is only exact to fp16's 11 bits if dS is brought into that range:
the kernel multiplies P, and so dS, by the per-(b, h) power of two
2^kq, kq = -(eo + ev), where max|dO| 2^-eo lies in [2^3, 2^4) and
max|V| 2^-ev in [2^2, 2^3), and divides it out of the fp32 result.  Then
|dS 2^kq| <= 2 d max|dO 2^-eo| max|V 2^-ev| < 2^15 for d <= 128.

This test reproduces only that rounding, in numpy (float16 keeps
subnormals), on exact fp64 P, dP, D of a causal problem, and checks that

* with the scale, dQ stays within 5e-3 of its own size for every gradient
  magnitude from dO x 1e-9 to dO, V x 300 (the parity gates are 1e-2 and
  2e-2), and no value overflows;
* without it (the form the kernel had before), gradients of training size
  lose a large part of dQ to fp16's subnormal range, and large dO, V
  overflow to inf — so the emulation is sensitive to what it guards.

No GPU code is run or imported; P, dP, D follow the oracle's definition and
the unrounded emulation is checked against oracle.attention_bwd.
"""

import numpy as np
import pytest

from oracle import attention_bwd
from workloads import Workload, make_inputs, round_to_dtype

N, D_HEAD = 1024, 64


def scale_exp(mx, t):
    """e with mx 2^-e in [2^t, 2^(t+1)), clamped to [-60, 60]; 0 for mx = 0."""
    if mx == 0.0:
        return 0
    return int(np.clip(np.floor(np.log2(mx)) - t, -60, 60))


def exact_terms(q, k, v, dO, scale):
    """P, dP - D (fp64) of one causal head, by the definition."""
    S = scale * (q @ k.T)
    S[np.triu_indices(len(q), 1)] = -np.inf
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    dP = dO @ v.T
    Drow = (P * dP).sum(axis=1, keepdims=True)
    return P, dP - Drow


def emulated_dq(q, k, v, dO, scale, scaled):
    P, dPD = exact_terms(q, k, v, dO, scale)
    kq = -(scale_exp(np.abs(dO).max(), 3) + scale_exp(np.abs(v).max(), 2)) if scaled else 0
    with np.errstate(over="ignore", invalid="ignore"):
        dS16 = (np.ldexp(P, kq) * dPD).astype(np.float16).astype(np.float64)
        dq = np.ldexp(scale * (dS16 @ k), -kq)
    return dq, int((dS16 == 0).sum() - (P * dPD == 0).sum())


@pytest.fixture(scope="module")
def base():
    x = make_inputs(Workload("dq_rounding", 1, 1, N, D_HEAD, "bf16", seed=71))
    return {n: x[n][0, 0] for n in ("q", "k", "v", "dO")}, x["scale"]


def scaled_inputs(base, fdo, fv):
    t, _ = base
    out = dict(t)
    out["dO"] = round_to_dtype((t["dO"] * fdo).astype(np.float32), "bf16").astype(np.float64)
    out["v"] = round_to_dtype((t["v"] * fv).astype(np.float32), "bf16").astype(np.float64)
    out["q"], out["k"] = t["q"].astype(np.float64), t["k"].astype(np.float64)
    return out


def test_unrounded_emulation_is_the_oracle(base):
    t, scale = base
    P, dPD = exact_terms(*(t[n].astype(np.float64) for n in ("q", "k", "v", "dO")), scale)
    dq = scale * ((P * dPD) @ t["k"].astype(np.float64))
    ref = attention_bwd(*(t[n][None, None] for n in ("q", "k", "v", "dO")), scale, causal=True)[0]
    assert np.abs(dq - ref[0, 0]).max() <= 1e-12 * np.abs(ref).max()


@pytest.mark.parametrize("fdo,fv", [(1.0, 1.0), (1e-3, 1.0), (1e-6, 1.0), (1e-9, 1.0),
                                    (30.0, 30.0), (100.0, 100.0), (300.0, 300.0)])
def test_scaled_ds_keeps_dq_within_gate(base, fdo, fv):
    x = scaled_inputs(base, fdo, fv)
    _, scale = base
    P, dPD = exact_terms(x["q"], x["k"], x["v"], x["dO"], scale)
    ref = scale * ((P * dPD) @ x["k"])
    got, flushed = emulated_dq(x["q"], x["k"], x["v"], x["dO"], scale, scaled=True)
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    print(f"dO x {fdo:g}, V x {fv:g}: max err / max|dQ| = {rel:.2e}, dS flushed {flushed}")
    assert np.isfinite(got).all()
    assert rel <= 5e-3


def test_unscaled_ds_fails_away_from_unit_scale(base):
    """The emulation sees the defect the scale removes."""
    _, scale = base
    x = scaled_inputs(base, 1e-6, 1.0)
    P, dPD = exact_terms(x["q"], x["k"], x["v"], x["dO"], scale)
    ref = scale * ((P * dPD) @ x["k"])
    got, flushed = emulated_dq(x["q"], x["k"], x["v"], x["dO"], scale, scaled=False)
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    print(f"unscaled, dO x 1e-6: max err / max|dQ| = {rel:.2e}, dS flushed {flushed}")
    assert rel > 2e-2 and flushed > 0
    x = scaled_inputs(base, 300.0, 300.0)
    got, _ = emulated_dq(x["q"], x["k"], x["v"], x["dO"], scale, scaled=False)
    assert not np.isfinite(got).all()
