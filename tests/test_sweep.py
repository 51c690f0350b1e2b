"""Parity on the sequence-length sweep: H = 16, N = 1K .. 16K, B = 16384 / N,
d = 64, bf16, causal and non-causal (the metric's length range at a fixed
token count).  The fp64 oracle checks sampled rows: O, lse and dQ of 256
query rows (plus the first and last), dK and dV of 64 key rows, drawn over
all B x H heads (without key padding, batches and heads are independent
and interchangeable, so they are flattened into one head axis)."""

import dataclasses

import numpy as np
import pytest

from helpers import TOL, assert_close, to_dev, to_np
from oracle import attention_key_grads, attention_rows
from workloads import SWEEP, Workload, make_inputs, sample_key_rows, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import io_aware_tiled_05_amd as fa
    fa.load()
    return fa


# ragged length with a grid of more than two 4-wave workgroups per compute
# unit (the small test shapes run the 2-wave forward)
RAGGED = tuple(Workload(f"ragged_{'causal' if c else 'full'}_1000", 16, 16, 1000, 64, "bf16",
                        causal=c, seed=120 + c, sample_rows=256, sample_keys=64)
               for c in (True, False))


@pytest.mark.parametrize("w", SWEEP + RAGGED, ids=[w.name for w in SWEEP + RAGGED])
def test_sweep_sampled_rows(fa, w):
    import torch
    x = make_inputs(w)
    B, H, N, d = x["q"].shape
    q, k, v, dO = (to_dev(x[n], w.dtype) for n in ("q", "k", "v", "dO"))
    print(f"[{w.name}: B={B} H={H} N={N}]", flush=True)
    o, lse = fa.fa_fwd(q, k, v, scale=x["scale"], causal=w.causal)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, dO, scale=x["scale"], causal=w.causal)
    torch.cuda.synchronize()
    flat = lambda a: a.reshape(1, B * H, N, d)  # noqa: E731
    O, L = flat(to_np(o)), to_np(lse).reshape(1, B * H, N)
    dq, dk, dv = (flat(to_np(t)) for t in (dq, dk, dv))
    xq, xk, xv, xo = (flat(x[n]) for n in ("q", "k", "v", "dO"))
    wf = dataclasses.replace(w, B=1, H=B * H)
    tol = TOL[w.dtype]
    rows = sample_rows(wf, B * H, N, w.sample_rows)
    for h in sorted({h for h, _ in rows}):
        ii = [i for hh, i in rows if hh == h]
        Or, lr, qr = attention_rows(xq, xk, xv, x["scale"], 0, h, ii, dO=xo, causal=w.causal)
        assert_close(f"O h={h}", O[0, h, ii], Or, tol)
        assert_close(f"lse h={h}", L[0, h, ii], lr, tol)
        assert_close(f"dq h={h}", dq[0, h, ii], qr, tol)
    keys = sample_key_rows(wf, B * H, N, w.sample_keys)
    for h in sorted({h for h, _ in keys}):
        jj = [j for hh, j in keys if hh == h]
        kr, vr = attention_key_grads(xq, xk, xv, xo, x["scale"], 0, h, jj, causal=w.causal)
        assert_close(f"dk h={h}", dk[0, h, jj], kr, tol)
        assert_close(f"dv h={h}", dv[0, h, jj], vr, tol)
