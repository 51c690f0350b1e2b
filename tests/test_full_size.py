"""Full-size GPU checks on every element, not a sample.

At the long workloads the materialising oracle can only be sampled.  Two
pins hold at any size:

* q = 0 closed forms (oracle/closed_forms.py, pinned against the definition
  in test_oracle.py): each row of P is uniform over its visible keys, so O,
  lse, dQ and dV follow from running or per-block sums and dK is exactly 0.
  Every element of the GPU results is compared with them, at the same
  tolerances as the other parity tests.
* the O box: every output row lies inside the componentwise range of the
  value rows it sees (P is a probability row), checked on all rows with the
  workload's own random inputs.
"""

import numpy as np
import pytest

from helpers import TOL, assert_close, to_dev, to_np
from oracle import q_zero_attention
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import io_aware_tiled_05_amd as fa
    fa.load()
    return fa


def gpu_fwd_bwd(fa, w, x, q):
    import torch
    dt = w.dtype
    k, v, dO = (to_dev(x[n], dt) for n in ("k", "v", "dO"))
    qd = to_dev(q, dt)
    s = x["scale"]
    if w.block_sparse:
        bm = torch.from_numpy(x["block_mask"]).cuda()
        o, lse = fa.fa_fwd_blocksparse(qd, k, v, bm, scale=s)
        dq, dk, dv = fa.fa_bwd_blocksparse(qd, k, v, o, lse, dO, bm, scale=s)
    else:
        kl = None if x["key_len"] is None else torch.from_numpy(x["key_len"]).cuda()
        o, lse = fa.fa_fwd(qd, k, v, scale=s, causal=w.causal, key_len=kl)
        dq, dk, dv = fa.fa_bwd(qd, k, v, o, lse, dO, scale=s, causal=w.causal, key_len=kl)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("name", ["long_causal", "long_causal_d128", "bert_large",
                                  "block_sparse"])
def test_q_zero_closed_forms_full_size(fa, name):
    w = WORKLOADS[name]
    x = make_inputs(w)
    q = np.zeros_like(x["q"])
    print(f"[q = 0 closed forms, {name}: B={x['B']} H={x['H']} N={x['N']} d={x['d']} "
          f"{w.dtype}]", flush=True)
    o, lse, dq, dk, dv = gpu_fwd_bwd(fa, w, x, q)
    cO, cl, cdq, _, cdv = q_zero_attention(x["k"], x["v"], x["dO"], x["scale"], causal=w.causal,
                                           key_len=x["key_len"], block_mask=x["block_mask"])
    tol = TOL[w.dtype]
    assert_close("o", to_np(o), cO, tol)
    assert_close("lse", to_np(lse), cl, tol)
    assert_close("dq", to_np(dq), cdq, tol)
    assert_close("dv", to_np(dv), cdv, tol)
    assert int((dk != 0).sum()) == 0, "dK must be exactly zero when q = 0"


@pytest.mark.parametrize("name", ["long_causal", "bert_large"])
def test_outputs_lie_in_the_box_of_visible_values(fa, name):
    w = WORKLOADS[name]
    x = make_inputs(w)
    print(f"[O box, {name}]", flush=True)
    o, _, _, _, _ = gpu_fwd_bwd(fa, w, x, x["q"])
    o = to_np(o)
    v = x["v"].astype(np.float64)
    tol = float(TOL[w.dtype])
    B, H, N, _ = v.shape
    for b in range(B):
        L = N if x["key_len"] is None else int(x["key_len"][b])
        for h in range(H):
            if w.causal:  # row i sees keys 0 .. min(i, L - 1)
                last = np.minimum(np.arange(N), L - 1)
                lo = np.minimum.accumulate(v[b, h], axis=0)[last]
                hi = np.maximum.accumulate(v[b, h], axis=0)[last]
            else:
                lo = np.broadcast_to(v[b, h, :L].min(0), (N, v.shape[-1]))
                hi = np.broadcast_to(v[b, h, :L].max(0), (N, v.shape[-1]))
            assert np.all(o[b, h] >= lo - tol) and np.all(o[b, h] <= hi + tol), (b, h)
