"""Decode parity: fa_decode (through the C ABI) vs the fp64 oracle.

A few queries against a longer key sequence, keys j >= key_len[b] hidden,
no causal order (the oracle's Nq != Nk case, pinned in test_oracle.py).
Tolerances (max abs error on O and lse): fp32 1e-5, fp16 1e-2, bf16 2e-2.
Shapes cover one and several chunks of keys, ragged chunk tails, query
counts that are not a multiple of the 4-query groups, empty key ranges and
the long-context shape (16 heads, 16384 cached keys).
"""

import numpy as np
import pytest

from helpers import TOL, assert_close, to_dev, to_np
from oracle import attention_fwd
from workloads import make_decode_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import io_aware_tiled_05_amd as fa
    fa.load()
    return fa


def run(fa, x, key_len=None):
    import torch
    q, k, v = (to_dev(x[n], x["dtype"]) for n in ("q", "k", "v"))
    kl = None if key_len is None else torch.tensor(key_len, dtype=torch.int32, device="cuda:0")
    o, lse = fa.fa_decode(q, k, v, scale=x["scale"], key_len=kl)
    torch.cuda.synchronize()
    return to_np(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 100), (3, 257), (5, 1000), (1, 4096), (8, 2500)])
def test_decode_shapes(fa, dtype, d, Nq, Nk):
    x = make_decode_inputs(2, 3, Nq, Nk, d, dtype, seed=Nq * 7919 + Nk)
    o, lse = run(fa, x)
    ro, rl = attention_fwd(x["q"], x["k"], x["v"], x["scale"])
    print(f"[decode {dtype} d={d} Nq={Nq} Nk={Nk}]")
    assert_close("o", o, ro, TOL[dtype])
    assert_close("lse", lse, rl, TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_key_lengths(fa, dtype):
    # batch 0: no visible key (O = 0, lse = -inf); 1: a single key; 2: a
    # length inside a chunk; 3: past the end (clamped to Nk)
    x = make_decode_inputs(4, 2, 3, 3000, 64, dtype, seed=77)
    key_len = np.array([0, 1, 1300, 5000])
    o, lse = run(fa, x, key_len)
    ro, rl = attention_fwd(x["q"], x["k"], x["v"], x["scale"], key_len=np.minimum(key_len, 3000))
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert_close("o", o, ro, TOL[dtype])
    assert_close("lse", lse, rl, TOL[dtype])


def test_decode_long_context(fa):
    # the long causal workload's heads and length, one new token each
    x = make_decode_inputs(1, 16, 1, 16384, 64, "bf16", seed=4)
    key_len = np.array([16000])
    o, lse = run(fa, x, key_len)
    ro, rl = attention_fwd(x["q"], x["k"], x["v"], x["scale"], key_len=key_len)
    assert_close("o", o, ro, TOL["bf16"])
    assert_close("lse", lse, rl, TOL["bf16"])


def test_decode_matches_forward_rows(fa):
    # decode of the last queries of a sequence == those rows of the
    # non-causal forward over the whole sequence (same inputs, two different
    # kernels; the forward sums P after rounding it to bf16, the decode in
    # fp32, so lse agrees to the bf16 gate, not to fp32 rounding)
    import torch
    from workloads import Workload, make_inputs
    x = make_inputs(Workload("dec", 2, 4, 600, 64, "bf16", seed=9))
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    o_full, lse_full = fa.fa_fwd(q, k, v, scale=x["scale"])
    o_dec, lse_dec = fa.fa_decode(q[:, :, -3:].contiguous(), k, v, scale=x["scale"])
    torch.cuda.synchronize()
    assert_close("o", to_np(o_dec), to_np(o_full[:, :, -3:]), TOL["bf16"])
    assert_close("lse", to_np(lse_dec), to_np(lse_full[:, :, -3:]), TOL["bf16"])
