"""The differentiable wrapper (io_aware_tiled_05_amd.autograd).

GPU tests: outputs and autograd gradients of ``attention`` against the
fp64 oracle (tolerances fp32 1e-5, fp16 1e-2, bf16 2e-2, max abs error), the
[B, N, H, d] layout and the SDPA-shaped entry point against the plain
[B, H, N, d] call (identical kernels, so bit-identical results).  CPU tests:
argument errors raised before any GPU work.
"""

import numpy as np
import pytest

from helpers import TOL, assert_close, to_dev, to_np
from oracle import attention_bwd, attention_fwd
from workloads import Workload, make_inputs


def inputs(dtype, N=200, d=64, B=2, H=3, seed=21):
    return make_inputs(Workload("autograd", B, H, N, d, dtype, seed=seed))


def leaf(x, dtype):
    return to_dev(x, dtype).requires_grad_(True)


def run(x, dtype, **kw):
    from io_aware_tiled_05_amd.autograd import attention
    q, k, v = (leaf(x[n], dtype) for n in ("q", "k", "v"))
    dO = to_dev(x["dO"], dtype)
    o = attention(q, k, v, scale=x["scale"], **kw)
    o.backward(dO)
    return o, q.grad, k.grad, v.grad


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "pad"])
def test_autograd_matches_oracle(dtype, d, mask):
    import torch
    x = inputs(dtype, d=d)
    causal = mask == "causal"
    key_len = np.array([200, 77]) if mask == "pad" else None
    kl = None if key_len is None else torch.tensor(key_len, dtype=torch.int32, device="cuda:0")
    o, dq, dk, dv = run(x, dtype, causal=causal, key_len=kl)
    ro, _ = attention_fwd(x["q"], x["k"], x["v"], x["scale"], causal=causal, key_len=key_len)
    rq, rk, rv = attention_bwd(x["q"], x["k"], x["v"], x["dO"], x["scale"], causal=causal,
                               key_len=key_len)
    print(f"[autograd {dtype} d={d} {mask}]")
    assert_close("o", to_np(o.detach()), ro, TOL[dtype])
    assert_close("dq", to_np(dq), rq, TOL[dtype])
    assert_close("dk", to_np(dk), rk, TOL[dtype])
    assert_close("dv", to_np(dv), rv, TOL[dtype])


@pytest.mark.gpu
def test_autograd_block_sparse():
    import torch
    dtype = "bf16"
    x = inputs(dtype, N=300)
    bm = np.random.default_rng(5).random((3, 3)) < 0.5
    bm[np.arange(3), np.arange(3)] = True
    bmd = torch.tensor(bm.astype(np.uint8), device="cuda:0")
    o, dq, dk, dv = run(x, dtype, block_mask=bmd)
    ro, _ = attention_fwd(x["q"], x["k"], x["v"], x["scale"], block_mask=bm)
    rq, rk, rv = attention_bwd(x["q"], x["k"], x["v"], x["dO"], x["scale"], block_mask=bm)
    assert_close("o", to_np(o.detach()), ro, TOL[dtype])
    assert_close("dq", to_np(dq), rq, TOL[dtype])
    assert_close("dk", to_np(dk), rk, TOL[dtype])
    assert_close("dv", to_np(dv), rv, TOL[dtype])


@pytest.mark.gpu
def test_bnhd_layout_and_sdpa_entry_are_the_same_kernels():
    import torch
    from io_aware_tiled_05_amd.autograd import attention, scaled_dot_product_attention
    dtype = "bf16"
    x = inputs(dtype, N=130)
    o, dq, dk, dv = run(x, dtype, causal=True)

    # [B, N, H, d] copies of the same values
    qn, kn, vn = (to_dev(x[n], dtype).transpose(1, 2).contiguous().requires_grad_(True)
                  for n in ("q", "k", "v"))
    on = attention(qn, kn, vn, causal=True, scale=x["scale"], layout="bnhd")
    on.backward(to_dev(x["dO"], dtype).transpose(1, 2))
    assert on.shape == qn.shape
    assert torch.equal(on.transpose(1, 2), o)
    assert torch.equal(qn.grad.transpose(1, 2), dq)
    assert torch.equal(kn.grad.transpose(1, 2), dk)
    assert torch.equal(vn.grad.transpose(1, 2), dv)

    qs, ks, vs = (leaf(x[n], dtype) for n in ("q", "k", "v"))
    os_ = scaled_dot_product_attention(qs, ks, vs, is_causal=True, scale=x["scale"])
    os_.backward(to_dev(x["dO"], dtype))
    assert torch.equal(os_, o)
    assert torch.equal(qs.grad, dq) and torch.equal(ks.grad, dk) and torch.equal(vs.grad, dv)


@pytest.mark.gpu
def test_fp32_forward_and_backward():
    x = inputs("f32", N=100, B=1, H=2)
    for causal in (False, True):
        o, dq, dk, dv = run(x, "f32", causal=causal)
        ro, _ = attention_fwd(x["q"], x["k"], x["v"], x["scale"], causal=causal)
        rq, rk, rv = attention_bwd(x["q"], x["k"], x["v"], x["dO"], x["scale"], causal=causal)
        assert_close("o", to_np(o.detach()), ro, TOL["f32"])
        assert_close("dq", to_np(dq), rq, TOL["f32"])
        assert_close("dk", to_np(dk), rk, TOL["f32"])
        assert_close("dv", to_np(dv), rv, TOL["f32"])


def test_argument_errors_before_gpu_work():
    import torch
    from io_aware_tiled_05_amd.autograd import attention, scaled_dot_product_attention
    t = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError, match="dropout"):
        scaled_dot_product_attention(t, t, t, dropout_p=1.0)
    with pytest.raises(ValueError, match="dropout"):
        attention(t, t, t, dropout_p=0.1, block_mask=torch.ones(1, 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="attn_mask"):
        scaled_dot_product_attention(t, t, t, attn_mask=torch.zeros(4, 4))
    with pytest.raises(ValueError, match="layout"):
        attention(t, t, t, layout="nhd")
    with pytest.raises(ValueError, match="block_mask"):
        attention(t, t, t, causal=True, block_mask=torch.ones(1, 1, dtype=torch.uint8))
