"""Strided tensor views through the C ABI (fa_fwd_strided, fa_bwd_strided).

The kernels address every tensor through (batch, head, row) strides, so a
view is read and written in place.  The arithmetic does not depend on the
addressing: on the same values, the strided calls must return bit for bit
what the packed calls return, and their outputs must land exactly where the
views point (the bytes between rows untouched).  One case per layout is
also held to the fp64 oracle.  Layouts: the [B, N, H, d] order of framework
activations; q, k, v as slices of one fused [B, N, 3, H, d] projection;
rows inside a wider padded buffer; and mixed layouts in one call.
"""

import numpy as np
import pytest

from helpers import TOL, assert_close, to_dev, to_np, torch_dtype
from oracle import attention_bwd, attention_fwd
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import io_aware_tiled_05_amd as fa
    fa.load()
    return fa


def views(x, dtype, layout):
    """q, k, v, dO as [B, H, N, d] views of the given layout holding the
    values of x (numpy [B, H, N, d])."""
    import torch
    dev, tdt = "cuda:0", torch_dtype(dtype)
    B, H, N, d = x["q"].shape
    t = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(dev, tdt) for n in ("q", "k", "v", "dO")}
    if layout == "bhnd":
        return t
    if layout == "bnhd":
        return {n: a.transpose(1, 2).contiguous().transpose(1, 2) for n, a in t.items()}
    if layout == "qkv_fused":  # [B, N, 3, H, d] storage, q/k/v its slices
        fused = torch.empty((B, N, 3, H, d), dtype=tdt, device=dev)
        out = {}
        for i, n in enumerate(("q", "k", "v")):
            fused[:, :, i] = t[n].transpose(1, 2)
            out[n] = fused[:, :, i].transpose(1, 2)
        out["dO"] = t["dO"].transpose(1, 2).contiguous().transpose(1, 2)
        return out
    if layout == "padded_rows":  # each row inside a buffer 16 elements wider
        out = {}
        for n, a in t.items():
            buf = torch.full((B, H, N, d + 16), float("nan"), dtype=tdt, device=dev)
            buf[..., :d] = a
            out[n] = buf[..., :d]
        return out
    raise ValueError(layout)


def out_like(t, layout):
    """An output view of the given layout (rows of padded buffers hold NaN
    between them, to show nothing is written there)."""
    import torch
    B, H, N, d = t.shape
    if layout == "padded_rows":
        buf = torch.full((B, H, N, d + 16), float("nan"), dtype=t.dtype, device=t.device)
        return buf[..., :d], buf
    if layout in ("bnhd", "qkv_fused"):
        o = torch.empty((B, N, H, d), dtype=t.dtype, device=t.device).transpose(1, 2)
        return o, o
    o = torch.empty_like(t)
    return o, o


LAYOUTS = ["bnhd", "qkv_fused", "padded_rows"]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("mask", ["none", "causal", "pad"])
@pytest.mark.parametrize("d", [64, 128])
def test_strided_equals_packed(fa, dtype, layout, mask, d):
    import torch
    N = 300 if d == 64 else 129
    x = make_inputs(Workload("strided", 2, 3, N, d, dtype, seed=61))
    causal = mask == "causal"
    kl = torch.tensor([N, 97], dtype=torch.int32, device="cuda:0") if mask == "pad" else None
    s = x["scale"]
    p = views(x, dtype, "bhnd")
    sv = views(x, dtype, layout)
    print(f"[strided {layout} {dtype} d={d} N={N} {mask}]", flush=True)
    o_ref, lse_ref = fa.fa_fwd(p["q"], p["k"], p["v"], scale=s, causal=causal, key_len=kl)
    g_ref = fa.fa_bwd(p["q"], p["k"], p["v"], o_ref, lse_ref, p["dO"], scale=s, causal=causal,
                      key_len=kl)
    o, obuf = out_like(sv["q"], layout)
    o, lse = fa.fa_fwd_strided(sv["q"], sv["k"], sv["v"], scale=s, causal=causal, key_len=kl,
                               out=o)
    outs = [out_like(sv[n], layout) for n in ("q", "k", "v")]
    g = fa.fa_bwd_strided(sv["q"], sv["k"], sv["v"], o, lse, sv["dO"], scale=s, causal=causal,
                          key_len=kl, dq=outs[0][0], dk=outs[1][0], dv=outs[2][0])
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    for name, a, b in zip(("dq", "dk", "dv"), g, g_ref):
        assert torch.equal(a, b), f"{name} differs from the packed call"
    if layout == "padded_rows":  # nothing written between the rows
        for _, buf in [(o, obuf)] + outs:
            assert bool(torch.isnan(buf[..., -16:].float()).all())
    if mask == "causal" and d == 64:
        ro, _ = attention_fwd(x["q"], x["k"], x["v"], s, causal=True)
        rq, rk, rv = attention_bwd(x["q"], x["k"], x["v"], x["dO"], s, causal=True)
        assert_close("o", to_np(o), ro, TOL[dtype])
        for name, a, r in zip(("dq", "dk", "dv"), g, (rq, rk, rv)):
            assert_close(name, to_np(a), r, TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_strided_block_sparse_and_dropout(fa, dtype):
    import torch
    N = 300
    x = make_inputs(Workload("strided", 1, 2, N, 64, dtype, seed=62))
    s = x["scale"]
    p = views(x, dtype, "bhnd")
    sv = views(x, dtype, "bnhd")
    nb = 3
    bm = torch.tensor((np.random.default_rng(9).random((nb, nb)) < 0.6) | np.eye(nb, dtype=bool),
                      dtype=torch.uint8, device="cuda:0")
    print(f"[strided block-sparse and dropout {dtype}]", flush=True)
    o_ref, lse_ref = fa.fa_fwd_blocksparse(p["q"], p["k"], p["v"], bm, scale=s)
    g_ref = fa.fa_bwd_blocksparse(p["q"], p["k"], p["v"], o_ref, lse_ref, p["dO"], bm, scale=s)
    o, lse = fa.fa_fwd_strided(sv["q"], sv["k"], sv["v"], scale=s, block_mask=bm)
    g = fa.fa_bwd_strided(sv["q"], sv["k"], sv["v"], o, lse, sv["dO"], scale=s, block_mask=bm)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    assert all(torch.equal(a, b) for a, b in zip(g, g_ref))

    o_ref, lse_ref = fa.fa_fwd_dropout(p["q"], p["k"], p["v"], 0.2, 123, 7, scale=s, causal=True)
    g_ref = fa.fa_bwd_dropout(p["q"], p["k"], p["v"], o_ref, lse_ref, p["dO"], 0.2, 123, 7,
                              scale=s, causal=True)
    o, lse = fa.fa_fwd_strided(sv["q"], sv["k"], sv["v"], scale=s, causal=True, dropout_p=0.2,
                               seed=123, offset=7)
    g = fa.fa_bwd_strided(sv["q"], sv["k"], sv["v"], o, lse, sv["dO"], scale=s, causal=True,
                          dropout_p=0.2, seed=123, offset=7)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    assert all(torch.equal(a, b) for a, b in zip(g, g_ref))


def test_mixed_layouts_in_one_call(fa):
    # q from a fused projection, k packed, v [B, N, H, d], dO padded rows,
    # outputs in yet another order
    import torch
    dtype = "bf16"
    x = make_inputs(Workload("strided", 2, 2, 257, 64, dtype, seed=63))
    s = x["scale"]
    p = views(x, dtype, "bhnd")
    q = views(x, dtype, "qkv_fused")["q"]
    v = views(x, dtype, "bnhd")["v"]
    dO = views(x, dtype, "padded_rows")["dO"]
    print("[strided mixed layouts]", flush=True)
    o_ref, lse_ref = fa.fa_fwd(p["q"], p["k"], p["v"], scale=s, causal=True)
    g_ref = fa.fa_bwd(p["q"], p["k"], p["v"], o_ref, lse_ref, p["dO"], scale=s, causal=True)
    o, lse = fa.fa_fwd_strided(q, p["k"], v, scale=s, causal=True)
    g = fa.fa_bwd_strided(q, p["k"], v, o, lse, dO, scale=s, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert all(torch.equal(a, b) for a, b in zip(g, g_ref))


def test_autograd_bnhd_reads_and_writes_in_place():
    """attention(layout="bnhd") hands the [B, N, H, d] tensors to the kernels
    as views: the only device memory it allocates is O, lse, the gradients
    and the backward's workspace, never a transposed copy of q, k, v or dO."""
    import torch
    from io_aware_tiled_05_amd import fa_bwd_workspace_size
    from io_aware_tiled_05_amd.autograd import attention
    B, N, H, d = 2, 1024, 8, 64
    torch.manual_seed(3)
    q, k, v = (torch.randn(B, N, H, d, device="cuda:0", dtype=torch.bfloat16).requires_grad_(True)
               for _ in range(3))
    dO = torch.randn(B, N, H, d, device="cuda:0", dtype=torch.bfloat16)
    tensor = B * N * H * d * 2
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    o = attention(q, k, v, causal=True, layout="bnhd")
    fwd_peak = torch.cuda.max_memory_allocated() - base
    assert o.is_contiguous() and o.shape == (B, N, H, d)
    o.backward(dO)
    torch.cuda.synchronize()
    bwd_peak = torch.cuda.max_memory_allocated() - base
    lse = B * H * N * 4
    ws = fa_bwd_workspace_size(B, H, N, d)
    print(f"forward peak {fwd_peak} B (O + lse = {tensor + lse}), backward peak {bwd_peak} B "
          f"(O + lse + 3 gradients + workspace = {4 * tensor + lse + ws})", flush=True)
    slack = 2 << 20  # allocator rounding
    assert fwd_peak <= tensor + lse + slack
    assert bwd_peak <= 4 * tensor + lse + ws + slack
    for t in (q, k, v):
        assert t.grad.is_contiguous() and t.grad.shape == (B, N, H, d)
