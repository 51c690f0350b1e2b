"""The backward as one call (fa_bwd: the D pass, then one launch that runs the
dK/dV and dQ workgroups together), as its three stages launched one at a
time, and as the D stage followed by the one-launch gradient stage
(fa_bwd_stage 1, 2, 3 and 1, 4) must give the same gradients bit for bit:
every output element is computed by the same arithmetic in all three.  The one-call form is
checked against the fp64 oracle by test_parity_bwd.py; one case here is
checked against it too, through the staged form.
"""

import numpy as np
import pytest

from helpers import TOL, assert_close, to_dev, to_np
from oracle import attention_bwd
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import io_aware_tiled_05_amd as fa
    fa.load()
    return fa


def both(fa, x, dtype, causal=False, key_len=None, block_mask=None):
    import torch
    q, k, v, dO = (to_dev(x[n], dtype) for n in ("q", "k", "v", "dO"))
    s = x["scale"]
    B, H, N, d = q.shape
    kl = None if key_len is None else torch.from_numpy(key_len.astype(np.int32)).cuda()
    bm = None if block_mask is None else torch.from_numpy(block_mask).cuda()
    if bm is not None:
        o, lse = fa.fa_fwd_blocksparse(q, k, v, bm, scale=s)
        one = fa.fa_bwd_blocksparse(q, k, v, o, lse, dO, bm, scale=s)
    else:
        o, lse = fa.fa_fwd(q, k, v, scale=s, causal=causal, key_len=kl)
        one = fa.fa_bwd(q, k, v, o, lse, dO, scale=s, causal=causal, key_len=kl)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d) // 4, dtype=torch.float32,
                     device=q.device)
    for st in (fa.FA_BWD_STAGE_D, fa.FA_BWD_STAGE_DKDV, fa.FA_BWD_STAGE_DQ):
        fa.fa_bwd_stage(st, q, k, v, o, lse, dO, dq, dk, dv, ws, scale=s, causal=causal,
                        key_len=kl, block_mask=bm)
    g4 = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    for st in (fa.FA_BWD_STAGE_D, fa.FA_BWD_STAGE_GRADS):
        fa.fa_bwd_stage(st, q, k, v, o, lse, dO, *g4, ws, scale=s, causal=causal, key_len=kl,
                        block_mask=bm)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), one, g4):
        assert bool((a == b).all()), f"{name} differs between fa_bwd and stages 1, 4"
    return one, (dq, dk, dv)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("N", [7, 129, 700])
@pytest.mark.parametrize("mask", ["none", "causal", "pad"])
def test_one_call_equals_stages(fa, dtype, d, N, mask):
    x = make_inputs(Workload("stages", 2, 3, N, d, dtype, seed=21))
    key_len = None
    if mask == "pad":
        key_len = np.random.default_rng(N + d).integers(1, N, size=2, endpoint=True)
    one, staged = both(fa, x, dtype, causal=mask == "causal", key_len=key_len)
    print(f"[bwd one call vs stages {dtype} d={d} N={N} {mask}]")
    for name, a, b in zip(("dq", "dk", "dv"), one, staged):
        assert bool((a == b).all()), f"{name} differs between fa_bwd and fa_bwd_stage"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_one_call_equals_stages_blocksparse(fa, dtype):
    N = 700
    nb = (N + 127) // 128
    bm = (np.random.default_rng(3).random((nb, nb)) < 0.5).astype(np.uint8)
    np.fill_diagonal(bm, 1)
    bm[1, :] = 0  # a block row without keys
    x = make_inputs(Workload("stages", 1, 2, N, 64, dtype, seed=22))
    one, staged = both(fa, x, dtype, block_mask=bm)
    print(f"[bwd one call vs stages block-sparse {dtype} N={N}]")
    for name, a, b in zip(("dq", "dk", "dv"), one, staged):
        assert bool((a == b).all()), f"{name} differs between fa_bwd and fa_bwd_stage"


def test_stages_against_oracle(fa):
    x = make_inputs(Workload("stages", 2, 2, 300, 64, "bf16", seed=23))
    _, staged = both(fa, x, "bf16", causal=True)
    ref = attention_bwd(x["q"], x["k"], x["v"], x["dO"], x["scale"], causal=True)
    print("[bwd stages vs oracle bf16 d=64 N=300 causal]")
    for name, got, want in zip(("dq", "dk", "dv"), staged, ref):
        assert_close(name, to_np(got), want, TOL["bf16"])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("N,mask", [(300, "causal"), (1024, "none"), (2048, "causal"),
                                    (517, "dropout")])
def test_one_launch_d_pass_equals_split(fa, dtype, d, N, mask):
    """With 32 or more heads of at most 2048 rows the D pass runs as one
    workgroup per head; otherwise as two launches over many workgroups per
    head.  Both write the same D, shift, maxima, fp16 copies and row terms,
    so the gradients of the first heads of a 32-head call must equal, bit
    for bit, those of a 4-head call holding only them (b = 0, so every head
    keeps its index, which the dropout draw depends on)."""
    import torch
    x = make_inputs(Workload("headprep", 1, 32, N, d, dtype, seed=71))
    q, k, v, dO = (to_dev(x[n], dtype) for n in ("q", "k", "v", "dO"))
    s = x["scale"]
    print(f"[one-launch D pass {dtype} d={d} N={N} {mask}]", flush=True)

    def grads(q, k, v, dO):
        if mask == "dropout":
            o, lse = fa.fa_fwd_dropout(q, k, v, 0.2, 99, 3, scale=s, causal=True)
            return fa.fa_bwd_dropout(q, k, v, o, lse, dO, 0.2, 99, 3, scale=s, causal=True)
        o, lse = fa.fa_fwd(q, k, v, scale=s, causal=mask == "causal")
        return fa.fa_bwd(q, k, v, o, lse, dO, scale=s, causal=mask == "causal")

    full = grads(q, k, v, dO)
    part = grads(*(t[:, :4].contiguous() for t in (q, k, v, dO)))
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), full, part):
        assert torch.equal(a[:, :4], b), f"{name}: one-launch and split D passes differ"
