"""fa_bwd_noalloc (the backward with the library's fixed workspace array)
against fa_bwd (the same backward with a caller-provided workspace),
through the C ABI.

Both run the same kernels in the same launch sequence, so their gradients
must agree bit for bit.  Two calls in a row, the second on a smaller
problem, check that a call does not depend on what the previous one left in
the shared array; the first call is also held to the fp64 oracle's
tolerance.  A problem of the bench workload's size (100 MiB of workspace)
uses most of the 128 MiB array.
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


def run_both(fa, x, dtype, causal, key_len):
    import torch
    q, k, v, dO = (to_dev(x[n], dtype) for n in ("q", "k", "v", "dO"))
    kl = None if key_len is None else torch.from_numpy(key_len.astype(np.int32)).cuda()
    s = x["scale"]
    o, lse = fa.fa_fwd(q, k, v, scale=s, causal=causal, key_len=kl)
    ref = fa.fa_bwd(q, k, v, o, lse, dO, scale=s, causal=causal, key_len=kl)
    got = tuple(torch.empty_like(q) for _ in range(3))
    fa.fa_bwd_noalloc(q, k, v, o, lse, dO, *got, scale=s, causal=causal, key_len=kl)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_noalloc_equals_fa_bwd_two_calls(fa, dtype):
    # first call: larger, causal; second: smaller, key padding
    x1 = make_inputs(Workload("noalloc", 2, 3, 700, 64, dtype, seed=31))
    print(f"[noalloc {dtype} B=2 H=3 N=700 causal]", flush=True)
    ref1, got1 = run_both(fa, x1, dtype, True, None)
    for name, a, b in zip(("dq", "dk", "dv"), ref1, got1):
        assert bool((a == b).all()), f"{name}: fa_bwd_noalloc differs from fa_bwd"
    want = attention_bwd(x1["q"], x1["k"], x1["v"], x1["dO"], x1["scale"], causal=True)
    for name, g, w in zip(("dq", "dk", "dv"), got1, want):
        assert_close(name, to_np(g), w, TOL[dtype])

    x2 = make_inputs(Workload("noalloc", 1, 2, 129, 64, dtype, seed=32))
    kl = np.array([77], dtype=np.int32)
    print(f"[noalloc {dtype} B=1 H=2 N=129 key_len=77]", flush=True)
    ref2, got2 = run_both(fa, x2, dtype, False, kl)
    for name, a, b in zip(("dq", "dk", "dv"), ref2, got2):
        assert bool((a == b).all()), f"{name}: second call differs from fa_bwd"


def test_noalloc_at_the_bench_size(fa):
    # B=1, H=16, N=16384, d=64 bf16 causal: 100 MiB of the 128 MiB array,
    # then a small call after it
    import torch
    torch.manual_seed(5)
    dev = torch.device("cuda:0")
    shape = (1, 16, 16384, 64)
    q, k, v, dO = (torch.randn(shape, device=dev).to(torch.bfloat16) for _ in range(4))
    print("[noalloc bf16 B=1 H=16 N=16384 d=64 causal]", flush=True)
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    ref = fa.fa_bwd(q, k, v, o, lse, dO, causal=True)
    got = tuple(torch.empty_like(q) for _ in range(3))
    fa.fa_bwd_noalloc(q, k, v, o, lse, dO, *got, causal=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert bool((a == b).all()), f"{name}: fa_bwd_noalloc differs from fa_bwd"
    x = make_inputs(Workload("noalloc", 1, 1, 64, 64, "bf16", seed=33))
    print("[noalloc bf16 B=1 H=1 N=64 after the large call]", flush=True)
    ref2, got2 = run_both(fa, x, "bf16", True, None)
    for name, a, b in zip(("dq", "dk", "dv"), ref2, got2):
        assert bool((a == b).all()), f"{name}: small call after the large one differs"


def test_noalloc_too_large_raises(fa):
    import torch
    shape = (1, 16, 16384, 128)  # 196 MiB of workspace
    t = torch.empty(shape, dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty(shape[:3], dtype=torch.float32, device="cuda:0")
    with pytest.raises(fa.FaError, match="fixed scratch buffer"):
        fa.fa_bwd_noalloc(t, t, t, t, lse, t, t, t, t, causal=True)
