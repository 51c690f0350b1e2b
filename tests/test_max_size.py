"""The largest problem the C ABI accepts: B = H = 1, d = 64 and
N = (2^31 - 1) // 64 rows, so q, k, v, o, dO, dq, dk, dv each hold
2^31 - 64 elements (4 GiB in bf16) and every kernel's row offsets reach
2^31 elements.  key_len = 128 keeps the work linear in N: every query row
sees the first 128 keys and no other.

Keys at or past key_len have weight exactly 0, so each query row's result
is the definition applied to that row against K[:128] and V[:128]: the fp64
oracle computes O, lse and dQ for sampled query rows (the first, the last
and rows around 2^24 and N / 2) from that sub-problem.  dK and dV must be
exactly 0 on every key row past 128 (sampled, the last one included); for
the 128 visible keys two identities of the backward hold at any size:
sum_j dK_j = 0 (every row of dS sums to 0) and sum_j dV_j = sum_i dO_i
(every row of P sums to 1).  Inputs are seeded N(0, 1) drawn on the GPU
(too large for a host-side generator in a test).
"""

import numpy as np
import pytest

from helpers import TOL, assert_close
from oracle import attention_rows

pytestmark = pytest.mark.gpu

D = 64
N = (2 ** 31 - 1) // D
KL = 128


@pytest.fixture(scope="module")
def fa():
    import io_aware_tiled_05_amd as fa
    fa.load()
    return fa


def test_largest_accepted_size(fa):
    import torch
    props = torch.cuda.get_device_properties(0)
    if props.total_memory < 96 * 2 ** 30:
        pytest.skip("needs about 50 GiB of device memory")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(31)
    shape = (1, 1, N, D)
    print(f"[max size: B=1 H=1 N={N} d={D} bf16, key_len={KL}]", flush=True)
    q, k, v, dO = (torch.randn(shape, device=dev, dtype=torch.bfloat16, generator=g)
                   for _ in range(4))
    kl = torch.tensor([KL], dtype=torch.int32, device=dev)
    scale = D ** -0.5
    o, lse = fa.fa_fwd(q, k, v, scale=scale, key_len=kl)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, dO, scale=scale, key_len=kl)
    torch.cuda.synchronize()

    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([
        [0, 1, 63, 64, 255, 256, N // 2, 2 ** 24 - 1, 2 ** 24, N - 257, N - 2, N - 1],
        rng.integers(0, N, 20)]))
    ri = torch.from_numpy(rows).to(dev)

    def host(t, idx=None):
        t = t[0, 0] if idx is None else t[0, 0].index_select(0, idx)
        return t.float().cpu().numpy().astype(np.float64)

    qs, dOs = host(q, ri), host(dO, ri)
    ks, vs = host(k[:, :, :KL]), host(v[:, :, :KL])
    O_ref, lse_ref, dq_ref = attention_rows(qs[None, None], ks[None, None], vs[None, None],
                                            scale, 0, 0, np.arange(rows.size),
                                            dO=dOs[None, None])
    assert_close("O rows", host(o, ri), O_ref, TOL["bf16"])
    assert_close("lse rows", lse[0, 0].index_select(0, ri).cpu().numpy().astype(np.float64),
                 lse_ref, TOL["bf16"])
    assert_close("dQ rows", host(dq, ri), dq_ref, TOL["bf16"])

    # key rows past key_len: no query sees them
    kz = np.unique(np.concatenate([[KL, KL + 1, N // 2, N - 64, N - 1],
                                   rng.integers(KL, N, 20)]))
    kzi = torch.from_numpy(kz).to(dev)
    assert bool((dk[0, 0].index_select(0, kzi) == 0).all()), "dK not 0 past key_len"
    assert bool((dv[0, 0].index_select(0, kzi) == 0).all()), "dV not 0 past key_len"

    # the 128 visible keys: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i
    dk_vis, dv_vis = host(dk[:, :, :KL]), host(dv[:, :, :KL])
    sum_dO = np.zeros(D)
    step = 1 << 22
    for r0 in range(0, N, step):
        sum_dO += dO[0, 0, r0:r0 + step].to(torch.float64).sum(dim=0).cpu().numpy()
    # each dK_j, dV_j is rounded to bf16 (relative 2^-9) and accumulated in
    # fp32 over N rows: bound the sums by 1 % of the sums of magnitudes
    tol_k = 1e-2 * np.abs(dk_vis).sum(axis=0) + 1e-3
    tol_v = 1e-2 * np.abs(dv_vis).sum(axis=0) + 1e-3
    err_k = np.abs(dk_vis.sum(axis=0))
    err_v = np.abs(dv_vis.sum(axis=0) - sum_dO)
    print(f"  sum dK: max {err_k.max():.3e} (tol {tol_k.min():.3e}..); "
          f"sum dV - sum dO: max {err_v.max():.3e} (|sum dO| max {np.abs(sum_dO).max():.1f})",
          flush=True)
    assert np.all(err_k <= tol_k)
    assert np.all(err_v <= tol_v)
    del q, k, v, dO, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("Nq", [1, 4])
def test_decode_largest_accepted_size(fa, Nq):
    """fa_decode with Nk = (2^31 - 1) // 64 cached keys (the largest the C
    ABI accepts): q = 0, so every key has weight 1 / Nk (any K), O is the
    mean of all V rows and lse = ln Nk.  V is a ramp in the key index (even
    columns rising, odd falling, bf16-rounded), so a key range read from the
    wrong place or skipped moves the mean; the expected mean is summed in
    fp64 from the same bf16 tensor, and lse pins the count of keys (fp32:
    1e-5 is about 335 keys of 33.5 million)."""
    import math
    import torch
    props = torch.cuda.get_device_properties(0)
    if props.total_memory < 32 * 2 ** 30:
        pytest.skip("needs about 10 GiB of device memory")
    dev = torch.device("cuda:0")
    Nk = N
    print(f"[decode max size: B=1 H=1 Nq={Nq} Nk={Nk} d={D} bf16, q = 0]", flush=True)
    g = torch.Generator(device=dev)
    g.manual_seed(32)
    k = torch.randn((1, 1, Nk, D), device=dev, dtype=torch.bfloat16, generator=g)
    ramp = torch.arange(Nk, device=dev, dtype=torch.float32) / Nk
    v = torch.empty((1, 1, Nk, D), device=dev, dtype=torch.bfloat16)
    v[0, 0, :, 0::2] = ramp[:, None].to(torch.bfloat16)
    v[0, 0, :, 1::2] = (1.0 - ramp)[:, None].to(torch.bfloat16)
    del ramp
    q = torch.zeros((1, 1, Nq, D), device=dev, dtype=torch.bfloat16)
    o, lse = fa.fa_decode(q, k, v, scale=D ** -0.5)
    torch.cuda.synchronize()
    mean = torch.zeros(D, dtype=torch.float64, device=dev)
    step = 1 << 22
    for r0 in range(0, Nk, step):
        mean += v[0, 0, r0:r0 + step].to(torch.float64).sum(dim=0)
    mean = (mean / Nk).cpu().numpy()
    O = o[0, 0].float().cpu().numpy().astype(np.float64)
    L = lse[0, 0].cpu().numpy().astype(np.float64)
    for i in range(Nq):
        assert_close(f"O row {i}", O[i], mean, TOL["bf16"])
    err_l = np.abs(L - math.log(Nk)).max()
    print(f"  lse: max|err| = {err_l:.3e} (tol 1e-05)", flush=True)
    assert err_l <= 1e-5
    # the rounded mean itself: half of the columns near 0.5 either way
    assert np.abs(O - mean[None]).max() <= 2.0 ** -9 + 1e-6
    del q, k, v, o, lse
    torch.cuda.empty_cache()
