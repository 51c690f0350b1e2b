"""The library's launches inside a captured HIP graph.

fa_fwd and the three backward launches allocate nothing and issue no
memsets (the maxima are cleared by a kernel), so a caller can capture them.
A graph of forward + backward on preallocated buffers is replayed several
times with eager work and synchronisations between the replays; every replay
must equal the eager result bit for bit (the kernels are deterministic).
"""

import pytest

from helpers import to_dev
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def test_forward_backward_replay_in_a_graph():
    import torch

    import io_aware_tiled_05_amd as fa
    fa.load()
    x = make_inputs(Workload("graph", 2, 4, 600, 64, "bf16", causal=True, seed=31))
    q, k, v, dO = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "dO"))
    B, H, N, d = q.shape
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d) // 4 + 64, dtype=torch.float32,
                     device=q.device)

    def step():
        fa.fa_fwd(q, k, v, scale=x["scale"], causal=True, out=o, lse=lse)
        fa.fa_bwd(q, k, v, o, lse, dO, scale=x["scale"], causal=True, dq=dq, dk=dk, dv=dv,
                  workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager result"
