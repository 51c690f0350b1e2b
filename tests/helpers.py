"""Shared helpers for the GPU parity tests (no attention arithmetic here)."""

import numpy as np

TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 2e-2}


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def to_dev(x, dtype):
    """float32 numpy array (already rounded to dtype) -> contiguous GPU tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0", torch_dtype(dtype)).contiguous()


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def max_err(got, ref, mask=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), "non-finite pattern differs"
    if mask is not None:
        fin &= mask
    if not fin.any():
        return 0.0
    return float(np.abs(got[fin] - ref[fin]).max())


def assert_close(name, got, ref, tol, mask=None):
    e = max_err(got, ref, mask)
    print(f"  {name}: max|err| = {e:.3e} (tol {tol:g})", flush=True)
    assert e <= tol, f"{name}: max|err| {e:.3e} > {tol:g}"
