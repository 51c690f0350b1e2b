"""Shared helpers for the GPU parity tests (no attention arithmetic here)."""

import numpy as np

class Tol(float):
    """A max-abs-error gate for outputs stored in ``dtype``."""

    def __new__(cls, value, dtype):
        t = super().__new__(cls, value)
        t.dtype = dtype
        return t


TOL = {"f32": Tol(1e-5, "f32"), "f16": Tol(1e-2, "f16"), "bf16": Tol(2e-2, "bf16")}

# stored significand bits (without the hidden bit) and smallest normal
# exponent of each output dtype
_MANT = {"f32": 23, "f16": 10, "bf16": 7}
_EMIN = {"f32": -126, "f16": -14, "bf16": -126}


def half_spacing(ref, dtype):
    """Half the distance between neighbouring ``dtype`` values at |ref|: the
    error that storing the exact result in that dtype can cost.  Below the
    dtype's normal range the spacing stays that of its subnormals (fp16:
    2^-24 under 2^-14)."""
    a = np.maximum(np.abs(np.asarray(ref, dtype=np.float64)), np.finfo(np.float64).tiny)
    e = np.maximum(np.floor(np.log2(a)).astype(np.int64), _EMIN[dtype])
    return np.ldexp(1.0, e - _MANT[dtype] - 1)


def allowance(ref, tol):
    """Per-element gate: tol, widened by the output dtype's half-spacing only
    where that half-spacing alone reaches tol (bf16 |x| >= 8, fp16 |x| >= 32,
    fp32 |x| >= 256), since there even the correctly rounded exact value can
    miss an absolute gate of tol."""
    if not isinstance(tol, Tol):
        return tol
    u = half_spacing(ref, tol.dtype)
    return np.where(u >= float(tol), float(tol) + u, float(tol))


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
    """max |got - ref| <= tol (per element: tol widened as in ``allowance``
    where the output dtype cannot hold values to within tol)."""
    e = max_err(got, ref, mask)
    print(f"  {name}: max|err| = {e:.3e} (tol {float(tol):g})", flush=True)
    if e <= tol:
        return
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref) if mask is None else np.isfinite(ref) & mask
    err, allow = np.abs(got[fin] - ref[fin]), allowance(ref[fin], tol)
    bad = err > allow
    assert not bad.any(), (f"{name}: max|err| {e:.3e} > {float(tol):g} (worst beyond the "
                           f"dtype allowance: {float((err - allow)[bad].max()):.3e})")
    print(f"  {name}: within the output dtype's rounding allowance above the gate", flush=True)
