"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no attention arithmetic: it only draws random numbers,
rounds them to the storage dtype, and builds the masks' structure (lengths,
block patterns) and the sampled row sets.  Both the oracle and the HIP path
consume exactly the arrays produced here.

Workloads (shapes of the workloads the pages quote; the data is synthetic
N(0, 1) because the datasets and trained models are not available):

* ``fp32_small``   B=1  H=1  N=128   d=64  fp32, no mask, forward only
* ``bert_large``   B=8  H=16 N=512   d=64  fp16, key padding, lengths U[256,512]
  (BERT-large at sequence length 512)
* ``gpt2_small``   B=8  H=12 N=1024  d=64  bf16, causal (GPT-2 at 1K)
* ``long_causal``  B=1  H=16 N=16384 d=64  bf16, causal (Path-X length 16K)
* ``long_causal_d128`` the same at d=128
* ``block_sparse`` B=1  H=8  N=65536 d=64  bf16, 128x128 block mask: a band of
  3 blocks either side of the diagonal plus seeded random off-band blocks to
  about 5 % density (Path-256 length 64K)
* ``sweep_{causal,full}_{1,2,4,8,16}k``  H=16, N=1K..16K, B=16384/N, d=64,
  bf16 (the metric's sequence-length range at a fixed token count)

Random streams: ``numpy.random.Generator(PCG64(SeedSequence(seed)))`` spawned
into independent child streams for q, k, v, dO, lengths/mask and samples.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool = False
    key_padding: bool = False
    block_sparse: bool = False
    fwd_only: bool = False
    seed: int = 0
    sample_rows: int | None = None  # sampled query rows (None: check all)
    sample_keys: int | None = None  # sampled key rows for dK/dV
    sample_key_heads: int = 2       # heads the key-row samples are drawn from
    sample_key_blocks: int | None = None  # if set: key rows drawn inside this
                                          # many random 128-key blocks

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    "fp32_small": Workload("fp32_small", 1, 1, 128, 64, "f32", fwd_only=True, seed=1),
    "bert_large": Workload("bert_large", 8, 16, 512, 64, "f16", key_padding=True, seed=2),
    "gpt2_small": Workload("gpt2_small", 8, 12, 1024, 64, "bf16", causal=True, seed=3),
    "long_causal": Workload("long_causal", 1, 16, 16384, 64, "bf16", causal=True, seed=4,
                            sample_rows=256, sample_keys=64),
    "long_causal_d128": Workload("long_causal_d128", 1, 16, 16384, 128, "bf16", causal=True,
                                 seed=4, sample_rows=256, sample_keys=64),
    "long_causal_d32": Workload("long_causal_d32", 1, 16, 16384, 32, "bf16", causal=True,
                                seed=4, sample_rows=256, sample_keys=64),
    "long_causal_d96": Workload("long_causal_d96", 1, 16, 16384, 96, "bf16", causal=True,
                                seed=4, sample_rows=256, sample_keys=64),
    "block_sparse": Workload("block_sparse", 1, 8, 65536, 64, "bf16", block_sparse=True,
                             seed=5, sample_rows=256, sample_keys=64, sample_key_heads=1,
                             sample_key_blocks=8),
}

# Sequence-length sweep: the same 16384 tokens per head at every length
# (B = 16384 / N), H = 16, d = 64, bf16, causal and non-causal; seed
# 100 + log2 N.
SWEEP_N = (1024, 2048, 4096, 8192, 16384)
SWEEP = tuple(
    Workload(f"sweep_{'causal' if c else 'full'}_{n // 1024}k", 16384 // n, 16, n, 64, "bf16",
             causal=c, seed=100 + int(math.log2(n)), sample_rows=256, sample_keys=64)
    for c in (True, False) for n in SWEEP_N)
WORKLOADS.update({w.name: w for w in SWEEP})


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype (round to nearest even).

    Returns float32 arrays holding exactly representable values, so that a
    later conversion to the device dtype is exact.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
        return u.astype(np.uint32).view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


def band_plus_random_block_mask(nblk: int, band: int, density: float,
                                rng: np.random.Generator) -> np.ndarray:
    """uint8 [nblk, nblk]: |i - j| <= band always on; off-band blocks drawn
    i.i.d. Bernoulli(p) with p chosen so the expected total density is
    ``density``."""
    i = np.arange(nblk)
    inband = np.abs(i[:, None] - i[None, :]) <= band
    n_band = int(inband.sum())
    p = (density * nblk * nblk - n_band) / (nblk * nblk - n_band)
    p = min(max(p, 0.0), 1.0)
    off = rng.random((nblk, nblk)) < p
    return (inband | off).astype(np.uint8)


def make_inputs(w: Workload, seed: int | None = None, N: int | None = None,
                B: int | None = None, H: int | None = None, d: int | None = None):
    """Seeded inputs for a workload (optionally with overridden sizes).

    Returns a dict of numpy arrays: q, k, v, dO (float32, values already
    rounded to ``w.dtype``), key_len (int32 [B] or None), block_mask
    (uint8 or None), plus the sizes.
    """
    seed = w.seed if seed is None else seed
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    d = w.d if d is None else d
    sq, sk, sv, sdo, smask, _ = _streams(seed, 6)
    shape = (B, H, N, d)
    q = round_to_dtype(sq.standard_normal(shape, dtype=np.float32), w.dtype)
    k = round_to_dtype(sk.standard_normal(shape, dtype=np.float32), w.dtype)
    v = round_to_dtype(sv.standard_normal(shape, dtype=np.float32), w.dtype)
    dO = round_to_dtype(sdo.standard_normal(shape, dtype=np.float32), w.dtype)
    key_len = None
    if w.key_padding:
        lo, hi = min(256, N), N if N < 512 else 512
        lo = max(1, min(lo, hi))
        key_len = smask.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    block_mask = None
    if w.block_sparse:
        nblk = (N + 127) // 128
        block_mask = band_plus_random_block_mask(nblk, 3, 0.05, smask)
    return dict(q=q, k=k, v=v, dO=dO, key_len=key_len, block_mask=block_mask,
                B=B, H=H, N=N, d=d, scale=1.0 / math.sqrt(d), dtype=w.dtype,
                causal=w.causal)


def make_decode_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, seed: int):
    """Seeded decode inputs: q [B, H, Nq, d] against k, v [B, H, Nk, d]
    (float32 arrays holding values rounded to ``dtype``), N(0, 1) like the
    other workloads."""
    sq, sk, sv = _streams(seed, 3)
    q = round_to_dtype(sq.standard_normal((B, H, Nq, d), dtype=np.float32), dtype)
    k = round_to_dtype(sk.standard_normal((B, H, Nk, d), dtype=np.float32), dtype)
    v = round_to_dtype(sv.standard_normal((B, H, Nk, d), dtype=np.float32), dtype)
    return dict(q=q, k=k, v=v, scale=1.0 / math.sqrt(d), dtype=dtype)


def sample_rows(w: Workload, H: int, N: int, n: int, seed: int | None = None):
    """(h, i) query rows: n drawn uniformly without replacement over all
    heads and positions, plus the forced rows (0, 0) and (H-1, N-1)."""
    rng = _streams(w.seed if seed is None else seed, 6)[5]
    flat = rng.choice(H * N, size=min(n, H * N), replace=False)
    pairs = {(int(f // N), int(f % N)) for f in flat}
    pairs |= {(0, 0), (H - 1, N - 1)}
    return sorted(pairs)


def sample_key_rows(w: Workload, H: int, N: int, n: int, seed: int | None = None):
    """(h, j) key rows for dK/dV checks: ``w.sample_key_heads`` heads drawn
    at random, n key positions spread over them (inside
    ``w.sample_key_blocks`` random 128-key blocks when that is set, which
    bounds the oracle's work under a block mask), plus j = 0 and j = N-1 in
    the first drawn head."""
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence((w.seed if seed is None else seed, 77))))
    nh = min(w.sample_key_heads, H)
    heads = sorted(int(h) for h in rng.choice(H, size=nh, replace=False))
    pairs = set()
    per = max(1, n // nh)
    for h in heads:
        if w.sample_key_blocks:
            nb = (N + 127) // 128
            blocks = rng.choice(nb, size=min(w.sample_key_blocks, nb), replace=False)
            pool = np.concatenate([np.arange(bk * 128, min(N, bk * 128 + 128)) for bk in blocks])
        else:
            pool = np.arange(N)
        for j in rng.choice(pool, size=min(per, pool.size), replace=False):
            pairs.add((h, int(j)))
    pairs |= {(heads[0], 0), (heads[0], N - 1)}
    return sorted(pairs)
