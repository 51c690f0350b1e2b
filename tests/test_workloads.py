"""The seeded input generators (no attention arithmetic lives there)."""

import numpy as np
import pytest

from workloads import (WORKLOADS, band_plus_random_block_mask, make_inputs,
                       round_to_dtype, sample_key_rows, sample_rows)


def test_round_to_dtype_matches_torch_rne():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]  # ties
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        ref = torch.from_numpy(x).to(tdt).float().numpy()
        np.testing.assert_array_equal(round_to_dtype(x, dt), ref)
    np.testing.assert_array_equal(round_to_dtype(x, "f32"), x)


def test_inputs_are_seeded_and_shaped():
    w = WORKLOADS["bert_large"]
    a = make_inputs(w, N=64, B=3, H=2)
    b = make_inputs(w, N=64, B=3, H=2)
    for key in ("q", "k", "v", "dO", "key_len"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["q"].shape == (3, 2, 64, 64)
    full = make_inputs(w, H=1, N=512)
    assert full["key_len"].min() >= 256 and full["key_len"].max() <= 512
    assert not np.array_equal(a["q"], a["k"])


def test_block_mask_structure():
    bm = band_plus_random_block_mask(512, 3, 0.05, np.random.default_rng(5))
    i = np.arange(512)
    assert np.all(bm[np.abs(i[:, None] - i[None, :]) <= 3] == 1)
    assert 0.045 < bm.mean() < 0.055


def test_samples():
    w = WORKLOADS["long_causal"]
    r = sample_rows(w, 16, 16384, 256)
    assert (0, 0) in r and (15, 16383) in r and len(r) >= 256
    kr = sample_key_rows(w, 16, 16384, 64)
    assert len({h for h, _ in kr}) <= w.sample_key_heads and len(kr) >= 64
