"""The Lloyd-Max level helper used by the non-affine study (host code, no GPU).

Pins: the two end levels stay at 0 and M - 1 (every min-max normalised stream
has values there); the levels increase; for a symmetric source they are
symmetric about (M - 1) / 2 up to sampling noise; and nearest rounding to them
has a lower mean squared error than rounding to the affine grid on a fresh
sample (a Lloyd-Max quantiser minimises that error for the source it was
fitted on)."""

import numpy as np
import pytest

from kv_cache_entropy_amd.studies import lloyd_max_levels


@pytest.mark.parametrize("M", [4, 6, 8])
def test_lloyd_max_levels(M):
    n = 256
    lv = np.array(lloyd_max_levels(M, n, streams=1500, iters=40, seed=1))
    assert lv[0] == 0.0 and lv[-1] == M - 1
    assert np.all(np.diff(lv) > 0)
    assert np.max(np.abs(lv + lv[::-1] - (M - 1))) < 0.02
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1500, n))
    u = (x - x.min(1, keepdims=True)) / (x.max(1, keepdims=True) - x.min(1, keepdims=True)) * (M - 1)
    mse = lambda v: np.min((u[..., None] - v) ** 2, axis=-1).mean()
    assert mse(lv) < 0.9 * mse(np.arange(M, dtype=float))
