"""Pins for the oracle's four-level Lloyd-Max codebook (oracle/codebook.py):
closed-form fixed points, symmetry, the centroid condition, an exhaustive
search on the 1/32 grid, brute-force nearest-level encoding, and agreement
with the uniform quantizer for the uniform codebook."""

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import quant


def test_uniform_density_gives_uniform_levels():
    # a deterministic uniform density on [0, 3]: the uniform quantizer is the
    # fixed point (each interior cell [k - 1/2, k + 1/2) has mean k)
    t = (np.arange(30000) + 0.5) / 10000
    assert np.array_equal(cb.lloyd_max(t), [0.0, 1.0, 2.0, 3.0])


def test_symmetric_density_gives_symmetric_levels():
    rng = np.random.default_rng(1)
    half = np.clip(rng.normal(1.5, 0.6, 20000), 0, 3)
    t = np.concatenate([half, 3 - half])
    lv = cb.lloyd_max_unrounded(t)
    assert abs(lv[1] + lv[2] - 3) < 1e-9
    r = cb.lloyd_max(t)
    assert r[1] + r[2] == 3 and r[1] > 1  # mass near the middle pulls the levels inward
    assert cb.check_levels(r)


def test_centroid_condition_at_the_fixed_point():
    rng = np.random.default_rng(2)
    t = np.clip(rng.normal(1.4, 0.7, 50000), -0.2, 3.2)
    lv = cb.lloyd_max_unrounded(t, iterations=400)
    b = cb.thresholds(lv)
    for k in (1, 2):
        cell = t[(t >= b[k - 1]) & (t < b[k])]
        assert abs(cell.mean() - lv[k]) < 1e-10


def _mse(t, lv):
    q = np.asarray(lv)[cb.encode(t, lv)]
    return np.mean((t - q) ** 2)


def test_lloyd_optimum_matches_exhaustive_search_on_the_grid():
    """A unimodal density: the fixed-end Lloyd-Max levels, rounded to the
    grid, are within one grid step of the best pair found by exhaustive
    search over all interior levels on the 1/32 grid."""
    rng = np.random.default_rng(3)
    t = np.clip(rng.normal(1.5, 0.55, 4000), 0, 3).astype(np.float32)
    grid = np.arange(1, 96) / 32.0
    best, best_lv = np.inf, None
    for i, a in enumerate(grid):
        for c in grid[i + 1:]:
            lv = np.array([0.0, a, c, 3.0])
            m = _mse(t, lv)
            if m < best:
                best, best_lv = m, lv
    lv = cb.lloyd_max(t)
    assert np.all(np.abs(lv - best_lv) <= 1 / 32 + 1e-12), (lv, best_lv)
    assert _mse(t, lv) <= best * 1.001


def test_encode_is_nearest_level_ties_down():
    lv = np.array([0.0, 1.125, 1.90625, 3.0])
    rng = np.random.default_rng(4)
    b = cb.thresholds(lv)
    t = np.concatenate([rng.uniform(-0.3, 3.3, 2000), b, np.nextafter(b, 9), np.nextafter(b, -9), [0.0, 3.0]])
    t = t.astype(np.float32)
    codes = cb.encode(t, lv)
    for x, c in zip(t.tolist(), codes.tolist()):
        d = [abs(x - l) for l in lv]
        m = min(d)
        want = min(k for k in range(4) if d[k] == m)  # the lower level on a tie
        assert c == want, (x, c, want)


def test_uniform_codebook_equals_the_uniform_quantizer():
    """With levels 0, 1, 2, 3 the codebook quantizer is W1-W7's except where
    t falls exactly on k + 1/2 (round-half-even there, ties down here)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    r, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    r = r.astype(np.float32)
    c1, s1, z1 = cb.quantize_tokens(x, r, np.float32(2.5), 64, cb.UNIFORM)
    c0, s0, z0 = quant.quantize_tokens(x, r, np.float32(2.5), 64)
    assert np.array_equal(s1, s0) and np.array_equal(z1, z0)
    t = cb.normalized_values(x, r, np.float32(2.5), 64)
    tie = (t * 2) == np.round(t * 2)
    tie &= (np.round(t * 2) % 2 == 1)
    assert np.array_equal(c1[~tie], c0[~tie])


def test_dequantize_reconstructs_levels_exactly():
    lv = np.array([0.0, 0.96875, 2.125, 3.0])
    rng = np.random.default_rng(6)
    n, d, g = 8, 64, 32
    codes = rng.integers(0, 4, (n, d)).astype(np.uint8)
    codes[:, 0], codes[:, 1], codes[:, 32], codes[:, 33] = 0, 3, 0, 3  # every group spans 0..3
    s = np.full((n, d // g), 0.5, np.float32)
    z = np.full((n, d // g), 1.0, np.float32)
    x = cb.dequantize(codes, s, z, g, lv)
    assert np.array_equal(x, 0.5 * (lv[codes] - 1.0))
    # quantizing the reconstruction (no rotation, no clip) gives the codes back
    c2, s2, z2 = cb.quantize_tokens(x, None, np.inf, g, lv)
    assert np.array_equal(c2, codes) and np.all(s2 == 0.5) and np.all(z2 == 1.0)


@pytest.mark.parametrize("lv,ok", [([0, 1, 2, 3], True), ([0, 1.03125, 1.96875, 3], True),
                                   ([0, 1.01, 2, 3], False), ([0, 2, 1, 3], False), ([0.5, 1, 2, 3], False),
                                   ([0, 1, 2, 2.96875], False)])
def test_level_constraints(lv, ok):
    assert bool(cb.check_levels(lv)) == ok
