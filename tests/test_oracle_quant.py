"""Pins for the oracle quantizer (W1-W7) against brute force and closed-form
properties of 4-level asymmetric min-max quantization."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import dequantize, quantize_tokens
from oracle.numerics import round_bf16


def _groups(rng, n, d, outliers=True):
    x = rng.standard_normal((n, d)).astype(np.float32)
    if outliers:
        x[:, rng.choice(d, 4, replace=False)] *= 20
    return round_bf16(x)


@pytest.mark.parametrize("gs", [32, 64, 128])
def test_codes_are_nearest_level(gs):
    """Each code is the argmin over the 4 levels s (k - z) of |c - level|,
    computed exactly in fp64 with the stored (bf16) scale and zero; a
    different choice is only allowed where c lies within fp32 rounding of the
    midpoint between two levels (the pages fix no finer decision rule)."""
    rng = np.random.default_rng(gs)
    x = _groups(rng, 4000, 128)
    codes, s, z, y, c = quantize_tokens(x, None, np.float32(np.inf), gs, return_intermediate=True)
    ng = 128 // gs
    cg = c.reshape(-1, ng, gs).astype(np.float64)
    lv = s[:, :, None, None].astype(np.float64) * (np.arange(4)[None, None, None, :] - z[:, :, None, None])
    err = np.abs(cg[..., None] - lv)  # [n, ng, gs, 4]
    best = err.argmin(axis=-1)
    got = codes.reshape(-1, ng, gs)
    mism = best != got
    if mism.any():
        e_got = np.take_along_axis(err, got[..., None].astype(np.int64), -1)[..., 0]
        e_best = err.min(-1)
        slack = 4 * np.finfo(np.float32).eps * (np.abs(cg) + s[:, :, None] * (3 + np.abs(z[:, :, None])))
        assert np.all((e_got - e_best)[mism] <= slack[mism])
    assert mism.mean() < 1e-4


def test_scale_zero_closed_form_bounds():
    rng = np.random.default_rng(5)
    x = _groups(rng, 3000, 128)
    codes, s, z, y, c = quantize_tokens(x, None, np.float32(np.inf), 64, return_intermediate=True)
    cg = c.reshape(-1, 2, 64).astype(np.float64)
    mn, mx = cg.min(-1), cg.max(-1)
    exact_s = (mx - mn) / 3
    # s is (mx - mn)/3 up to one fp32 and one bf16 rounding
    assert np.all(np.abs(s - exact_s) <= exact_s * (2**-8 + 2**-23))
    # level 0 sits at the group minimum and level 3 at the maximum, up to the
    # bf16 rounding of z (half an ulp of z, in code units) and of s
    dz = np.abs(z) * 2**-8 + 1e-30
    assert np.all(np.abs(s * (0 - z) - mn) <= s * dz + 1e-6 * np.abs(mn))
    assert np.all(np.abs(s * (3 - z) - mx) <= s * dz + 3 * np.abs(s - exact_s) + 1e-6 * np.abs(mx))


def test_min_max_codes_and_four_levels():
    rng = np.random.default_rng(7)
    x = _groups(rng, 3000, 128)
    codes, s, z, y, c = quantize_tokens(x, None, np.float32(np.inf), 128, return_intermediate=True)
    assert np.all(np.abs(z) < 64)
    i_min, i_max = c.argmin(1), c.argmax(1)
    ar = np.arange(len(c))
    assert np.all(codes[ar, i_min] == 0)
    assert np.all(codes[ar, i_max] == 3)
    deq = dequantize(codes, s, z, 128)
    for row in deq[:200]:
        assert len(np.unique(row)) <= 4
    # reconstruction error within half a level plus the bf16 rounding of z
    err = np.abs(deq - c)
    assert np.all(err <= s[:, 0:1] * (0.5 + np.abs(z) * 2**-8) + 1e-5)


def test_ties_to_even_and_constant_group():
    # group spanning exactly [0, 3]: s = 1, z = 0; midpoints 0.5, 1.5, 2.5
    x = np.array([[0, 3, 0.5, 1.5, 2.5, 1, 2, 0.25]], np.float32)
    codes, s, z = quantize_tokens(x, None, np.float32(np.inf), 8)
    assert s[0, 0] == 1 and z[0, 0] == 0
    assert list(codes[0]) == [0, 3, 0, 2, 2, 1, 2, 0]
    # constant group: d = 0 -> s = 1, z = -value, every code rne(0) = 0
    x = np.full((1, 8), 5.0, np.float32)
    codes, s, z = quantize_tokens(x, None, np.float32(np.inf), 8)
    assert s[0, 0] == 1 and z[0, 0] == -5 and np.all(codes == 0)
    assert np.all(dequantize(codes, s, z, 8) == 5.0)


def test_clip_applies_after_rotation():
    rng = np.random.default_rng(9)
    x = _groups(rng, 64, 64)
    r = np.linalg.qr(rng.standard_normal((64, 64)))[0].astype(np.float32)
    tau = np.float32(2.5)
    codes, s, z, y, c = quantize_tokens(x, r, tau, 64, return_intermediate=True)
    assert np.all(np.abs(c) <= tau)
    inside = np.abs(y) <= tau
    assert np.array_equal(c[inside], y[inside])
    assert np.all(c[y > tau] == tau) and np.all(c[y < -tau] == -tau)


def test_rotation_is_row_vector_times_r_within_one_ulp():
    """y = x R (row vector on the left), within 1 fp32 ulp of the exact
    rational product; the transposed product would fail."""
    rng = np.random.default_rng(13)
    x = _groups(rng, 3, 16)
    r = rng.standard_normal((16, 16)).astype(np.float32)
    _, _, _, y, _ = quantize_tokens(x, r, np.float32(np.inf), 16, return_intermediate=True)
    for i in range(3):
        for j in range(16):
            exact = sum(Fraction(float(x[i, k])) * Fraction(float(r[k, j])) for k in range(16))
            ulp = np.spacing(np.float32(abs(float(exact))))
            assert abs(float(y[i, j]) - float(exact)) <= ulp
    ident = quantize_tokens(x, np.eye(16, dtype=np.float32), np.float32(np.inf), 16, True)[3]
    assert np.array_equal(ident, x)
