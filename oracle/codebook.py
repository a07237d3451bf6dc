"""Four-level Lloyd-Max codebook for the INT2 history, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The ModelScope/CSDN page (closing section) states that OSCAR's attention-aware
rotation has been combined with a Lloyd-Max codebook to push compression
further, and nothing more.  The reading taken here keeps the 2.25-bit layout
and the per-group scale and zero of the uniform quantizer (``quant``):

  L1  a codebook is four levels in code units, 0 = L[0] < L[1] < L[2] < L[3]
      = 3, so a group's minimum and maximum are still reconstructed exactly;
      L[1], L[2] are multiples of 1/32 (the decode kernels feed 32 L[code] to
      the int8 matrix cores);
  L2  quantization: W1-W5 of the uniform quantizer give c, s and z; then
      t = fl32(fl32(c / s) + z) and the code is the number of thresholds
      b_k = (L[k] + L[k+1]) / 2 strictly below t (a tie goes to the lower
      level; the thresholds are exact in fp32);
  L3  dequantization: x^ = s (L[code] - z);
  L4  calibration: Lloyd-Max with the end levels held at 0 and 3 on the
      normalized values t of a calibration set: each interior level is the
      mean of the values in its cell [b_{k-1}, b_k), the thresholds the
      midpoints; 100 iterations from the uniform levels, then each interior
      level rounded to the nearest multiple of 1/32 (half to even); an empty
      cell keeps its level.  A layer has one codebook for keys and one for
      values, fitted on the normalized values of all its KV heads.

Pinned by ``tests/test_oracle_codebook.py``.
"""

import numpy as np

from .numerics import round_bf16

UNIFORM = np.array([0.0, 1.0, 2.0, 3.0])
GRID = 32.0
ITERATIONS = 100


def thresholds(levels):
    levels = np.asarray(levels, np.float64)
    return (levels[:-1] + levels[1:]) / 2


def check_levels(levels):
    """L1: the constraints a codebook must meet."""
    levels = np.asarray(levels, np.float64)
    return (levels.shape == (4,) and levels[0] == 0.0 and levels[3] == 3.0 and
            np.all(np.diff(levels) > 0) and np.all(levels * GRID == np.round(levels * GRID)))


def _normalize(x, r, tau, group_size):
    """W1-W5 of the uniform quantizer, then t = fl32(fl32(c / s) + z).
    Returns (t [N, D], s [N, D/G], z [N, D/G]) as float32."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    y = x.astype(np.float32) if r is None else (x @ np.asarray(r, np.float32).astype(np.float64)).astype(np.float32)
    t32 = np.float32(tau)
    c = np.minimum(np.maximum(y, -t32), t32).astype(np.float32)
    cg = c.reshape(n, d // group_size, group_size)
    mn, mx = cg.min(axis=2), cg.max(axis=2)
    dlt = (mx - mn).astype(np.float32)
    s = round_bf16((dlt / np.float32(3.0)).astype(np.float32))
    s = np.where((dlt == 0) | (s == 0), np.float32(1.0), s).astype(np.float32)
    z = round_bf16(((-mn) / s).astype(np.float32))
    t = ((cg / s[:, :, None]).astype(np.float32) + z[:, :, None]).astype(np.float32)
    return t.reshape(n, d), s, z


def normalized_values(x, r, tau, group_size):
    """The normalized values t [N, D] of x [N, D] (r None: no rotation)."""
    return _normalize(x, r, tau, group_size)[0]


def lloyd_max_unrounded(t, iterations=ITERATIONS):
    """L4 before the final rounding to the 1/32 grid."""
    t = np.asarray(t, np.float64).ravel()
    lv = UNIFORM.copy()
    for _ in range(iterations):
        b = thresholds(lv)
        for k in (1, 2):
            cell = t[(t >= b[k - 1]) & (t < b[k])]
            if cell.size:
                lv[k] = cell.mean()
    return lv


def lloyd_max(t, iterations=ITERATIONS):
    """L4: the codebook for normalized values t (any shape)."""
    lv = lloyd_max_unrounded(t, iterations)
    lv[1:3] = np.round(lv[1:3] * GRID) / GRID
    return lv


def encode(t, levels):
    """L2: codes of normalized values t."""
    b = thresholds(levels).astype(np.float32)
    t = np.asarray(t, np.float32)
    return ((t[..., None] > b).sum(axis=-1)).astype(np.uint8)


def quantize_tokens(x, r, tau, group_size, levels):
    """L2 for N token vectors of one KV head: codes [N, D] uint8 and the
    bf16 scale and zero [N, D/G] (float32 holding bf16 values), as
    ``quant.quantize_tokens`` returns them."""
    t, s, z = _normalize(x, r, tau, group_size)
    return encode(t, levels), s, z


def dequantize(codes, s, z, group_size, levels):
    """L3: x^ = s (L[code] - z) per group, fp64."""
    lv = np.asarray(levels, np.float64)[np.asarray(codes, np.int64)]
    shp = lv.shape
    lg = lv.reshape(shp[:-1] + (shp[-1] // group_size, group_size))
    out = np.asarray(s, np.float64)[..., None] * (lg - np.asarray(z, np.float64)[..., None])
    return out.reshape(shp)
