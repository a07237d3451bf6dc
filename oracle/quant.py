"""Write path of one token-head vector: rotate, clip, quantize, pack.

Follows the MarkTechPost article, "The Serving System" (each token is rotated,
clipped to a calibration-derived threshold, then quantized with per-token
asymmetric INT2 in groups of G channels), the ModelScope/CSDN page's design
section (four 2-bit values packed per byte; dequantization by scale and zero
point), and the article's "Why INT2 KV Cache Quantization is Hard" section
(four representable levels).

Steps (the pages leave the exact formulas open; the readings taken are):
  W1  y = x R in fp64, rounded once to fp32 (no R: y = x exactly).
  W2  c = min(max(y, -tau), +tau) in fp32.
  W3  per group of G consecutive channels: mn = min c, mx = max c.
  W4  d = fl32(mx - mn); s = bf16(fl32(d / 3)); if d == 0 or s == 0 then s = 1.
  W5  z = bf16(fl32(-mn / s))         (zero point in code units: x^ = s (q - z)).
  W6  q = clamp(rne(fl32(fl32(c / s) + z)), 0, 3), IEEE fp32 divide, no FMA.
  W7  4 codes per byte, channel 4b+k in bits 2k..2k+1 of byte b (LSB first).
"""

import numpy as np

from .numerics import round_bf16


def quantize_tokens(x, r, tau, group_size: int, return_intermediate: bool = False):
    """Quantize N token vectors of one KV head.

    x: [N, D] bf16 values (any float dtype); r: [D, D] float32 rotation or
    None; tau: fp32 clip threshold (np.inf disables clipping).
    Returns codes [N, D] uint8, scale [N, D/G] and zero [N, D/G] as float32
    holding bf16 values.  With ``return_intermediate`` also returns the fp32
    rotated values y and the clipped values c.
    """
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    assert d % group_size == 0
    # W1
    if r is None:
        y = x.astype(np.float32)
    else:
        y = (x @ np.asarray(r, dtype=np.float32).astype(np.float64)).astype(np.float32)
    # W2
    t32 = np.float32(tau)
    c = np.minimum(np.maximum(y, -t32), t32).astype(np.float32)
    # W3
    cg = c.reshape(n, d // group_size, group_size)
    mn = cg.min(axis=2)
    mx = cg.max(axis=2)
    # W4
    dlt = (mx - mn).astype(np.float32)
    s = round_bf16((dlt / np.float32(3.0)).astype(np.float32))
    s = np.where((dlt == 0) | (s == 0), np.float32(1.0), s).astype(np.float32)
    # W5
    z = round_bf16(((-mn) / s).astype(np.float32))
    # W6
    t = ((cg / s[:, :, None]).astype(np.float32) + z[:, :, None]).astype(np.float32)
    codes = np.clip(np.rint(t), 0, 3).astype(np.uint8).reshape(n, d)
    if return_intermediate:
        return codes, s, z, y, c
    return codes, s, z


def quantize_token(x, r, tau, group_size: int):
    """One token-head vector [D]; see ``quantize_tokens``."""
    codes, s, z = quantize_tokens(np.asarray(x)[None, :], r, tau, group_size)
    return codes[0], s[0], z[0]


def dequantize(codes, s, z, group_size: int) -> np.ndarray:
    """x^ = s (q - z) per group, in fp64.  codes [..., D], s/z [..., D/G]."""
    codes = np.asarray(codes, dtype=np.float64)
    shp = codes.shape
    cg = codes.reshape(shp[:-1] + (shp[-1] // group_size, group_size))
    out = np.asarray(s, np.float64)[..., None] * (cg - np.asarray(z, np.float64)[..., None])
    return out.reshape(shp)


def pack_codes(codes) -> np.ndarray:
    """[..., D] codes in 0..3 -> [..., D/4] bytes, channel 4b+k at bits 2k."""
    c = np.asarray(codes, dtype=np.uint8)
    shp = c.shape
    c = c.reshape(shp[:-1] + (shp[-1] // 4, 4))
    out = np.zeros(c.shape[:-1], dtype=np.uint8)
    for k in range(4):
        out |= (c[..., k] & 3) << (2 * k)
    return out


def unpack_codes(packed) -> np.ndarray:
    """Inverse of ``pack_codes``."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.stack([(p >> (2 * k)) & 3 for k in range(4)], axis=-1)
    return out.reshape(p.shape[:-1] + (p.shape[-1] * 4,)).astype(np.uint8)
