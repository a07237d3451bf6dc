"""Pins for the oracle's rounding helpers and the 4-codes-per-byte packing."""

import numpy as np
import torch

from oracle import pack_codes, round_bf16, unpack_codes


def test_bf16_rounding_matches_torch():
    # torch's CPU float->bfloat16 conversion is an independent RNE implementation
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 10 ** rng.uniform(-30, 30, 200_000).astype(np.float32),
        rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = round_bf16(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_bf16_ties_go_to_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: the even one (1) wins
    assert round_bf16(np.float32(1 + 2**-8)) == np.float32(1.0)
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert round_bf16(np.float32(1 + 3 * 2**-8)) == np.float32(1 + 2**-6)
    assert round_bf16(np.float32(1 + 2**-8 + 2**-20)) == np.float32(1 + 2**-7)
    assert round_bf16(np.float32(-1 - 2**-8)) == np.float32(-1.0)


def test_pack_unpack_exhaustive_bytes():
    allbytes = np.arange(256, dtype=np.uint8)
    codes = unpack_codes(allbytes[:, None])  # [256, 4]
    assert codes.shape == (256, 4)
    # byte b holds code k in bits 2k..2k+1 (LSB first)
    for b in range(256):
        assert [int(c) for c in codes[b]] == [(b >> (2 * k)) & 3 for k in range(4)]
    assert np.array_equal(pack_codes(codes)[:, 0], allbytes)


def test_pack_roundtrip_random_rows():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 4, size=(50, 8, 128), dtype=np.uint8)
    packed = pack_codes(codes)
    assert packed.shape == (50, 8, 32)
    assert np.array_equal(unpack_codes(packed), codes)
