"""CPU tests: the test-side pool layout against the bit positions include/oscar.h
documents, and the C ABI's loading, exports and host-side validation (no
kernel is launched: every call here fails validation before any HIP call)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import pool_io
from oracle.numerics import round_bf16

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oscar.h")


def test_int2_layout_bit_positions():
    d, ng = 128, 1
    kc = np.zeros((1, 16, d), np.uint8)
    vc = np.zeros((1, 16, d), np.uint8)
    z = np.zeros((1, 16, ng), np.float32)
    kc[0, 5, 70] = 3  # token 5, channel 70 = 1*64 + 0*16 + 6 -> record 5, K word 1, bits 12..13
    vc[0, 6, 37] = 2  # token 6 = 4*1 + 2, channel 37 = (4*0 + 2)*16 + 5 -> record 21, V word 0, bits 10..11
    blk = pool_io.pack_int2_blocks(kc, z, z, vc, z, z)[0]
    words = blk[: 8 * d].view("<u4").reshape(64, 4)
    assert words[5, 1] == 3 << 12
    assert words[21, 2] == 2 << 10
    assert np.count_nonzero(words) == 2
    # scales: token 9 (quad 2, slot 1) K scale/zero, V scale
    ks = np.zeros((1, 16, 1), np.float32)
    ks[0, 9, 0] = 1.5
    vs = np.zeros((1, 16, 1), np.float32)
    vs[0, 9, 0] = -2.0
    blk = pool_io.pack_int2_blocks(kc * 0, ks, z, vc * 0, vs, z)[0]
    sc = blk[8 * d:].view("<u2")
    assert sc[2 * 16 + 0 * 8 + 1 * 2 + 0] == 0x3FC0  # bf16(1.5)
    assert sc[2 * 16 + 1 * 8 + 1 * 2 + 0] == 0xC000  # bf16(-2)
    assert blk.size == 8 * d + 128 * ng == 1152


@pytest.mark.parametrize("d,ng", [(128, 1), (128, 2), (64, 1)])
def test_int2_roundtrip(d, ng):
    rng = np.random.default_rng(d + ng)
    n = 7
    kc, vc = (rng.integers(0, 4, (n, 16, d), dtype=np.uint8) for _ in range(2))
    sc = [round_bf16(rng.standard_normal((n, 16, ng)).astype(np.float32)) for _ in range(4)]
    blocks = pool_io.pack_int2_blocks(kc, sc[0], sc[1], vc, sc[2], sc[3])
    assert blocks.shape == (n, 8 * d + 128 * ng)
    out = pool_io.unpack_int2_blocks(blocks, d, ng)
    for a, b in zip(out, (kc, sc[0], sc[1], vc, sc[2], sc[3])):
        assert np.array_equal(a, b)
    # 4 codes per byte: the code bytes carry exactly 2 bits per code
    assert blocks[:, : 8 * d].size * 8 == 2 * kc.size + 2 * vc.size


def test_bf16_layout():
    rng = np.random.default_rng(0)
    d = 64
    k = round_bf16(rng.standard_normal((3, 16, d)).astype(np.float32))
    v = round_bf16(rng.standard_normal((3, 16, d)).astype(np.float32))
    blk = pool_io.pack_bf16_blocks(k, v)
    u = blk[0].view("<u2")
    assert u[5 * d + 7] == pool_io.bf16_bits(k[0, 5, 7])  # K [token][channel]
    assert u[16 * d + (9 // 4) * d * 4 + 7 * 4 + 9 % 4] == pool_io.bf16_bits(v[0, 9, 7])  # V [quad][channel][slot]
    k2, v2 = pool_io.unpack_bf16_blocks(blk, d)
    assert np.array_equal(k2, k) and np.array_equal(v2, v)


# ------------------------------------------------------------------ ABI --
def header_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(oscar_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_header_function():
    import long_context_decode_oscar_amd as oscar
    lib = oscar.load()
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", oscar.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (oscar_\w+)", out))
    assert set(names) <= exported
    assert set(names) == set(oscar.EXPORTED)


def _cfg(**kw):
    import long_context_decode_oscar_amd as oscar
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, group_size=128)
    base.update(kw)
    return oscar.PoolConfig(**base)


def test_pool_create_validation_and_layout():
    import long_context_decode_oscar_amd as oscar
    p = oscar.OscarPool(_cfg())
    assert p.int2_head_block_bytes == 1152 and p.int2_page_bytes == 8 * 1152
    assert p.bf16_head_block_bytes == 8192 and p.bf16_page_bytes == 8 * 8192
    assert oscar.OscarPool(_cfg(head_dim=64, group_size=64, num_q_heads=4, num_kv_heads=2)).int2_head_block_bytes == 640
    assert oscar.OscarPool(_cfg(group_size=64)).int2_head_block_bytes == 8 * 128 + 256
    assert oscar.OscarPool(_cfg(v_absorbed=0)).int2_page_bytes == 8 * 1152  # values not absorbed
    cases = [
        (dict(num_q_heads=30), oscar.OSCAR_ERR_INVALID),
        (dict(group_size=96), oscar.OSCAR_ERR_INVALID),
        (dict(sink_tokens=60), oscar.OSCAR_ERR_INVALID),
        (dict(recent_tokens=0), oscar.OSCAR_ERR_INVALID),
        (dict(sm_scale=float("nan")), oscar.OSCAR_ERR_INVALID),
        (dict(head_dim=256, group_size=128), oscar.OSCAR_ERR_UNSUPPORTED),
        (dict(group_size=32), oscar.OSCAR_ERR_UNSUPPORTED),
        (dict(page_size=32, sink_tokens=64), oscar.OSCAR_ERR_UNSUPPORTED),
        (dict(num_q_heads=8), oscar.OSCAR_ERR_UNSUPPORTED),
        (dict(v_absorbed=2), oscar.OSCAR_ERR_INVALID),
        (dict(codebook=2), oscar.OSCAR_ERR_INVALID),
        (dict(codebook=1, levels_k=(0, 1.01, 2, 3)), oscar.OSCAR_ERR_INVALID),   # not on the 1/32 grid
        (dict(codebook=1, levels_v=(0, 2, 1, 3)), oscar.OSCAR_ERR_INVALID),      # not increasing
        (dict(codebook=1, levels_k=(0.5, 1, 2, 3)), oscar.OSCAR_ERR_INVALID),    # ends must be 0 and 3
    ]
    assert oscar.OscarPool(_cfg(codebook=1, levels_k=(0, 1.125, 1.875, 3), levels_v=(0, 0.03125, 2.96875, 3)))
    # without the codebook flag the levels are ignored
    assert oscar.OscarPool(_cfg(codebook=0, levels_k=(0, 2, 1, 3)))
    for kw, status in cases:
        with pytest.raises(oscar.OscarError) as e:
            oscar.OscarPool(_cfg(**kw))
        assert e.value.status == status, kw
    lib = oscar.load()
    assert lib.oscar_pool_create(None, None, None) == oscar.OSCAR_ERR_INVALID
    assert lib.oscar_status_string(3) == b"OSCAR_ERR_WORKSPACE"


def test_workspace_bytes_grows_with_batch_and_length():
    import long_context_decode_oscar_amd as oscar
    p = oscar.OscarPool(_cfg())
    a = p.workspace_bytes(1, 100_000)
    assert a > 0 and a % 256 == 0
    assert p.workspace_bytes(32, 32_768) > a
    assert p.workspace_bytes(0, 10) == 0
    assert p.workspace_bytes(1, 100_000, bf16_only=True) > 0


@pytest.mark.parametrize("group_size,chunk_pages", [(128, 1024), (64, 512)])
def test_decode_plan_chunk_limit(group_size, chunk_pages):
    """The split-K planner gives one (sequence, KV head) at most 1024 INT2
    chunks, of at most 1024 pages at D = 128 with one scale group per head
    (two batches of page ids per decode wave) and 512 pages otherwise: a
    history of exactly 1024 chunks fits, one page more is rejected as
    unsupported before any launch."""
    import ctypes
    import long_context_decode_oscar_amd as oscar
    lib = oscar.load()
    p = oscar.OscarPool(_cfg(group_size=group_size))
    n = ctypes.c_size_t()
    at_limit = 64 + 256 + 1024 * chunk_pages * 16  # sink + recent + history tokens
    assert lib.oscar_decode_workspace_bytes(p.handle, 1, at_limit, 0, ctypes.byref(n)) == oscar.OSCAR_OK
    assert n.value > 0
    assert lib.oscar_decode_workspace_bytes(p.handle, 1, at_limit + 16, 0, ctypes.byref(n)) == \
        oscar.OSCAR_ERR_UNSUPPORTED
    assert b"split-K chunks" in lib.oscar_last_error()


def test_decode_validation_fails_before_launch():
    import long_context_decode_oscar_amd as oscar
    lib = oscar.load()
    p = oscar.OscarPool(_cfg())
    F = 1 << 20  # fake, aligned, never-dereferenced addresses
    host = oscar.HostLengths([1000])
    args = dict(q=F, lens=F, hlens=None, bpt=F, bs=8, bn=4, ipt=F, istr=8, inn=4, bpool=F, ipool=F, rk=F, rv=None,
                out=F, ws=F, wsb=16, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return lib.oscar_decode_attention(p.handle, 1, 1000, a["q"], a["lens"], a["hlens"], a["bpt"], a["bs"],
                                          a["bn"], a["ipt"], a["istr"], a["inn"], a["bpool"], a["ipool"], a["rk"],
                                          a["rv"], a["out"], a["ws"], a["wsb"], a["stream"])
    assert call(q=None) == oscar.OSCAR_ERR_INVALID
    assert call(ipool=F + 4) == oscar.OSCAR_ERR_INVALID  # misaligned
    assert call(bs=0) == oscar.OSCAR_ERR_INVALID
    assert call(rv=F) == oscar.OSCAR_ERR_INVALID  # r_v given although V is absorbed
    assert call() == oscar.OSCAR_ERR_WORKSPACE  # 16 bytes is too small
    assert call(hlens=host.ptr) == oscar.OSCAR_ERR_WORKSPACE  # with host lengths too
    assert call(ws=F + 64, wsb=1 << 30) == oscar.OSCAR_ERR_WORKSPACE  # misaligned workspace
    assert b"workspace" in lib.oscar_last_error()
    assert lib.oscar_decode_attention(p.handle, 0, 0, None, None, None, None, 0, 0, None, 0, 0, None, None, None,
                                      None, None, None, 0, None) == oscar.OSCAR_OK  # empty batch
    assert lib.oscar_merge(4, 96, F, F, F, F, None) == oscar.OSCAR_ERR_UNSUPPORTED
    assert lib.oscar_merge(4, 128, None, F, F, F, None) == oscar.OSCAR_ERR_INVALID
    assert lib.oscar_quantize_pack(p.handle, 16, F, F, F, 0, F, F, None, F, F, None) == oscar.OSCAR_ERR_INVALID
    assert lib.oscar_append_demote(p.handle, 1, F, F, F, F, 8, 4, F, 8, 4, F, F, F, F, F, F, None) == \
        oscar.OSCAR_ERR_INVALID  # r_v given although V is absorbed
    # values not absorbed: r_v is required
    pn = oscar.OscarPool(_cfg(v_absorbed=0))
    assert lib.oscar_append_demote(pn.handle, 1, F, F, F, F, 8, 4, F, 8, 4, F, F, F, None, F, F, None) == \
        oscar.OSCAR_ERR_INVALID
    assert lib.oscar_quantize_pack(pn.handle, 16, F, F, F, 4, F, F, None, F, F, None) == oscar.OSCAR_ERR_INVALID
    assert lib.oscar_decode_attention(pn.handle, 1, 1000, F, F, None, F, 8, 4, F, 8, 4, F, F, F, None, F, F, 16,
                                      None) == oscar.OSCAR_ERR_INVALID
    assert lib.oscar_bf16_decode_attention(p.handle, 1, 100, F, F, F, 8, 4, F, F, F, 0, None) == \
        oscar.OSCAR_ERR_WORKSPACE


def test_calibration_validation_fails_before_launch():
    import long_context_decode_oscar_amd as oscar
    lib = oscar.load()
    F = 1 << 20  # fake, aligned, never-dereferenced addresses
    n = ctypes.c_size_t()
    assert lib.oscar_calib_gram_workspace_bytes(8, 8192, 128, ctypes.byref(n)) == oscar.OSCAR_OK
    assert n.value >= 8 * 128 * 128 * 4
    assert lib.oscar_calib_gram_workspace_bytes(8, 8192, 96, ctypes.byref(n)) == oscar.OSCAR_ERR_UNSUPPORTED
    assert lib.oscar_calib_clip_workspace_bytes(8, 2048, 128, ctypes.byref(n)) == oscar.OSCAR_OK
    assert n.value >= 8 * 2048 * 128 * 4  # one key per rotated value
    assert lib.oscar_calib_workspace_bytes(8, 4, 2048, 128, ctypes.byref(n)) == oscar.OSCAR_OK
    assert n.value >= 8 * 4 * 2048 * 128 * 4  # the attention outputs
    # gram: bad dims, null input, strides, workspace
    assert lib.oscar_calib_gram(8, 64, 96, F, 64 * 96, 96, 1.0, F, F, 1 << 30, None) == oscar.OSCAR_ERR_UNSUPPORTED
    assert lib.oscar_calib_gram(8, 64, 128, None, 64 * 128, 128, 1.0, F, F, 1 << 30, None) == oscar.OSCAR_ERR_INVALID
    assert lib.oscar_calib_gram(8, 64, 128, F, 64 * 128, 100, 1.0, F, F, 1 << 30, None) == oscar.OSCAR_ERR_INVALID
    assert lib.oscar_calib_gram(8, 64, 128, F, 64 * 128, 128, 1.0, F, F, 16, None) == oscar.OSCAR_ERR_WORKSPACE
    assert lib.oscar_calib_gram(1, 1 << 22, 128, F, 0, 128, 1.0, F, F, 1 << 40, None) == \
        oscar.OSCAR_ERR_UNSUPPORTED  # a 2 GiB head span
    # attention: shapes, alignment, strides
    assert lib.oscar_calib_attention(8, 4, 0, 128, 0.0, F, F, F, 2048 * 128, 128, F, None, None) == \
        oscar.OSCAR_ERR_INVALID
    assert lib.oscar_calib_attention(8, 4, 64, 128, 0.0, F + 4, F, F, 64 * 128, 128, F, None, None) == \
        oscar.OSCAR_ERR_INVALID
    assert lib.oscar_calib_attention(8, 4, 64, 128, 0.0, F, F, F, 64 * 128, 64, F, None, None) == \
        oscar.OSCAR_ERR_INVALID  # token stride below head_dim
    assert lib.oscar_calib_attention(8, 4, 64, 128, 0.0, F, F, F, 64 * 128, 128, None, None, None) == \
        oscar.OSCAR_ERR_INVALID
    # rotation / clip / whole calibration
    assert lib.oscar_calib_rotation(8, 128, F, 2, F, None, None) == oscar.OSCAR_ERR_INVALID
    assert lib.oscar_calib_rotation(8, 32, F, 1, F, None, None) == oscar.OSCAR_ERR_UNSUPPORTED
    assert lib.oscar_calib_clip(8, 64, 128, F, 64 * 128, 128, None, 1.5, F, F, 1 << 30, None) == \
        oscar.OSCAR_ERR_INVALID
    assert lib.oscar_calib_clip(8, 64, 128, F, 64 * 128, 128, None, 0.995, F, F, 64, None) == \
        oscar.OSCAR_ERR_WORKSPACE
    assert lib.oscar_calibrate(8, 4, 64, 128, 0.0, F, F, F, 64 * 128, 128, 0.995, F, F, F, F, None, None, F + 64,
                               1 << 30, None) == oscar.OSCAR_ERR_WORKSPACE  # misaligned workspace
    assert lib.oscar_calibrate(8, 4, 64, 128, 0.0, F, F, F, 64 * 128, 128, 0.995, None, F, F, F, None, None, F,
                               1 << 30, None) == oscar.OSCAR_ERR_INVALID
    # dequantize / error chain
    p = oscar.OscarPool(_cfg())
    assert lib.oscar_dequantize(p.handle, 32, F, 0, F, None, None, F, F, None) == oscar.OSCAR_ERR_INVALID
    assert lib.oscar_dequantize(p.handle, 0, None, 0, None, None, None, None, None, None) == oscar.OSCAR_OK
    assert lib.oscar_attention_error(8, 4, 64, 128, 0.0, F, F, F, None, F, 64 * 128, 128, F, None) == \
        oscar.OSCAR_ERR_INVALID
    assert lib.oscar_calib_codebook_workspace_bytes(8, 2048, 128, ctypes.byref(n)) == oscar.OSCAR_OK
    assert n.value >= 8 * 2048 * 128 * 4
    assert lib.oscar_calib_codebook(8, 64, 128, 96, F, 64 * 128, 128, None, F, F, F, 1 << 30, None) == \
        oscar.OSCAR_ERR_UNSUPPORTED  # group size
    assert lib.oscar_calib_codebook(8, 64, 128, 128, F, 64 * 128, 128, None, None, F, F, 1 << 30, None) == \
        oscar.OSCAR_ERR_INVALID  # tau
    assert lib.oscar_calib_codebook(8, 64, 128, 128, F, 64 * 128, 128, None, F, F, F, 64, None) == \
        oscar.OSCAR_ERR_WORKSPACE


def test_cascade_validation_fails_before_launch():
    import long_context_decode_oscar_amd as oscar
    lib = oscar.load()
    p = oscar.OscarPool(_cfg(num_q_heads=64))  # GQA 8: two sequences per prefix unit
    F = 1 << 20
    n = ctypes.c_size_t()

    def ws_bytes(groups, batch=8, stride=8192):
        arr, ng = oscar._groups(groups)
        ptr = ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None
        return lib.oscar_decode_cascade_workspace_bytes(p.handle, batch, 131072, stride, ptr, ng, ctypes.byref(n))
    assert ws_bytes([]) == oscar.OSCAR_OK
    plain = n.value
    assert ws_bytes([(0, 4, 4092)]) == oscar.OSCAR_OK and n.value > plain  # prefix partial slots
    assert ws_bytes([(0, 4, 0)]) == oscar.OSCAR_OK and n.value == plain    # nothing shared
    assert ws_bytes([(2, 2, 10), (0, 2, 10)]) == oscar.OSCAR_ERR_INVALID   # not ordered
    assert ws_bytes([(0, 3, 10), (2, 2, 10)]) == oscar.OSCAR_ERR_INVALID   # overlapping
    assert ws_bytes([(6, 3, 10)]) == oscar.OSCAR_ERR_INVALID               # past the batch
    assert ws_bytes([(0, 2, 9000)]) == oscar.OSCAR_ERR_INVALID             # beyond the table
    assert ws_bytes([(0, 66, 10)], batch=66) == oscar.OSCAR_ERR_UNSUPPORTED  # 33 units of 2
    arr, ng = oscar._groups([(0, 4, 100)])
    assert lib.oscar_decode_attention_cascade(p.handle, 8, 131072, F, F, None, F, 8, 4, F, 8192, 4, F, F, F, None, F,
                                              ctypes.cast(arr, ctypes.c_void_p), ng, F, 16, None) == \
        oscar.OSCAR_ERR_WORKSPACE
    assert lib.oscar_decode_attention_cascade(p.handle, 8, 131072, F, F, None, F, 8, 4, F, 8192, 4, F, F, F, None, F,
                                              None, 2, F, 1 << 30, None) == oscar.OSCAR_ERR_INVALID
