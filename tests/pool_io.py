"""Test-side writer and reader of the paged pool layout documented in
include/oscar.h, in numpy.  It shares no code with the HIP library: it
uploads oracle-built pools for decode tests and decodes GPU-written pages
back into logical codes, scales and zeros for write-path tests."""

import numpy as np

PAGE = 16


def bf16_bits(x) -> np.ndarray:
    """bf16-representable float32 values -> uint16 bit patterns."""
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, np.uint32) << 16).astype(np.uint32).view(np.float32)


def int2_block_bytes(d, ng):
    return 8 * d + 128 * ng


def bf16_block_bytes(d):
    return 64 * d


# ----------------------------------------------------------- INT2 blocks --
def pack_int2_blocks(kc, ks, kz, vc, vs, vz):
    """kc/vc [N, 16, D] uint8 codes, ks/kz/vs/vz [N, 16, NG] bf16 values ->
    [N, 8D + 128 NG] uint8 head blocks."""
    kc = np.asarray(kc, np.uint32)
    vc = np.asarray(vc, np.uint32)
    n, _, d = kc.shape
    ng = ks.shape[2]
    kw = d // 64
    # K record (j, r) word w: channel w*64 + j*16 + m at bits 2m
    k5 = kc.reshape(n, 16, kw, 4, 16)  # [n, r, w, j, m]
    kwords = (k5 << (2 * np.arange(16, dtype=np.uint32))).sum(axis=-1, dtype=np.uint64).astype(np.uint32)
    kwords = kwords.transpose(0, 3, 1, 2)  # [n, j, r, w]
    # V record (j, r) word w: channel (4w + bb)*16 + r of token 4j + i at
    # bits 16*(i&1) + 2*(2*bb + (i>>1))
    v6 = vc.reshape(n, 4, 4, kw, 4, 16)  # [n, j, i, w, bb, r]
    i_ = np.arange(4)[:, None]
    bb_ = np.arange(4)[None, :]
    shift = (16 * (i_ & 1) + 2 * (2 * bb_ + (i_ >> 1))).astype(np.uint32)  # [i, bb]
    vshift = v6 << shift[None, None, :, None, :, None]
    vwords = vshift.sum(axis=(2, 4), dtype=np.uint64).astype(np.uint32)  # [n, j, w, r]
    vwords = vwords.transpose(0, 1, 3, 2)  # [n, j, r, w]
    rec = np.concatenate([kwords, vwords], axis=-1).reshape(n, 64, 2 * kw)  # [n, lam, words]
    codes = rec.astype("<u4").view(np.uint8).reshape(n, 8 * d)
    # scales: [quad j][K/V][token i][group g][s, z]
    sc = np.zeros((n, 4, 2, 4, ng, 2), np.uint16)
    for which, (s, z) in enumerate(((ks, kz), (vs, vz))):
        sc[:, :, which, :, :, 0] = bf16_bits(s).reshape(n, 4, 4, ng)
        sc[:, :, which, :, :, 1] = bf16_bits(z).reshape(n, 4, 4, ng)
    scb = sc.astype("<u2").view(np.uint8).reshape(n, 128 * ng)
    return np.concatenate([codes, scb], axis=1)


def unpack_int2_blocks(blocks, d, ng):
    """Inverse of pack_int2_blocks."""
    blocks = np.asarray(blocks, np.uint8)
    n = blocks.shape[0]
    kw = d // 64
    rec = blocks[:, : 8 * d].copy().view("<u4").reshape(n, 4, 16, 2 * kw)  # [n, j, r, words]
    kwords, vwords = rec[..., :kw], rec[..., kw:]
    m = np.arange(16, dtype=np.uint32)
    kcodes = (kwords[..., None] >> (2 * m)) & 3  # [n, j, r, w, m]
    kc = kcodes.transpose(0, 2, 3, 1, 4).reshape(n, 16, d).astype(np.uint8)
    i_ = np.arange(4)[:, None]
    bb_ = np.arange(4)[None, :]
    shift = (16 * (i_ & 1) + 2 * (2 * bb_ + (i_ >> 1))).astype(np.uint32)  # [i, bb]
    vw = vwords.transpose(0, 1, 3, 2)  # [n, j, w, r]
    vcodes = (vw[:, :, None, :, None, :] >> shift[None, None, :, None, :, None]) & 3  # [n, j, i, w, bb, r]
    vc = vcodes.reshape(n, 16, d).astype(np.uint8)
    sc = blocks[:, 8 * d:].copy().view("<u2").reshape(n, 4, 2, 4, ng, 2)
    out = []
    for which in range(2):
        s = bits_to_f32(sc[:, :, which, :, :, 0]).reshape(n, 16, ng)
        z = bits_to_f32(sc[:, :, which, :, :, 1]).reshape(n, 16, ng)
        out.append((s, z))
    return kc, out[0][0], out[0][1], vc, out[1][0], out[1][1]


# ----------------------------------------------------------- BF16 blocks --
def pack_bf16_blocks(k, v):
    """k, v [N, 16, D] bf16 values -> [N, 64 D] uint8 head blocks."""
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    n, _, d = k.shape
    kb = bf16_bits(k).reshape(n, 16 * d)
    vb = bf16_bits(v).reshape(n, 4, 4, d).transpose(0, 1, 3, 2).reshape(n, 16 * d)  # [quad][channel][token]
    return np.concatenate([kb, vb], axis=1).astype("<u2").view(np.uint8).reshape(n, 64 * d)


def unpack_bf16_blocks(blocks, d):
    blocks = np.asarray(blocks, np.uint8)
    n = blocks.shape[0]
    u = blocks.copy().view("<u2").reshape(n, 32 * d)
    k = bits_to_f32(u[:, : 16 * d]).reshape(n, 16, d)
    v = bits_to_f32(u[:, 16 * d:]).reshape(n, 4, d, 4).transpose(0, 1, 3, 2).reshape(n, 16, d)
    return k, v


# ----------------------------------------------------------------- pools --
def bf16_positions_needed(L, sink, recent):
    r0 = max(sink, L - recent)
    return [p for p in range((L + PAGE - 1) // PAGE)
            if p * PAGE < min(L, sink) or ((p + 1) * PAGE > r0 and p * PAGE < L)]


def build_pools(seqs, hkv, d, ng, sink, recent, seed=0, extra_bf16_pages=None, garbage=True,
                int2_slack=0, bf16_for_all=False, int2_capacity=None):
    """Lay out oracle sequences (oracle.SeqPool) in paged pools with random
    physical page ids.  BF16 pages hold the sink and recent pages (all pages
    if ``bf16_for_all``); positions outside those segments are filled with
    NaN / garbage bit patterns unless ``garbage`` is False.  ``int2_capacity``
    (logical pages per sequence) and ``extra_bf16_pages`` reserve table
    entries for tokens a later append / demotion writes.

    Returns dict(int2_pool [P2, Hkv*blk2] u8, bf16_pool, int2_pt [B, S2] i32,
    bf16_pt [B, S16] i32)."""
    rng = np.random.default_rng(seed)
    blk2, blk16 = int2_block_bytes(d, ng), bf16_block_bytes(d)
    n_int2 = [(s.n_hist + PAGE - 1) // PAGE for s in seqs]
    if int2_capacity is not None:
        n_int2 = [max(a, int(c)) for a, c in zip(n_int2, int2_capacity)]
    b16_lists = [list(range((s.L + PAGE - 1) // PAGE)) if bf16_for_all else bf16_positions_needed(s.L, sink, recent)
                 for s in seqs]
    if extra_bf16_pages:
        for b, extra in extra_bf16_pages.items():
            b16_lists[b] = sorted(set(b16_lists[b]) | set(extra))
    n_int2_phys = sum(n_int2) + int2_slack + 1
    n_b16_phys = sum(len(x) for x in b16_lists) + 1
    perm2 = rng.permutation(n_int2_phys)
    perm16 = rng.permutation(n_b16_phys)
    int2_pool = rng.integers(0, 256, size=(n_int2_phys, hkv * blk2), dtype=np.uint8)
    bf16_pool = rng.integers(0, 256, size=(n_b16_phys, hkv * blk16), dtype=np.uint8)
    s2 = max(max(n_int2), 1)
    s16 = max([(s.L + PAGE - 1) // PAGE for s in seqs] + [max(x) + 1 for x in b16_lists if x]) + 2
    int2_pt = np.full((len(seqs), s2 + 1), -1, np.int32)
    bf16_pt = np.full((len(seqs), s16), -1, np.int32)
    p2 = p16 = 0
    for b, s in enumerate(seqs):
        for lp in range(n_int2[b]):
            phys = int(perm2[p2])
            p2 += 1
            int2_pt[b, lp] = phys
            t0, t1 = lp * PAGE, max(min((lp + 1) * PAGE, s.n_hist), lp * PAGE)
            kc = np.zeros((hkv, PAGE, d), np.uint8)
            vc = np.zeros((hkv, PAGE, d), np.uint8)
            ks, kz, vs, vz = (np.zeros((hkv, PAGE, ng), np.float32) for _ in range(4))
            kc[:, : t1 - t0] = s.kc[t0:t1].transpose(1, 0, 2)
            vc[:, : t1 - t0] = s.vc[t0:t1].transpose(1, 0, 2)
            for arr, src in ((ks, s.ks), (kz, s.kz), (vs, s.vs), (vz, s.vz)):
                arr[:, : t1 - t0] = src[t0:t1].transpose(1, 0, 2)
            int2_pool[phys] = pack_int2_blocks(kc, ks, kz, vc, vs, vz).reshape(-1)
        for lp in b16_lists[b]:
            phys = int(perm16[p16])
            p16 += 1
            bf16_pt[b, lp] = phys
            k = np.zeros((hkv, PAGE, d), np.float32)
            v = np.zeros((hkv, PAGE, d), np.float32)
            for sl in range(PAGE):
                pos = lp * PAGE + sl
                if pos < s.L:
                    k[:, sl] = s.k[pos]
                    v[:, sl] = s.v[pos]
                elif garbage:
                    k[:, sl] = np.nan
                    v[:, sl] = np.nan
            if garbage and not bf16_for_all:
                # positions demoted to history: stale bf16 garbage (NaN)
                r0 = max(sink, s.L - recent)
                for sl in range(PAGE):
                    pos = lp * PAGE + sl
                    if sink <= pos < r0:
                        k[:, sl] = np.nan
                        v[:, sl] = np.nan
            bf16_pool[phys] = pack_bf16_blocks(k, v).reshape(-1)
    return dict(int2_pool=int2_pool, bf16_pool=bf16_pool, int2_pt=int2_pt, bf16_pt=bf16_pt)


def read_history(int2_pool, int2_pt_row, n_hist, hkv, d, ng):
    """Logical history (codes, scales, zeros) of one sequence from a pool."""
    blk2 = int2_block_bytes(d, ng)
    npg = (n_hist + PAGE - 1) // PAGE
    pages = int2_pool[int2_pt_row[:npg]].reshape(npg * hkv, blk2)
    kc, ks, kz, vc, vs, vz = unpack_int2_blocks(pages, d, ng)

    def arr(x):
        x = x.reshape(npg, hkv, PAGE, *x.shape[2:]).swapaxes(1, 2)
        return x.reshape(npg * PAGE, hkv, *x.shape[3:])[:n_hist]
    return tuple(arr(x) for x in (kc, ks, kz, vc, vs, vz))
