"""Pins for the oracle's pool model and decode attention (R1-R3)."""

import math

import numpy as np
import pytest
import torch

from oracle import SeqPool, bf16_decode_attention, decode_attention, dequantize
from oracle.numerics import round_bf16


def _orth(rng, d):
    return np.linalg.qr(rng.standard_normal((d, d)))[0].astype(np.float32)


def _bf16(rng, *shape, scale=1.0):
    return round_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def test_tiny_bruteforce_pure_python():
    """D=4, 9 tokens, sink 2 | history 4 | recent 3, two query heads on one
    KV head; the reference below is written with Python loops only."""
    rng = np.random.default_rng(1)
    d, sink, recent, L = 4, 2, 3, 9
    k = _bf16(rng, L, 1, d, scale=2)
    v = _bf16(rng, L, 1, d)
    r_k, r_v = _orth(rng, d)[None], _orth(rng, d)[None]
    tau = np.array([1.7], np.float32)
    for absorbed in (True, False):
        seq = SeqPool(1, d, 2, sink=sink, recent=recent, v_absorbed=absorbed)
        seq.prefill(k, v, r_k, tau, tau, r_v)
        assert seq.n_hist == 4
        q = _bf16(rng, 1, 2, d)
        out, lse = decode_attention([seq], q, r_k, r_v)

        keys, vals = [], []
        for t in range(L):
            if t < sink or t >= L - recent:
                keys.append([float(a) for a in k[t, 0]])
                vals.append([float(a) for a in v[t, 0]])
            else:
                i = t - sink
                kq = [float(seq.ks[i, 0, c // 2]) * (int(seq.kc[i, 0, c]) - float(seq.kz[i, 0, c // 2])) for c in range(d)]
                vq = [float(seq.vs[i, 0, c // 2]) * (int(seq.vc[i, 0, c]) - float(seq.vz[i, 0, c // 2])) for c in range(d)]
                # inverse rotation x = x' R^T
                keys.append([sum(kq[j] * float(r_k[0, c, j]) for j in range(d)) for c in range(d)])
                if absorbed:
                    vals.append(vq)
                else:
                    vals.append([sum(vq[j] * float(r_v[0, c, j]) for j in range(d)) for c in range(d)])
        for h in range(2):
            lg = [sum(float(q[0, h, c]) * keys[t][c] for c in range(d)) / math.sqrt(d) for t in range(L)]
            m = max(lg)
            e = [math.exp(x - m) for x in lg]
            tot = sum(e)
            ref = [sum(e[t] * vals[t][c] for t in range(L)) / tot for c in range(d)]
            assert np.allclose(out[0, h], ref, rtol=1e-12, atol=1e-12)
            assert abs(lse[0, h] - (m + math.log(tot))) < 1e-12


@pytest.mark.parametrize("L", [1, 63, 64, 65, 200, 320])
def test_no_history_is_textbook_attention(L):
    """With L <= S0 + W every token is BF16: plain softmax attention (checked
    against torch's scaled_dot_product_attention in float64 on the CPU)."""
    rng = np.random.default_rng(L)
    d, hkv, hq = 64, 2, 4
    k = _bf16(rng, L, hkv, d, scale=3)
    v = _bf16(rng, L, hkv, d)
    eye = np.stack([np.eye(d, dtype=np.float32)] * hkv)
    inf = np.full(hkv, np.inf, np.float32)
    seq = SeqPool(hkv, d, 64).prefill(k, v, eye, inf, inf)
    assert seq.n_hist == 0
    q = _bf16(rng, 1, hq, d)
    out, _ = decode_attention([seq], q, eye)
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).repeat_interleave(2, 0)
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).repeat_interleave(2, 0)
    qt = torch.from_numpy(q[0].astype(np.float64))[:, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0].numpy()
    assert np.allclose(out[0], ref, rtol=1e-12, atol=1e-13)


def test_on_grid_history_is_lossless():
    """History values that already sit on a 4-level grid s (q - z) (with the
    group's min and max on levels 0 and 3) quantize exactly, so INT2 decode
    equals all-BF16 decode on the same values."""
    rng = np.random.default_rng(4)
    d, hkv, L = 64, 2, 700
    s = np.float32(0.5)
    z = rng.choice(np.array([-1.5, 0.0, 1.5, 2.0, 4.0], np.float32), size=(L, hkv))
    codes = rng.integers(0, 4, size=(L, hkv, d))
    codes[:, :, 0], codes[:, :, 1] = 0, 3
    k = (s * (codes - z[:, :, None])).astype(np.float32)
    codes_v = rng.integers(0, 4, size=(L, hkv, d))
    codes_v[:, :, 5], codes_v[:, :, 9] = 0, 3
    v = (s * (codes_v - z[:, :, None])).astype(np.float32)
    assert np.array_equal(round_bf16(k), k) and np.array_equal(round_bf16(v), v)
    eye = np.stack([np.eye(d, dtype=np.float32)] * hkv)
    inf = np.full(hkv, np.inf, np.float32)
    seq = SeqPool(hkv, d, 64).prefill(k, v, eye, inf, inf)
    assert seq.n_hist == L - 64 - 256
    q = _bf16(rng, 1, 4, d)
    out, lse = decode_attention([seq], q, eye)
    ref, ref_lse = bf16_decode_attention([k], [v], q, [L])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, ref_lse, rtol=1e-13)


def test_on_codebook_history_is_lossless():
    """The same with a four-level codebook: values s (L[q] - z) quantize
    exactly with the codebook quantizer, so the decode equals all-BF16 decode
    on them."""
    rng = np.random.default_rng(14)
    d, hkv, L = 64, 2, 640
    lk = np.array([0.0, 1.125, 1.875, 3.0])
    lv = np.array([0.0, 0.90625, 2.03125, 3.0])
    s = np.float32(0.5)
    z = rng.choice(np.array([-1.5, 0.0, 1.5, 2.0], np.float32), size=(L, hkv))
    codes = rng.integers(0, 4, size=(L, hkv, d))
    codes[:, :, 0], codes[:, :, 1] = 0, 3
    k = (s * (lk[codes] - z[:, :, None])).astype(np.float32)
    codes_v = rng.integers(0, 4, size=(L, hkv, d))
    codes_v[:, :, 5], codes_v[:, :, 9] = 0, 3
    v = (s * (lv[codes_v] - z[:, :, None])).astype(np.float32)
    assert np.array_equal(round_bf16(k), k) and np.array_equal(round_bf16(v), v)
    eye = np.stack([np.eye(d, dtype=np.float32)] * hkv)
    inf = np.full(hkv, np.inf, np.float32)
    seq = SeqPool(hkv, d, 64, levels_k=lk, levels_v=lv).prefill(k, v, eye, inf, inf)
    assert np.array_equal(seq.kc, codes[64:L - 256]) and np.array_equal(seq.vc, codes_v[64:L - 256])
    q = _bf16(rng, 1, 4, d)
    out, lse = decode_attention([seq], q, eye)
    ref, ref_lse = bf16_decode_attention([k], [v], q, [L])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, ref_lse, rtol=1e-13)


def test_logit_error_identity_weights_by_query_covariance():
    """||Q K^T - Q K^^T||_F^2 = tr((K - K^) Q^T Q (K - K^)^T) (MarkTechPost
    article, "What OSCAR Does Differently"), with K^ the oracle's dequantized,
    inverse-rotated keys."""
    rng = np.random.default_rng(8)
    d, L = 64, 600
    k = _bf16(rng, L, 1, d, scale=2)
    v = _bf16(rng, L, 1, d)
    r = _orth(rng, d)[None]
    tau = np.array([4.0], np.float32)
    seq = SeqPool(1, d, 64).prefill(k, v, r, tau, tau)
    _, hist, _ = seq.segments()
    kk = k[hist, 0].astype(np.float64)
    kh = dequantize(seq.kc[:, 0], seq.ks[:, 0], seq.kz[:, 0], 64) @ r[0].astype(np.float64).T
    q = rng.standard_normal((50, d))
    lhs = np.linalg.norm(q @ kk.T - q @ kh.T) ** 2
    e = kk - kh
    rhs = np.trace(e @ q.T @ q @ e.T)
    assert abs(lhs - rhs) <= 1e-10 * abs(lhs)
    assert lhs > 0


def test_query_rotation_form_equals_inverse_rotated_keys():
    """sm s (q' . q_K - z sum(q')) with q' = q R_K equals sm q . k^ where
    k^ = s (q_K - z) R_K^T (R_K^T R_K = I); the GPU uses the first form."""
    rng = np.random.default_rng(10)
    d = 128
    r = np.linalg.qr(rng.standard_normal((d, d)))[0]
    qv = rng.standard_normal(d)
    codes = rng.integers(0, 4, d)
    s, z = 0.37, 1.25
    sm = 1 / math.sqrt(d)
    qp = qv @ r
    a = sm * s * (qp @ codes - z * qp.sum())
    b = sm * qv @ (s * (codes - z) @ r.T)
    assert abs(a - b) <= 1e-12 * (1 + abs(b))


@pytest.mark.parametrize("L", [1, 63, 64, 65, 319, 320, 321, 336, 337, 512])
def test_segment_boundaries(L):
    seq = SeqPool(1, 64, 64)
    rng = np.random.default_rng(L)
    eye = np.eye(64, dtype=np.float32)[None]
    inf = np.full(1, np.inf, np.float32)
    seq.prefill(_bf16(rng, L, 1, 64), _bf16(rng, L, 1, 64), eye, inf, inf)
    sink, hist, recent = seq.segments()
    assert len(sink) == min(L, 64)
    assert len(hist) == max(0, L - 320)
    assert len(recent) == L - min(L, 64) - max(0, L - 320)
    assert len(sink) + len(hist) + len(recent) == L
    assert seq.n_hist == len(hist)


def test_prefill_equals_token_by_token_demotion():
    rng = np.random.default_rng(12)
    d, hkv, L0, steps = 64, 2, 300, 90
    k = _bf16(rng, L0 + steps, hkv, d, scale=2)
    v = _bf16(rng, L0 + steps, hkv, d)
    r = np.stack([_orth(rng, d) for _ in range(hkv)])
    tk = np.array([3.0, 2.0], np.float32)
    tv = np.array([1.5, 2.5], np.float32)
    inc = SeqPool(hkv, d, 32).prefill(k[:L0], v[:L0], r, tk, tv)
    demoted = [inc.append_demote(k[L0 + i], v[L0 + i], r, tk, tv) for i in range(steps)]
    assert demoted[0] is None and demoted[-1] == L0 + steps - 1 - 256
    bulk = SeqPool(hkv, d, 32).prefill(k, v, r, tk, tv)
    for n in ("kc", "ks", "kz", "vc", "vs", "vz"):
        assert np.array_equal(getattr(inc, n), getattr(bulk, n))
