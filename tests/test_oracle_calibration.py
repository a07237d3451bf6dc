"""Pins for the oracle's offline calibration (C1-C5) and error chain (E1-E2).

Each check goes through a route other than the oracle's own formula: closed
forms, hand-computed small cases, pure-Python brute force, and the invariants
the pages state (orthogonality, Lemma 1, the trace form of the logit error).
"""

import math

import numpy as np
import pytest

from oracle import calibration as cal
from oracle import quantize_tokens
from synthetic import draw_calibration


@pytest.fixture(scope="module")
def calib():
    draws = draw_calibration(num_kv_heads=2, gqa=2, head_dim=64, seed=0, n_cal=512)
    return draws, cal.calibrate([(d.q, d.k, d.v) for d in draws])


# -- C4 building blocks ------------------------------------------------------

def test_bit_reversal_table_and_involution():
    p = cal.bit_reversal_permutation(128)
    assert p[1] == 64 and p[3] == 96 and p[2] == 32 and p[127] == 127 and p[0] == 0
    assert np.array_equal(p[p], np.arange(128))
    p6 = cal.bit_reversal_permutation(64)
    assert p6[1] == 32 and p6[5] == 40  # 000101 -> 101000
    # every power-of-two group of consecutive output channels takes one input
    # from each importance band (MarkTechPost article, P_br bullet)
    for gsz in (2, 4, 8, 16, 32, 64):
        for start in range(0, 128, gsz):
            bands = sorted(int(i) // (128 // gsz) for i in p[start:start + gsz])
            assert bands == list(range(gsz))


def test_hadamard_orthonormal_sylvester():
    h = cal.hadamard_matrix(64)
    assert np.allclose(h @ h.T, np.eye(64), atol=1e-14)
    assert np.allclose(np.abs(h), 1 / 8)
    h2 = cal.hadamard_matrix(32)
    assert np.allclose(h[:32, :32], h2 / np.sqrt(2)) and np.allclose(h[32:, 32:], -h2 / np.sqrt(2))
    # entry (i, j) = (-1)^popcount(i & j) / sqrt(d)
    for i, j in ((3, 5), (7, 7), (12, 10), (63, 1)):
        assert h[i, j] == (-1) ** bin(i & j).count("1") / 8


def test_mix_matrix_columns():
    """(y H P_br)[j] = (y H)[br(j)]: column j of the mix is column br(j) of H."""
    m = cal.mix_matrix(16)
    h = cal.hadamard_matrix(16)
    y = np.arange(16.0)
    br = cal.bit_reversal_permutation(16)
    assert np.allclose(y @ m, (y @ h)[br])
    assert np.allclose(m[:, 1], h[:, 8]) and np.allclose(m[:, 2], h[:, 4])


# -- C1 / C3 -------------------------------------------------------------------

def test_query_covariance_by_hand():
    q = np.array([[1.0, 2.0], [3.0, -1.0], [0.0, 4.0]])
    # (1/3) [[1+9, 2-3], [2-3, 4+1+16]]
    assert np.allclose(cal.query_covariance(q), np.array([[10.0, -1.0], [-1.0, 21.0]]) / 3)
    # leading axes are pooled: two heads of rows equal one head of all rows
    assert np.allclose(cal.query_covariance(np.stack([q[:2], q[1:]])),
                       cal.query_covariance(np.concatenate([q[:2], q[1:]])))


def test_eigenbasis_permutation_case():
    u, w = cal.eigenbasis(np.diag([3.0, 1.0, 2.0]))
    assert np.allclose(w, [3.0, 2.0, 1.0])
    assert np.allclose(u, np.eye(3)[:, [0, 2, 1]])


def test_eigenbasis_golden_ratio_case():
    """[[2, 1], [1, 3]]: eigenvalues (5 +- sqrt5)/2, eigenvectors (1, phi) and
    (1, -1/phi) up to scale; the sign convention makes the larger-magnitude
    entry positive."""
    phi = (1 + math.sqrt(5)) / 2
    u, w = cal.eigenbasis(np.array([[2.0, 1.0], [1.0, 3.0]]))
    assert np.allclose(w, [(5 + math.sqrt(5)) / 2, (5 - math.sqrt(5)) / 2], atol=1e-14)
    assert np.allclose(u[:, 0], np.array([1.0, phi]) / math.sqrt(1 + phi * phi), atol=1e-14)
    assert np.allclose(u[:, 1], np.array([1.0, -1 / phi]) / math.sqrt(1 + 1 / phi ** 2), atol=1e-14)


def test_eigenbasis_sign_convention_random():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((12, 12))
    c = a @ a.T
    u, w = cal.eigenbasis(c)
    assert np.allclose(c @ u, u * w, atol=1e-10)
    assert np.all(np.diff(w) <= 0)
    for j in range(12):
        assert u[np.argmax(np.abs(u[:, j])), j] > 0


# -- C2 ----------------------------------------------------------------------

def _causal_attention_loops(q, k, v, sm):
    n, d = len(q), len(q[0])
    out = []
    for i in range(n):
        ls = [sm * sum(q[i][c] * k[t][c] for c in range(d)) for t in range(i + 1)]
        m = max(ls)
        e = [math.exp(x - m) for x in ls]
        tot = sum(e)
        out.append([sum(e[t] * v[t][c] for t in range(i + 1)) / tot for c in range(d)])
    return out


def test_causal_attention_brute_force():
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((6, 3)) for _ in range(3))
    o, lse = cal.causal_attention(q, k, v, sm=0.7)
    assert np.allclose(o, _causal_attention_loops(q.tolist(), k.tolist(), v.tolist(), 0.7), atol=1e-13)
    assert np.allclose(o[0], v[0])
    assert np.isclose(lse[0], 0.7 * q[0] @ k[0])


def test_score_weighted_covariance_zero_queries():
    """q = 0 makes every causal row uniform: o_n is the mean of v_0..v_n."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal((9, 4))
    k = rng.standard_normal((9, 4))
    means = np.cumsum(v, axis=0) / np.arange(1, 10)[:, None]
    want = sum(np.outer(m, m) for m in means) / 9
    assert np.allclose(cal.score_weighted_covariance(np.zeros((2, 9, 4)), k, v), want, atol=1e-14)


def test_score_weighted_covariance_averages_heads():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 7, 4))
    k, v = rng.standard_normal((7, 4)), rng.standard_normal((7, 4))
    per = [cal.score_weighted_covariance(q[h:h + 1], k, v) for h in range(3)]
    assert np.allclose(cal.score_weighted_covariance(q, k, v), sum(per) / 3, atol=1e-14)


# -- C4 on calibration data ----------------------------------------------------

def test_rotations_orthogonal(calib):
    _, c = calib
    for key in ("r_k64", "r_v64"):
        for r in c[key]:
            assert np.max(np.abs(r @ r.T - np.eye(r.shape[0]))) < 1e-12


def test_lemma1_equalises_query_energy(calib):
    """diag(R_K^T C_Q R_K) = tr(C_Q)/D for every channel (MarkTechPost article,
    Lemma 1).  Holds only for the row-vector convention x' = x R with U_Q the
    eigenbasis of C_Q; the transposed R or a basis that does not diagonalise
    C_Q breaks it."""
    _, c = calib
    for rk, cq in zip(c["r_k64"], c["c_q"]):
        dg = np.diag(rk.T @ cq @ rk)
        assert np.allclose(dg, np.trace(cq) / cq.shape[0], rtol=1e-10)
        assert not np.allclose(np.diag(rk @ cq @ rk.T), np.trace(cq) / cq.shape[0], rtol=1e-2)


def test_u_diagonalises_covariances(calib):
    _, c = calib
    m = cal.mix_matrix(64)
    for r, cov in [(r, cq) for r, cq in zip(c["r_k64"], c["c_q"])] + \
                  [(r, cs) for r, cs in zip(c["r_v64"], c["c_s"])]:
        u = r @ m.T  # undo H P_br
        lam = u.T @ cov @ u
        off = lam - np.diag(np.diag(lam))
        assert np.max(np.abs(off)) < 1e-10 * np.max(np.abs(lam))
        assert np.all(np.diff(np.diag(lam)) <= 1e-12 * np.max(np.abs(lam)))


def test_query_covariance_tracks_generator_spectrum(calib):
    """The draw has Sigma_Q = U diag(lambda) U^T; with 1024 samples per head
    the empirical top eigenvector aligns with U's first column."""
    draws, c = calib
    for d, cq in zip(draws, c["c_q"]):
        u, _ = cal.eigenbasis(cq)
        assert abs(u[:, 0] @ d.u[:, 0]) > 0.99


# -- C5 ------------------------------------------------------------------------

def _quantile_type7(values, p):
    xs = sorted(values)
    h = (len(xs) - 1) * p
    lo = math.floor(h)
    hi = min(lo + 1, len(xs) - 1)
    return xs[lo] + (h - lo) * (xs[hi] - xs[lo])


def test_clip_threshold_closed_form():
    # |x| = 0..200 evenly spaced: the 0.995 quantile is exactly 199
    x = np.arange(201.0).reshape(-1, 1) * np.where(np.arange(201) % 2, -1.0, 1.0)[:, None]
    assert cal.clip_threshold(x, None) == np.float32(199.0)


def test_clip_threshold_brute_force_rotated():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((37, 8))
    r, _ = np.linalg.qr(rng.standard_normal((8, 8)))
    want = _quantile_type7(np.abs(x @ r).ravel().tolist(), 0.995)
    assert cal.clip_threshold(x, r) == np.float32(want)
    # the sign of the input does not matter
    assert cal.clip_threshold(-x, r) == cal.clip_threshold(x, r)


def test_clip_thresholds_on_calibration(calib):
    _, c = calib
    assert c["tau_k"].dtype == np.float32 and np.all(c["tau_k"] > 0)
    # the Hadamard factor spreads the x20 outlier channels: rotated keys are
    # far below 20
    assert np.all(c["tau_k"] < 20) and np.all(c["tau_v"] < 5)


# -- E1 / E2 ---------------------------------------------------------------------

def test_kl_closed_forms():
    a, b = 0.3, 0.6
    want = a * math.log(a / b) + (1 - a) * math.log((1 - a) / (1 - b))
    assert math.isclose(cal.kl_divergence([a, 1 - a], [b, 1 - b]), want, rel_tol=1e-14)
    assert cal.kl_divergence([0.2, 0.8], [0.2, 0.8]) == 0.0
    assert cal.kl_divergence([0.0, 1.0], [0.5, 0.5]) == pytest.approx(math.log(2.0), rel=1e-14)


def _error_rows_loops(q, k, v, kh, vh, sm):
    n, d = len(q), len(q[0])
    kl, l2, ose = [], [], []
    for i in range(n):
        ls = [sm * sum(q[i][c] * k[t][c] for c in range(d)) for t in range(i + 1)]
        lh = [sm * sum(q[i][c] * kh[t][c] for c in range(d)) for t in range(i + 1)]
        z = sum(math.exp(x) for x in ls)
        zh = sum(math.exp(x) for x in lh)
        p = [math.exp(x) / z for x in ls]
        ph = [math.exp(x) / zh for x in lh]
        kl.append(sum(p[t] * math.log(p[t] / ph[t]) for t in range(i + 1)))
        l2.append(sum((lh[t] - ls[t]) ** 2 for t in range(i + 1)))
        o = [sum(p[t] * v[t][c] for t in range(i + 1)) for c in range(d)]
        oh = [sum(ph[t] * vh[t][c] for t in range(i + 1)) for c in range(d)]
        ose.append(sum((o[c] - oh[c]) ** 2 for c in range(d)))
    return kl, l2, ose


def test_attention_error_rows_brute_force():
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((5, 4)) for _ in range(3))
    kh = k + 0.1 * rng.standard_normal((5, 4))
    vh = v + 0.1 * rng.standard_normal((5, 4))
    kl, l2, ose, osq = cal.attention_error_rows(q, k, v, kh, vh, sm=0.5)
    bk, bl, bo = _error_rows_loops(q.tolist(), k.tolist(), v.tolist(), kh.tolist(), vh.tolist(), 0.5)
    assert np.allclose(kl, bk, atol=1e-14) and np.allclose(l2, bl, atol=1e-13) and np.allclose(ose, bo, atol=1e-14)
    assert kl[0] == pytest.approx(0.0, abs=1e-15)  # one key: both distributions are [1]
    assert np.all(kl >= 0)


def test_logit_error_trace_form():
    """Summed over causal pairs, (q_n . e_t)^2 = e_t (sum_{n >= t} q_n^T q_n) e_t^T
    (the logit-error identity of the MarkTechPost article, "What OSCAR Does
    Differently", restricted to the queries that see key t)."""
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((11, 6)) for _ in range(3))
    kh = k + 0.05 * rng.standard_normal((11, 6))
    _, l2, _, _ = cal.attention_error_rows(q, k, v, kh, v, sm=1.0)
    outer = np.einsum("ni,nj->nij", q, q)
    suffix = np.cumsum(outer[::-1], axis=0)[::-1]  # sum over n >= t
    e = kh - k
    want = sum(e[t] @ suffix[t] @ e[t] for t in range(11))
    assert np.isclose(l2.sum(), want, rtol=1e-12)


def test_error_chain_lossless_grid():
    """Values already on a 4-level grid per group, no rotation, no clipping:
    the quantizer is lossless, so every error is zero."""
    rng = np.random.default_rng(8)
    n, d, g = 16, 8, 4
    lev = rng.integers(0, 4, size=(n, d)).astype(np.float64)
    lev[:, 0], lev[:, 1], lev[:, 4], lev[:, 5] = 0, 3, 0, 3  # every group spans 0..3
    k = 0.5 * (lev - 1)    # s = 0.5, z = 1
    v = 0.25 * (lev - 2)   # s = 0.25, z = 2
    q = rng.standard_normal((2, n, d))
    rows, summ = cal.error_chain(q, k, v, None, None, np.inf, np.inf, g)
    assert np.array_equal(cal.quantize_roundtrip(k, None, np.inf, g), k)
    assert summ["logit_mse"] == 0 and summ["out_rel_mse"] == 0
    assert np.allclose(rows[0], 0, atol=1e-15)


def test_roundtrip_matches_quantizer_and_rotation():
    """E1 = dequantize(quantize(x R)) R^T: undoing the rotation of exactly
    representable codes returns the dequantized rotated vector."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, 8)).astype(np.float32)
    r, _ = np.linalg.qr(rng.standard_normal((8, 8)))
    r32 = r.astype(np.float32)
    codes, s, z = quantize_tokens(x, r32, np.inf, 4)
    y_hat = np.repeat(s, 4, axis=1) * (codes - np.repeat(z, 4, axis=1))
    assert np.allclose(cal.quantize_roundtrip(x, r32, np.inf, 4) @ r32.astype(np.float64), y_hat, atol=1e-12)


def test_error_chain_rotations_beat_no_rotation(calib):
    """Sanity check on the synthetic draw (not a pin): both rotations cut the
    logit error and the score KL of plain INT2 several times over.  (Which of
    the two rotations wins depends on the recipe: with axis-aligned key
    outliers and a query basis drawn independently of them, the Hadamard
    transform alone bounds each rotated key's range best.)"""
    draws, c = calib
    d = draws[0]
    q = d.q[:, :256]
    k, v = d.k[:256].astype(np.float64), d.v[:256].astype(np.float64)
    mix = cal.mix_matrix(64)
    res = {}
    for name, rk, rv in (("none", None, None), ("hadamard", mix, mix), ("oscar", c["r_k64"][0], c["r_v64"][0])):
        tk = np.inf if rk is None else cal.clip_threshold(d.k, rk)
        tv = np.inf if rv is None else cal.clip_threshold(d.v, rv)
        res[name] = cal.error_chain(q, k, v, rk, rv, tk, tv, 64)[1]
    for name in ("hadamard", "oscar"):
        assert res[name]["logit_mse"] < 0.5 * res["none"]["logit_mse"], res
        assert res[name]["kl"] < 0.5 * res["none"]["kl"], res


def test_summarize_hand_computed():
    """Hand-worked summary of two query heads' rows at N = 3 (ModelScope/CSDN
    page, motivation section, Figure 1: score KL and output error).  Causal
    pairs per head are 1 + 2 + 3 = 6, so 12 in all; the KL is averaged over
    the 6 query rows; the output error is one ratio of sums.  The literals
    below were worked out by hand: 12 / 12 pairs, 1.8 / 6 rows, 8 / 80."""
    kl = [[0.0, 0.3, 0.6], [0.0, 0.9, 0.0]]
    lse2 = [[0.5, 1.0, 4.5], [0.0, 3.0, 3.0]]
    ose = [[1.0, 2.0, 3.0], [0.0, 0.0, 2.0]]
    osq = [[10.0, 10.0, 10.0], [10.0, 10.0, 30.0]]
    s = cal.summarize(np.array([kl, lse2, ose, osq]))
    # n^2 normalization would give 2/3, a per-row mean 2.0
    assert s["logit_mse"] == pytest.approx(1.0, rel=1e-15)
    # a summed KL would give 1.8
    assert s["kl"] == pytest.approx(0.3, rel=1e-15)
    # the mean of per-row ratios would give 1/9
    assert s["out_rel_mse"] == pytest.approx(0.1, rel=1e-15)
    # the leading axes are only a stack: one head alone has 6 pairs, 3 rows
    s0 = cal.summarize(np.array([kl[0], lse2[0], ose[0], osq[0]]))
    assert s0["logit_mse"] == pytest.approx(1.0, rel=1e-15)
    assert s0["kl"] == pytest.approx(0.3, rel=1e-15)
    assert s0["out_rel_mse"] == pytest.approx(0.2, rel=1e-15)


def _grid_keys(rng, n, d, g):
    """Keys already on a 4-level grid in every group: lossless without
    rotation or clipping (s = 0.5, z = 1)."""
    lev = rng.integers(0, 4, size=(n, d)).astype(np.float64)
    for j in range(0, d, g):
        lev[:, j], lev[:, j + 1] = 0, 3
    return 0.5 * (lev - 1)


def test_error_chain_routes_key_and_value_parameters():
    """error_chain must quantize the keys with (r_k, tau_k) and the values
    with (r_v, tau_v).  Keys on the grid with no rotation and no clip are
    lossless, so the logit error and the KL are exactly zero while the
    values, rotated and clipped, carry an output error; swapping the
    rotations or the thresholds would make the keys lossy.  The output error
    is checked against pure-Python loops fed the value round trip (E1)."""
    rng = np.random.default_rng(11)
    n, d, g = 9, 8, 4
    k = _grid_keys(rng, n, d, g)
    v = rng.standard_normal((n, d))
    r_v, _ = np.linalg.qr(rng.standard_normal((d, d)))
    r_v = r_v.astype(np.float32)
    tau_v = np.float32(0.6)  # clips the rotated values, and would clip the keys (|k| up to 1)
    q = rng.standard_normal((2, n, d))
    rows, summ = cal.error_chain(q, k, v, None, r_v, np.inf, tau_v, g, sm=0.5)
    assert summ["logit_mse"] == 0.0 and summ["kl"] == 0.0
    assert summ["out_rel_mse"] > 1e-3
    vh = cal.quantize_roundtrip(v, r_v, tau_v, g)
    for h in range(2):
        bk, bl, bo = _error_rows_loops(q[h].tolist(), k.tolist(), v.tolist(), k.tolist(), vh.tolist(), 0.5)
        assert np.allclose(rows[2, h], bo, rtol=1e-12, atol=1e-15)
        assert np.all(rows[0, h] == 0) and np.all(rows[1, h] == 0)
    # the swapped routes are lossy on the keys
    for rk, tk in ((r_v, np.inf), (None, tau_v)):
        _, bad = cal.error_chain(q, k, v, rk, None, tk, np.inf, g, sm=0.5)
        assert bad["logit_mse"] > 1e-4

    # reversed roles: lossless values, rotated and clipped keys
    vg = _grid_keys(rng, n, d, g)
    r_k, _ = np.linalg.qr(rng.standard_normal((d, d)))
    r_k = r_k.astype(np.float32)
    tau_k = np.float32(0.7)
    rows, summ = cal.error_chain(q, k, vg, r_k, None, tau_k, np.inf, g, sm=0.5)
    kh = cal.quantize_roundtrip(k, r_k, tau_k, g)
    for h in range(2):
        bk, bl, bo = _error_rows_loops(q[h].tolist(), k.tolist(), vg.tolist(), kh.tolist(), vg.tolist(), 0.5)
        assert np.allclose(rows[0, h], bk, rtol=1e-10, atol=1e-14)
        assert np.allclose(rows[1, h], bl, rtol=1e-12, atol=1e-14)
        assert np.allclose(rows[2, h], bo, rtol=1e-10, atol=1e-14)
    assert summ["logit_mse"] > 1e-4
