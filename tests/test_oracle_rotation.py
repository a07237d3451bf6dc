"""Pins for the offline rotation recipe R = U H P_br that the inputs use."""

import numpy as np
import pytest

from synthetic import bit_reversal_permutation, calibrate, hadamard_matrix


@pytest.fixture(scope="module")
def calib():
    return calibrate(num_kv_heads=2, gqa=2, head_dim=64, seed=0, n_cal=1024)


def test_bit_reversal_table_and_involution():
    p = bit_reversal_permutation(128)
    assert p[1] == 64 and p[3] == 96 and p[2] == 32 and p[127] == 127 and p[0] == 0
    assert np.array_equal(p[p], np.arange(128))
    p6 = bit_reversal_permutation(64)
    assert p6[1] == 32 and p6[5] == 40  # 000101 -> 101000
    # every power-of-two group of consecutive output channels takes one input
    # from each importance band (MarkTechPost article, P_br bullet)
    for gsz in (2, 4, 8, 16, 32, 64):
        for start in range(0, 128, gsz):
            bands = sorted(int(i) // (128 // gsz) for i in p[start:start + gsz])
            assert bands == list(range(gsz))


def test_hadamard_orthonormal_sylvester():
    h = hadamard_matrix(64)
    assert np.allclose(h @ h.T, np.eye(64), atol=1e-14)
    assert np.allclose(np.abs(h), 1 / 8)
    h2 = hadamard_matrix(32)
    assert np.allclose(h[:32, :32], h2 / np.sqrt(2)) and np.allclose(h[32:, 32:], -h2 / np.sqrt(2))


def test_rotations_orthogonal(calib):
    for r in (calib.r_k, calib.r_v):
        for rk in r:
            rk = rk.astype(np.float64)
            assert np.max(np.abs(rk @ rk.T - np.eye(rk.shape[0]))) < 1e-6


def test_lemma1_equalises_query_energy(calib):
    """diag(R_K^T C_Q R_K) = tr(C_Q)/D for every channel (MarkTechPost article,
    Lemma 1).  Holds only for the row-vector convention x' = x R with U_Q the
    eigenbasis of C_Q; the transposed R or a basis that does not diagonalise
    C_Q breaks it."""
    for rk, cq in zip(calib.r_k, calib.c_q):
        rk = rk.astype(np.float64)
        dg = np.diag(rk.T @ cq @ rk)
        assert np.allclose(dg, np.trace(cq) / cq.shape[0], rtol=2e-5)
        assert not np.allclose(np.diag(rk @ cq @ rk.T), np.trace(cq) / cq.shape[0], rtol=1e-2)


def test_u_diagonalises_covariances(calib):
    h = hadamard_matrix(64)
    p = np.zeros((64, 64))
    p[np.arange(64), bit_reversal_permutation(64)] = 1
    for rk, cq, rv, cs in zip(calib.r_k, calib.c_q, calib.r_v, calib.c_s):
        for r, c in ((rk, cq), (rv, cs)):
            u = r.astype(np.float64) @ p.T @ h.T  # undo H P_br
            lam = u.T @ c @ u
            off = lam - np.diag(np.diag(lam))
            assert np.max(np.abs(off)) < 1e-5 * np.max(np.abs(lam))
            assert np.all(np.diff(np.diag(lam)) <= 1e-9 * np.max(np.abs(lam)))  # descending


def test_clip_thresholds_are_quantiles(calib):
    assert calib.tau_k.dtype == np.float32 and np.all(calib.tau_k > 0)
    # outlier keys are spread by the Hadamard factor: rotated keys are far
    # from the x20 outliers, so tau_K is well below 20
    assert np.all(calib.tau_k < 20) and np.all(calib.tau_v < 5)
