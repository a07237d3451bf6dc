"""GPU parity of the offline calibration and the rotation error chain
(oscar_calib_gram, oscar_calib_attention, oscar_calib_rotation,
oscar_calib_clip, oscar_calibrate, oscar_dequantize, oscar_attention_error)
against the oracle's fp64 calibration (oracle/calibration.py).

Tolerances (fp32 arithmetic in the kernels, fp64 in the oracle):
  * covariances and attention outputs: max abs error <= 1e-5 * the largest
    magnitude of the reference (fp32 sums of a few thousand terms);
  * rotations: orthogonal to 2e-5; Lemma 1's equal diagonal to 1e-4 of
    tr(C)/D; eigenvalues to 1e-5 of the largest; each eigenvector whose
    eigenvalue is separated from its neighbours by >= 1e-2 of the largest
    agrees with the oracle's to |u . u_ref| >= 1 - 1e-4, with the same sign
    where the column's two largest magnitudes differ by >= 1e-3;
  * clip thresholds: exactly the oracle's order statistics without rotation
    (within one fp32 ulp of numpy's quantile); 1e-5 relative with a given
    rotation; at the end of the whole calibration, where R is the library's
    own, 1e-5 relative to the quantile of |x R| for that R, and 5e-4 relative
    to the oracle's tau when every column of U has the oracle's sign: the
    eigenvectors of clustered small eigenvalues are only defined to
    ~eps * lambda_max / gap, and the fp32 covariance alone moves tau by up to
    ~1e-4 (the same Jacobi emulated in numpy fp32 does).  A column whose two
    largest magnitudes differ by less than its fp32 accuracy may take either
    sign (several results are correct); then only the property is checked;
  * dequantization: 1e-5 relative to each vector's norm; error statistics:
    KL to 2e-5 + 2e-3 KL, squared errors to 1e-3 relative.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import pool_io
from harness import log, pool_config, to_dev
from oracle import calibration as cal
from synthetic import CONFIGS, draw_calibration, make_workload

pytestmark = pytest.mark.gpu


def _rel_max(got, ref):
    return np.max(np.abs(np.asarray(got, np.float64) - ref)) / np.max(np.abs(ref))


def _draw(hkv, g, d, n, seed):
    draws = draw_calibration(hkv, g, d, seed, n_cal=n)
    q = np.stack([dr.q for dr in draws])  # [Hkv, g, N, D]
    k = np.stack([dr.k for dr in draws])  # [Hkv, N, D]
    v = np.stack([dr.v for dr in draws])
    return draws, q, k, v


def _token_major(x):
    """[Hkv, N, D] host array -> a device [Hkv, N, D] view of a [N, Hkv, D]
    buffer (the cache's token-major layout)."""
    return to_dev(np.ascontiguousarray(np.transpose(x, (1, 0, 2)))).transpose(0, 1)


@pytest.mark.parametrize("d,rows,strided", [(128, 8192, False), (64, 333, True), (128, 100, True)])
def test_gram_matches_numpy(gpu_lib, d, rows, strided):
    oscar = gpu_lib
    rng = np.random.default_rng(d + rows)
    heads = 3
    x = (rng.standard_normal((heads, rows, d)) * rng.uniform(0.1, 10, d)).astype(np.float32)
    xd = _token_major(x) if strided else to_dev(x)
    out = torch.empty(heads, d, d, dtype=torch.float32, device="cuda")
    log(f"gram d={d} rows={rows} strided={strided}")
    oscar.oscar_calib_gram(xd, 1.0 / rows, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for h in range(heads):
        ref = cal.query_covariance(x[h])
        err = _rel_max(got[h], ref)
        assert err <= 1e-5, (h, err)
    log(f"gram: worst {max(_rel_max(got[h], cal.query_covariance(x[h])) for h in range(heads)):.2e}")


@pytest.mark.parametrize("d,n,g", [(64, 77, 2), (128, 300, 4), (128, 2048, 4)])
def test_calibration_attention_matches_oracle(gpu_lib, d, n, g):
    oscar = gpu_lib
    hkv = 2
    _, q, k, v = _draw(hkv, g, d, n, seed=d + n)
    out = torch.empty(hkv, g, n, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(hkv, g, n, dtype=torch.float32, device="cuda")
    log(f"calibration attention d={d} n={n} g={g}")
    oscar.oscar_calib_attention(to_dev(q), _token_major(k), _token_major(v), out, lse)
    torch.cuda.synchronize()
    o_g, l_g = out.cpu().numpy(), lse.cpu().numpy()
    rows = range(n) if n <= 300 else sorted(set(np.random.default_rng(0).integers(0, n, 64).tolist()) | {0, n - 1})
    rows = list(rows)
    for h in range(hkv):
        for j in range(g):
            o_r, l_r = cal.causal_attention(q[h, j], k[h], v[h])
            for r in rows:
                nrm = np.linalg.norm(o_r[r])
                assert np.max(np.abs(o_g[h, j, r] - o_r[r])) <= 1e-5 * max(nrm, 1.0), (h, j, r)
                assert abs(l_g[h, j, r] - l_r[r]) <= 1e-5 * max(1.0, abs(l_r[r])), (h, j, r)


def _check_rotation(r_gpu, eig_gpu, c, mix, what):
    d = c.shape[0]
    r = np.asarray(r_gpu, np.float64)
    assert np.max(np.abs(r @ r.T - np.eye(d))) <= 2e-5, what
    u_ref, w_ref = cal.eigenbasis(c)
    lam_max = np.max(np.abs(w_ref))
    assert np.max(np.abs(np.asarray(eig_gpu, np.float64) - w_ref)) <= 1e-5 * lam_max, what
    u = r @ cal.mix_matrix(d).T if mix else r
    if mix:
        dg = np.diag(r.T @ c @ r)
        assert np.max(np.abs(dg - np.trace(c) / d)) <= 1e-4 * np.trace(c) / d, what  # Lemma 1
    gaps = np.abs(np.diff(w_ref))
    sep = np.minimum(np.r_[np.inf, gaps], np.r_[gaps, np.inf]) >= 1e-2 * lam_max
    checked = 0
    for i in np.nonzero(sep)[0]:
        dot = float(u[:, i] @ u_ref[:, i])
        assert abs(dot) >= 1 - 1e-4, (what, i, dot)
        mags = np.sort(np.abs(u_ref[:, i]))
        if mags[-1] - mags[-2] >= 1e-3:
            assert dot > 0, (what, i, "sign convention")
        checked += 1
    return checked


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_of_calibration_covariances(gpu_lib, d):
    oscar = gpu_lib
    hkv = 3
    draws, q, k, v = _draw(hkv, 2, d, 1024, seed=d)
    covs = np.stack([cal.query_covariance(dr.q) for dr in draws] +
                    [cal.score_weighted_covariance(dr.q, dr.k, dr.v) for dr in draws]).astype(np.float32)
    for mix in (True, False):
        r = torch.empty(2 * hkv, d, d, dtype=torch.float32, device="cuda")
        eig = torch.empty(2 * hkv, d, dtype=torch.float32, device="cuda")
        log(f"rotation d={d} mix={mix}")
        oscar.oscar_calib_rotation(to_dev(covs), r, eig, mix=mix)
        torch.cuda.synchronize()
        rg, eg = r.cpu().numpy(), eig.cpu().numpy()
        n = sum(_check_rotation(rg[i], eg[i], covs[i].astype(np.float64), mix, f"head {i} mix {mix}")
                for i in range(2 * hkv))
        log(f"rotation d={d} mix={mix}: {n} separated eigenvectors aligned")
        assert n >= 2 * hkv  # at least the top direction of each head


def test_rotation_closed_form_diagonal(gpu_lib):
    """A diagonal covariance with distinct entries: U is the permutation that
    sorts them (no Jacobi rotation is needed), and R = U H P_br exactly."""
    oscar = gpu_lib
    d = 128
    rng = np.random.default_rng(5)
    diag = rng.permutation(np.arange(1, d + 1)).astype(np.float32)
    c = np.diag(diag)[None]
    r = torch.empty(1, d, d, dtype=torch.float32, device="cuda")
    eig = torch.empty(1, d, dtype=torch.float32, device="cuda")
    oscar.oscar_calib_rotation(to_dev(c), r, eig, mix=True)
    torch.cuda.synchronize()
    u = np.eye(d)[:, np.argsort(-diag, kind="stable")]
    assert np.array_equal(eig.cpu().numpy()[0], np.sort(diag)[::-1])
    assert np.allclose(r.cpu().numpy()[0], u @ cal.mix_matrix(d), atol=1e-7)


@pytest.mark.parametrize("d,rows", [(128, 2048), (64, 203)])
def test_clip_threshold(gpu_lib, d, rows):
    oscar = gpu_lib
    heads = 3
    rng = np.random.default_rng(rows)
    x = (rng.standard_normal((heads, rows, d)) * np.where(np.arange(d) % 17 == 0, 20.0, 1.0)).astype(np.float32)
    xd = _token_major(x)
    tau = torch.empty(heads, dtype=torch.float32, device="cuda")
    log(f"clip d={d} rows={rows} unrotated")
    oscar.oscar_calib_clip(xd, None, 0.995, tau)
    torch.cuda.synchronize()
    got = tau.cpu().numpy()
    for h in range(heads):
        ref = np.float32(np.quantile(np.abs(x[h].astype(np.float64)), 0.995))
        ulp = np.spacing(ref)
        assert abs(float(got[h]) - float(ref)) <= ulp, (h, got[h], ref)
        assert got[h] == cal.clip_threshold(x[h], None) or abs(float(got[h]) - float(ref)) <= ulp
    # rotated: R from a seeded orthogonal matrix (an input, not a result of the library)
    rr = np.stack([np.linalg.qr(rng.standard_normal((d, d)))[0] for _ in range(heads)]).astype(np.float32)
    log(f"clip d={d} rows={rows} rotated")
    oscar.oscar_calib_clip(xd, to_dev(rr), 0.995, tau)
    torch.cuda.synchronize()
    got = tau.cpu().numpy()
    for h in range(heads):
        ref = cal.clip_threshold(x[h], rr[h].astype(np.float64))
        assert abs(float(got[h]) - float(ref)) <= 1e-5 * float(ref), (h, got[h], ref)
    # other quantiles, including both ends
    for qq in (0.0, 0.5, 1.0):
        oscar.oscar_calib_clip(xd, None, qq, tau)
        torch.cuda.synchronize()
        for h in range(heads):
            ref = np.float32(np.quantile(np.abs(x[h].astype(np.float64)), qq))
            assert abs(float(tau.cpu().numpy()[h]) - float(ref)) <= np.spacing(ref), (qq, h)


@pytest.mark.parametrize("hkv,g,d,n", [(2, 2, 64, 512), (8, 4, 128, 2048)])
def test_calibrate_matches_oracle(gpu_lib, hkv, g, d, n):
    """The whole calibration (the last case is the Qwen3-8B layer shape with
    the 2048-token calibration draw)."""
    oscar = gpu_lib
    draws, q, k, v = _draw(hkv, g, d, n, seed=hkv * 100 + d)
    log(f"calibrate hkv={hkv} g={g} d={d} n={n}")
    res = oscar.oscar_calibrate(to_dev(q), _token_major(k), _token_major(v), clip_quantile=0.995)
    torch.cuda.synchronize()
    got = {name: t.cpu().numpy() for name, t in res.items()}
    ref = cal.calibrate([(dr.q, dr.k, dr.v) for dr in draws])
    for h in range(hkv):
        assert _rel_max(got["c_q"][h], ref["c_q"][h]) <= 1e-5, h
        assert _rel_max(got["c_s"][h], ref["c_s"][h]) <= 1e-5, h
        for key, cov, tkey, x in (("r_k", "c_q", "tau_k", draws[h].k), ("r_v", "c_s", "tau_v", draws[h].v)):
            r = got[key][h].astype(np.float64)
            assert np.max(np.abs(r @ r.T - np.eye(d))) <= 2e-5, (key, h)
            dg = np.diag(r.T @ ref[cov][h] @ r)
            assert np.max(np.abs(dg - np.trace(ref[cov][h]) / d)) <= 1e-4 * np.trace(ref[cov][h]) / d, (key, h)
            u = r @ cal.mix_matrix(d).T
            u_ref = ref[key + "64"][h] @ cal.mix_matrix(d).T
            # the attention-importance direction: U's first column matches
            assert float(u[:, 0] @ u_ref[:, 0]) >= 1 - 1e-4, (key, h)
            # column signs: the convention (largest-magnitude entry positive)
            # decides a sign only where that entry stands out beyond the
            # eigenvectors' fp32 accuracy; elsewhere either sign is a valid
            # result, and through H P_br the sign moves tau
            dots = np.sum(u * u_ref, axis=0)
            mags = np.sort(np.abs(u_ref), axis=0)
            flipped = np.nonzero(dots < 0)[0]
            assert np.all(mags[-1, flipped] - mags[-2, flipped] < 1e-3), (key, h, flipped)
            # tau is the quantile of |x R| for the R returned (a property of the
            # result, checked in fp64 here)
            want = np.float32(np.quantile(np.abs(x.astype(np.float64) @ r), 0.995))
            assert abs(float(got[tkey][h]) - float(want)) <= 1e-5 * float(want), (tkey, h)
            if flipped.size == 0:
                assert abs(float(got[tkey][h]) - float(ref[tkey][h])) <= 5e-4 * float(ref[tkey][h]), (tkey, h)
            else:
                log(f"{key} head {h}: columns {flipped.tolist()} signed the other way (tie within fp32)")
    log(f"calibrate: tau_k {got['tau_k'][:4]} vs {ref['tau_k'][:4]}")


def _oracle_pool(wl, k, v, r_k, r_v, tau_k, tau_v, seed):
    """INT2 pages written by the oracle quantizer through the documented
    layout (independent of the write kernels)."""
    t, hkv, d = k.shape
    npg = (t + 15) // 16
    blocks = []
    for h in range(hkv):
        kc, ks, kz = oracle.quantize_tokens(k[:, h], r_k[h], tau_k[h], wl.group_size)
        vc, vs, vz = oracle.quantize_tokens(v[:, h], r_v[h], tau_v[h], wl.group_size)
        pad = npg * 16 - t

        def pg(a):
            return np.concatenate([a, np.zeros((pad,) + a.shape[1:], a.dtype)]).reshape(npg, 16, -1)
        blocks.append(pool_io.pack_int2_blocks(pg(kc), pg(ks), pg(kz), pg(vc), pg(vs), pg(vz)))
    rng = np.random.default_rng(seed)
    n_phys = npg + 5
    ids = rng.permutation(n_phys)[:npg].astype(np.int32)
    pool = rng.integers(0, 256, (n_phys, hkv, blocks[0].shape[1]), dtype=np.uint8)
    for h in range(hkv):
        pool[ids, h] = blocks[h]
    return pool.reshape(n_phys, -1), ids


@pytest.mark.parametrize("d,g_size,t", [(128, 128, 200), (128, 64, 77), (64, 64, 64)])
def test_dequantize_matches_oracle(gpu_lib, d, g_size, t):
    oscar = gpu_lib
    wl = make_workload(CONFIGS["qwen3-8b-l100k"] if d == 128 else CONFIGS["tiny-d64-l512"],
                       num_q_heads=4, num_kv_heads=2, group_size=g_size, batch=1, seq_lens=(t,), seed=3)
    rng = np.random.default_rng(t)
    k = pool_io.bits_to_f32(pool_io.bf16_bits(rng.standard_normal((t, 2, d)) * 3))
    v = pool_io.bits_to_f32(pool_io.bf16_bits(rng.standard_normal((t, 2, d))))
    r_k = np.stack([np.linalg.qr(rng.standard_normal((d, d)))[0] for _ in range(2)]).astype(np.float32)
    r_v = np.stack([np.linalg.qr(rng.standard_normal((d, d)))[0] for _ in range(2)]).astype(np.float32)
    tau = np.array([6.0, 5.0], np.float32)
    host_pool, ids = _oracle_pool(wl, k, v, r_k, r_v, tau, tau, seed=t)
    pool = oscar.OscarPool(pool_config(wl, v_absorbed=False))
    k_out = torch.empty(t, 2, d, dtype=torch.float32, device="cuda")
    v_out = torch.empty(t, 2, d, dtype=torch.float32, device="cuda")
    log(f"dequantize d={d} G={g_size} T={t}")
    oscar.oscar_dequantize(pool, t, to_dev(ids), to_dev(host_pool), to_dev(r_k), to_dev(r_v), k_out, v_out)
    torch.cuda.synchronize()
    kg, vg = k_out.cpu().numpy(), v_out.cpu().numpy()
    for h in range(2):
        for x, xg, r in ((k, kg, r_k), (v, vg, r_v)):
            ref = cal.quantize_roundtrip(x[:, h], r[h], tau[h], g_size)
            err = np.abs(xg[:, h] - ref).max(axis=1) / np.linalg.norm(ref, axis=1)
            assert np.all(err <= 1e-5), err.max()
    # without rotations: the stored basis
    oscar.oscar_dequantize(pool, t, to_dev(ids), to_dev(host_pool), None, None, k_out, v_out)
    torch.cuda.synchronize()
    codes, s, z = oracle.quantize_tokens(k[:, 1], r_k[1], tau[1], g_size)
    assert np.allclose(k_out.cpu().numpy()[:, 1], oracle.dequantize(codes, s, z, g_size), rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("d,n,g", [(64, 130, 2), (128, 512, 4)])
def test_attention_error_matches_oracle(gpu_lib, d, n, g):
    oscar = gpu_lib
    hkv = 2
    draws, q, k, v = _draw(hkv, g, d, n, seed=7 * n)
    k = pool_io.bits_to_f32(pool_io.bf16_bits(k))
    v = pool_io.bits_to_f32(pool_io.bf16_bits(v))
    mix = cal.mix_matrix(d)
    kh = np.stack([cal.quantize_roundtrip(k[h], mix.astype(np.float32), cal.clip_threshold(k[h], mix), 64)
                   for h in range(hkv)]).astype(np.float32)
    vh = np.stack([cal.quantize_roundtrip(v[h], mix.astype(np.float32), cal.clip_threshold(v[h], mix), 64)
                   for h in range(hkv)]).astype(np.float32)
    stats = torch.empty(hkv, g, n, 4, dtype=torch.float32, device="cuda")
    log(f"attention error d={d} n={n} g={g}")
    oscar.oscar_attention_error(to_dev(q), _token_major(k), _token_major(v), _token_major(kh), _token_major(vh),
                                stats)
    torch.cuda.synchronize()
    sg = stats.cpu().numpy()
    for h in range(hkv):
        for j in range(g):
            kl, l2, ose, osq = cal.attention_error_rows(q[h, j], k[h], v[h], kh[h], vh[h])
            assert np.all(np.abs(sg[h, j, :, 0] - kl) <= 2e-5 + 2e-3 * kl), (h, j)
            for c, ref in ((1, l2), (2, ose), (3, osq)):
                assert np.all(np.abs(sg[h, j, :, c] - ref) <= 1e-3 * ref + 1e-6), (h, j, c)


def _summary_by_loops(st):
    """The chain's three figures from the kernel's per-row statistics
    st [Hkv, g, N, 4], written out without the oracle's summarize: row n of
    a causal attention sees n + 1 keys, so the logit error is averaged over
    sum_n (n + 1) pairs per query head, the KL over the rows, and the output
    error is one ratio of sums."""
    hkv, g, n, _ = st.shape
    kl_sum = l2_sum = e_sum = o_sum = 0.0
    pairs = rows = 0
    for h in range(hkv):
        for j in range(g):
            for r in range(n):
                kl_sum += float(st[h, j, r, 0])
                l2_sum += float(st[h, j, r, 1])
                e_sum += float(st[h, j, r, 2])
                o_sum += float(st[h, j, r, 3])
                pairs += r + 1
                rows += 1
    return {"logit_mse": l2_sum / pairs, "kl": kl_sum / rows, "out_rel_mse": e_sum / o_sum}


def test_error_chain_on_gpu_matches_oracle(gpu_lib):
    """quantize_pack -> dequantize -> attention_error with the oracle's
    rotations and thresholds, against the oracle's chain on the same bf16
    inputs.  The kernels may flip a code that lies on a rounding boundary
    within the rotation's fp32 error, so the summaries agree to 2 %."""
    oscar = gpu_lib
    hkv, g, d, n = 2, 2, 128, 512
    draws, q, k, v = _draw(hkv, g, d, n, seed=99)
    kb = pool_io.bits_to_f32(pool_io.bf16_bits(k))
    vb = pool_io.bits_to_f32(pool_io.bf16_bits(v))
    ref = cal.calibrate([(dr.q, dr.k, dr.v) for dr in draws])
    wl = make_workload(CONFIGS["qwen3-8b-l100k"], num_q_heads=hkv * g, num_kv_heads=hkv, batch=1, seq_lens=(n,),
                       seed=1)
    pool = oscar.OscarPool(pool_config(wl, v_absorbed=False))
    npg = n // 16
    ids = torch.arange(npg, dtype=torch.int32, device="cuda")
    int2 = torch.zeros(npg, pool.int2_page_bytes, dtype=torch.uint8, device="cuda")
    k_tok = to_dev(np.ascontiguousarray(kb.transpose(1, 0, 2)), torch.bfloat16)
    v_tok = to_dev(np.ascontiguousarray(vb.transpose(1, 0, 2)), torch.bfloat16)
    r_k, r_v = to_dev(ref["r_k"]), to_dev(ref["r_v"])
    oscar.oscar_quantize_pack(pool, k_tok, v_tok, ids, int2, r_k, to_dev(ref["tau_k"]), to_dev(ref["tau_v"]), r_v=r_v)
    kh = torch.empty(n, hkv, d, dtype=torch.float32, device="cuda")
    vh = torch.empty(n, hkv, d, dtype=torch.float32, device="cuda")
    oscar.oscar_dequantize(pool, n, ids, int2, r_k, r_v, kh, vh)
    stats = torch.empty(hkv, g, n, 4, dtype=torch.float32, device="cuda")
    oscar.oscar_attention_error(to_dev(q), k_tok.float().transpose(0, 1), v_tok.float().transpose(0, 1),
                                kh.transpose(0, 1), vh.transpose(0, 1), stats)
    torch.cuda.synchronize()
    got = _summary_by_loops(stats.cpu().numpy().astype(np.float64))
    want = cal.summarize(np.stack([cal.error_chain(q[h], kb[h], vb[h], ref["r_k"][h], ref["r_v"][h], ref["tau_k"][h],
                                                   ref["tau_v"][h], 128)[0] for h in range(hkv)], axis=1))
    log(f"error chain gpu {got} oracle {want}")
    for key in want:
        assert abs(got[key] - want[key]) <= 2e-2 * want[key], (key, got[key], want[key])
