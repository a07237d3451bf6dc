"""Test-side helpers for the GPU parity tests: build cases from the seeded
generator and the oracle, upload pools, and apply the acceptance rules.

Tolerances (stated for the path's fp32 accumulation with bf16 I/O):
  * decode output: per (sequence, query head), max_c |o_gpu - o_ref| <=
    2e-3 * ||o_ref||_2;
  * write path, pre-rotated input (no rotation): codes, scales and zeros
    bit-exact;
  * write path with the key rotation: scale/zero may differ by one bf16 step
    only where the oracle's value before rounding lies within the rotation
    error of a rounding midpoint; a code may differ from the one the oracle
    picks with the GPU's scale and zero only where the clipped value lies
    within 1e-5 * scale of the boundary between the two codes.
"""

import functools
import math
import sys

import numpy as np
import torch

import oracle
import pool_io
import synthetic

DECODE_TOL = 2e-3
FLIP_TOL = 1e-5


def log(msg):
    print(msg, file=sys.stderr, flush=True)


@functools.lru_cache(maxsize=16)
def _oracle_calibration(num_kv_heads, gqa, head_dim, seed):
    draws = synthetic.draw_calibration(num_kv_heads, gqa, head_dim, seed)
    c = oracle.calibrate([(d.q, d.k, d.v) for d in draws])
    return synthetic.make_calibration(draws, c["r_k"], c["r_v"], c["tau_k"], c["tau_v"])


def calibration(wl):
    """Offline parameters for a workload, from the oracle's calibration of the
    seeded calibration draw."""
    return _oracle_calibration(wl.num_kv_heads, wl.gqa, wl.head_dim, wl.seed)


def draw_inputs(wl, calib=None, **kw):
    """The seeded cache tensors and queries of a workload, with the oracle's
    offline parameters unless ``calib`` is given."""
    return synthetic.draw_inputs(wl, calibration(wl) if calib is None else calib, **kw)


def make_seqs(wl, inputs, r_k=None, tau_k=None, tau_v=None, r_v=None, levels=None):
    """Oracle pool state for every sequence of an Inputs draw.  With r_v the
    pool does not absorb V: the history stores V R_V.  levels = (levels_k,
    levels_v): the four-level codebook quantizer."""
    c = inputs.calib
    r_k = c.r_k if r_k is None else r_k
    tau_k = c.tau_k if tau_k is None else tau_k
    tau_v = c.tau_v if tau_v is None else tau_v
    seqs = []
    for b, L in enumerate(wl.seq_lens):
        k = inputs.k[b][:L].float().numpy()
        v = inputs.v[b][:L].float().numpy()
        lk, lv = (None, None) if levels is None else levels
        s = oracle.SeqPool(wl.num_kv_heads, wl.head_dim, wl.group_size, wl.sink, wl.recent,
                           v_absorbed=r_v is None, levels_k=lk, levels_v=lv)
        seqs.append(s.prefill(k, v, r_k, tau_k, tau_v, r_v))
    return seqs


def pool_config(wl, v_absorbed=True, levels=None):
    """Pool configuration of a workload; ``levels`` = (levels_k, levels_v)
    selects the four-level codebook."""
    import long_context_decode_oscar_amd as oscar
    if levels is None:
        return oscar.PoolConfig(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.group_size, 16, wl.sink,
                                wl.recent, 1 if v_absorbed else 0, 0.0)
    return oscar.PoolConfig(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.group_size, 16, wl.sink, wl.recent,
                            1 if v_absorbed else 0, 0.0, 1, tuple(float(x) for x in levels[0]),
                            tuple(float(x) for x in levels[1]))


def to_dev(x, dtype=None):
    t = torch.as_tensor(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def upload(pools):
    return {k: to_dev(v) for k, v in pools.items()}


def check_decode(out_gpu, ref, pairs=None, tol=DECODE_TOL, what=""):
    """Per (b, h) max abs error relative to ||o_ref||_2."""
    out = out_gpu.float().cpu().numpy().astype(np.float64)
    bsz, hq, _ = ref.shape
    pairs = pairs or [(b, h) for b in range(bsz) for h in range(hq)]
    worst = 0.0
    for b, h in pairs:
        nrm = np.linalg.norm(ref[b, h])
        err = np.max(np.abs(out[b, h] - ref[b, h]))
        assert np.all(np.isfinite(out[b, h])), (what, b, h)
        rel = err / max(nrm, 1e-30)
        worst = max(worst, rel)
        assert err <= tol * nrm, f"{what} b={b} h={h}: max err {err:.3e} > {tol} * {nrm:.3e}"
    log(f"{what}: worst max-err / ||o|| = {worst:.2e} over {len(pairs)} heads")
    return worst


def _bf16_neighbors_ok(got, ref, pre, slack):
    """got/ref bf16 values (float32), pre the fp32 value before rounding:
    equal, or one bf16 step apart with pre within `slack` of their midpoint."""
    if got == ref:
        return True
    gb = int(np.float32(got).view(np.uint32) >> 16)
    rb = int(np.float32(ref).view(np.uint32) >> 16)
    if abs(gb - rb) != 1:
        return False
    mid = (float(got) + float(ref)) / 2
    return abs(float(pre) - mid) <= slack


def check_write(gpu, x, r, tau, gs, what, rot_err_rel=4e-5, levels=None):
    """gpu = (codes [N, D], s [N, NG], z [N, NG]) read back from the pool;
    x [N, D] bf16 inputs; r rotation (None for pre-rotated input); levels: a
    four-level codebook (None: the uniform levels)."""
    codes_g, s_g, z_g = gpu
    codes_o, s_o, z_o, y_o, c_o = oracle.quantize_tokens(x, r, tau, gs, return_intermediate=True)
    if levels is not None:
        # scale and zero are the uniform quantizer's; the codes the codebook's
        codes_o = oracle.codebook.quantize_tokens(x, r, tau, gs, levels)[0]
    n, d = codes_o.shape
    ng = d // gs
    if r is None:
        assert np.array_equal(s_g.view(np.uint32), s_o.view(np.uint32)), f"{what}: scales differ"
        assert np.array_equal(z_g.view(np.uint32), z_o.view(np.uint32)), f"{what}: zeros differ"
        bad = np.argwhere(codes_g != codes_o)
        assert bad.size == 0, f"{what}: {len(bad)} codes differ, first {bad[:5].tolist()}"
        log(f"{what}: {n} tokens bit-exact")
        return 0
    cg = c_o.reshape(n, ng, gs).astype(np.float64)
    mn, mx = cg.min(-1), cg.max(-1)
    eps_y = rot_err_rel * np.abs(y_o).max(axis=1)  # rotation error bound per token
    pre_s = (mx - mn).astype(np.float32) / np.float32(3)
    sz_mism = 0
    for i, g in zip(*np.nonzero((s_g != s_o) | (z_g != z_o))):
        sz_mism += 1
        assert _bf16_neighbors_ok(s_g[i, g], s_o[i, g], pre_s[i, g], 2 * eps_y[i] / 3 + 1e-6 * abs(pre_s[i, g])) \
            or s_g[i, g] == s_o[i, g], f"{what}: scale token {i} group {g}: {s_g[i, g]} vs {s_o[i, g]}"
        if s_g[i, g] == s_o[i, g]:
            pre_z = -mn[i, g] / s_o[i, g]
            assert _bf16_neighbors_ok(z_g[i, g], z_o[i, g], pre_z, eps_y[i] / s_o[i, g] + 1e-6 * abs(pre_z)), \
                f"{what}: zero token {i} group {g}: {z_g[i, g]} vs {z_o[i, g]}"
        else:
            assert abs(float(z_g[i, g]) - float(z_o[i, g])) <= 2 * 2.0 ** (math.floor(math.log2(abs(z_o[i, g]) + 1e-30)) - 7) + 1e-30
    assert sz_mism <= max(3, 1e-3 * n * ng), f"{what}: {sz_mism} scale/zero mismatches"
    # codes, re-evaluated with the GPU's scale and zero on the oracle's clipped values
    sgb = np.repeat(s_g, gs, axis=1)
    zgb = np.repeat(z_g, gs, axis=1)
    t = ((c_o / sgb).astype(np.float32) + zgb).astype(np.float32)
    if levels is None:
        ref = np.clip(np.rint(t), 0, 3).astype(np.int64)
        mids = np.array([0.5, 1.5, 2.5])
    else:
        ref = oracle.codebook.encode(t, levels).astype(np.int64)
        mids = oracle.codebook.thresholds(levels)
    got = codes_g.astype(np.int64)
    flips = np.argwhere(ref != got)
    for i, c in flips:
        assert abs(int(ref[i, c]) - int(got[i, c])) == 1, f"{what}: code jump at token {i} ch {c}"
        k = min(ref[i, c], got[i, c])
        boundary = float(sgb[i, c]) * (mids[k] - float(zgb[i, c]))
        assert abs(float(c_o[i, c]) - boundary) <= FLIP_TOL * float(sgb[i, c]), \
            f"{what}: flip at token {i} ch {c}: c={c_o[i, c]} boundary={boundary} s={sgb[i, c]}"
    log(f"{what}: {n} tokens, {sz_mism} scale/zero one-step differences, {len(flips)} allowed code flips")
    return len(flips)


def dense_kv(inputs, b, L=None):
    k = inputs.k[b] if L is None else inputs.k[b][:L]
    v = inputs.v[b] if L is None else inputs.v[b][:L]
    return k.float().numpy(), v.float().numpy()
