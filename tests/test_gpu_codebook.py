"""GPU parity of the four-level codebook variant (oscar_config.codebook = 1)
against the oracle's codebook quantizer and decode (oracle/codebook.py):
the write paths (bulk and decode-time), decode (plain and prefix-shared,
V absorbed or not), dequantization, and the Lloyd-Max fit of the levels.

Tolerances are those of the uniform path: codes, scales and zeros bit-exact
for pre-rotated input, the flip rule (with the codebook's thresholds as the
code boundaries) under a fused rotation, decode within 2e-3 of each head's
norm.  The fitted levels must equal the oracle's, or differ by one 1/32 step
only where the oracle's level before rounding lies within 1e-4 of a rounding
midpoint.
"""

import numpy as np
import pytest
import torch

import oracle
import pool_io
from harness import check_decode, check_write, draw_inputs, log, make_seqs, pool_config, to_dev, upload
from oracle import calibration as cal
from oracle import codebook as cb
from synthetic import CONFIGS, draw_calibration, make_workload

pytestmark = pytest.mark.gpu

TINY = CONFIGS["tiny-d64-l512"]
QWEN = CONFIGS["qwen3-8b-l100k"]
# codebooks of the shape the fit gives on the synthetic draws (interior
# levels pulled toward the middle), and a lopsided one
LEVELS = {
    "fit-like": (np.array([0.0, 1.125, 1.875, 3.0]), np.array([0.0, 1.09375, 1.90625, 3.0])),
    "lopsided": (np.array([0.0, 0.71875, 2.40625, 3.0]), np.array([0.0, 1.5, 1.53125, 3.0])),
}
WL = {
    "d128-g128": make_workload(QWEN, num_q_heads=8, num_kv_heads=2, batch=1, seq_lens=(1000,), seed=41),
    "d128-g64": make_workload(QWEN, num_q_heads=8, num_kv_heads=2, group_size=64, batch=1, seq_lens=(1000,),
                              seed=42),
    "d64-g64": make_workload(TINY, batch=1, seq_lens=(1000,), seed=43),
}


def _identity(hkv, d):
    return np.stack([np.eye(d, dtype=np.float32)] * hkv)


def _bulk(oscar, wl, k, v, r_k, tau_k, tau_v, levels, seed=0, r_v=None):
    t = k.shape[0]
    npg = (t + 15) // 16
    pool = oscar.OscarPool(pool_config(wl, v_absorbed=r_v is None, levels=levels))
    rng = np.random.default_rng(seed)
    n_phys = npg + 3
    ids = rng.permutation(n_phys)[:npg].astype(np.int32)
    int2 = torch.randint(0, 256, (n_phys, pool.int2_page_bytes), dtype=torch.uint8, device="cuda")
    log(f"quantize_pack (codebook) T={t}")
    oscar.oscar_quantize_pack(pool, to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16), to_dev(ids), int2,
                              to_dev(r_k), to_dev(tau_k), to_dev(tau_v), r_v=None if r_v is None else to_dev(r_v))
    torch.cuda.synchronize()
    return pool_io.read_history(int2.cpu().numpy(), ids, t, wl.num_kv_heads, wl.head_dim, wl.n_groups)


@pytest.mark.parametrize("lv", list(LEVELS))
@pytest.mark.parametrize("name", list(WL))
@pytest.mark.parametrize("rotated", [False, True, "values too"])
def test_quantize_pack_codebook(gpu_lib, name, lv, rotated):
    wl = WL[name]
    levels = LEVELS[lv]
    inp = draw_inputs(wl, with_q=False)
    k, v = inp.k[0][:1000].float().numpy(), inp.v[0][:1000].float().numpy()
    c = inp.calib
    r_k = c.r_k if rotated else _identity(wl.num_kv_heads, wl.head_dim)
    r_v = c.r_v if rotated == "values too" else None
    kc, ks, kz, vc, vs, vz = _bulk(gpu_lib, wl, k, v, r_k, c.tau_k, c.tau_v, levels, seed=wl.seed, r_v=r_v)
    for h in range(wl.num_kv_heads):
        check_write((kc[:, h], ks[:, h], kz[:, h]), k[:, h], r_k[h] if rotated else None, c.tau_k[h],
                    wl.group_size, f"{name} {lv} K head {h} rotated={rotated}", levels=levels[0])
        check_write((vc[:, h], vs[:, h], vz[:, h]), v[:, h], None if r_v is None else r_v[h], c.tau_v[h],
                    wl.group_size, f"{name} {lv} V head {h}", levels=levels[1])


@pytest.mark.parametrize("lv", list(LEVELS))
@pytest.mark.parametrize("name", list(WL))
def test_quantize_pack_codebook_degenerate_groups(gpu_lib, name, lv):
    """The codebook encoding on groups that leave the reciprocal fast path
    (constant groups, scales below 2^-70, values near 1e20, zero points of
    several hundred): pre-rotated input, no clipping, bit-exact codes,
    scales and zeros."""
    from test_gpu_write import _degenerate_rows
    wl = WL[name]
    levels = LEVELS[lv]
    rng = np.random.default_rng(wl.seed + 60)
    t = 45
    k = np.stack([_degenerate_rows(t, wl.head_dim, wl.group_size, rng) for _ in range(wl.num_kv_heads)], axis=1)
    v = np.stack([_degenerate_rows(t, wl.head_dim, wl.group_size, rng) for _ in range(wl.num_kv_heads)], axis=1)
    tau = np.full(wl.num_kv_heads, 1e30, np.float32)
    kc, ks, kz, vc, vs, vz = _bulk(gpu_lib, wl, k, v, _identity(wl.num_kv_heads, wl.head_dim), tau, tau, levels,
                                   seed=wl.seed + 61)
    for h in range(wl.num_kv_heads):
        check_write((kc[:, h], ks[:, h], kz[:, h]), k[:, h], None, tau[h], wl.group_size,
                    f"{name} {lv} K head {h} degenerate groups", levels=levels[0])
        check_write((vc[:, h], vs[:, h], vz[:, h]), v[:, h], None, tau[h], wl.group_size,
                    f"{name} {lv} V head {h} degenerate groups", levels=levels[1])


@pytest.mark.parametrize("name", ["d128-g128", "d64-g64"])
@pytest.mark.parametrize("rotated", [False, True])
def test_append_demote_codebook(gpu_lib, name, rotated):
    """20 decode-time appends on two sequences; the demoted tokens' codes
    against the oracle's codebook quantizer, then decode of the pool."""
    base = WL[name]
    levels = LEVELS["fit-like"]
    steps = 20
    l0 = (700, 330)
    wl = make_workload(base, batch=2, seq_lens=tuple(x + steps for x in l0), seed=base.seed + 100)
    inp = draw_inputs(wl)
    c = inp.calib
    r_k = c.r_k if rotated else _identity(wl.num_kv_heads, wl.head_dim)
    seqs = []
    for b in range(2):
        k, v = inp.k[b][: l0[b]].float().numpy(), inp.v[b][: l0[b]].float().numpy()
        seqs.append(oracle.SeqPool(wl.num_kv_heads, wl.head_dim, wl.group_size, wl.sink, wl.recent,
                                   levels_k=levels[0], levels_v=levels[1]).prefill(k, v, r_k, c.tau_k, c.tau_v))
    cap = [(max(0, x + steps - 320) + 15) // 16 + 1 for x in l0]
    extra = {b: list(range((l0[b] + steps + 15) // 16)) for b in range(2)}
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=5,
                                int2_capacity=cap, extra_bf16_pages=extra, garbage=False)
    dev = upload(pools)
    pool = gpu_lib.OscarPool(pool_config(wl, levels=levels))
    rk, tk, tv = to_dev(r_k), to_dev(c.tau_k), to_dev(c.tau_v)
    for st in range(steps):
        lens = torch.tensor([x + st for x in l0], dtype=torch.int32, device="cuda")
        kn = torch.stack([inp.k[b][l0[b] + st] for b in range(2)]).cuda()
        vn = torch.stack([inp.v[b][l0[b] + st] for b in range(2)]).cuda()
        gpu_lib.oscar_append_demote(pool, kn, vn, lens, dev["bf16_pt"], dev["int2_pt"], dev["bf16_pool"],
                                    dev["int2_pool"], rk, tk, tv)
        for b in range(2):
            seqs[b].append_demote(kn[b].float().cpu().numpy(), vn[b].float().cpu().numpy(), r_k, c.tau_k, c.tau_v)
    torch.cuda.synchronize()
    host2 = dev["int2_pool"].cpu().numpy()
    for b, s in enumerate(seqs):
        kc, ks, kz, vc, vs, vz = pool_io.read_history(host2, pools["int2_pt"][b], s.n_hist, wl.num_kv_heads,
                                                      wl.head_dim, wl.n_groups)
        new = np.arange(max(0, l0[b] - 320), s.n_hist)
        for h in range(wl.num_kv_heads):
            pos = wl.sink + new
            check_write((kc[new, h], ks[new, h], kz[new, h]), s.k[pos, h], r_k[h] if rotated else None, c.tau_k[h],
                        wl.group_size, f"{name} demoted K seq {b} head {h}", levels=levels[0])
            check_write((vc[new, h], vs[new, h], vz[new, h]), s.v[pos, h], None, c.tau_v[h], wl.group_size,
                        f"{name} demoted V seq {b} head {h}", levels=levels[1])
    lens = torch.tensor([s.L for s in seqs], dtype=torch.int32, device="cuda")
    out = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = pool.alloc_workspace(2, max(s.L for s in seqs))
    gpu_lib.oscar_decode_attention(pool, inp.q.cuda(), lens, max(s.L for s in seqs), dev["bf16_pt"], dev["int2_pt"],
                                   dev["bf16_pool"], dev["int2_pool"], rk, out, ws)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), r_k)
    check_decode(out, ref, what=f"{name} codebook decode after demotion")


DECODE = {
    "d128-gqa4-ragged": make_workload(QWEN, num_q_heads=8, num_kv_heads=2, batch=3, seq_lens=(1000, 5000, 333),
                                      seed=47),
    "d128-g64-gqa8": make_workload(QWEN, num_q_heads=16, num_kv_heads=2, group_size=64, batch=2,
                                   seq_lens=(4100, 700), seed=48),
    "d64-gqa2": make_workload(TINY, batch=2, seq_lens=(3000, 900), seed=49),
}


@pytest.mark.parametrize("lv", list(LEVELS))
@pytest.mark.parametrize("name", list(DECODE))
def test_decode_codebook_matches_oracle(gpu_lib, name, lv):
    wl = DECODE[name]
    levels = LEVELS[lv]
    inp = draw_inputs(wl)
    seqs = make_seqs(wl, inp, levels=levels)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=wl.seed)
    pool = gpu_lib.OscarPool(pool_config(wl, levels=levels))
    dev = upload(pools)
    lens = torch.tensor([s.L for s in seqs], dtype=torch.int32, device="cuda")
    max_len = max(s.L for s in seqs)
    out = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = pool.alloc_workspace(len(seqs), max_len)
    log(f"codebook decode {name} {lv}")
    gpu_lib.oscar_decode_attention(pool, inp.q.cuda(), lens, max_len, dev["bf16_pt"], dev["int2_pt"],
                                   dev["bf16_pool"], dev["int2_pool"], to_dev(inp.calib.r_k), out, ws)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k)
    check_decode(out, ref, what=f"{name} codebook {lv}")
    # the uniform decode of the same pages differs: the levels are used
    if lv == "lopsided":
        uni = torch.empty_like(out)
        upool = gpu_lib.OscarPool(pool_config(wl))
        uws = upool.alloc_workspace(len(seqs), max_len)
        gpu_lib.oscar_decode_attention(upool, inp.q.cuda(), lens, max_len, dev["bf16_pt"], dev["int2_pt"],
                                       dev["bf16_pool"], dev["int2_pool"], to_dev(inp.calib.r_k), uni, uws)
        torch.cuda.synchronize()
        assert not torch.equal(uni.view(torch.int16), out.view(torch.int16))


def test_decode_codebook_values_not_absorbed_and_cascade(gpu_lib):
    """V rotated at demotion with a codebook, and the prefix-shared decode of
    two sequences sharing 40 history pages, both against the oracle."""
    wl = make_workload(QWEN, num_q_heads=16, num_kv_heads=2, batch=3, seq_lens=(1500, 2000, 900), seed=51,
                       shared_prefix_tokens=64 + 16 * 40, shared_prefix_seqs=2)
    levels = LEVELS["fit-like"]
    inp = draw_inputs(wl)
    r_v = inp.calib.r_v
    seqs = make_seqs(wl, inp, r_v=r_v, levels=levels)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=wl.seed)
    pt = pools["int2_pt"].copy()
    pt[1, :40] = pt[0, :40]  # the shared pages exist once
    pools = dict(pools, int2_pt=pt)
    pool = gpu_lib.OscarPool(pool_config(wl, v_absorbed=False, levels=levels))
    dev = upload(pools)
    lens = torch.tensor([s.L for s in seqs], dtype=torch.int32, device="cuda")
    max_len = max(s.L for s in seqs)
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k, r_v)
    for groups in ([], [(0, 2, 40)]):
        out = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        nbytes = gpu_lib.cascade_workspace_bytes(pool, wl.batch, max_len, dev["int2_pt"].shape[1], groups)
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        gpu_lib.oscar_decode_attention_cascade(pool, inp.q.cuda(), lens, max_len, dev["bf16_pt"], dev["int2_pt"],
                                               dev["bf16_pool"], dev["int2_pool"], to_dev(inp.calib.r_k), out, ws,
                                               groups, r_v=to_dev(r_v))
        torch.cuda.synchronize()
        check_decode(out, ref, what=f"codebook, V not absorbed, groups {groups}")


def test_dequantize_codebook(gpu_lib):
    wl = WL["d128-g64"]
    levels = LEVELS["lopsided"]
    rng = np.random.default_rng(7)
    t, d = 77, wl.head_dim
    k = pool_io.bits_to_f32(pool_io.bf16_bits(rng.standard_normal((t, 2, d)) * 3))
    v = pool_io.bits_to_f32(pool_io.bf16_bits(rng.standard_normal((t, 2, d))))
    r_k = np.stack([np.linalg.qr(rng.standard_normal((d, d)))[0] for _ in range(2)]).astype(np.float32)
    tau = np.float32(6.0)
    npg = (t + 15) // 16
    blocks = []
    for h in range(2):
        kc, ks, kz = cb.quantize_tokens(k[:, h], r_k[h], tau, wl.group_size, levels[0])
        vc, vs, vz = cb.quantize_tokens(v[:, h], None, tau, wl.group_size, levels[1])
        pad = npg * 16 - t

        def pg(a):
            return np.concatenate([a, np.zeros((pad,) + a.shape[1:], a.dtype)]).reshape(npg, 16, -1)
        blocks.append(pool_io.pack_int2_blocks(pg(kc), pg(ks), pg(kz), pg(vc), pg(vs), pg(vz)))
    host = np.stack(blocks, axis=1).reshape(npg, -1)
    pool = gpu_lib.OscarPool(pool_config(wl, levels=levels))
    k_out = torch.empty(t, 2, d, dtype=torch.float32, device="cuda")
    v_out = torch.empty(t, 2, d, dtype=torch.float32, device="cuda")
    gpu_lib.oscar_dequantize(pool, t, to_dev(np.arange(npg, dtype=np.int32)), to_dev(host), to_dev(r_k), None,
                             k_out, v_out)
    torch.cuda.synchronize()
    for h in range(2):
        kc, ks, kz = cb.quantize_tokens(k[:, h], r_k[h], tau, wl.group_size, levels[0])
        ref = cb.dequantize(kc, ks, kz, wl.group_size, levels[0]) @ r_k[h].astype(np.float64).T
        err = np.abs(k_out.cpu().numpy()[:, h] - ref).max(axis=1) / np.linalg.norm(ref, axis=1)
        assert np.all(err <= 1e-5)
        vc, vs, vz = cb.quantize_tokens(v[:, h], None, tau, wl.group_size, levels[1])
        assert np.allclose(v_out.cpu().numpy()[:, h], cb.dequantize(vc, vs, vz, wl.group_size, levels[1]),
                           rtol=1e-6, atol=1e-6)


def _levels_agree(got, t_ref):
    ref = cb.lloyd_max(t_ref)
    raw = cb.lloyd_max_unrounded(t_ref)
    for k in (1, 2):
        if got[k] != ref[k]:
            assert abs(got[k] - ref[k]) == 1 / 32, (got, ref)
            frac = raw[k] * 32 - np.floor(raw[k] * 32)
            assert abs(frac - 0.5) < 32e-4, (got, ref, raw)
    assert got[0] == 0 and got[3] == 3


@pytest.mark.parametrize("hkv,g,d,gs,n", [(2, 2, 64, 64, 512), (8, 4, 128, 128, 2048), (2, 4, 128, 64, 700)])
def test_codebook_fit_matches_oracle(gpu_lib, hkv, g, d, gs, n):
    """oscar_calib_codebook on the calibration draw (keys with the oracle's
    R_K and tau_K, values with R_V and tau_V; the last case has G = 64)."""
    draws = draw_calibration(hkv, g, d, 60 + d + gs, n_cal=n)
    ref = cal.calibrate([(dr.q, dr.k, dr.v) for dr in draws])
    for x_name, r_name, t_name in (("k", "r_k", "tau_k"), ("v", "r_v", "tau_v")):
        x = np.stack([getattr(dr, x_name) for dr in draws])  # [Hkv, N, D]
        xd = to_dev(np.ascontiguousarray(x.transpose(1, 0, 2))).transpose(0, 1)  # token-major buffer
        log(f"codebook fit {x_name} hkv={hkv} d={d} G={gs} n={n}")
        lv = gpu_lib.oscar_calib_codebook(xd, to_dev(ref[r_name]), to_dev(ref[t_name]), gs)
        torch.cuda.synchronize()
        got = lv.cpu().numpy().astype(np.float64)
        t_ref = np.concatenate([cb.normalized_values(x[h], ref[r_name][h], ref[t_name][h], gs).ravel()
                                for h in range(hkv)])
        _levels_agree(got, t_ref)
        log(f"codebook {x_name}: {got.tolist()}")
    # no rotation: the normalized values are the oracle's exactly
    x = np.stack([dr.v for dr in draws])
    lv = gpu_lib.oscar_calib_codebook(to_dev(x), None, to_dev(ref["tau_v"]), gs)
    torch.cuda.synchronize()
    t_ref = np.concatenate([cb.normalized_values(x[h], None, ref["tau_v"][h], gs).ravel() for h in range(hkv)])
    assert np.array_equal(lv.cpu().numpy().astype(np.float64), cb.lloyd_max(t_ref))
