"""GPU parity of the write path: oscar_quantize_pack (bulk) and
oscar_append_demote (decode-time), read back through the documented layout
and compared with the oracle quantizer; then end-to-end decode on the
GPU-written pool against oracle write + oracle decode."""

import numpy as np
import pytest
import torch

import oracle
import pool_io
from harness import check_decode, check_write, log, make_seqs, pool_config, to_dev, upload
from synthetic import CONFIGS, make_workload
from harness import draw_inputs

pytestmark = pytest.mark.gpu

TINY = CONFIGS["tiny-d64-l512"]
QWEN = CONFIGS["qwen3-8b-l100k"]

WL = {
    "d128-g128": make_workload(QWEN, num_q_heads=8, num_kv_heads=2, batch=1, seq_lens=(1000,), seed=21),
    "d128-g64": make_workload(QWEN, num_q_heads=8, num_kv_heads=2, group_size=64, batch=1, seq_lens=(1000,), seed=22),
    "d64-g64": make_workload(TINY, batch=1, seq_lens=(1000,), seed=23),
}


def _identity(hkv, d):
    return np.stack([np.eye(d, dtype=np.float32)] * hkv)


def _bulk(oscar, wl, k, v, r_k, tau_k, tau_v, seed=0, r_v=None):
    """Quantize dense k, v [T, Hkv, D] into fresh random pages; returns the
    logical history read back per head.  With r_v, V is rotated too."""
    t = k.shape[0]
    npg = (t + 15) // 16
    pool = oscar.OscarPool(pool_config(wl, v_absorbed=r_v is None))
    rng = np.random.default_rng(seed)
    n_phys = npg + 3
    ids = rng.permutation(n_phys)[:npg].astype(np.int32)
    int2 = torch.randint(0, 256, (n_phys, pool.int2_page_bytes), dtype=torch.uint8, device="cuda")
    log(f"quantize_pack launch: T={t} pages={npg}")
    oscar.oscar_quantize_pack(pool, to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16), to_dev(ids), int2,
                              to_dev(r_k), to_dev(tau_k), to_dev(tau_v), r_v=None if r_v is None else to_dev(r_v))
    torch.cuda.synchronize()
    host = int2.cpu().numpy()
    hist = pool_io.read_history(host, ids, t, wl.num_kv_heads, wl.head_dim, wl.n_groups)
    # slots past the last token are zero-filled
    if t % 16:
        last = host[ids[-1]].reshape(wl.num_kv_heads, -1)
        kc, ks, kz, vc, vs, vz = pool_io.unpack_int2_blocks(last, wl.head_dim, wl.n_groups)
        for a in (kc, ks, kz, vc, vs, vz):
            assert np.all(a[:, t % 16:] == 0)
    return hist


@pytest.mark.parametrize("name", list(WL))
@pytest.mark.parametrize("rotated", [False, True])
def test_quantize_pack_matches_oracle(gpu_lib, name, rotated):
    wl = WL[name]
    inp = draw_inputs(wl, with_q=False)
    k, v = inp.k[0][:1000].float().numpy(), inp.v[0][:1000].float().numpy()
    c = inp.calib
    r_k = c.r_k if rotated else _identity(wl.num_kv_heads, wl.head_dim)
    kc, ks, kz, vc, vs, vz = _bulk(gpu_lib, wl, k, v, r_k, c.tau_k, c.tau_v, seed=wl.seed)
    for h in range(wl.num_kv_heads):
        check_write((kc[:, h], ks[:, h], kz[:, h]), k[:, h], r_k[h] if rotated else None, c.tau_k[h],
                    wl.group_size, f"{name} K head {h} rotated={rotated}")
        check_write((vc[:, h], vs[:, h], vz[:, h]), v[:, h], None, c.tau_v[h], wl.group_size,
                    f"{name} V head {h}")


@pytest.mark.parametrize("ppb", [8, 20, 64])
@pytest.mark.parametrize("name", ["d128-g64", "d64-g64"])
def test_quantize_pack_page_split(gpu_lib, monkeypatch, name, ppb):
    """Workgroups covering 8, 20 and 64 pages of a 63-page input: waves take
    one to eight pages each and the last workgroup's range is ragged."""
    monkeypatch.setenv("OSCAR_QP_PAGES_PER_BLOCK", str(ppb))
    wl = WL[name]
    inp = draw_inputs(wl, with_q=False)
    k, v = inp.k[0][:1000].float().numpy(), inp.v[0][:1000].float().numpy()
    c = inp.calib
    kc, ks, kz, vc, vs, vz = _bulk(gpu_lib, wl, k, v, c.r_k, c.tau_k, c.tau_v, seed=ppb)
    for h in range(wl.num_kv_heads):
        check_write((kc[:, h], ks[:, h], kz[:, h]), k[:, h], c.r_k[h], c.tau_k[h], wl.group_size,
                    f"{name} K head {h} pages/block={ppb}")
        check_write((vc[:, h], vs[:, h], vz[:, h]), v[:, h], None, c.tau_v[h], wl.group_size,
                    f"{name} V head {h} pages/block={ppb}")


@pytest.mark.parametrize("identity", [True, False])
@pytest.mark.parametrize("name", list(WL))
def test_quantize_pack_values_rotated(gpu_lib, name, identity):
    """v_absorbed = 0: V is rotated by R_V on the matrix cores like K.  With
    R_V = I the V codes are bit-exact; with the calibrated R_V the flip rule
    applies."""
    wl = WL[name]
    inp = draw_inputs(wl, with_q=False)
    k, v = inp.k[0][:1000].float().numpy(), inp.v[0][:1000].float().numpy()
    c = inp.calib
    r_v = _identity(wl.num_kv_heads, wl.head_dim) if identity else c.r_v
    kc, ks, kz, vc, vs, vz = _bulk(gpu_lib, wl, k, v, c.r_k, c.tau_k, c.tau_v, seed=wl.seed + 7, r_v=r_v)
    for h in range(wl.num_kv_heads):
        check_write((kc[:, h], ks[:, h], kz[:, h]), k[:, h], c.r_k[h], c.tau_k[h], wl.group_size,
                    f"{name} K head {h} (V rotated too)")
        check_write((vc[:, h], vs[:, h], vz[:, h]), v[:, h], None if identity else r_v[h], c.tau_v[h],
                    wl.group_size, f"{name} V head {h} rotated (R_V = I: {identity})")


def test_quantize_pack_full_size_sampled(gpu_lib):
    """Bulk prefill of 131,072 tokens x 8 KV heads x 128 (the bulk workload);
    every page is read back and a sample of pages checked against the oracle."""
    wl = CONFIGS["bulk-quant-t131k"]
    inp = draw_inputs(wl, with_q=False)
    k, v = inp.k[0].float().numpy(), inp.v[0].float().numpy()
    c = inp.calib
    kc, ks, kz, vc, vs, vz = _bulk(gpu_lib, wl, k, v, c.r_k, c.tau_k, c.tau_v, seed=3)
    rng = np.random.default_rng(0)
    pages = np.sort(rng.choice(k.shape[0] // 16, 64, replace=False))
    tok = (pages[:, None] * 16 + np.arange(16)).reshape(-1)
    for h in range(wl.num_kv_heads):
        check_write((kc[tok, h], ks[tok, h], kz[tok, h]), k[tok, h], c.r_k[h], c.tau_k[h], wl.group_size,
                    f"bulk K head {h} (64 sampled pages)")
        check_write((vc[tok, h], vs[tok, h], vz[tok, h]), v[tok, h], None, c.tau_v[h], wl.group_size,
                    f"bulk V head {h} (64 sampled pages)")


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).bfloat16().float().numpy()


def _degenerate_rows(n, d, gs, rng):
    """Token rows whose groups hit every special case of the quantizer's
    scale/zero rule (W4-W6): constant groups (d = 0, so s = 1, including a
    zero point far from the code range), spreads so small that the scale is
    below 2^-70, values beyond 2^56, zero points beyond 128 in magnitude, and
    a group with one outlier; the rest are plain Gaussian groups."""
    patterns = [
        lambda: np.zeros(gs),
        lambda: np.full(gs, 1.5),
        lambda: np.full(gs, -200.0),
        lambda: rng.uniform(1e-30, 3e-30, gs) * rng.choice([-1.0, 1.0]),
        lambda: rng.uniform(-1e20, 1e20, gs),
        lambda: 1000.0 + 8.0 * rng.integers(0, 3, gs),
        lambda: np.r_[np.full(gs - 1, 7.0), 7.0 + 1.0 / 32],
        lambda: rng.standard_normal(gs),
    ]
    x = np.empty((n, d), np.float32)
    for i in range(n):
        for g in range(d // gs):
            x[i, g * gs:(g + 1) * gs] = patterns[(i + 3 * g) % len(patterns)]()
    return _bf16(x)


@pytest.mark.parametrize("name", list(WL))
def test_quantize_pack_degenerate_groups(gpu_lib, name):
    """Pre-rotated input (R_K = I, V absorbed) whose groups take the bulk
    kernel off its reciprocal fast path: codes, scales and zeros must still
    be bit-exact against the oracle.  Clipping is disabled (tau = 1e30)."""
    wl = WL[name]
    rng = np.random.default_rng(wl.seed + 50)
    t = 45  # two full pages and a ragged third
    k = np.stack([_degenerate_rows(t, wl.head_dim, wl.group_size, rng) for _ in range(wl.num_kv_heads)], axis=1)
    v = np.stack([_degenerate_rows(t, wl.head_dim, wl.group_size, rng) for _ in range(wl.num_kv_heads)], axis=1)
    tau = np.full(wl.num_kv_heads, 1e30, np.float32)
    r_k = _identity(wl.num_kv_heads, wl.head_dim)
    kc, ks, kz, vc, vs, vz = _bulk(gpu_lib, wl, k, v, r_k, tau, tau, seed=wl.seed + 51)
    for h in range(wl.num_kv_heads):
        check_write((kc[:, h], ks[:, h], kz[:, h]), k[:, h], None, tau[h], wl.group_size,
                    f"{name} K head {h} degenerate groups")
        check_write((vc[:, h], vs[:, h], vz[:, h]), v[:, h], None, tau[h], wl.group_size,
                    f"{name} V head {h} degenerate groups")


@pytest.mark.parametrize("rotated", [False, True, "values too"])
@pytest.mark.parametrize("name", ["d128-g128", "d64-g64", "d128-g64"])
def test_append_demote_steps_then_decode(gpu_lib, name, rotated):
    """Three sequences (one still too short to demote) take 40 decode-time
    appends; the GPU pool must hold the oracle's history and BF16 tokens, and
    GPU decode over it must match oracle decode."""
    base = WL[name]
    steps = 40
    l0 = (700, 330, 150)
    wl = make_workload(base, batch=3, seq_lens=tuple(x + steps for x in l0), seed=base.seed + 100)
    inp = draw_inputs(wl)
    c = inp.calib
    r_k = c.r_k if rotated else _identity(wl.num_kv_heads, wl.head_dim)
    r_v = c.r_v if rotated == "values too" else None  # V not absorbed: rotated at demotion
    seqs = []
    for b in range(3):
        k, v = inp.k[b][: l0[b]].float().numpy(), inp.v[b][: l0[b]].float().numpy()
        seqs.append(oracle.SeqPool(wl.num_kv_heads, wl.head_dim, wl.group_size, wl.sink, wl.recent,
                                   v_absorbed=r_v is None).prefill(k, v, r_k, c.tau_k, c.tau_v, r_v))
    cap = [(max(0, x + steps - 320) + 15) // 16 + 1 for x in l0]
    extra = {b: list(range((l0[b] + steps + 15) // 16)) for b in range(3)}
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=5,
                                int2_capacity=cap, extra_bf16_pages=extra, garbage=False)
    dev = upload(pools)
    pool = gpu_lib.OscarPool(pool_config(wl, v_absorbed=r_v is None))
    rk, tk, tv = to_dev(r_k), to_dev(c.tau_k), to_dev(c.tau_v)
    rv = None if r_v is None else to_dev(r_v)
    for st in range(steps):
        lens = torch.tensor([x + st for x in l0], dtype=torch.int32, device="cuda")
        kn = torch.stack([inp.k[b][l0[b] + st] for b in range(3)]).cuda()
        vn = torch.stack([inp.v[b][l0[b] + st] for b in range(3)]).cuda()
        gpu_lib.oscar_append_demote(pool, kn, vn, lens, dev["bf16_pt"], dev["int2_pt"], dev["bf16_pool"],
                                    dev["int2_pool"], rk, tk, tv, r_v=rv)
        for b in range(3):
            seqs[b].append_demote(kn[b].float().cpu().numpy(), vn[b].float().cpu().numpy(), r_k, c.tau_k, c.tau_v,
                                  r_v)
    torch.cuda.synchronize()
    host2 = dev["int2_pool"].cpu().numpy()
    host16 = dev["bf16_pool"].cpu().numpy()
    pt2 = pools["int2_pt"]
    for b, s in enumerate(seqs):
        if s.n_hist:
            kc, ks, kz, vc, vs, vz = pool_io.read_history(host2, pt2[b], s.n_hist, wl.num_kv_heads, wl.head_dim,
                                                          wl.n_groups)
            new = np.arange(max(0, l0[b] - 320), s.n_hist)  # tokens demoted by the GPU
            for h in range(wl.num_kv_heads):
                hist_pos = wl.sink + new
                check_write((kc[new, h], ks[new, h], kz[new, h]), s.k[hist_pos, h], r_k[h] if rotated else None,
                            c.tau_k[h], wl.group_size, f"{name} demoted K seq {b} head {h}")
                check_write((vc[new, h], vs[new, h], vz[new, h]), s.v[hist_pos, h],
                            None if r_v is None else r_v[h], c.tau_v[h], wl.group_size,
                            f"{name} demoted V seq {b} head {h}")
        # appended tokens landed in the BF16 pool
        for pos in range(l0[b], l0[b] + steps):
            blk = host16[pools["bf16_pt"][b, pos // 16]].reshape(wl.num_kv_heads, -1)
            kk, vv = pool_io.unpack_bf16_blocks(blk, wl.head_dim)
            assert np.array_equal(kk[:, pos % 16], s.k[pos]) and np.array_equal(vv[:, pos % 16], s.v[pos])
    # end to end: decode the GPU-written pool
    lens = torch.tensor([s.L for s in seqs], dtype=torch.int32, device="cuda")
    out = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = pool.alloc_workspace(3, max(s.L for s in seqs))
    gpu_lib.oscar_decode_attention(pool, inp.q.cuda(), lens, max(s.L for s in seqs), dev["bf16_pt"], dev["int2_pt"],
                                   dev["bf16_pool"], dev["int2_pool"], rk, out, ws, r_v=rv)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), r_k, r_v)
    check_decode(out, ref, what=f"{name} decode after demotion rotated={rotated}")


@pytest.mark.parametrize("name", list(WL))
def test_append_demote_degenerate_groups(gpu_lib, name):
    """Decode-time demotion of tokens whose groups take every special case of
    the scale/zero rule (see _degenerate_rows): with R_K = I, V absorbed and
    no clipping, the codes, scales and zeros the GPU writes for the demoted
    tokens are bit-exact against the oracle."""
    wl = make_workload(WL[name], batch=1, seq_lens=(370,), seed=WL[name].seed + 200)
    rng = np.random.default_rng(wl.seed)
    steps, l0 = 40, 330  # the appends demote positions 74 .. 113
    n = l0 + steps
    k = np.stack([_degenerate_rows(n, wl.head_dim, wl.group_size, rng) for _ in range(wl.num_kv_heads)], axis=1)
    v = np.stack([_degenerate_rows(n, wl.head_dim, wl.group_size, rng) for _ in range(wl.num_kv_heads)], axis=1)
    tau = np.full(wl.num_kv_heads, 1e30, np.float32)
    r_k = _identity(wl.num_kv_heads, wl.head_dim)
    seq = oracle.SeqPool(wl.num_kv_heads, wl.head_dim, wl.group_size, wl.sink, wl.recent).prefill(
        k[:l0], v[:l0], r_k, tau, tau)
    cap = [(n - 320 + 15) // 16 + 1]
    pools = pool_io.build_pools([seq], wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=6,
                                int2_capacity=cap, extra_bf16_pages={0: list(range((n + 15) // 16))}, garbage=False)
    dev = upload(pools)
    pool = gpu_lib.OscarPool(pool_config(wl))
    rk, tk = to_dev(r_k), to_dev(tau)
    for st in range(steps):
        lens = torch.tensor([l0 + st], dtype=torch.int32, device="cuda")
        kn = to_dev(k[l0 + st][None], torch.bfloat16)
        vn = to_dev(v[l0 + st][None], torch.bfloat16)
        gpu_lib.oscar_append_demote(pool, kn, vn, lens, dev["bf16_pt"], dev["int2_pt"], dev["bf16_pool"],
                                    dev["int2_pool"], rk, tk, tk)
        seq.append_demote(k[l0 + st], v[l0 + st], r_k, tau, tau)
    torch.cuda.synchronize()
    kc, ks, kz, vc, vs, vz = pool_io.read_history(dev["int2_pool"].cpu().numpy(), pools["int2_pt"][0], seq.n_hist,
                                                  wl.num_kv_heads, wl.head_dim, wl.n_groups)
    new = np.arange(l0 - 320, seq.n_hist)  # history slots written by the GPU
    assert len(new) == steps
    for h in range(wl.num_kv_heads):
        pos = wl.sink + new
        check_write((kc[new, h], ks[new, h], kz[new, h]), k[pos, h], None, tau[h], wl.group_size,
                    f"{name} demoted degenerate K head {h}")
        check_write((vc[new, h], vs[new, h], vz[new, h]), v[pos, h], None, tau[h], wl.group_size,
                    f"{name} demoted degenerate V head {h}")
