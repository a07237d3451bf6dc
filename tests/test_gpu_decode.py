"""GPU parity: oscar_decode_attention, oscar_bf16_decode_attention and
oscar_merge against the fp64 oracle, on oracle-built pools uploaded through
the documented layout (so decode is tested independently of the write path).
"""

import numpy as np
import pytest
import torch

import oracle
import pool_io
from harness import DECODE_TOL, check_decode, log, make_seqs, pool_config, to_dev, upload
from synthetic import CONFIGS, make_workload
from harness import draw_inputs

pytestmark = pytest.mark.gpu

TINY = CONFIGS["tiny-d64-l512"]
QWEN = CONFIGS["qwen3-8b-l100k"]

CASES = {
    "tiny-d64-gqa2-l512": make_workload(TINY),
    "d64-gqa2-boundary-lengths": make_workload(TINY, batch=10, seq_lens=(1, 63, 64, 65, 319, 320, 321, 336, 337, 1000),
                                               seed=5),
    "d64-gqa8-ragged": make_workload(TINY, num_q_heads=16, batch=2, seq_lens=(3000, 50), seed=6),
    "d128-gqa4-ragged": make_workload(QWEN, num_q_heads=8, num_kv_heads=2, batch=3, seq_lens=(1000, 5000, 333), seed=7),
    "d128-g64-gqa4": make_workload(QWEN, num_q_heads=8, num_kv_heads=2, group_size=64, batch=2, seq_lens=(3100, 520),
                                   seed=12),
    "d128-g64-gqa8": make_workload(QWEN, num_q_heads=16, num_kv_heads=2, group_size=64, batch=2, seq_lens=(4100, 700),
                                   seed=8),
    "d128-gqa2": make_workload(QWEN, num_q_heads=4, num_kv_heads=2, batch=1, seq_lens=(2500,), seed=9),
    "d128-gqa4-long": make_workload(QWEN, num_q_heads=16, num_kv_heads=4, batch=1, seq_lens=(20000,), seed=10),
}


def _decode(oscar, wl, seqs, q, pools, r_k, max_len=None, r_v=None, host_lens=None):
    pool = oscar.OscarPool(pool_config(wl, v_absorbed=r_v is None))
    dev = upload(pools)
    lens = torch.tensor([s.L for s in seqs], dtype=torch.int32, device="cuda")
    max_len = max_len or max(s.L for s in seqs)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = pool.alloc_workspace(len(seqs), max_len)
    log(f"decode launch: batch={len(seqs)} max_len={max_len} host lengths={host_lens is not None}")
    oscar.oscar_decode_attention(pool, q.cuda(), lens, max_len, dev["bf16_pt"], dev["int2_pt"], dev["bf16_pool"],
                                 dev["int2_pool"], to_dev(r_k), out, ws, r_v=None if r_v is None else to_dev(r_v),
                                 seq_lens_host=host_lens)
    torch.cuda.synchronize()
    return out, (pool, dev, lens, ws, max_len)


@pytest.mark.parametrize("plan", ["max-length", "host-lengths"])
@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_oracle(gpu_lib, name, plan):
    """Both split-K plans: every sequence planned for max_seq_len, and the
    length-aware plan from the host copy of the lengths."""
    wl = CASES[name]
    log(f"case {name} ({plan} plan): {wl}")
    inp = draw_inputs(wl)
    seqs = make_seqs(wl, inp)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=wl.seed)
    host = list(wl.seq_lens) if plan == "host-lengths" else None
    out, _ = _decode(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k, host_lens=host)
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k)
    check_decode(out, ref, what=f"{name} ({plan} plan)")


def test_decode_host_lengths_longer_than_device(gpu_lib):
    """Host lengths above the device ones plan more chunks than the device
    lengths fill: the extra workgroups exit, the ticket counts only real
    partials, and the result is the decode at the device lengths; repeated
    calls are bit-identical and leave the tickets at zero."""
    wl = CASES["d128-gqa4-ragged"]
    inp = draw_inputs(wl)
    seqs = make_seqs(wl, inp)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=wl.seed)
    host = [L + 700 for L in wl.seq_lens]
    out, (pool, dev, lens, ws, max_len) = _decode(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k,
                                                  max_len=max(host), host_lens=host)
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k)
    check_decode(out, ref, what="host lengths above device lengths")
    rk = to_dev(inp.calib.r_k)
    for _ in range(3):
        o = torch.zeros_like(out)
        gpu_lib.oscar_decode_attention(pool, inp.q.cuda(), lens, max_len, dev["bf16_pt"], dev["int2_pt"],
                                       dev["bf16_pool"], dev["int2_pool"], rk, o, ws, seq_lens_host=host)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), out.view(torch.int16))
    assert int(ws[: 128 * wl.batch * wl.num_kv_heads].view(torch.int32).abs().sum()) == 0


def test_decode_empty_sequences_give_zero_rows(gpu_lib):
    """Lengths of 0 (and negative ones, clamped to 0) select no token: those
    rows of the output are exactly zero, and the other sequences of the batch
    are unaffected."""
    wl = make_workload(QWEN, num_q_heads=8, num_kv_heads=2, batch=4, seq_lens=(700, 2000, 333, 1500), seed=12)
    inp = draw_inputs(wl)
    seqs = make_seqs(wl, inp)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=wl.seed)
    pool = gpu_lib.OscarPool(pool_config(wl))
    dev = upload(pools)
    lens = torch.tensor([0, 2000, -5, 1500], dtype=torch.int32, device="cuda")
    out = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = pool.alloc_workspace(wl.batch, 2000)
    log("decode launch: lengths (0, 2000, -5, 1500)")
    gpu_lib.oscar_decode_attention(pool, inp.q.cuda(), lens, 2000, dev["bf16_pt"], dev["int2_pt"], dev["bf16_pool"],
                                   dev["int2_pool"], to_dev(inp.calib.r_k), out, ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[0].float()) == 0 and torch.count_nonzero(out[2].float()) == 0
    ref, _ = oracle.decode_attention([seqs[1], seqs[3]], inp.q[[1, 3]].float().numpy(), inp.calib.r_k)
    check_decode(out[[1, 3]], ref, what="non-empty sequences of a batch with empty ones")


@pytest.mark.parametrize("name", ["d64-gqa2-boundary-lengths", "d128-gqa4-ragged", "d128-g64-gqa4", "d128-g64-gqa8"])
def test_decode_values_not_absorbed(gpu_lib, name):
    """v_absorbed = 0: the BF16 segments hold V, the history V R_V; decode
    rotates the merged history partial back by R_V^T."""
    wl = CASES[name]
    inp = draw_inputs(wl)
    r_v = inp.calib.r_v
    seqs = make_seqs(wl, inp, r_v=r_v)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=wl.seed)
    out, _ = _decode(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k, r_v=r_v)
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k, r_v)
    check_decode(out, ref, what=f"{name} (V not absorbed)")


def test_decode_deterministic_and_workspace_reusable(gpu_lib):
    wl = CASES["d128-gqa4-ragged"]
    inp = draw_inputs(wl)
    seqs = make_seqs(wl, inp)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=1)
    out1, (pool, dev, lens, ws, max_len) = _decode(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k)
    rk = to_dev(inp.calib.r_k)
    outs = []
    for _ in range(3):
        o = torch.zeros_like(out1)
        gpu_lib.oscar_decode_attention(pool, inp.q.cuda(), lens, max_len, dev["bf16_pt"], dev["int2_pt"],
                                       dev["bf16_pool"], dev["int2_pool"], rk, o, ws)
        outs.append(o)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), out1.view(torch.int16))
    # the per-head tickets (one 128-byte line each, at the start of the
    # workspace) are left at zero after every call
    assert int(ws[: 128 * wl.batch * wl.num_kv_heads].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("bf16_pages_per_unit", [None, "8"])
@pytest.mark.parametrize("name", ["d64-gqa8-ragged", "d128-gqa4-ragged", "d128-gqa4-long"])
def test_decode_multi_round_plan(gpu_lib, name, bf16_pages_per_unit, monkeypatch):
    """A plan of 340-620 workgroups (the planner aimed at 1,024), i.e. more
    than the GPU's CUs: the workgroup order that runs each XCD's INT2 chunks
    before its BF16 units, with one or three BF16 units per (sequence, KV
    head) and, in the ragged cases, chunks past a sequence's own history that
    exit at once.  Nine calls are bitwise equal."""
    monkeypatch.setenv("OSCAR_TARGET_WGS", "1024")
    if bf16_pages_per_unit:
        monkeypatch.setenv("OSCAR_BF16_PAGES_PER_UNIT", bf16_pages_per_unit)
    wl = CASES[name]
    log(f"case {name}: multi-round plan, BF16 pages per unit {bf16_pages_per_unit or 'default'}")
    inp = draw_inputs(wl)
    seqs = make_seqs(wl, inp)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=wl.seed)
    out, (pool, dev, lens, ws, max_len) = _decode(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k)
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k)
    check_decode(out, ref, what=f"{name} (multi-round plan)")
    # several calls: with GQA <= 4 the q' prologue's waves meet at an LDS
    # counter rather than a workgroup barrier, and a shared-memory write
    # left outside that ordering shows as an occasional differing call
    rk, qd = to_dev(inp.calib.r_k), inp.q.cuda()
    for i in range(8):
        again = torch.zeros_like(out)
        gpu_lib.oscar_decode_attention(pool, qd, lens, max_len, dev["bf16_pt"], dev["int2_pt"],
                                       dev["bf16_pool"], dev["int2_pool"], rk, again, ws)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), out.view(torch.int16)), f"call {i + 2} differs"


LONG_CHUNK_CASES = {
    "d128-gqa4-long": CASES["d128-gqa4-long"],
    "d128-gqa8-long": make_workload(QWEN, num_q_heads=16, num_kv_heads=2, batch=2, seq_lens=(20000, 9000), seed=13),
    "d128-gqa2-long": make_workload(QWEN, num_q_heads=4, num_kv_heads=2, batch=1, seq_lens=(18000,), seed=14),
}


@pytest.mark.parametrize("plan", ["max-length", "host-lengths"])
@pytest.mark.parametrize("name", list(LONG_CHUNK_CASES))
def test_decode_long_chunks(gpu_lib, name, plan, monkeypatch):
    """Chunks of up to 1,024 history pages (the planner aimed at 4
    workgroups): each wave takes the ids of its tiles past the first 64 pages
    from a second batch.  Sequences of 9,000-20,000 tokens give one full
    chunk and a shorter last one; repeated calls are bitwise equal."""
    monkeypatch.setenv("OSCAR_TARGET_WGS", "4")
    wl = LONG_CHUNK_CASES[name]
    log(f"case {name} ({plan} plan): chunks of up to 1,024 pages")
    inp = draw_inputs(wl)
    seqs = make_seqs(wl, inp)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=wl.seed)
    host = list(wl.seq_lens) if plan == "host-lengths" else None
    out, (pool, dev, lens, ws, max_len) = _decode(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k, host_lens=host)
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k)
    check_decode(out, ref, what=f"{name} ({plan} plan, long chunks)")
    again = torch.zeros_like(out)
    gpu_lib.oscar_decode_attention(pool, inp.q.cuda(), lens, max_len, dev["bf16_pt"], dev["int2_pt"],
                                   dev["bf16_pool"], dev["int2_pool"], to_dev(inp.calib.r_k), again, ws,
                                   seq_lens_host=host)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), out.view(torch.int16))


def test_decode_full_size_headline_sampled(gpu_lib):
    """Qwen3-8B-shaped layer at 100,000 tokens, in the launch configuration
    bench.py times; the oracle computes a sample of query heads."""
    wl = QWEN
    inp = draw_inputs(wl)
    log("oracle quantization of 99,680 x 8 history tokens")
    seqs = make_seqs(wl, inp)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=wl.seed)
    out, (pool, dev, lens, ws, max_len) = _decode(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k,
                                                  host_lens=list(wl.seq_lens))
    pairs = [(0, 0), (0, 5), (0, 13), (0, 22), (0, 31)]
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k, pairs=pairs)
    check_decode(out, ref, pairs=pairs, what="qwen3-8b-l100k sampled")
    # the same launch ten times more: bitwise equal outputs (the fold order
    # of the split-K partials does not depend on which workgroup ends last),
    # and the per-head tickets back at zero after each call
    rk = to_dev(inp.calib.r_k)
    qd = inp.q.cuda()
    n_tickets = 128 * wl.batch * wl.num_kv_heads // 4
    for i in range(10):
        o = torch.zeros_like(out)
        gpu_lib.oscar_decode_attention(pool, qd, lens, max_len, dev["bf16_pt"], dev["int2_pt"], dev["bf16_pool"],
                                       dev["int2_pool"], rk, o, ws, seq_lens_host=list(wl.seq_lens))
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), out.view(torch.int16)), f"call {i + 1} differs"
        assert int(ws[: 4 * n_tickets].view(torch.int32).abs().sum()) == 0, f"tickets not reset after call {i + 1}"


@pytest.mark.parametrize("name", ["tiny-d64-gqa2-l512", "d128-gqa4-ragged", "d128-g64-gqa8"])
def test_bf16_only_decode_matches_oracle(gpu_lib, name):
    wl = CASES[name]
    inp = draw_inputs(wl)
    seqs = make_seqs(wl, inp)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=3,
                                bf16_for_all=True)
    pool = gpu_lib.OscarPool(pool_config(wl))
    dev = upload(pools)
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    out = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = pool.alloc_workspace(wl.batch, max(wl.seq_lens), bf16_only=True)
    gpu_lib.oscar_bf16_decode_attention(pool, inp.q.cuda(), lens, max(wl.seq_lens), dev["bf16_pt"], dev["bf16_pool"],
                                        out, ws)
    torch.cuda.synchronize()
    ks = [s.k for s in seqs]
    vs = [s.v for s in seqs]
    ref, _ = oracle.bf16_decode_attention(ks, vs, inp.q.float().numpy(), list(wl.seq_lens))
    check_decode(out, ref, what=f"bf16-only {name}")


@pytest.mark.parametrize("d", [64, 128])
def test_merge_matches_oracle(gpu_lib, d):
    rng = np.random.default_rng(d)
    rows = 37
    counts = rng.integers(0, 9, rows)
    counts[3] = 0
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    nnz = int(offs[-1])
    o = rng.standard_normal((nnz, d)).astype(np.float32)
    lse = (rng.standard_normal(nnz) * 20).astype(np.float32)
    lse[rng.random(nnz) < 0.15] = -np.inf
    a, bnd = int(offs[5]), int(offs[6])
    lse[a:bnd] = -np.inf  # a row whose partials are all empty
    out = torch.full((rows, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    gpu_lib.oscar_merge(to_dev(offs), to_dev(o), to_dev(lse), out)
    torch.cuda.synchronize()
    ref = np.stack([oracle.merge_partials(o[offs[i]:offs[i + 1]], lse[offs[i]:offs[i + 1]])[0] for i in range(rows)])
    got = out.float().cpu().numpy()
    for i in range(rows):
        nrm = np.linalg.norm(ref[i])
        assert np.max(np.abs(got[i] - ref[i])) <= DECODE_TOL * max(nrm, 1e-30) + (0 if nrm > 0 else 0), i
    assert np.all(got[3] == 0) and np.all(got[5] == 0)


def _value_scaled(inp, factor):
    """The draw with every value multiplied by factor(t) (a scalar or an
    array over token positions), rounded to bf16 like the cache content."""
    vs = []
    for v in inp.v:
        f = torch.as_tensor(factor(v.shape[0]) if callable(factor) else factor, dtype=torch.float32)
        f = f.reshape(-1, 1, 1) if f.ndim == 1 else f
        vs.append((v.float() * f).to(torch.bfloat16))
    inp.v = vs
    return inp


@pytest.mark.parametrize("gqa", [4, 8])
@pytest.mark.parametrize("vscale", [1e-8, 1e-3, 300.0, 1e12])
def test_decode_value_range_unclipped(gpu_lib, gqa, vscale):
    """Values far from N(0, 1) with no value clip (tau_V = +inf): the value
    scales s_V run from ~1e-8 to ~1e12, so the fp16 P.V weights p * s_V
    would leave fp16's range without the scale exponent the kernel keeps
    beside its running max.  Tolerance as everywhere (2e-3 of each head's
    norm)."""
    wl = make_workload(QWEN, num_q_heads=2 * gqa, num_kv_heads=2, batch=2, seq_lens=(3000, 777), seed=20 + gqa)
    log(f"value range case gqa={gqa} scale={vscale}")
    inp = _value_scaled(draw_inputs(wl), vscale)
    tau_v = np.full(wl.num_kv_heads, np.inf, np.float32)
    seqs = make_seqs(wl, inp, tau_v=tau_v)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=wl.seed)
    out, _ = _decode(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k)
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k)
    check_decode(out, ref, what=f"gqa {gqa}, values x{vscale:g}, no value clip")


@pytest.mark.parametrize("gqa", [4, 8])
def test_decode_value_scale_ramp(gpu_lib, gqa):
    """Value magnitudes growing 2^(t/400) along the sequence (64x over the
    history), so the scale exponent is raised several times inside a wave's
    tiles and the accumulated state is rescaled each time."""
    wl = make_workload(QWEN, num_q_heads=2 * gqa, num_kv_heads=2, batch=1, seq_lens=(2700,), seed=30 + gqa)
    inp = _value_scaled(draw_inputs(wl), lambda n: 2.0 ** (np.arange(n) / 400.0))
    tau_v = np.full(wl.num_kv_heads, np.inf, np.float32)
    seqs = make_seqs(wl, inp, tau_v=tau_v)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=wl.seed)
    out, _ = _decode(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k)
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k)
    check_decode(out, ref, what=f"gqa {gqa}, value scale ramp")


@pytest.mark.parametrize("gqa", [4, 8])
def test_decode_dominant_query_channel(gpu_lib, gqa):
    """R_K = I and one query channel 50x the others: q' = q, so the int8
    split of q' is scaled by that one channel and the other channels keep
    fewer significant bits.  Keys are unrotated and unclipped."""
    wl = make_workload(QWEN, num_q_heads=2 * gqa, num_kv_heads=2, batch=2, seq_lens=(4000, 900), seed=40 + gqa)
    inp = draw_inputs(wl)
    q = inp.q.float()
    q[:, :, 17] *= 50.0
    inp.q = q.to(torch.bfloat16)
    eye = np.broadcast_to(np.eye(wl.head_dim, dtype=np.float32), (wl.num_kv_heads, wl.head_dim, wl.head_dim)).copy()
    tau_k = np.full(wl.num_kv_heads, np.inf, np.float32)
    seqs = make_seqs(wl, inp, r_k=eye, tau_k=tau_k)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=wl.seed)
    out, _ = _decode(gpu_lib, wl, seqs, inp.q, pools, eye)
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), eye)
    check_decode(out, ref, what=f"gqa {gqa}, one query channel x50, R_K = I")
