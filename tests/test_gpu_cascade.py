"""GPU parity of the prefix-shared ("cascade") decode,
oscar_decode_attention_cascade, against the fp64 oracle.

The pools are built by the oracle's quantizer (as in test_gpu_decode.py);
sequences of a prefix group draw identical tokens for the shared prefix, and
their INT2 page tables are then pointed at the longest member's physical pages
for the shared history pages, so the shared pages exist once.  The expected
result is plain decode attention per sequence (the oracle decodes each
sequence on its own), within the decode tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
import pool_io
from harness import check_decode, draw_inputs, log, make_seqs, pool_config, to_dev, upload
from synthetic import CONFIGS, make_workload

pytestmark = pytest.mark.gpu

TINY = CONFIGS["tiny-d64-l512"]
QWEN = CONFIGS["qwen3-8b-l100k"]


def _shared_tokens(pages, sink=64):
    return sink + 16 * pages


# name -> (workload, groups as (first_seq, num_seqs, shared_pages))
CASES = {
    # GQA 8: two sequences per prefix unit; member 2's history (580 tokens)
    # is shorter than the 640-token shared range
    "d128-gqa8": (make_workload(QWEN, num_q_heads=16, num_kv_heads=2, batch=6,
                                seq_lens=(1500, 1200, 900, 2000, 1000, 333), seed=31,
                                shared_prefix_tokens=_shared_tokens(40), shared_prefix_seqs=4),
                  [(0, 4, 40)]),
    # GQA 4: four sequences per unit; the group starts at sequence 1
    "d128-gqa4": (make_workload(QWEN, num_q_heads=8, num_kv_heads=2, batch=5,
                                seq_lens=(700, 3000, 2500, 1400, 2600), seed=32), [(1, 3, 50)]),
    # G = 64 at D = 128 (two scale groups), GQA 8, ragged shared range
    "d128-g64-gqa8": (make_workload(QWEN, num_q_heads=16, num_kv_heads=2, group_size=64, batch=3,
                                    seq_lens=(2300, 4100, 3000), seed=33), [(0, 3, 75)]),
    # D = 64, GQA 2: eight sequences per unit, a group of 5 plus a group of 2
    "d64-gqa2": (make_workload(TINY, batch=8, seq_lens=(900, 1300, 1100, 700, 1600, 800, 2000, 1900), seed=34),
                 [(0, 5, 20), (6, 2, 60)]),
}


def _prefix_inputs(wl, groups):
    """Inputs whose groups share their first tokens: the tokens of the first
    member are copied into the other members for the shared range."""
    inp = draw_inputs(wl)
    for first, n, pages in groups:
        t = _shared_tokens(pages)
        for m in range(first + 1, first + n):
            t_m = min(t, wl.seq_lens[m])
            inp.k[m][:t_m] = inp.k[first][:t_m]
            inp.v[m][:t_m] = inp.v[first][:t_m]
    return inp


def _share_tables(pools, seqs, groups):
    """Point every member's table entries of the shared pages (as far as its
    own history reaches) at the physical pages of the group's longest member
    (the data there is identical)."""
    pt = pools["int2_pt"].copy()
    for first, n, pages in groups:
        members = range(first, first + n)
        src = max(members, key=lambda m: seqs[m].n_hist)
        for m in members:
            k = min(pages, (seqs[m].n_hist + 15) // 16)
            pt[m, :k] = pt[src, :k]
    return dict(pools, int2_pt=pt)


def _run(oscar, wl, seqs, q, pools, r_k, groups, r_v=None, host_lens=None):
    pool = oscar.OscarPool(pool_config(wl, v_absorbed=r_v is None))
    dev = upload(pools)
    lens = torch.tensor([s.L for s in seqs], dtype=torch.int32, device="cuda")
    max_len = max(s.L for s in seqs)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    nbytes = oscar.cascade_workspace_bytes(pool, len(seqs), max_len, dev["int2_pt"].shape[1], groups)
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    log(f"cascade decode: batch={len(seqs)} groups={groups}")
    rv = None if r_v is None else to_dev(r_v)
    oscar.oscar_decode_attention_cascade(pool, q.cuda(), lens, max_len, dev["bf16_pt"], dev["int2_pt"],
                                         dev["bf16_pool"], dev["int2_pool"], to_dev(r_k), out, ws, groups, r_v=rv,
                                         seq_lens_host=host_lens)
    torch.cuda.synchronize()
    return out, (pool, dev, lens, ws, max_len)


@pytest.mark.parametrize("name", list(CASES))
def test_cascade_matches_oracle(gpu_lib, name):
    wl, groups = CASES[name]
    inp = _prefix_inputs(wl, groups)
    seqs = make_seqs(wl, inp)
    pools = _share_tables(pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent,
                                              seed=wl.seed), seqs, groups)
    out, (pool, dev, lens, ws, max_len) = _run(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k, groups)
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k)
    check_decode(out, ref, what=f"{name} cascade")
    # the same pools through the plain decode agree as well, and the
    # workspace's tickets are back at zero after the cascade call
    assert int(ws[: 128 * wl.batch * wl.num_kv_heads].view(torch.int32).abs().sum()) == 0
    plain = torch.empty_like(out)
    pws = pool.alloc_workspace(wl.batch, max_len)
    gpu_lib.oscar_decode_attention(pool, inp.q.cuda(), lens, max_len, dev["bf16_pt"], dev["int2_pt"],
                                   dev["bf16_pool"], dev["int2_pool"], to_dev(inp.calib.r_k), plain, pws)
    torch.cuda.synchronize()
    check_decode(plain, ref, what=f"{name} plain")


def test_cascade_values_not_absorbed(gpu_lib):
    wl, groups = CASES["d128-gqa8"]
    inp = _prefix_inputs(wl, groups)
    r_v = inp.calib.r_v
    seqs = make_seqs(wl, inp, r_v=r_v)
    pools = _share_tables(pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent,
                                              seed=wl.seed), seqs, groups)
    out, _ = _run(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k, groups, r_v=r_v)
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k, r_v)
    check_decode(out, ref, what="cascade, V not absorbed")


def test_cascade_without_groups_is_plain_decode(gpu_lib):
    """No group (or only groups with no shared pages): the call is the plain
    decode, bit for bit."""
    wl, _ = CASES["d128-gqa4"]
    inp = draw_inputs(wl)
    seqs = make_seqs(wl, inp)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=3)
    a, (pool, dev, lens, ws, max_len) = _run(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k, [(0, 2, 0)])
    b = torch.empty_like(a)
    pws = pool.alloc_workspace(wl.batch, max_len)
    gpu_lib.oscar_decode_attention(pool, inp.q.cuda(), lens, max_len, dev["bf16_pt"], dev["int2_pt"],
                                   dev["bf16_pool"], dev["int2_pool"], to_dev(inp.calib.r_k), b, pws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_cascade_repeated_calls_deterministic(gpu_lib):
    wl, groups = CASES["d64-gqa2"]
    inp = _prefix_inputs(wl, groups)
    seqs = make_seqs(wl, inp)
    pools = _share_tables(pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent,
                                              seed=wl.seed), seqs, groups)
    out1, (pool, dev, lens, ws, max_len) = _run(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k, groups)
    for _ in range(2):
        o = torch.zeros_like(out1)
        gpu_lib.oscar_decode_attention_cascade(pool, inp.q.cuda(), lens, max_len, dev["bf16_pt"], dev["int2_pt"],
                                               dev["bf16_pool"], dev["int2_pool"], to_dev(inp.calib.r_k), o, ws,
                                               groups)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), out1.view(torch.int16))


def test_cascade_group_with_empty_member(gpu_lib):
    """A prefix group whose member has length 0 this step: its rows are
    exactly zero, and the other members still match the oracle."""
    wl, groups = CASES["d128-gqa4"]
    inp = _prefix_inputs(wl, groups)
    seqs = make_seqs(wl, inp)
    pools = _share_tables(pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent,
                                              seed=wl.seed), seqs, groups)
    pool = gpu_lib.OscarPool(pool_config(wl))
    dev = upload(pools)
    lens_h = [s.L for s in seqs]
    empty = groups[0][0] + 1  # second member of the group
    lens_h[empty] = 0
    lens = torch.tensor(lens_h, dtype=torch.int32, device="cuda")
    max_len = max(lens_h)
    out = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    nbytes = gpu_lib.cascade_workspace_bytes(pool, len(seqs), max_len, dev["int2_pt"].shape[1], groups)
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    log(f"cascade decode with an empty member {empty}: lengths {lens_h}")
    gpu_lib.oscar_decode_attention_cascade(pool, inp.q.cuda(), lens, max_len, dev["bf16_pt"], dev["int2_pt"],
                                           dev["bf16_pool"], dev["int2_pool"], to_dev(inp.calib.r_k), out, ws, groups)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[empty].float()) == 0
    keep = [b for b in range(len(seqs)) if b != empty]
    ref, _ = oracle.decode_attention([seqs[b] for b in keep], inp.q[keep].float().numpy(), inp.calib.r_k)
    check_decode(out[keep], ref, what="cascade, group with an empty member")


@pytest.mark.parametrize("vscale", [1e-6, 500.0])
def test_cascade_value_range_unclipped(gpu_lib, vscale):
    """The prefix kernel keeps the same value-scale exponent as the decode
    kernel: values x1e-6 and x500 with no value clip (tau_V = +inf), GQA 8."""
    wl, groups = CASES["d128-gqa8"]
    inp = _prefix_inputs(wl, groups)
    inp.v = [(v.float() * vscale).to(torch.bfloat16) for v in inp.v]
    seqs = make_seqs(wl, inp, tau_v=np.full(wl.num_kv_heads, np.inf, np.float32))
    pools = _share_tables(pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent,
                                              seed=wl.seed), seqs, groups)
    out, _ = _run(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k, groups)
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k)
    check_decode(out, ref, what=f"cascade, values x{vscale:g}, no value clip")


@pytest.mark.parametrize("name", ["d128-gqa8", "d64-gqa2"])
def test_cascade_host_length_plan(gpu_lib, name):
    """The prefix-shared decode with the length-aware plan: each member's own
    chunks and its prefix slots in the per-sequence partial layout."""
    wl, groups = CASES[name]
    inp = _prefix_inputs(wl, groups)
    seqs = make_seqs(wl, inp)
    pools = _share_tables(pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent,
                                              seed=wl.seed), seqs, groups)
    out, _ = _run(gpu_lib, wl, seqs, inp.q, pools, inp.calib.r_k, groups, host_lens=[s.L for s in seqs])
    ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k)
    check_decode(out, ref, what=f"cascade {name}, host-length plan")
