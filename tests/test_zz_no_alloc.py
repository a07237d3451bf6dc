"""The allocation-free decode, oscar_decode_attention_noalloc, against the
workspace entry point oscar_decode_attention: two calls in a row on the
library's own device scratch, the second with a smaller batch and shorter
sequences, each bit-identical to the workspace call on the same inputs and
within the decode tolerance of the oracle.  A request whose workspace would
exceed the scratch is rejected before anything is launched."""

import pytest
import torch

import long_context_decode_oscar_amd as oscar_mod
import oracle
import pool_io
from harness import check_decode, draw_inputs, log, make_seqs, pool_config, to_dev, upload
from synthetic import CONFIGS, make_workload

pytestmark = pytest.mark.gpu

QWEN = CONFIGS["qwen3-8b-l100k"]


def _case(wl):
    inp = draw_inputs(wl)
    seqs = make_seqs(wl, inp)
    pools = pool_io.build_pools(seqs, wl.num_kv_heads, wl.head_dim, wl.n_groups, wl.sink, wl.recent, seed=wl.seed)
    return inp, seqs, upload(pools)


def test_noalloc_decode_matches_workspace_decode(gpu_lib):
    big = make_workload(QWEN, num_q_heads=16, num_kv_heads=4, batch=3, seq_lens=(9000, 2500, 400), seed=61)
    small = make_workload(QWEN, num_q_heads=16, num_kv_heads=4, batch=1, seq_lens=(700,), seed=62)
    for name, wl in (("first call, 3 sequences", big), ("second call, 1 shorter sequence", small)):
        inp, seqs, dev = _case(wl)
        pool = gpu_lib.OscarPool(pool_config(wl))
        lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
        max_len = max(wl.seq_lens)
        q, rk = inp.q.cuda(), to_dev(inp.calib.r_k)
        ws = pool.alloc_workspace(wl.batch, max_len)
        assert ws.numel() <= oscar_mod.NOALLOC_SCRATCH_BYTES
        ref_out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        log(f"noalloc case: {name}: workspace decode")
        gpu_lib.oscar_decode_attention(pool, q, lens, max_len, dev["bf16_pt"], dev["int2_pt"], dev["bf16_pool"],
                                       dev["int2_pool"], rk, ref_out, ws)
        out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        log(f"noalloc case: {name}: allocation-free decode")
        gpu_lib.oscar_decode_attention_noalloc(pool, q, lens, max_len, dev["bf16_pt"], dev["int2_pt"],
                                               dev["bf16_pool"], dev["int2_pool"], rk, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), name
        ref, _ = oracle.decode_attention(seqs, inp.q.float().numpy(), inp.calib.r_k)
        check_decode(out, ref, what=f"allocation-free decode, {name}")


def test_noalloc_decode_rejects_oversized_requests(gpu_lib):
    """512 sequences of 100,000 tokens need more decode scratch than the
    allocation-free entry point holds: OSCAR_ERR_UNSUPPORTED on the host,
    nothing launched, the output left untouched."""
    wl = QWEN
    pool = gpu_lib.OscarPool(pool_config(wl))
    batch = 512
    assert pool.workspace_bytes(batch, 100_000) > oscar_mod.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(batch, wl.num_q_heads, wl.head_dim, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    lens = torch.full((batch,), 100_000, dtype=torch.int32, device="cuda")
    pt = torch.zeros(batch, 1, dtype=torch.int32, device="cuda")
    b16 = torch.zeros(1, pool.bf16_page_bytes, dtype=torch.uint8, device="cuda")
    i2 = torch.zeros(1, pool.int2_page_bytes, dtype=torch.uint8, device="cuda")
    rk = torch.zeros(wl.num_kv_heads, wl.head_dim, wl.head_dim, dtype=torch.float32, device="cuda")
    with pytest.raises(oscar_mod.OscarError) as ei:
        gpu_lib.oscar_decode_attention_noalloc(pool, q, lens, 100_000, pt, pt, b16, i2, rk, out)
    assert ei.value.status == oscar_mod.OSCAR_ERR_UNSUPPORTED
    assert "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out.float() == 7.0).all())
