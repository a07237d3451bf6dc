"""GPU parity on the batched workloads at their full sizes, end to end: the
pools are written by the library's own write path (oscar_write_bf16,
oscar_quantize_pack, and for the demote workload oscar_append_demote inside
the step) and decoded by oscar_decode_attention.  On a sample of sequences
and KV heads (all query heads of each sampled KV head) the written history
is checked against the oracle's quantization and the decode output against
the oracle's decode of that history."""

import numpy as np
import pytest
import torch

import oracle
import pool_io
from harness import check_decode, check_write, log, pool_config
from synthetic import CONFIGS
from harness import draw_inputs

pytestmark = pytest.mark.gpu


def _gpu_pools(oscar, wl, inp, seed, pre_append=False, share=True):
    """Pools written through the library with random physical page ids.
    Sequences below wl.shared_prefix_seqs map the INT2 pages and BF16 sink
    pages of their common prefix to sequence 0's pages.  pre_append: the
    BF16 window also holds the token the step's append/demote moves."""
    rng = np.random.default_rng(seed)
    pool = oscar.OscarPool(pool_config(wl))
    lists16, n2 = [], []
    for L in wl.seq_lens:
        r0 = max(wl.sink, L - wl.recent - (1 if pre_append else 0))
        lists16.append([p for p in range((L + 15) // 16)
                        if p * 16 < min(L, wl.sink) or ((p + 1) * 16 > r0 and p * 16 < L)])
        n2.append((wl.hist_len(L) + 15) // 16)
    n_sh = wl.shared_prefix_seqs if share else 0
    sh2 = (wl.shared_prefix_tokens - wl.sink) // 16 if n_sh else 0
    sh16 = min(wl.sink, wl.shared_prefix_tokens) // 16 if n_sh else 0
    tot16 = sum(len(x) for x in lists16) + 7
    tot2 = sum(n2) + 13
    p16, p2 = iter(rng.permutation(tot16)), iter(rng.permutation(tot2))
    bpt = np.full((wl.batch, max((L + 15) // 16 for L in wl.seq_lens) + 1), -1, np.int32)
    ipt = np.full((wl.batch, max(n2)), -1, np.int32)
    for b in range(wl.batch):
        for lp in lists16[b]:
            bpt[b, lp] = bpt[0, lp] if 0 < b < n_sh and lp < sh16 else next(p16)
        for lp in range(n2[b]):
            ipt[b, lp] = ipt[0, lp] if 0 < b < n_sh and lp < sh2 else next(p2)
    dev = {"bf16_pt": torch.from_numpy(bpt).cuda(), "int2_pt": torch.from_numpy(ipt).cuda(),
           "bf16_pool": torch.full((tot16, pool.bf16_page_bytes), 0x7F, dtype=torch.uint8, device="cuda"),
           "int2_pool": torch.randint(0, 256, (tot2, pool.int2_page_bytes), dtype=torch.uint8, device="cuda")}
    c = inp.calib
    r_k, tau_k, tau_v = (torch.as_tensor(x).cuda() for x in (c.r_k, c.tau_k, c.tau_v))
    for b, L in enumerate(wl.seq_lens):
        k, v = inp.k[b], inp.v[b]
        sink = min(L, wl.sink)
        oscar.oscar_write_bf16(pool, k[:sink].contiguous(), v[:sink].contiguous(), 0, dev["bf16_pt"][b],
                               dev["bf16_pool"])
        r0 = max(wl.sink, L - wl.recent - (1 if pre_append else 0))
        if r0 < L:
            oscar.oscar_write_bf16(pool, k[r0:L].contiguous(), v[r0:L].contiguous(), r0, dev["bf16_pt"][b],
                                   dev["bf16_pool"])
        h = wl.hist_len(L)
        if h:
            oscar.oscar_quantize_pack(pool, k[wl.sink:wl.sink + h].contiguous(), v[wl.sink:wl.sink + h].contiguous(),
                                      dev["int2_pt"][b, :n2[b]].contiguous(), dev["int2_pool"], r_k, tau_k, tau_v)
    torch.cuda.synchronize()
    return pool, dev, (r_k, tau_k, tau_v)


def _oracle(wl, inp, seqs_idx, kv_heads, dev, pre_append=False):
    """Oracle reference for the sampled sequences and KV heads (heads are
    independent).  The GPU-written history of those heads is checked against
    the oracle's quantization first (V bit-exact, K within the rotation flip
    rule); the oracle then decodes that GPU-written history, so the output
    comparison measures the decode kernel alone and not the allowed flips
    (one flipped key code can move a sharply peaked head's output by more
    than the output tolerance).  Returns (ref, query heads)."""
    c = inp.calib
    rk, tk, tv = c.r_k[kv_heads], c.tau_k[kv_heads], c.tau_v[kv_heads]
    host2 = dev["int2_pool"].cpu().numpy()
    ipt = dev["int2_pt"].cpu().numpy()
    seqs = []
    for b in seqs_idx:
        L = wl.seq_lens[b]
        k = inp.k[b][:L][:, kv_heads].float().cpu().numpy()
        v = inp.v[b][:L][:, kv_heads].float().cpu().numpy()
        s = oracle.SeqPool(len(kv_heads), wl.head_dim, wl.group_size, wl.sink, wl.recent)
        if pre_append:
            s.prefill(k[:L - 1], v[:L - 1], rk, tk, tv)
            s.append_demote(k[L - 1], v[L - 1], rk, tk, tv)
        else:
            s.prefill(k, v, rk, tk, tv)
        g = pool_io.read_history(host2, ipt[b], s.n_hist, wl.num_kv_heads, wl.head_dim, wl.n_groups)
        kc, ks, kz, vc, vs, vz = (x[:, kv_heads] for x in g)
        hist = wl.sink + np.arange(s.n_hist)
        for i, h in enumerate(kv_heads):
            check_write((kc[:, i], ks[:, i], kz[:, i]), k[hist, i], rk[i], tk[i], wl.group_size,
                        f"seq {b} KV head {h} keys")
            check_write((vc[:, i], vs[:, i], vz[:, i]), v[hist, i], None, tv[i], wl.group_size,
                        f"seq {b} KV head {h} values")
        s.kc, s.ks, s.kz = kc.copy(), ks.astype(np.float32), kz.astype(np.float32)
        s.vc, s.vs, s.vz = vc.copy(), vs.astype(np.float32), vz.astype(np.float32)
        seqs.append(s)
    g = wl.gqa
    qh = [h for kv in kv_heads for h in range(kv * g, (kv + 1) * g)]
    q = inp.q[seqs_idx][:, qh].float().cpu().numpy()
    ref, _ = oracle.decode_attention(seqs, q, rk)
    return ref, qh


def test_batched_demote_step_full_size_sampled(gpu_lib):
    """32 sequences of 32,768 tokens (32 q / 8 KV heads, D 128): one step of
    append + demote + decode on GPU-written pools, as bench.py times it."""
    wl = CONFIGS["qwen3-8b-b32-l32k-demote"]
    inp = draw_inputs(wl, device="cuda")
    log("writing 32 x 32,768-token pools through the library")
    pool, dev, (r_k, tau_k, tau_v) = _gpu_pools(gpu_lib, wl, inp, seed=11, pre_append=True)
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    k_new = torch.stack([inp.k[b][L - 1] for b, L in enumerate(wl.seq_lens)]).contiguous()
    v_new = torch.stack([inp.v[b][L - 1] for b, L in enumerate(wl.seq_lens)]).contiguous()
    gpu_lib.oscar_append_demote(pool, k_new, v_new, lens - 1, dev["bf16_pt"], dev["int2_pt"], dev["bf16_pool"],
                                dev["int2_pool"], r_k, tau_k, tau_v)
    out = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = pool.alloc_workspace(wl.batch, max(wl.seq_lens))
    gpu_lib.oscar_decode_attention(pool, inp.q.contiguous(), lens, max(wl.seq_lens), dev["bf16_pt"], dev["int2_pt"],
                                   dev["bf16_pool"], dev["int2_pool"], r_k, out, ws)
    torch.cuda.synchronize()
    seqs_idx, kv_heads = [0, 9, 22, 31], [2, 7]
    log(f"oracle write + decode of sequences {seqs_idx}, KV heads {kv_heads}")
    ref, qh = _oracle(wl, inp, seqs_idx, kv_heads, dev, pre_append=True)
    check_decode(out[seqs_idx][:, qh], ref, what="batched demote step (sampled)")


def test_mixed_prefix_gqa8_full_size_sampled(gpu_lib):
    """8 sequences of 30K-121K tokens, 64 q / 8 KV heads (GQA 8), four
    sharing a 65,536-token prefix through common page-table entries."""
    wl = CONFIGS["qwen3-32b-b8-mixed-prefix"]
    inp = draw_inputs(wl, device="cuda")
    log(f"writing pools for lengths {wl.seq_lens} through the library")
    pool, dev, (r_k, _, _) = _gpu_pools(gpu_lib, wl, inp, seed=12)
    ipt = dev["int2_pt"].cpu().numpy()
    assert (ipt[1, :4092] == ipt[0, :4092]).all() and (ipt[3, :4092] == ipt[0, :4092]).all()
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    out = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = pool.alloc_workspace(wl.batch, max(wl.seq_lens))
    gpu_lib.oscar_decode_attention(pool, inp.q.contiguous(), lens, max(wl.seq_lens), dev["bf16_pt"], dev["int2_pt"],
                                   dev["bf16_pool"], dev["int2_pool"], r_k, out, ws)
    torch.cuda.synchronize()
    # the same step through the prefix-shared decode: the 4,092 shared pages
    # attended once per pair of sequences
    groups = [(0, wl.shared_prefix_seqs, (wl.shared_prefix_tokens - wl.sink) // 16)]
    nbytes = gpu_lib.cascade_workspace_bytes(pool, wl.batch, max(wl.seq_lens), dev["int2_pt"].shape[1], groups)
    cws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out_c = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    log(f"cascade decode with groups {groups}")
    gpu_lib.oscar_decode_attention_cascade(pool, inp.q.contiguous(), lens, max(wl.seq_lens), dev["bf16_pt"],
                                           dev["int2_pt"], dev["bf16_pool"], dev["int2_pool"], r_k, out_c, cws,
                                           groups)
    torch.cuda.synchronize()
    # both paths again with the length-aware plan (host copy of the lengths),
    # the launch configuration bench.py times
    out_h = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    gpu_lib.oscar_decode_attention(pool, inp.q.contiguous(), lens, max(wl.seq_lens), dev["bf16_pt"], dev["int2_pt"],
                                   dev["bf16_pool"], dev["int2_pool"], r_k, out_h, ws, seq_lens_host=wl.seq_lens)
    out_ch = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    gpu_lib.oscar_decode_attention_cascade(pool, inp.q.contiguous(), lens, max(wl.seq_lens), dev["bf16_pt"],
                                           dev["int2_pt"], dev["bf16_pool"], dev["int2_pool"], r_k, out_ch, cws,
                                           groups, seq_lens_host=wl.seq_lens)
    torch.cuda.synchronize()
    seqs_idx, kv_heads = list(range(8)), [5]
    log(f"oracle write + decode of all 8 sequences, KV head {kv_heads}")
    ref, qh = _oracle(wl, inp, seqs_idx, kv_heads, dev)
    check_decode(out[seqs_idx][:, qh], ref, what="mixed prefix GQA8 (sampled)")
    check_decode(out_c[seqs_idx][:, qh], ref, what="mixed prefix GQA8, cascade (sampled)")
    check_decode(out_h[seqs_idx][:, qh], ref, what="mixed prefix GQA8, host-length plan (sampled)")
    check_decode(out_ch[seqs_idx][:, qh], ref, what="mixed prefix GQA8, cascade, host-length plan (sampled)")
