#!/usr/bin/env python3
"""Benchmark of the OSCAR INT2 decode-attention hot path on one MI355X.

A step is one decode-attention pass (oscar_decode_attention: q rotation,
INT2 history split-K, BF16 sink/recent, LSE merge) of one layer for the whole
batch; the demote workload adds one oscar_append_demote per step.  The pools
are built on the GPU by the library's own write path (oscar_quantize_pack,
oscar_write_bf16) from seeded synthetic tensors.

Timing protocol: the pool working set of one step (58.7 MB at 100K tokens)
fits the 256 MB Infinity Cache, so steps rotate through independent pool
copies totalling >= 2 GiB (cold-cache), one pool tensor per copy like the
per-layer KV caches of a model, all sharing the sequences' page tables as a
model's layers do; the K timed steps are replayed from a HIP graph and
bracketed by HIP events on the launch stream.  The median of
several repeats is reported; warm (single copy) and eager-launch numbers are
reported beside it.

Prints one JSON line.
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "INT2 decode-attn KV GB/s & tokens/s at 100K ctx; % of HBM peak"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


_CALIB_CACHE = {}


def gpu_calibration(oscar, wl):
    """Offline parameters of a workload from the library's calibration kernels
    (oscar_calibrate) on the seeded 2048-token calibration draw."""
    import torch
    from synthetic import draw_calibration, make_calibration
    key = (wl.num_kv_heads, wl.gqa, wl.head_dim, wl.seed)
    if key not in _CALIB_CACHE:
        draws = draw_calibration(*key)
        q = torch.from_numpy(np.stack([d.q for d in draws])).cuda()
        k = torch.from_numpy(np.stack([d.k for d in draws])).cuda()
        v = torch.from_numpy(np.stack([d.v for d in draws])).cuda()
        res = oscar.oscar_calibrate(q, k, v, clip_quantile=0.995)
        torch.cuda.synchronize()
        _CALIB_CACHE[key] = make_calibration(draws, *(res[n].cpu().numpy() for n in ("r_k", "r_v", "tau_k", "tau_v")))
    return _CALIB_CACHE[key]


_CODEBOOK_CACHE = {}


def gpu_codebook(oscar, wl):
    """Four-level codebooks (keys, values) of a workload's layer from
    oscar_calib_codebook on the calibration draw, with the rotations and
    thresholds of gpu_calibration."""
    import torch
    from synthetic import draw_calibration
    key = (wl.num_kv_heads, wl.gqa, wl.head_dim, wl.group_size, wl.seed)
    if key not in _CODEBOOK_CACHE:
        c = gpu_calibration(oscar, wl)
        draws = draw_calibration(wl.num_kv_heads, wl.gqa, wl.head_dim, wl.seed)
        out = []
        for name, r, tau in (("k", c.r_k, c.tau_k), ("v", c.r_v, c.tau_v)):
            x = torch.from_numpy(np.stack([getattr(d, name) for d in draws])).cuda()
            lv = oscar.oscar_calib_codebook(x, torch.from_numpy(r).cuda(), torch.from_numpy(tau).cuda(),
                                            wl.group_size)
            out.append(tuple(float(a) for a in lv.cpu().numpy()))
        _CODEBOOK_CACHE[key] = tuple(out)
    return _CODEBOOK_CACHE[key]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3-8b-l100k")
    ap.add_argument("--cold-bytes", type=float, default=2 * 2**30)
    ap.add_argument("--repeats", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=1e3 * SETTLE_S,
                    help="untimed back-to-back runs of the timed steps before each measurement")
    ap.add_argument("--no-bf16", action="store_true", help="skip the BF16-only comparator")
    ap.add_argument("--no-codebook", action="store_true", help="skip the four-level codebook variant")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run N eager decode steps over the cold pool copies, then one plain copy of "
                         "--probe-bytes (for rocprofv3 counters); prints no JSON")
    ap.add_argument("--probe-bytes", type=int, default=256 * 2**20)
    ap.add_argument("--phase-stamps", action="store_true",
                    help="load the profiling build liboscar_stamps.so, replay the 100K-token step over cold pool "
                         "copies and print its per-wave phase timeline (no JSON metric line)")
    ap.add_argument("--only", default="all", choices=["all", "headline", "bulk", "demote", "mixed", "calib", "batch-bf16"],
                    help="run one section only (the JSON line then holds what was measured)")
    return ap.parse_args()


class Decoder:
    """Pre-marshalled oscar_decode_attention calls, one per pool copy."""

    def __init__(self, oscar, pool, wl, q, lens, copies, r_k, out, ws, bf16_only=False, groups=None,
                 host_lengths=True):
        import torch
        lib = oscar.load()
        self.lib = lib
        self.bf16_only = bf16_only
        self.torch = torch
        # the sequences' lengths on the host: the length-aware split-K plan
        # (host_lengths=False: every sequence planned for the longest)
        self.host_lens = oscar.HostLengths(wl.seq_lens)
        hptr = self.host_lens.ptr if host_lengths else None
        self.args = []
        # r_k: one tensor for every copy, or one per copy (a layer's own R_K)
        rks = r_k if isinstance(r_k, (list, tuple)) else [r_k] * len(copies)
        for c, rk in zip(copies, rks):
            b16, i2 = c["bf16_pool"], c["int2_pool"]
            if bf16_only:
                self.args.append((pool.handle, wl.batch, max(wl.seq_lens), q.data_ptr(), lens.data_ptr(),
                                  c["bf16_pt"].data_ptr(), c["bf16_pt"].shape[1], b16.shape[0],
                                  b16.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel()))
            else:
                self.args.append((pool.handle, wl.batch, max(wl.seq_lens), q.data_ptr(), lens.data_ptr(), hptr,
                                  c["bf16_pt"].data_ptr(), c["bf16_pt"].shape[1], b16.shape[0],
                                  c["int2_pt"].data_ptr(), c["int2_pt"].shape[1], i2.shape[0],
                                  b16.data_ptr(), i2.data_ptr(), rk.data_ptr(), None,
                                  out.data_ptr(), ws.data_ptr(), ws.numel()))
        self.fn = lib.oscar_bf16_decode_attention if bf16_only else lib.oscar_decode_attention
        if groups:
            # prefix groups: oscar_decode_attention_cascade (group array
            # inserted before the workspace arguments)
            arr, ng = oscar._groups(groups)
            self._groups = arr
            gp = ctypes.cast(arr, ctypes.c_void_p)
            self.args = [a[:-2] + (gp, ng) + a[-2:] for a in self.args]
            self.fn = lib.oscar_decode_attention_cascade

    def __call__(self, i):
        # launch on the current stream (the capture stream inside a graph capture)
        st = self.fn(*self.args[i % len(self.args)], self.torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(self.lib.oscar_last_error().decode())


def build_pools(oscar, pool, wl, inp, n_copies, bf16_only=False, seed=0, shared_tables=True, pre_append=False):
    """n_copies independent pools of one workload, written by the library.

    shared_tables=True models one layer's KV cache per copy: every copy has
    its own pool tensor (a slice of one allocation) and all copies share the
    sequences' page tables, as the layers of a model share a sequence's page
    table.  shared_tables=False gives every copy its own page tables over one
    big pool (the page-table reads are then cold as well); the INT2 pool then
    spans the workload's INT2 arena (wl.int2_arena_bytes) when that is larger,
    pages scattered over it at random.

    pre_append=True builds the state before the step's append: the BF16
    window also holds the token that the step's oscar_append_demote moves to
    the INT2 history.  Sequences 0..wl.shared_prefix_seqs-1 share the INT2
    pages and BF16 sink pages of their common prefix (one physical copy)."""
    import numpy as np
    import torch
    rng = np.random.Generator(np.random.PCG64(seed + 300))
    c = inp.calib
    r_k = torch.as_tensor(c.r_k).cuda()
    tau_k = torch.as_tensor(c.tau_k).cuda()
    tau_v = torch.as_tensor(c.tau_v).cuda()
    max_pages = max((L + 15) // 16 for L in wl.seq_lens)
    b16_lists, i2_counts = [], []
    for L in wl.seq_lens:
        if bf16_only:
            b16_lists.append(list(range((L + 15) // 16)))
            i2_counts.append(0)
        else:
            r0 = max(wl.sink, L - wl.recent - (1 if pre_append else 0))
            b16_lists.append([p for p in range((L + 15) // 16)
                              if p * 16 < min(L, wl.sink) or ((p + 1) * 16 > r0 and p * 16 < L)])
            i2_counts.append((wl.hist_len(L) + 15) // 16)
    # prefix sharing: logical pages below these counts map to sequence 0's pages
    n_sh_seq = wl.shared_prefix_seqs if (wl.shared_prefix_seqs and not bf16_only) else 0
    n_sh2 = max(0, wl.shared_prefix_tokens - wl.sink) // 16 if n_sh_seq else 0
    n_sh16 = min(wl.sink, wl.shared_prefix_tokens) // 16 if n_sh_seq else 0
    saved16 = max(0, n_sh_seq - 1) * n_sh16
    saved2 = max(0, n_sh_seq - 1) * n_sh2
    n16c = max(sum(len(x) for x in b16_lists) - saved16, 1)  # physical pages per copy
    n2c = max(sum(i2_counts) - saved2, 1)
    arena2 = n2c * n_copies
    if not shared_tables and wl.int2_arena_bytes:
        arena2 = max(arena2, wl.int2_arena_bytes // pool.int2_page_bytes)
    bf16_all = torch.empty((n16c * n_copies, pool.bf16_page_bytes), dtype=torch.uint8, device="cuda")
    int2_all = torch.empty((arena2, pool.int2_page_bytes), dtype=torch.uint8, device="cuda")

    def tables(phys16, phys2):
        """Page tables over the given physical page ids (consumed in order)."""
        bpt = np.full((wl.batch, max_pages + 1), -1, np.int32)
        ipt = np.full((wl.batch, max(max(i2_counts), 1)), -1, np.int32)
        p16 = p2 = 0
        for b in range(wl.batch):
            for lp in b16_lists[b]:
                if 0 < b < n_sh_seq and lp < n_sh16:
                    bpt[b, lp] = bpt[0, lp]
                else:
                    bpt[b, lp] = phys16[p16]
                    p16 += 1
            for lp in range(i2_counts[b]):
                if 0 < b < n_sh_seq and lp < n_sh2:
                    ipt[b, lp] = ipt[0, lp]
                else:
                    ipt[b, lp] = phys2[p2]
                    p2 += 1
        assert p16 <= len(phys16) and p2 <= len(phys2)
        return torch.from_numpy(bpt).cuda(), torch.from_numpy(ipt).cuda()

    if shared_tables:
        shared = tables(rng.permutation(n16c), rng.permutation(n2c))
    else:
        glob16 = rng.permutation(n16c * n_copies)
        glob2 = rng.choice(arena2, n2c * n_copies, replace=False) if arena2 > n2c * n_copies else \
            rng.permutation(arena2)
    copies = []
    for ci in range(n_copies):
        if shared_tables:
            bpt, ipt = shared
            b16, i2 = bf16_all[ci * n16c:(ci + 1) * n16c], int2_all[ci * n2c:(ci + 1) * n2c]
        else:
            # distinct tables over the whole allocation; copy ci owns the
            # pages its slice of the global draw names
            bpt, ipt = tables(glob16[ci * n16c:(ci + 1) * n16c], glob2[ci * n2c:(ci + 1) * n2c])
            b16, i2 = bf16_all, int2_all
        cp = {"bf16_pt": bpt, "int2_pt": ipt, "bf16_pool": b16, "int2_pool": i2}
        for b, L in enumerate(wl.seq_lens):
            k, v = inp.k[b], inp.v[b]
            if bf16_only:
                oscar.oscar_write_bf16(pool, k[:L].contiguous(), v[:L].contiguous(), 0, bpt[b], b16)
                continue
            sink = min(L, wl.sink)
            oscar.oscar_write_bf16(pool, k[:sink].contiguous(), v[:sink].contiguous(), 0, bpt[b], b16)
            r0 = max(wl.sink, L - wl.recent - (1 if pre_append else 0))
            if r0 < L:
                oscar.oscar_write_bf16(pool, k[r0:L].contiguous(), v[r0:L].contiguous(), r0, bpt[b], b16)
            h = wl.hist_len(L)
            if h:
                oscar.oscar_quantize_pack(pool, k[wl.sink:wl.sink + h].contiguous(), v[wl.sink:wl.sink + h].contiguous(),
                                          ipt[b, :i2_counts[b]].contiguous(), i2, r_k, tau_k, tau_v)
        copies.append(cp)
    torch.cuda.synchronize()
    return copies, r_k


class DemoteDecoder:
    """One decode step with the append/demote folded in, per pool copy:
    oscar_append_demote (token L-1 appended, token L-1-W demoted to INT2),
    then oscar_decode_attention at length L, both on the current stream."""

    def __init__(self, oscar, pool, wl, q, copies, r_k, tau_k, tau_v, k_new, v_new, lens_pre, lens, out, ws):
        import torch
        self.torch = torch
        self.lib = oscar.load()
        self.dec = Decoder(oscar, pool, wl, q, lens, copies, r_k, out, ws)
        self.args = []
        for c in copies:
            b16, i2 = c["bf16_pool"], c["int2_pool"]
            self.args.append((pool.handle, wl.batch, k_new.data_ptr(), v_new.data_ptr(), lens_pre.data_ptr(),
                              c["bf16_pt"].data_ptr(), c["bf16_pt"].shape[1], b16.shape[0],
                              c["int2_pt"].data_ptr(), c["int2_pt"].shape[1], i2.shape[0],
                              b16.data_ptr(), i2.data_ptr(), r_k.data_ptr(), None, tau_k.data_ptr(),
                              tau_v.data_ptr()))

    def __call__(self, i):
        st = self.lib.oscar_append_demote(*self.args[i % len(self.args)],
                                          self.torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(self.lib.oscar_last_error().decode())
        self.dec(i)


def unique_kv_bytes(wl):
    """HBM bytes of one decode step counting pages shared by a prefix once."""
    kv = wl.kv_bytes()
    if not wl.shared_prefix_seqs:
        return kv["total"]
    n_sh2 = max(0, wl.shared_prefix_tokens - wl.sink) // 16
    n_sh16 = min(wl.sink, wl.shared_prefix_tokens)
    dup = (wl.shared_prefix_seqs - 1) * wl.num_kv_heads * (
        n_sh2 * 16 * wl.int2_bytes_per_token_head() + n_sh16 * wl.bf16_bytes_per_token_head())
    return kv["total"] - dup


def bench_decode_workload(oscar, name, steps, warmup, repeats, cold_bytes, profile_launches=0):
    """Decode steps of a batched workload, timed like the headline: HIP-graph
    replay over cold pool copies.  With wl.demote every step also appends one
    token per sequence and demotes one to the INT2 history.  profile_launches
    > 0 only runs that many eager steps (for rocprofv3 counters) and returns
    None."""
    import torch
    from synthetic import CONFIGS, draw_inputs
    wl = CONFIGS[name]
    kv = wl.kv_bytes()
    uniq = unique_kv_bytes(wl)
    inp = draw_inputs(wl, gpu_calibration(oscar, wl), device="cuda")
    pool = oscar.OscarPool(oscar.PoolConfig(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.group_size, 16,
                                            wl.sink, wl.recent, 1, 0.0))
    n_copies = max(2, math.ceil(cold_bytes / uniq))
    copies, r_k = build_pools(oscar, pool, wl, inp, n_copies, seed=wl.seed, shared_tables=not wl.demote,
                              pre_append=wl.demote)
    q = inp.q.contiguous()
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = pool.alloc_workspace(wl.batch, max(wl.seq_lens))
    if wl.demote:
        c = inp.calib
        tau_k = torch.as_tensor(c.tau_k).cuda()
        tau_v = torch.as_tensor(c.tau_v).cuda()
        k_new = torch.stack([inp.k[b][L - 1] for b, L in enumerate(wl.seq_lens)]).contiguous()
        v_new = torch.stack([inp.v[b][L - 1] for b, L in enumerate(wl.seq_lens)]).contiguous()
        lens_pre = lens - 1
        step = DemoteDecoder(oscar, pool, wl, q, copies, r_k, tau_k, tau_v, k_new, v_new, lens_pre, lens, out, ws)
    else:
        step = Decoder(oscar, pool, wl, q, lens, copies, r_k, out, ws)
    if profile_launches:
        for i in range(profile_launches):
            step(i)
        torch.cuda.synchronize()
        log(f"profile run: {profile_launches} {name} steps done")
        return None
    ms, ms_min = time_steps(step, steps, warmup, repeats, use_graph=True)
    uniform = None
    if wl.batch > 1 and len(set(wl.seq_lens)) > 1:
        # the same step with every sequence planned for the longest one
        ustep = Decoder(oscar, pool, wl, q, lens, copies, r_k, out, ws, host_lengths=False)
        ms_u, _ = time_steps(ustep, steps, warmup, repeats, use_graph=True)
        uniform = {"us_per_step": round(ms_u * 1e3, 3), "host_length_plan_speedup": round(ms_u / ms, 3)}
        log(f"{name} max-length plan: {ms_u * 1e3:.2f} us/step ({ms_u / ms:.2f}x the host-length plan)")
        del ustep
    cascade = None
    if wl.shared_prefix_seqs:
        # the same step with the shared prefix pages attended once per group
        # of sequences (oscar_decode_attention_cascade)
        groups = [(0, wl.shared_prefix_seqs, max(0, wl.shared_prefix_tokens - wl.sink) // 16)]
        cws_n = oscar.cascade_workspace_bytes(pool, wl.batch, max(wl.seq_lens), copies[0]["int2_pt"].shape[1], groups)
        cws = torch.zeros(cws_n, dtype=torch.uint8, device="cuda")
        out_c = torch.empty_like(q)
        cstep = Decoder(oscar, pool, wl, q, lens, copies, r_k, out_c, cws, groups=groups)
        ms_c, ms_c_min = time_steps(cstep, steps, warmup, repeats, use_graph=True)
        step(0)
        cstep(0)
        torch.cuda.synchronize()
        # the two paths agree to the decode tolerance (2e-3 of each head's norm)
        dif = (out.float() - out_c.float()).abs().amax(dim=-1) / out.float().norm(dim=-1).clamp_min(1e-30)
        cascade = {"groups": groups, "us_per_step": round(ms_c * 1e3, 3), "us_min": round(ms_c_min * 1e3, 3),
                   "speedup_vs_plain": round(ms / ms_c, 3), "max_rel_diff_vs_plain": round(float(dif.max()), 6),
                   "GBps_unique": round(uniq / (ms_c * 1e-3) / 1e9, 2),
                   "pct_hbm_peak_unique": round(100 * uniq / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}
        log(f"{name} cascade: {ms_c * 1e3:.2f} us/step ({ms / ms_c:.2f}x), max rel diff {float(dif.max()):.2e}")
        del cstep, cws
    # append/demote (and the write it does) counted on top of the KV read
    # (per sequence and KV head: bf16 K, V written by the append and read by
    # the demotion, the INT2 token written)
    extra = wl.batch * wl.num_kv_heads * (2 * (2 * wl.head_dim * 2) + wl.int2_bytes_per_token_head()) \
        if wl.demote else 0
    log(f"{name}: {ms * 1e3:.2f} us/step ({'append/demote + ' if wl.demote else ''}decode), "
        f"{uniq / (ms * 1e-3) / 1e9:.1f} GB/s unique KV")
    res = {"workload": name, "batch": wl.batch, "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
           "context": list(wl.seq_lens) if wl.batch <= 8 else f"{wl.batch} x {wl.seq_lens[0]}",
           "us_per_step": round(ms * 1e3, 3), "us_min": round(ms_min * 1e3, 3),
           "tokens_per_s": round(wl.batch / (ms * 1e-3), 1),
           "kv_bytes_per_step": kv["total"], "unique_kv_bytes_per_step": uniq,
           "GBps": round((uniq + extra) / (ms * 1e-3) / 1e9, 2),
           "pct_hbm_peak": round(100 * (uniq + extra) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
           "pool_copies": n_copies}
    if wl.demote:
        res["append_demote"] = "one token appended and one demoted per sequence inside every timed step"
        res["int2_arena_GiB"] = round(wl.int2_arena_bytes / 2**30, 1)
    if uniform:
        res["max_length_plan"] = uniform
    if wl.shared_prefix_seqs:
        res["shared_prefix"] = f"{wl.shared_prefix_seqs} sequences share {wl.shared_prefix_tokens} tokens"
        res["logical_GBps"] = round(kv["total"] / (ms * 1e-3) / 1e9, 2)
        res["cascade"] = cascade
    del step, copies
    torch.cuda.empty_cache()
    return res


def bench_batch_comparator(oscar, name, steps, warmup, repeats, cold_bytes, min_bf16_copies=3):
    """Decode only (no append/demote) of a batched workload, INT2 pool against
    the BF16-only comparator on the same sequences, both timed like the
    headline: HIP-graph replay over cold pool copies (the BF16 pools are
    several GB each, so at least min_bf16_copies of them rotate)."""
    import torch
    from synthetic import CONFIGS, draw_inputs
    wl = CONFIGS[name]
    kv = wl.kv_bytes()
    inp = draw_inputs(wl, gpu_calibration(oscar, wl), device="cuda")
    pool = oscar.OscarPool(oscar.PoolConfig(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.group_size, 16,
                                            wl.sink, wl.recent, 1, 0.0))
    q = inp.q.contiguous()
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    n2 = max(2, math.ceil(cold_bytes / kv["total"]))
    copies, r_k = build_pools(oscar, pool, wl, inp, n2, seed=wl.seed + 5)
    ws = pool.alloc_workspace(wl.batch, max(wl.seq_lens))
    dec = Decoder(oscar, pool, wl, q, lens, copies, r_k, out, ws)
    ms2, _ = time_steps(dec, steps, warmup, repeats, use_graph=True)
    del dec, copies, ws
    torch.cuda.empty_cache()
    n16 = max(min_bf16_copies, math.ceil(cold_bytes / kv["bf16_only_total"]))
    bcopies, _ = build_pools(oscar, pool, wl, inp, n16, bf16_only=True, seed=wl.seed + 6)
    bws = pool.alloc_workspace(wl.batch, max(wl.seq_lens), bf16_only=True)
    bdec = Decoder(oscar, pool, wl, q, lens, bcopies, r_k, out, bws, bf16_only=True)
    ms16, _ = time_steps(bdec, steps, warmup, repeats, use_graph=True)
    del bdec, bcopies, bws, inp
    torch.cuda.empty_cache()
    log(f"{name} decode only: INT2 {ms2 * 1e3:.2f} us/step, BF16-only {ms16 * 1e3:.2f} us/step "
        f"({ms16 / ms2:.2f}x)")
    return {"workload": name, "batch": wl.batch, "context": f"{wl.batch} x {wl.seq_lens[0]}",
            "decode_only": "no append/demote in the timed step",
            "int2": {"us_per_step": round(ms2 * 1e3, 3), "kv_bytes_per_step": kv["total"],
                     "GBps": round(kv["total"] / (ms2 * 1e-3) / 1e9, 2), "pool_copies": n2,
                     "tokens_per_s": round(wl.batch / (ms2 * 1e-3), 1)},
            "bf16_only": {"us_per_step": round(ms16 * 1e3, 3), "kv_bytes_per_step": kv["bf16_only_total"],
                          "GBps": round(kv["bf16_only_total"] / (ms16 * 1e-3) / 1e9, 2), "pool_copies": n16,
                          "tokens_per_s": round(wl.batch / (ms16 * 1e-3), 1)},
            "int2_speedup": round(ms16 / ms2, 3)}


SETTLE_S = 0.05


def time_steps(step, n_steps, warmup, repeats, use_graph=True):
    """Median and min ms per step over `repeats` runs of n_steps steps.

    After the `warmup` eager steps (and the graph capture) the same n_steps
    steps run untimed, back to back, for SETTLE_S seconds before the timed
    runs: the first ~10 ms of decode work after the GPU idled (pool building
    is mostly host work) run up to 7 % slower than the steady state that a
    serving loop sees, whatever the number of steps per replay."""
    import torch
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for i in range(n_steps):
                    step(warmup + i)
        torch.cuda.synchronize()
    t_end = time.perf_counter() + SETTLE_S
    n_settle = 0
    while True:
        if graph is not None:
            graph.replay()
        else:
            for i in range(n_steps):
                step(warmup + i)
        torch.cuda.synchronize()
        n_settle += 1
        if time.perf_counter() >= t_end:
            break
    log(f"timing: {warmup} warm-up steps, {n_settle} untimed runs of {n_steps} steps, {repeats} timed runs")
    times = []
    for _ in range(repeats):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(n_steps):
                step(warmup + i)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / n_steps)
    return statistics.median(times), min(times)


def copy_ceiling_gbps():
    import torch
    n = 2 * 2**30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 5
    del x, y
    return 2 * n / ms / 1e6


DECODE_SOURCES = ("decode.hip", "common.h", "kernels.h")
BULK_SOURCES = ("write.hip", "common.h", "kernels.h")


def source_sha(files):
    """Hash of the kernel sources with comments and blank space removed, so
    that it changes with the code and not with its commentary."""
    import re
    h = hashlib.sha256()
    for f in files:
        text = open(os.path.join(ROOT, "long_context_decode_oscar_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_for(workload, files=DECODE_SOURCES):
    """HBM bytes per launch from committed rocprofv3 PMC counters, if they
    were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("kernel_source_sha") != source_sha(files):
        return None
    return t.get("hbm_bytes_per_launch")


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, repeats=3):
    """The oracle timed on this host's cores, the whole 100K-token step:
    its write path (W1-W7: rotate, clip, quantize and pack every history
    token of every KV head, the pool's prefill) once, and its decode (R1-R3:
    dequantize, inverse-rotate, one softmax over the concatenated pool) with
    all BLAS threads (median of `repeats`) and with one thread (one run).
    Inputs come from the oracle's own calibration of the same seeded draws
    (not timed)."""
    import oracle
    from synthetic import draw_calibration, draw_inputs, make_calibration
    draws = draw_calibration(wl.num_kv_heads, wl.gqa, wl.head_dim, wl.seed)
    oc = oracle.calibrate([(d.q, d.k, d.v) for d in draws])
    c = make_calibration(draws, oc["r_k"], oc["r_v"], oc["tau_k"], oc["tau_v"])
    inp = draw_inputs(wl, c, device="cpu")
    seqs = []
    t_write = 0.0
    hist_tokens = 0
    for b, L in enumerate(wl.seq_lens):
        k = inp.k[b][:L].float().cpu().numpy()
        v = inp.v[b][:L].float().cpu().numpy()
        s = oracle.SeqPool(wl.num_kv_heads, wl.head_dim, wl.group_size, wl.sink, wl.recent)
        t0 = time.perf_counter()
        s.prefill(k, v, c.r_k, c.tau_k, c.tau_v)
        t_write += time.perf_counter() - t0
        hist_tokens += wl.hist_len(L)
        seqs.append(s)
    q = inp.q.float().cpu().numpy()
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        oracle.decode_attention(seqs, q, c.r_k)
        times.append(time.perf_counter() - t0)
    dt = statistics.median(times)
    kv = wl.kv_bytes()
    cores = os.cpu_count()
    dt1 = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.decode_attention(seqs, q, c.r_k)
            dt1 = time.perf_counter() - t0
    except Exception:
        pass
    tok_heads = hist_tokens * wl.num_kv_heads
    res = {"value": round(kv["total"] / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
           "sample": f"whole step: fp64 numpy oracle decode (dequantize, inverse-rotate, one softmax) of all "
                     f"{wl.num_kv_heads} KV heads / {wl.num_q_heads} query heads of {wl.batch} sequence(s) at "
                     f"{list(wl.seq_lens)[:4]} tokens; step KV bytes / median wall time of {repeats} runs "
                     f"({dt:.2f} s) with {cores} BLAS threads; host has {os.cpu_count()} logical CPUs",
           "cpu_model": _cpu_model(),
           "write_path": {"token_heads_per_s": round(tok_heads / t_write, 1), "s": round(t_write, 3),
                          "sample": f"oracle W1-W7 of {hist_tokens} history tokens x {wl.num_kv_heads} KV heads "
                                    f"(R_K rotation, clip, quantize, pack), one run"}}
    if dt1 is not None:
        res["single_thread"] = {"value": round(kv["total"] / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                                "s": round(dt1, 3)}
    return res


def bench_bulk_quant(oscar, steps=10, warmup=3, repeats=5, profile_launches=0):
    """Write-path bulk quantization: K, V of 131,072 tokens x 8 KV heads x 128
    (bf16) rotated (K), clipped, quantized and packed into 8,192 pages per
    head, one oscar_quantize_pack launch per step.  Algorithmic bytes: the
    bf16 K and V read once plus the packed pages written once."""
    import numpy as np
    import torch
    from synthetic import CONFIGS, draw_inputs
    wl = CONFIGS["bulk-quant-t131k"]
    inp = draw_inputs(wl, gpu_calibration(oscar, wl), with_q=False, device="cuda")
    k, v = inp.k[0].contiguous(), inp.v[0].contiguous()
    t = k.shape[0]
    c = inp.calib
    r_k, tau_k, tau_v = (torch.as_tensor(x).cuda() for x in (c.r_k, c.tau_k, c.tau_v))
    pool = oscar.OscarPool(oscar.PoolConfig(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.group_size, 16,
                                            wl.sink, wl.recent, 1, 0.0))
    npg = (t + 15) // 16
    rng = np.random.Generator(np.random.PCG64(wl.seed + 500))
    ids = torch.from_numpy(rng.permutation(npg).astype(np.int32)).cuda()
    int2 = torch.empty((npg, pool.int2_page_bytes), dtype=torch.uint8, device="cuda")

    def step(i):
        oscar.oscar_quantize_pack(pool, k, v, ids, int2, r_k, tau_k, tau_v)

    if profile_launches:
        for i in range(profile_launches):
            step(i)
        torch.cuda.synchronize()
        log(f"profile run: {profile_launches} bulk quantize launches done")
        return None
    ms, ms_min = time_steps(step, steps, warmup, repeats, use_graph=True)
    nbytes = k.numel() * 2 + v.numel() * 2 + npg * pool.int2_page_bytes
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"bulk quantize ({t} tokens x {wl.num_kv_heads} heads): {ms * 1e3:.2f} us/launch, {gbps:.1f} GB/s")
    del k, v, int2, inp
    torch.cuda.empty_cache()
    return {"workload": wl.name, "tokens": t, "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
            "us_per_launch": round(ms * 1e3, 3), "us_min": round(ms_min * 1e3, 3), "bytes_per_launch": nbytes,
            "GBps": round(gbps, 2), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
            "hbm_traffic_bytes": traffic_for(wl.name, BULK_SOURCES),
            "kernel": "k_quantize_pack (bf16-MFMA key rotation + clip + quantize + pack)"}


FP32_MFMA_PEAK_TFLOPS = 157.3


def bench_calibration(oscar, steps=10, warmup=2, repeats=5, profile_launches=0):
    """Offline calibration of one layer at the Qwen3-8B shape (8 KV heads x 4
    query heads, D = 128) from the seeded 2048-token calibration draw:
    oscar_calibrate (query covariance, causal calibration attention, score-
    weighted value covariance, two Jacobi eigenbases + Hadamard mixes, two
    clip quantiles), then the rotation error chain (quantize, dequantize,
    reference-vs-quantized attention) for the calibrated rotation, the
    Hadamard transform alone and no rotation."""
    import torch
    from synthetic import CONFIGS, draw_calibration
    wl = CONFIGS["qwen3-8b-l100k"]
    hkv, g, d = wl.num_kv_heads, wl.gqa, wl.head_dim
    draws = draw_calibration(hkv, g, d, wl.seed)
    n = draws[0].k.shape[0]
    q = torch.from_numpy(np.stack([x.q for x in draws])).cuda()
    k = torch.from_numpy(np.stack([x.k for x in draws])).cuda()
    v = torch.from_numpy(np.stack([x.v for x in draws])).cuda()
    ws = oscar._ws(oscar._size_out("oscar_calib_workspace_bytes", hkv, g, n, d), "cuda")
    res = oscar.oscar_calibrate(q, k, v, workspace=ws)
    attn_out = torch.empty(hkv, g, n, d, dtype=torch.float32, device="cuda")
    if profile_launches:
        for _ in range(profile_launches):
            oscar.oscar_calibrate(q, k, v, workspace=ws)
        torch.cuda.synchronize()
        log(f"profile run: {profile_launches} calibrations done")
        return None
    ms_cal, _ = time_steps(lambda i: oscar.oscar_calibrate(q, k, v, workspace=ws), steps, warmup, repeats)
    ms_attn, _ = time_steps(lambda i: oscar.oscar_calib_attention(q, k, v, attn_out), steps, warmup, repeats)
    flops = hkv * g * 4 * d * n * (n + 1) // 2  # Q K^T and P V over the causal pairs
    tflops = flops / (ms_attn * 1e-3) / 1e12
    log(f"calibration: {ms_cal * 1e3:.1f} us per layer; causal attention {ms_attn * 1e3:.1f} us "
        f"({tflops:.1f} TFLOP/s fp32)")

    # rotation error chain
    eye = torch.eye(d, dtype=torch.float32, device="cuda").expand(hkv, d, d).contiguous()
    had = torch.empty_like(eye)
    oscar.oscar_calib_rotation(eye, had, mix=True)  # identity covariance: U = I, R = H P_br
    tau_h = {x: torch.empty(hkv, dtype=torch.float32, device="cuda") for x in "kv"}
    oscar.oscar_calib_clip(k, had, 0.995, tau_h["k"])
    oscar.oscar_calib_clip(v, had, 0.995, tau_h["v"])
    inf = torch.full((hkv,), float("inf"), dtype=torch.float32, device="cuda")
    variants = {"oscar": (res["r_k"], res["r_v"], res["tau_k"], res["tau_v"]),
                "oscar_lloyd_max": (res["r_k"], res["r_v"], res["tau_k"], res["tau_v"]),
                "hadamard_only": (had, had, tau_h["k"], tau_h["v"]),
                "none": (eye, eye, inf, inf)}
    pool = oscar.OscarPool(oscar.PoolConfig(wl.num_q_heads, hkv, d, wl.group_size, 16, wl.sink, wl.recent, 0, 0.0))
    # the layer's codebooks, fitted on the same draw with the calibrated
    # rotations and thresholds
    lv_k = oscar.oscar_calib_codebook(k, res["r_k"], res["tau_k"], wl.group_size).cpu().numpy()
    lv_v = oscar.oscar_calib_codebook(v, res["r_v"], res["tau_v"], wl.group_size).cpu().numpy()
    lm_pool = oscar.OscarPool(oscar.PoolConfig(wl.num_q_heads, hkv, d, wl.group_size, 16, wl.sink, wl.recent, 0, 0.0,
                                               1, tuple(map(float, lv_k)), tuple(map(float, lv_v))))
    npg = (n + 15) // 16
    ids = torch.arange(npg, dtype=torch.int32, device="cuda")
    int2 = torch.zeros(npg, pool.int2_page_bytes, dtype=torch.uint8, device="cuda")
    k_tok = k.transpose(0, 1).to(torch.bfloat16).contiguous()  # the cache's bf16 content, [N, Hkv, D]
    v_tok = v.transpose(0, 1).to(torch.bfloat16).contiguous()
    k_ref, v_ref = k_tok.float().transpose(0, 1), v_tok.float().transpose(0, 1)
    kh = torch.empty(n, hkv, d, dtype=torch.float32, device="cuda")
    vh = torch.empty_like(kh)
    stats = torch.empty(hkv, g, n, 4, dtype=torch.float32, device="cuda")
    pairs = hkv * g * n * (n + 1) / 2
    chain = {}
    for name, (rk, rv, tk, tv) in variants.items():
        pl = lm_pool if name == "oscar_lloyd_max" else pool

        def run(i, rk=rk, rv=rv, tk=tk, tv=tv, pl=pl):
            oscar.oscar_quantize_pack(pl, k_tok, v_tok, ids, int2, rk, tk, tv, r_v=rv)
            oscar.oscar_dequantize(pl, n, ids, int2, rk, rv, kh, vh)
            oscar.oscar_attention_error(q, k_ref, v_ref, kh.transpose(0, 1), vh.transpose(0, 1), stats)
        run(0)
        torch.cuda.synchronize()
        st = stats.double()
        chain[name] = {"logit_mse": round(float(st[..., 1].sum() / pairs), 5),
                       "score_kl": round(float(st[..., 0].mean()), 5),
                       "out_rel_mse": round(float(st[..., 2].sum() / st[..., 3].sum()), 5)}
        if name == "oscar":
            ms_chain, _ = time_steps(run, steps, warmup, repeats)
    log(f"error chain: {chain}")
    del ws, attn_out, int2
    torch.cuda.empty_cache()
    return {"workload": f"calibration of one layer: {hkv} KV heads x {g} query heads, D={d}, {n}-token draw",
            "us_per_calibration": round(ms_cal * 1e3, 1),
            "calib_attention": {"us_per_launch": round(ms_attn * 1e3, 1), "flops_per_launch": flops,
                                "TFLOPs": round(tflops, 2), "pct_fp32_mfma_peak": round(100 * tflops /
                                                                                      FP32_MFMA_PEAK_TFLOPS, 2),
                                "kernel": "k_calib_attention (fp32 MFMA causal attention)"},
            "error_chain": chain, "us_per_error_chain": round(ms_chain * 1e3, 1),
            "codebooks": {"levels_k": [float(x) for x in lv_k], "levels_v": [float(x) for x in lv_v]},
            "error_chain_note": "quantize_pack -> dequantize -> attention_error on the calibration draw itself; "
                                "logit_mse per causal pair, score_kl per query row, out_rel_mse = "
                                "sum ||o - o^||^2 / sum ||o||^2"}


# the profiling build's stamp area (kStampSlots, kStampWaves, kStampWgs in
# the library's kernels.h): slots per wave, waves per workgroup, workgroups
STAMP_SLOTS, STAMP_WAVES, STAMP_WGS = 16, 8, 2048
PHASES = ["start", "first tiles requested", "q' partials ready", "q' split barrier", "first score MFMAs issued",
          "loop end", "wave merge barrier", "partial stores acknowledged", "ticket taken", "fold written", None,
          "q' FMAs done (R_K arrived)", "q' split written", "wave epilogue written to LDS",
          "ticket returned (wave 0)", "acquire done (wave 0)"]


def int2_workgroup_phases(st, rel, wg_used):
    """Medians over the INT2 workgroups of a stamped step, each on its own
    clock (the workgroups of a plan with several rounds start at different
    times): first tile request, first score MFMA, loop end and ticket, in us
    after the workgroup's start, and the share of the workgroup's life spent
    before its first score MFMA and after its loop."""
    import warnings
    import numpy as np
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)  # rows of unused workgroups are all NaN

        def pt(k):
            return np.where(st[:, :, k] > 0, rel[:, :, k], np.nan)
        wstart = np.nanmin(pt(0), axis=1)
        int2 = wg_used & np.isfinite(pt(4)).any(axis=1)

        def med(k, reduce):
            v = reduce(pt(k), axis=1) - wstart
            return round(float(np.nanmedian(v[int2])), 2)
        mfma, lend, tick = med(4, np.nanmedian), med(5, np.nanmax), med(8, np.nanmax)
        return {"workgroups": int(int2.sum()), "first_request": med(1, np.nanmedian), "first_score_mfma": mfma,
                "loop_end": lend, "ticket": tick, "fixed_share": round((mfma + tick - lend) / tick, 3)}


def phase_timeline(steps, warmup, workload="qwen3-8b-l100k"):
    """Per-wave phase times of one cold decode step (plain decode, host-length
    plan) from the profiling build (s_memrealtime at fixed points of
    k_decode, 100 MHz), relative to the earliest workgroup start of the
    step."""
    import numpy as np
    import torch
    import long_context_decode_oscar_amd as oscar
    from long_context_decode_oscar_amd import build as obuild
    from synthetic import CONFIGS, draw_inputs
    if not os.path.exists(obuild.STAMPS_LIB):
        raise SystemExit("the profiling build is missing: python -m long_context_decode_oscar_amd.build --phase-stamps")
    oscar.load(obuild.STAMPS_LIB)
    wl = CONFIGS[workload]
    kv = wl.kv_bytes()
    inp = draw_inputs(wl, gpu_calibration(oscar, wl), device="cuda")
    pool = oscar.OscarPool(oscar.PoolConfig(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.group_size, 16,
                                            wl.sink, wl.recent, 1, 0.0))
    n_copies = max(1, math.ceil(2 * 2**30 / kv["total"]))
    copies, r_k = build_pools(oscar, pool, wl, inp, n_copies, seed=wl.seed)
    q = inp.q.contiguous()
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = pool.alloc_workspace(wl.batch, max(wl.seq_lens))  # includes the stamp area in this build
    slots, waves, wgs = STAMP_SLOTS, STAMP_WAVES, STAMP_WGS
    nbytes = wgs * waves * slots * 8
    off = (ws.numel() - nbytes) // 256 * 256  # where the library puts the stamp area
    area = ws[off:off + nbytes]
    area.zero_()
    dec = Decoder(oscar, pool, wl, q, lens, copies, r_k, out, ws)
    ms, _ = time_steps(dec, steps, warmup, 1, use_graph=True)
    st = area.view(torch.int64).cpu().numpy().reshape(wgs, waves, slots).astype(np.float64)
    used = st[:, :, 0] > 0
    t0 = st[:, :, 0][used].min()
    rel = (st - t0) * 1e-2  # 100 MHz ticks -> us
    rows = []
    for k, name in enumerate(PHASES):
        if name is None:
            continue
        v = rel[:, :, k][st[:, :, k] > 0]
        if len(v):
            rows.append({"point": k, "phase": name, "n": int(len(v)), "min": round(float(v.min()), 2),
                         "median": round(float(np.median(v)), 2), "p90": round(float(np.percentile(v, 90)), 2),
                         "max": round(float(v.max()), 2)})
    folded = st[:, 0, 10] > 0
    wg_used = used.any(axis=1)
    loop_end = np.where(st[:, :, 5] > 0, rel[:, :, 5], np.nan)
    per_wg = {"wgs": int(wg_used.sum()), "wg_duration_us": None}
    starts = np.where(st[:, :, 0] > 0, rel[:, :, 0], np.nan)
    ends = np.where(st[:, :, 8] > 0, rel[:, :, 8], np.nan)
    dur_wg = np.nanmax(ends[wg_used], axis=1) - np.nanmin(starts[wg_used], axis=1)
    per_wg["wg_duration_us"] = {"min": round(float(np.nanmin(dur_wg)), 2), "median": round(float(np.nanmedian(dur_wg)), 2),
                                "max": round(float(np.nanmax(dur_wg)), 2)}
    per_wg["int2_workgroup_us"] = int2_workgroup_phases(st, rel, wg_used)
    res = {"workload": wl.name, "steps": steps, "step_us": round(ms * 1e3, 3), "phases": rows, "workgroups": per_wg,
           "fold_end_per_head_us": sorted(round(float(x), 2) for x in rel[folded, 0, 9]),
           "wg_loop_end_us": {"min": round(float(np.nanmin(np.nanmax(loop_end[wg_used], axis=1))), 2),
                              "median": round(float(np.nanmedian(np.nanmax(loop_end[wg_used], axis=1))), 2),
                              "max": round(float(np.nanmax(loop_end[wg_used])), 2)},
           "wave_loop_end_spread_in_wg_us": round(float(np.nanmedian(
               np.nanmax(loop_end[wg_used], axis=1) - np.nanmin(loop_end[wg_used], axis=1))), 2)}
    # the last workgroup of each head: its latest wave at every point
    fold_pts = {}
    for k in (0, 1, 4, 5, 13, 6, 7, 14, 15, 8, 9):
        v = np.where(st[folded, :, k] > 0, rel[folded, :, k], np.nan)
        if np.isfinite(v).any():
            fold_pts[k] = round(float(np.nanmedian(np.nanmax(v, axis=1))), 2)
    res["fold_wg_points_us"] = fold_pts
    log(f"phase timeline of the last of {steps} cold graph steps ({ms * 1e3:.2f} us/step in this build)")
    for r in rows:
        log(f"  {r['point']} {r['phase']:28s} n={r['n']:5d} min {r['min']:6.2f} med {r['median']:6.2f} "
            f"p90 {r['p90']:6.2f} max {r['max']:6.2f}")
    log("  last workgroups (median over heads of the latest wave): " +
        ", ".join(f"{k}: {v:.2f}" for k, v in fold_pts.items()))
    w = per_wg["int2_workgroup_us"]
    log(f"  INT2 workgroups on their own clocks ({w['workgroups']}, medians): first request {w['first_request']:.2f}, "
        f"first score MFMA {w['first_score_mfma']:.2f}, loop end {w['loop_end']:.2f}, ticket {w['ticket']:.2f} us; "
        f"start-to-first-MFMA plus loop-end-to-ticket = {100 * w['fixed_share']:.1f} % of the workgroup's life")
    return res


def copy_probe(nbytes):
    """One plain device copy of known size, for scaling HBM byte counters."""
    import torch
    x = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    # an elementwise kernel (a device memcpy may run on a DMA engine, which
    # carries no per-dispatch counters): reads nbytes, writes nbytes
    torch.bitwise_not(x, out=y)
    torch.cuda.synchronize()
    log(f"copy probe: bitwise_not kernel, {nbytes} bytes read, {nbytes} bytes written")


def main():
    global SETTLE_S
    args = parse()
    SETTLE_S = args.settle_ms * 1e-3
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import long_context_decode_oscar_amd as oscar
    from synthetic import CONFIGS, draw_inputs

    if args.phase_stamps:
        print(json.dumps({"phase_timeline": phase_timeline(args.steps, args.warmup, args.workload)}), flush=True)
        return
    oscar.load()
    if args.only in ("demote", "mixed"):
        name = "qwen3-8b-b32-l32k-demote" if args.only == "demote" else "qwen3-32b-b8-mixed-prefix"
        if args.profile_steps:
            bench_decode_workload(oscar, name, 0, 0, 0, args.cold_bytes, profile_launches=args.profile_steps)
            copy_probe(args.probe_bytes)
            return
        print(json.dumps({args.only: bench_decode_workload(oscar, name, max(10, args.steps // 4), args.warmup,
                                                           args.repeats, args.cold_bytes)}), flush=True)
        return
    if args.only == "batch-bf16":
        print(json.dumps({"batched_decode_vs_bf16": bench_batch_comparator(
            oscar, "qwen3-8b-b32-l32k-demote", max(10, args.steps // 10), 5, 3, args.cold_bytes)}), flush=True)
        return
    if args.only == "calib":
        if args.profile_steps:
            bench_calibration(oscar, profile_launches=args.profile_steps)
            return
        print(json.dumps({"calibration": bench_calibration(oscar)}), flush=True)
        return
    if args.only == "bulk":
        if args.profile_steps:
            bench_bulk_quant(oscar, profile_launches=args.profile_steps)
            copy_probe(args.probe_bytes)
            return
        print(json.dumps({"bulk_quantize": bench_bulk_quant(oscar)}), flush=True)
        return
    wl = CONFIGS[args.workload]
    kv = wl.kv_bytes()
    log(f"workload {wl.name}: KV bytes/step {kv['total']:,} (INT2 {kv['int2']:,}, BF16 {kv['bf16']:,})")
    inp = draw_inputs(wl, gpu_calibration(oscar, wl), device="cuda")
    pool = oscar.OscarPool(oscar.PoolConfig(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.group_size, 16,
                                            wl.sink, wl.recent, 1, 0.0))
    n_copies = max(1, math.ceil(args.cold_bytes / kv["total"]))
    copies, r_k = build_pools(oscar, pool, wl, inp, n_copies, seed=wl.seed)
    log(f"built {n_copies} pool copies ({n_copies * kv['total'] / 2**30:.2f} GiB of KV)")
    q = inp.q.contiguous()
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = pool.alloc_workspace(wl.batch, max(wl.seq_lens))
    dec = Decoder(oscar, pool, wl, q, lens, copies, r_k, out, ws)
    if args.profile_steps:
        for i in range(args.profile_steps):
            dec(i)
        torch.cuda.synchronize()
        log(f"profile run: {args.profile_steps} decode steps done")
        copy_probe(args.probe_bytes)
        return

    ms, ms_min = time_steps(dec, args.steps, args.warmup, args.repeats, use_graph=True)
    log(f"INT2 decode (graph, cold): {ms * 1e3:.2f} us/step (min {ms_min * 1e3:.2f})")
    ms_eager, _ = time_steps(dec, args.steps, args.warmup, 3, use_graph=False)
    log(f"INT2 decode (eager, cold): {ms_eager * 1e3:.2f} us/step")
    warm = Decoder(oscar, pool, wl, q, lens, copies[:1], r_k, out, ws)
    ms_warm, _ = time_steps(warm, args.steps, args.warmup, 3, use_graph=True)
    log(f"INT2 decode (graph, warm single copy): {ms_warm * 1e3:.2f} us/step")
    del warm, dec, copies
    torch.cuda.empty_cache()
    # the same protocol with a private page table per copy (page-table reads cold too)
    pcopies, _ = build_pools(oscar, pool, wl, inp, n_copies, seed=wl.seed + 2, shared_tables=False)
    pdec = Decoder(oscar, pool, wl, q, lens, pcopies, r_k, out, ws)
    ms_priv, _ = time_steps(pdec, args.steps, args.warmup, 3, use_graph=True)
    log(f"INT2 decode (graph, cold, private page table per copy): {ms_priv * 1e3:.2f} us/step")
    # ... and a rotation matrix of its own per copy too, as each layer of a
    # model has its own R_K (the pools hold the same codes; only where R_K
    # sits in memory differs)
    rk_copies = [r_k.clone() for _ in pcopies]
    rdec = Decoder(oscar, pool, wl, q, lens, pcopies, rk_copies, out, ws)
    ms_prk, _ = time_steps(rdec, args.steps, args.warmup, 3, use_graph=True)
    log(f"INT2 decode (graph, cold, private page table and R_K per copy): {ms_prk * 1e3:.2f} us/step")
    del pdec, rdec, pcopies, rk_copies
    torch.cuda.empty_cache()

    gbps = kv["total"] / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int2-kv/int8+bf16-mfma/fp32-acc", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "group_size": wl.group_size, "context": list(wl.seq_lens)[:4],
                   "sink": wl.sink, "recent": wl.recent, "page_size": 16, "pool_copies": n_copies,
                   "timing": "HIP-graph replay of the timed steps, cold cache: rotating over per-layer pool "
                             "copies that share the sequence's page tables; the same replay runs untimed, back "
                             f"to back, for {args.settle_ms:g} ms before the timed replays"},
        "tokens_per_s": round(wl.batch / (ms * 1e-3), 1),
        "kv_tokens_scanned_per_s": round(sum(wl.seq_lens) / (ms * 1e-3), 1),
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "kv_bytes_per_step": kv["total"],
        "eager_ms_per_step": round(ms_eager, 6),
        "warm_ms_per_step": round(ms_warm, 6),
        "private_tables_ms_per_step": round(ms_priv, 6),
        "private_tables_and_rk_ms_per_step": round(ms_prk, 6),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic_for(wl.name),
                     "kernel": "k_decode (INT2 split-K + BF16 sink/recent + LSE merge, one launch per step)"},
    }
    if not args.no_codebook:
        # the same step over pools written with the layer's Lloyd-Max codebook
        levels = gpu_codebook(oscar, wl)
        lpool = oscar.OscarPool(oscar.PoolConfig(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.group_size, 16,
                                                 wl.sink, wl.recent, 1, 0.0, 1, levels[0], levels[1]))
        lcopies, _ = build_pools(oscar, lpool, wl, inp, n_copies, seed=wl.seed + 3)
        ldec = Decoder(oscar, lpool, wl, q, lens, lcopies, r_k, out, ws)
        ms_lm, ms_lm_min = time_steps(ldec, args.steps, args.warmup, args.repeats, use_graph=True)
        log(f"INT2 decode with the codebook (graph, cold): {ms_lm * 1e3:.2f} us/step, levels {levels}")
        result["codebook_variant"] = {"levels_k": levels[0], "levels_v": levels[1],
                                      "ms_per_step": round(ms_lm, 6), "ms_min": round(ms_lm_min, 6),
                                      "GBps": round(kv["total"] / (ms_lm * 1e-3) / 1e9, 2),
                                      "slowdown_vs_uniform": round(ms_lm / ms, 3)}
        del ldec, lcopies
        torch.cuda.empty_cache()
    if not args.no_bf16:
        n16 = max(1, math.ceil(args.cold_bytes / kv["bf16_only_total"]))
        bcopies, _ = build_pools(oscar, pool, wl, inp, n16, bf16_only=True, seed=wl.seed + 1)
        bws = pool.alloc_workspace(wl.batch, max(wl.seq_lens), bf16_only=True)
        bdec = Decoder(oscar, pool, wl, q, lens, bcopies, r_k, out, bws, bf16_only=True)
        ms16, _ = time_steps(bdec, max(20, args.steps // 4), args.warmup, args.repeats, use_graph=True)
        log(f"BF16-only decode (graph, cold): {ms16 * 1e3:.2f} us/step")
        result["bf16_comparator"] = {"ms_per_step": round(ms16, 6),
                                     "kv_GBps": round(kv["bf16_only_total"] / (ms16 * 1e-3) / 1e9, 2),
                                     "kv_bytes_per_step": kv["bf16_only_total"], "pool_copies": n16,
                                     "int2_speedup": round(ms16 / ms, 3)}
        del bcopies
        torch.cuda.empty_cache()
    if args.only == "all":
        # the other workloads, measured the same way (not the headline)
        result["other_workloads"] = {
            "batched_demote": bench_decode_workload(oscar, "qwen3-8b-b32-l32k-demote", max(10, args.steps // 4),
                                                    args.warmup, args.repeats, args.cold_bytes),
            "batched_decode_vs_bf16": bench_batch_comparator(oscar, "qwen3-8b-b32-l32k-demote",
                                                             max(10, args.steps // 10), 5, 3, args.cold_bytes),
            "mixed_prefix_gqa8": bench_decode_workload(oscar, "qwen3-32b-b8-mixed-prefix", max(10, args.steps // 4),
                                                       args.warmup, args.repeats, args.cold_bytes),
            "bulk_quantize": bench_bulk_quant(oscar),
            "calibration": bench_calibration(oscar),
        }
    result["copy_ceiling_GBps"] = round(copy_ceiling_gbps(), 1)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, repeats=7)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
