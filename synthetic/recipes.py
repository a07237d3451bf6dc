"""Workload shapes, offline calibration parameters and seeded tensor draws.

Distributions (one recipe for every workload):
  * keys   ~ N(0, 1) in the model basis, with 4 seeded outlier channels per KV
             head scaled by 20 (the channel-wise outliers the MarkTechPost
             article, "Why INT2 KV Cache Quantization is Hard", describes);
  * queries ~ N(0, Sigma_Q), Sigma_Q = U diag(lambda) U^T with a seeded Haar U
             per KV head (shared by its query heads) and lambda_i ~ i^-1.5
             normalised to trace D;
  * values ~ N(0, 1), stored in the pool already multiplied by R_V (the pages
             fold R_V into the projection weights offline, MarkTechPost
             article, "The Serving System"), then rounded to bf16.

Calibration activations (per KV head, a separate 2048-token draw, rounded to
fp32): the group's queries, keys with the same outlier recipe, values in the
model basis.  This module draws them; the offline parameters computed from
them (R_K, R_V, tau_K, tau_V) come from the library's calibration kernels in
the benchmark and from the oracle in the tests, and are passed back in through
``make_calibration``.

Row-vector convention throughout: a rotated vector is x' = x R with R stored
row-major as [D_in][D_out].

Random streams: numpy PCG64(seed) for the calibration draw (per KV head in
head order: Haar basis, outlier channels, calibration queries, keys, values), and a
torch generator seeded with ``seed * 1000 + 7`` on the requested device for the
bulk tensors (keys, values, queries, new tokens, in that order).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

PAGE_SIZE = 16
SINK_TOKENS = 64
RECENT_TOKENS = 256
CALIB_TOKENS = 2048
OUTLIER_CHANNELS = 4
OUTLIER_SCALE = 20.0
EIG_POWER = 1.5
CLIP_QUANTILE = 0.995


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one decode (or bulk-quantize) workload."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    group_size: int
    seq_lens: tuple  # L per sequence, counting the token appended this step
    seed: int
    page_size: int = PAGE_SIZE
    sink: int = SINK_TOKENS
    recent: int = RECENT_TOKENS
    demote: bool = False  # the step includes one append+demote per sequence
    shared_prefix_tokens: int = 0  # tokens shared through common pages
    shared_prefix_seqs: int = 0  # sequences 0..n-1 share the prefix
    int2_arena_bytes: int = 0  # size of the INT2 page arena (0: just enough)
    bulk_tokens: int = 0  # >0: a bulk rotate-clip-quantize-pack workload

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def n_groups(self) -> int:
        return self.head_dim // self.group_size

    def hist_len(self, L: int) -> int:
        """History tokens of a sequence of length L: [S0, max(S0, L - W))."""
        return max(0, max(self.sink, L - self.recent) - self.sink)

    def recent_start(self, L: int) -> int:
        return max(self.sink, L - self.recent)

    def int2_bytes_per_token_head(self) -> int:
        # K and V codes (2 bits each) + bf16 scale and zero per group for K and V
        return 2 * self.head_dim // 4 + 2 * self.n_groups * 2 * 2

    def bf16_bytes_per_token_head(self) -> int:
        return 2 * self.head_dim * 2

    def kv_bytes(self) -> dict:
        """Algorithmic KV bytes one decode step reads, counted per sequence."""
        int2 = sum(self.hist_len(L) for L in self.seq_lens) * self.num_kv_heads * \
            self.int2_bytes_per_token_head()
        bf16 = sum(min(L, self.sink) + (L - self.recent_start(L)) for L in self.seq_lens) * \
            self.num_kv_heads * self.bf16_bytes_per_token_head()
        full = sum(self.seq_lens) * self.num_kv_heads * self.bf16_bytes_per_token_head()
        return {"int2": int2, "bf16": bf16, "total": int2 + bf16, "bf16_only_total": full}


def _mixed_lengths(seed: int) -> tuple:
    """Lengths of the Qwen3-32B-shaped mixed batch: 4 sequences sharing a
    65,536-token prefix draw L ~ U[65536 + 257, 131072]; the other 4 draw
    L ~ U[16384, 131072] (integers, inclusive)."""
    rng = np.random.Generator(np.random.PCG64(seed + 100))
    shared = rng.integers(65536 + RECENT_TOKENS + 1, 131072, size=4, endpoint=True)
    other = rng.integers(16384, 131072, size=4, endpoint=True)
    return tuple(int(x) for x in np.concatenate([shared, other]))


CONFIGS = {
    "tiny-d64-l512": Workload(
        name="tiny-d64-l512", batch=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
        group_size=64, seq_lens=(512,), seed=0),
    "qwen3-8b-l100k": Workload(
        name="qwen3-8b-l100k", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
        group_size=128, seq_lens=(100_000,), seed=1),
    "qwen3-8b-b32-l32k-demote": Workload(
        name="qwen3-8b-b32-l32k-demote", batch=32, num_q_heads=32, num_kv_heads=8,
        head_dim=128, group_size=128, seq_lens=(32_768,) * 32, seed=2, demote=True,
        int2_arena_bytes=40 * 2**30),
    "bulk-quant-t131k": Workload(
        name="bulk-quant-t131k", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
        group_size=128, seq_lens=(131_072,), seed=3, bulk_tokens=131_072),
    "qwen3-32b-b8-mixed-prefix": Workload(
        name="qwen3-32b-b8-mixed-prefix", batch=8, num_q_heads=64, num_kv_heads=8,
        head_dim=128, group_size=128, seq_lens=_mixed_lengths(4), seed=4,
        shared_prefix_tokens=65_536, shared_prefix_seqs=4),
}


def make_workload(base: Workload, **changes) -> Workload:
    return dataclasses.replace(base, **changes)


# --------------------------------------------------------------------------
# offline calibration (produces the hot path's fixed inputs)
# --------------------------------------------------------------------------

def _haar(rng: np.random.Generator, d: int) -> np.ndarray:
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))


def query_eigenvalues(d: int) -> np.ndarray:
    lam = np.arange(1, d + 1, dtype=np.float64) ** (-EIG_POWER)
    return lam * (d / lam.sum())


@dataclasses.dataclass
class CalibrationDraw:
    """Seeded calibration activations of one KV head's group (fp32 values)."""
    q: np.ndarray  # [gqa, n, d] queries of the group's query heads
    k: np.ndarray  # [n, d] keys (with the outlier channels)
    v: np.ndarray  # [n, d] values (model basis)
    u: np.ndarray  # [d, d] fp64 Haar basis of Sigma_Q
    outliers: np.ndarray  # [4] outlier channels of k


def draw_calibration(num_kv_heads: int, gqa: int, head_dim: int, seed: int,
                     n_cal: int = CALIB_TOKENS) -> list:
    """Calibration activations per KV head (random draws only)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    d = head_dim
    lam = query_eigenvalues(d)
    draws = []
    for _ in range(num_kv_heads):
        u = _haar(rng, d)
        outl = np.sort(rng.choice(d, OUTLIER_CHANNELS, replace=False))
        z = rng.standard_normal((gqa, n_cal, d))
        q_cal = (z * np.sqrt(lam)) @ u.T
        k_cal = rng.standard_normal((n_cal, d))
        k_cal[:, outl] *= OUTLIER_SCALE
        v_cal = rng.standard_normal((n_cal, d))
        draws.append(CalibrationDraw(q=q_cal.astype(np.float32), k=k_cal.astype(np.float32),
                                     v=v_cal.astype(np.float32), u=u, outliers=outl))
    return draws


@dataclasses.dataclass
class Calibration:
    """Offline parameters of the hot path (computed elsewhere: by the oracle
    in tests, by the library's calibration kernels in the benchmark) plus the
    draw parameters the bulk tensors are generated from."""
    r_k: np.ndarray  # [Hkv, D, D] float32
    r_v: np.ndarray  # [Hkv, D, D] float32
    tau_k: np.ndarray  # [Hkv] float32
    tau_v: np.ndarray  # [Hkv] float32
    q_basis: np.ndarray  # [Hkv, D, D] float64, the Haar U of Sigma_Q
    q_eigs: np.ndarray  # [D] float64
    outliers: np.ndarray  # [Hkv, 4] int64


def make_calibration(draws: list, r_k, r_v, tau_k, tau_v) -> Calibration:
    """Bundle offline parameters with the draws' basis and outlier channels."""
    return Calibration(
        r_k=np.ascontiguousarray(r_k, dtype=np.float32), r_v=np.ascontiguousarray(r_v, dtype=np.float32),
        tau_k=np.asarray(tau_k, dtype=np.float32).reshape(-1),
        tau_v=np.asarray(tau_v, dtype=np.float32).reshape(-1),
        q_basis=np.stack([d.u for d in draws]), q_eigs=query_eigenvalues(draws[0].u.shape[0]),
        outliers=np.stack([d.outliers for d in draws]))


# --------------------------------------------------------------------------
# bulk tensors and page tables
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Inputs:
    """Per-sequence dense caches (bf16 values held as torch bfloat16 tensors).

    k[b], v[b]: [L_b, Hkv, D]; k is in the model basis, v in the rotated V
    basis the pool stores.  The last position of each sequence is the token
    appended by this step.  q: [B, Hq, D] (model basis).
    """

    workload: Workload
    calib: Calibration
    k: list
    v: list
    q: object


def draw_inputs(wl: Workload, calib: Calibration, device="cpu", with_q: bool = True) -> Inputs:
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed * 1000 + 7)
    d, hkv = wl.head_dim, wl.num_kv_heads
    outl = torch.as_tensor(calib.outliers, device=device)
    r_v = torch.as_tensor(calib.r_v, device=device)
    scale = torch.ones(hkv, d, device=device)
    scale[torch.arange(hkv, device=device)[:, None], outl] = OUTLIER_SCALE

    def draw_kv(n: int):
        k = torch.randn(n, hkv, d, generator=gen, device=device) * scale
        v = torch.randn(n, hkv, d, generator=gen, device=device)
        v = torch.einsum("nhd,hde->nhe", v, r_v)
        return k.to(torch.bfloat16), v.to(torch.bfloat16)

    ks, vs = [], []
    prefix = None
    for b, L in enumerate(wl.seq_lens):
        if wl.shared_prefix_seqs and b < wl.shared_prefix_seqs:
            if prefix is None:
                prefix = draw_kv(wl.shared_prefix_tokens)
            k_tail, v_tail = draw_kv(L - wl.shared_prefix_tokens)
            ks.append(torch.cat([prefix[0], k_tail]))
            vs.append(torch.cat([prefix[1], v_tail]))
        else:
            k, v = draw_kv(L)
            ks.append(k)
            vs.append(v)
    q = None
    if with_q:
        lam = torch.as_tensor(np.sqrt(calib.q_eigs), dtype=torch.float32, device=device)
        u = torch.as_tensor(calib.q_basis, dtype=torch.float32, device=device)
        z = torch.randn(wl.batch, wl.num_q_heads, d, generator=gen, device=device) * lam
        kv_of_head = torch.arange(wl.num_q_heads, device=device) // wl.gqa
        q = torch.einsum("bhd,hed->bhe", z, u[kv_of_head]).to(torch.bfloat16).contiguous()
    return Inputs(workload=wl, calib=calib, k=ks, v=vs, q=q)


def random_page_table(n_pages: Sequence[int], n_physical: int, seed: int,
                      shared: Optional[tuple] = None) -> np.ndarray:
    """Page table [B, max_pages] of distinct random physical page ids (-1 pad).

    ``shared=(n_seqs, n_pages_shared)``: sequences 0..n_seqs-1 map their first
    n_pages_shared logical pages to the same physical pages.
    """
    rng = np.random.Generator(np.random.PCG64(seed + 200))
    n_pages = [int(x) for x in n_pages]
    need = sum(n_pages)
    if shared:
        need -= (shared[0] - 1) * shared[1]
    assert need <= n_physical, (need, n_physical)
    phys = rng.choice(n_physical, size=need, replace=False) if n_physical > 4 * need \
        else rng.permutation(n_physical)[:need]
    table = np.full((len(n_pages), max(n_pages + [1])), -1, dtype=np.int32)
    pos = 0
    common = None
    for b, n in enumerate(n_pages):
        if shared and b < shared[0]:
            if common is None:
                common = phys[pos:pos + shared[1]]
                pos += shared[1]
            table[b, :shared[1]] = common
            rest = n - shared[1]
            table[b, shared[1]:n] = phys[pos:pos + rest]
            pos += rest
        else:
            table[b, :n] = phys[pos:pos + n]
            pos += n
    return table
