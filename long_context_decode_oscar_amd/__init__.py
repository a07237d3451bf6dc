"""Python binding of liboscar, the OSCAR INT2 KV-cache decode library for
AMD MI355X (gfx950).

The binding only marshals arguments: it checks dtypes, shapes and devices of
torch tensors, passes their device pointers and the current HIP stream to the
C ABI (include/oscar.h), and raises on a non-OK status.  Every step of the
hot path runs in the library's HIP kernels.  The shared library must have
been built (``python -m long_context_decode_oscar_amd.build``); nothing falls
back to another implementation.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboscar.so")

OSCAR_OK, OSCAR_ERR_INVALID, OSCAR_ERR_UNSUPPORTED, OSCAR_ERR_WORKSPACE, OSCAR_ERR_HIP = range(5)

EXPORTED = (
    "oscar_pool_create", "oscar_pool_destroy", "oscar_decode_workspace_bytes", "oscar_append_demote",
    "oscar_decode_attention", "oscar_merge", "oscar_quantize_pack", "oscar_bf16_decode_attention",
    "oscar_write_bf16", "oscar_status_string", "oscar_last_error",
    "oscar_calib_gram_workspace_bytes", "oscar_calib_gram", "oscar_calib_attention", "oscar_calib_rotation",
    "oscar_calib_clip_workspace_bytes", "oscar_calib_clip", "oscar_calib_workspace_bytes", "oscar_calibrate",
    "oscar_dequantize", "oscar_attention_error",
    "oscar_decode_cascade_workspace_bytes", "oscar_decode_attention_cascade",
    "oscar_calib_codebook_workspace_bytes", "oscar_calib_codebook", "oscar_decode_attention_noalloc",
)


class OscarError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        self.status = status
        super().__init__(f"{func}: status {status} ({msg})")


class CConfig(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("group_size", ctypes.c_int32), ("page_size", ctypes.c_int32), ("sink_tokens", ctypes.c_int32),
        ("recent_tokens", ctypes.c_int32), ("v_absorbed", ctypes.c_int32), ("sm_scale", ctypes.c_float),
        ("codebook", ctypes.c_int32), ("levels_k", ctypes.c_float * 4), ("levels_v", ctypes.c_float * 4),
    ]


class CPrefixGroup(ctypes.Structure):
    _fields_ = [("first_seq", ctypes.c_int32), ("num_seqs", ctypes.c_int32), ("shared_pages", ctypes.c_int32)]


class CLayout(ctypes.Structure):
    _fields_ = [
        ("int2_page_bytes", ctypes.c_size_t), ("bf16_page_bytes", ctypes.c_size_t),
        ("int2_head_block_bytes", ctypes.c_size_t), ("bf16_head_block_bytes", ctypes.c_size_t),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Load liboscar.so and declare the C prototypes.  Raises if missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"liboscar.so not built at {path}; run python -m long_context_decode_oscar_amd.build")
    # torch first: the library then binds to the HIP runtime torch already
    # loaded, so torch's streams and device memory are valid in its calls
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I, S, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    lib.oscar_pool_create.argtypes = [ctypes.POINTER(CConfig), ctypes.POINTER(P), ctypes.POINTER(CLayout)]
    lib.oscar_pool_destroy.argtypes = [P]
    lib.oscar_pool_destroy.restype = None
    lib.oscar_decode_workspace_bytes.argtypes = [P, I, I, I, ctypes.POINTER(S)]
    lib.oscar_append_demote.argtypes = [P, I, P, P, P, P, I, I, P, I, I, P, P, P, P, P, P, P]
    lib.oscar_decode_attention.argtypes = [P, I, I, P, P, P, P, I, I, P, I, I, P, P, P, P, P, P, S, P]
    lib.oscar_decode_attention_noalloc.argtypes = [P, I, I, P, P, P, P, I, I, P, I, I, P, P, P, P, P, P]
    lib.oscar_merge.argtypes = [I, I, P, P, P, P, P]
    lib.oscar_quantize_pack.argtypes = [P, I, P, P, P, I, P, P, P, P, P, P]
    lib.oscar_bf16_decode_attention.argtypes = [P, I, I, P, P, P, I, I, P, P, P, S, P]
    lib.oscar_write_bf16.argtypes = [P, I, I, P, P, P, I, I, P, P]
    L = ctypes.c_int64
    lib.oscar_calib_gram_workspace_bytes.argtypes = [I, I, I, ctypes.POINTER(S)]
    lib.oscar_calib_gram.argtypes = [I, I, I, P, L, L, F, P, P, S, P]
    lib.oscar_calib_attention.argtypes = [I, I, I, I, F, P, P, P, L, L, P, P, P]
    lib.oscar_calib_rotation.argtypes = [I, I, P, I, P, P, P]
    lib.oscar_calib_clip_workspace_bytes.argtypes = [I, I, I, ctypes.POINTER(S)]
    lib.oscar_calib_clip.argtypes = [I, I, I, P, L, L, P, ctypes.c_double, P, P, S, P]
    lib.oscar_calib_workspace_bytes.argtypes = [I, I, I, I, ctypes.POINTER(S)]
    lib.oscar_calibrate.argtypes = [I, I, I, I, F, P, P, P, L, L, ctypes.c_double, P, P, P, P, P, P, P, S, P]
    lib.oscar_dequantize.argtypes = [P, I, P, I, P, P, P, P, P, P]
    lib.oscar_attention_error.argtypes = [I, I, I, I, F, P, P, P, P, P, L, L, P, P]
    lib.oscar_decode_cascade_workspace_bytes.argtypes = [P, I, I, I, P, I, ctypes.POINTER(S)]
    lib.oscar_decode_attention_cascade.argtypes = [P, I, I, P, P, P, P, I, I, P, I, I, P, P, P, P, P, P, I, P, S, P]
    lib.oscar_calib_codebook_workspace_bytes.argtypes = [I, I, I, ctypes.POINTER(S)]
    lib.oscar_calib_codebook.argtypes = [I, I, I, I, P, L, L, P, P, P, P, S, P]
    lib.oscar_status_string.argtypes = [ctypes.c_int]
    lib.oscar_status_string.restype = ctypes.c_char_p
    lib.oscar_last_error.argtypes = []
    lib.oscar_last_error.restype = ctypes.c_char_p
    for name in EXPORTED:
        if name not in ("oscar_pool_destroy", "oscar_status_string", "oscar_last_error"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int, func: str):
    if status != OSCAR_OK:
        lib = load()
        raise OscarError(status, func, lib.oscar_last_error().decode() or lib.oscar_status_string(status).decode())


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t, name, dtype=None, device_needed=True):
    import torch
    if t is None:
        return None
    if device_needed and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


@dataclasses.dataclass(frozen=True)
class PoolConfig:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    group_size: int
    page_size: int = 16
    sink_tokens: int = 64
    recent_tokens: int = 256
    v_absorbed: int = 1
    sm_scale: float = 0.0
    codebook: int = 0
    levels_k: tuple = (0.0, 1.0, 2.0, 3.0)
    levels_v: tuple = (0.0, 1.0, 2.0, 3.0)


class OscarPool:
    """Handle from oscar_pool_create (host-only, immutable configuration)."""

    def __init__(self, cfg: PoolConfig):
        lib = load()
        self.cfg = cfg
        self._c = CConfig(cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.group_size, cfg.page_size,
                          cfg.sink_tokens, cfg.recent_tokens, cfg.v_absorbed, cfg.sm_scale, cfg.codebook,
                          (ctypes.c_float * 4)(*[float(x) for x in cfg.levels_k]),
                          (ctypes.c_float * 4)(*[float(x) for x in cfg.levels_v]))
        h = ctypes.c_void_p()
        lay = CLayout()
        _check(lib.oscar_pool_create(ctypes.byref(self._c), ctypes.byref(h), ctypes.byref(lay)), "oscar_pool_create")
        self.handle = h
        self.int2_page_bytes = lay.int2_page_bytes
        self.bf16_page_bytes = lay.bf16_page_bytes
        self.int2_head_block_bytes = lay.int2_head_block_bytes
        self.bf16_head_block_bytes = lay.bf16_head_block_bytes

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.oscar_pool_destroy(self.handle)
            self.handle = None

    def workspace_bytes(self, batch: int, max_seq_len: int, bf16_only: bool = False) -> int:
        n = ctypes.c_size_t()
        _check(load().oscar_decode_workspace_bytes(self.handle, batch, max_seq_len, int(bf16_only), ctypes.byref(n)),
               "oscar_decode_workspace_bytes")
        return n.value

    def alloc_workspace(self, batch: int, max_seq_len: int, bf16_only: bool = False, device="cuda"):
        import torch
        n = self.workspace_bytes(batch, max_seq_len, bf16_only)
        return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def oscar_pool_create(cfg: PoolConfig) -> OscarPool:
    return OscarPool(cfg)


def _pages(pool_tensor, page_bytes):
    return pool_tensor.numel() // page_bytes


class HostLengths:
    """Host copy of a batch's lengths for the length-aware split-K plan
    (seq_lens_host of the decode calls); keeps the int32 array alive."""

    def __init__(self, lengths):
        vals = [int(x) for x in lengths]
        self.array = (ctypes.c_int32 * max(len(vals), 1))(*vals)
        self.count = len(vals)

    @property
    def ptr(self):
        return ctypes.cast(self.array, ctypes.c_void_p)


def _host_lens(seq_lens_host, batch):
    if seq_lens_host is None:
        return None, None
    h = seq_lens_host if isinstance(seq_lens_host, HostLengths) else HostLengths(seq_lens_host)
    if h.count != batch:
        raise ValueError(f"seq_lens_host holds {h.count} lengths for a batch of {batch}")
    return h, h.ptr


def oscar_append_demote(pool: OscarPool, k_new, v_new, seq_lens, bf16_page_table, int2_page_table, bf16_pool,
                        int2_pool, r_k, tau_k, tau_v, r_v=None, stream=None):
    import torch
    b = k_new.shape[0]
    _check(load().oscar_append_demote(
        pool.handle, b, _ptr(k_new, "k_new", torch.bfloat16), _ptr(v_new, "v_new", torch.bfloat16),
        _ptr(seq_lens, "seq_lens", torch.int32),
        _ptr(bf16_page_table, "bf16_page_table", torch.int32), bf16_page_table.shape[1],
        _pages(bf16_pool, pool.bf16_page_bytes),
        _ptr(int2_page_table, "int2_page_table", torch.int32), int2_page_table.shape[1],
        _pages(int2_pool, pool.int2_page_bytes),
        _ptr(bf16_pool, "bf16_pool", torch.uint8), _ptr(int2_pool, "int2_pool", torch.uint8),
        _ptr(r_k, "r_k", torch.float32), _ptr(r_v, "r_v", torch.float32),
        _ptr(tau_k, "tau_k", torch.float32), _ptr(tau_v, "tau_v", torch.float32), _stream(stream)),
        "oscar_append_demote")


def oscar_decode_attention(pool: OscarPool, q, seq_lens, max_seq_len: int, bf16_page_table, int2_page_table,
                           bf16_pool, int2_pool, r_k, out, workspace, r_v=None, stream=None, seq_lens_host=None):
    """seq_lens_host: the lengths on the host (a sequence of ints or
    HostLengths) for the length-aware split-K plan, or None."""
    import torch
    keep, hptr = _host_lens(seq_lens_host, q.shape[0])
    _check(load().oscar_decode_attention(
        pool.handle, q.shape[0], int(max_seq_len), _ptr(q, "q", torch.bfloat16), _ptr(seq_lens, "seq_lens", torch.int32),
        hptr,
        _ptr(bf16_page_table, "bf16_page_table", torch.int32), bf16_page_table.shape[1],
        _pages(bf16_pool, pool.bf16_page_bytes),
        _ptr(int2_page_table, "int2_page_table", torch.int32), int2_page_table.shape[1],
        _pages(int2_pool, pool.int2_page_bytes),
        _ptr(bf16_pool, "bf16_pool", torch.uint8), _ptr(int2_pool, "int2_pool", torch.uint8),
        _ptr(r_k, "r_k", torch.float32), _ptr(r_v, "r_v", torch.float32), _ptr(out, "out", torch.bfloat16),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream)),
        "oscar_decode_attention")
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20  # OSCAR_NOALLOC_SCRATCH_BYTES


def oscar_decode_attention_noalloc(pool: OscarPool, q, seq_lens, max_seq_len: int, bf16_page_table, int2_page_table,
                                   bf16_pool, int2_pool, r_k, out, r_v=None, stream=None, seq_lens_host=None):
    """oscar_decode_attention without a workspace: the library's own device
    scratch holds the partials (calls that overlap on one GPU race)."""
    import torch
    keep, hptr = _host_lens(seq_lens_host, q.shape[0])
    _check(load().oscar_decode_attention_noalloc(
        pool.handle, q.shape[0], int(max_seq_len), _ptr(q, "q", torch.bfloat16), _ptr(seq_lens, "seq_lens", torch.int32),
        hptr,
        _ptr(bf16_page_table, "bf16_page_table", torch.int32), bf16_page_table.shape[1],
        _pages(bf16_pool, pool.bf16_page_bytes),
        _ptr(int2_page_table, "int2_page_table", torch.int32), int2_page_table.shape[1],
        _pages(int2_pool, pool.int2_page_bytes),
        _ptr(bf16_pool, "bf16_pool", torch.uint8), _ptr(int2_pool, "int2_pool", torch.uint8),
        _ptr(r_k, "r_k", torch.float32), _ptr(r_v, "r_v", torch.float32), _ptr(out, "out", torch.bfloat16),
        _stream(stream)),
        "oscar_decode_attention_noalloc")
    return out


def _groups(groups):
    """[(first_seq, num_seqs, shared_pages), ...] -> (ctypes array or None, count)."""
    groups = list(groups or [])
    if not groups:
        return None, 0
    arr = (CPrefixGroup * len(groups))(*[CPrefixGroup(int(a), int(b), int(c)) for a, b, c in groups])
    return arr, len(groups)


def cascade_workspace_bytes(pool: OscarPool, batch: int, max_seq_len: int, int2_pt_stride: int, groups) -> int:
    arr, ng = _groups(groups)
    n = ctypes.c_size_t()
    _check(load().oscar_decode_cascade_workspace_bytes(pool.handle, batch, max_seq_len, int2_pt_stride,
                                                       ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None,
                                                       ng, ctypes.byref(n)), "oscar_decode_cascade_workspace_bytes")
    return n.value


def oscar_decode_attention_cascade(pool: OscarPool, q, seq_lens, max_seq_len: int, bf16_page_table,
                                   int2_page_table, bf16_pool, int2_pool, r_k, out, workspace, groups, r_v=None,
                                   stream=None, seq_lens_host=None):
    """Decode with prefix groups [(first_seq, num_seqs, shared_pages), ...]
    whose INT2 page tables share their first shared_pages history pages."""
    import torch
    arr, ng = _groups(groups)
    keep, hptr = _host_lens(seq_lens_host, q.shape[0])
    _check(load().oscar_decode_attention_cascade(
        pool.handle, q.shape[0], int(max_seq_len), _ptr(q, "q", torch.bfloat16), _ptr(seq_lens, "seq_lens", torch.int32),
        hptr,
        _ptr(bf16_page_table, "bf16_page_table", torch.int32), bf16_page_table.shape[1],
        _pages(bf16_pool, pool.bf16_page_bytes),
        _ptr(int2_page_table, "int2_page_table", torch.int32), int2_page_table.shape[1],
        _pages(int2_pool, pool.int2_page_bytes),
        _ptr(bf16_pool, "bf16_pool", torch.uint8), _ptr(int2_pool, "int2_pool", torch.uint8),
        _ptr(r_k, "r_k", torch.float32), _ptr(r_v, "r_v", torch.float32), _ptr(out, "out", torch.bfloat16),
        ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None, ng,
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream)),
        "oscar_decode_attention_cascade")
    return out


def oscar_bf16_decode_attention(pool: OscarPool, q, seq_lens, max_seq_len: int, bf16_page_table, bf16_pool, out,
                                workspace, stream=None):
    import torch
    _check(load().oscar_bf16_decode_attention(
        pool.handle, q.shape[0], int(max_seq_len), _ptr(q, "q", torch.bfloat16), _ptr(seq_lens, "seq_lens", torch.int32),
        _ptr(bf16_page_table, "bf16_page_table", torch.int32), bf16_page_table.shape[1],
        _pages(bf16_pool, pool.bf16_page_bytes), _ptr(bf16_pool, "bf16_pool", torch.uint8),
        _ptr(out, "out", torch.bfloat16), _ptr(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream)),
        "oscar_bf16_decode_attention")
    return out


def oscar_merge(row_offsets, o_partials, lse_partials, out, stream=None):
    import torch
    rows, d = out.shape
    _check(load().oscar_merge(
        rows, d, _ptr(row_offsets, "row_offsets", torch.int32), _ptr(o_partials, "o_partials", torch.float32),
        _ptr(lse_partials, "lse_partials", torch.float32), _ptr(out, "out", torch.bfloat16), _stream(stream)),
        "oscar_merge")
    return out


def oscar_quantize_pack(pool: OscarPool, k, v, page_ids, int2_pool, r_k, tau_k, tau_v, r_v=None, stream=None):
    import torch
    _check(load().oscar_quantize_pack(
        pool.handle, k.shape[0], _ptr(k, "k", torch.bfloat16), _ptr(v, "v", torch.bfloat16),
        _ptr(page_ids, "page_ids", torch.int32), _pages(int2_pool, pool.int2_page_bytes),
        _ptr(int2_pool, "int2_pool", torch.uint8), _ptr(r_k, "r_k", torch.float32), _ptr(r_v, "r_v", torch.float32),
        _ptr(tau_k, "tau_k", torch.float32), _ptr(tau_v, "tau_v", torch.float32), _stream(stream)),
        "oscar_quantize_pack")


def oscar_write_bf16(pool: OscarPool, k, v, first_position: int, bf16_page_table_row, bf16_pool, stream=None):
    """Stage dense bf16 tokens k, v [T, Hkv, D] at positions first_position..
    of one sequence (bf16_page_table_row: int32 [stride])."""
    import torch
    _check(load().oscar_write_bf16(
        pool.handle, k.shape[0], int(first_position), _ptr(k, "k", torch.bfloat16), _ptr(v, "v", torch.bfloat16),
        _ptr(bf16_page_table_row, "bf16_page_table_row", torch.int32), bf16_page_table_row.numel(),
        _pages(bf16_pool, pool.bf16_page_bytes), _ptr(bf16_pool, "bf16_pool", torch.uint8), _stream(stream)),
        "oscar_write_bf16")


# ---------------------------------------------------------------------------
# offline calibration and the rotation error chain
# ---------------------------------------------------------------------------

def _rows_view(x, name):
    """A [heads, rows, D] fp32 device view whose last dimension is dense:
    returns (pointer, head stride, row stride) in elements."""
    import torch
    if not x.is_cuda or x.dtype != torch.float32 or x.dim() != 3 or x.stride(2) != 1:
        raise ValueError(f"{name} must be a float32 device tensor [heads, rows, D] with unit last stride")
    return x.data_ptr(), x.stride(0), x.stride(1)


def _ws(nbytes, device):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _size_out(fn, *args):
    n = ctypes.c_size_t()
    _check(getattr(load(), fn)(*args, ctypes.byref(n)), fn)
    return n.value


def oscar_calib_gram(x, scale: float, out, workspace=None, stream=None):
    """out[h] = scale * x[h]^T x[h] for x [heads, rows, D] (any head/row
    strides)."""
    import torch
    heads, rows, d = x.shape
    px, hs, rs = _rows_view(x, "x")
    if workspace is None:
        workspace = _ws(_size_out("oscar_calib_gram_workspace_bytes", heads, rows, d), x.device)
    _check(load().oscar_calib_gram(heads, rows, d, px, hs, rs, float(scale), _ptr(out, "out", torch.float32),
                                   _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream)),
           "oscar_calib_gram")
    return out


def oscar_calib_attention(q, k, v, out, lse=None, sm_scale: float = 0.0, stream=None):
    """Causal attention of the calibration draw: q [Hkv, g, N, D] contiguous,
    k and v [Hkv, N, D] views with unit last stride and equal strides."""
    import torch
    hkv, g, n, d = q.shape
    pk, hs, ns = _rows_view(k, "k")
    pv, hs2, ns2 = _rows_view(v, "v")
    if (hs, ns) != (hs2, ns2):
        raise ValueError("k and v must have the same strides")
    _check(load().oscar_calib_attention(hkv, g, n, d, float(sm_scale), _ptr(q, "q", torch.float32), pk, pv, hs, ns,
                                        _ptr(out, "out", torch.float32), _ptr(lse, "lse", torch.float32),
                                        _stream(stream)),
           "oscar_calib_attention")
    return out


def oscar_calib_rotation(cov, r, eigvals=None, mix: bool = True, stream=None):
    """Eigenbasis of cov [heads, D, D] and R = U H P_br (mix) or U."""
    import torch
    heads, d, _ = cov.shape
    _check(load().oscar_calib_rotation(heads, d, _ptr(cov, "cov", torch.float32), int(bool(mix)),
                                       _ptr(r, "r", torch.float32), _ptr(eigvals, "eigvals", torch.float32),
                                       _stream(stream)),
           "oscar_calib_rotation")
    return r


def oscar_calib_clip(x, r, quantile: float, tau, workspace=None, stream=None):
    """tau[h] = quantile of |x[h] R[h]| (r None: of |x[h]|); x [heads, rows, D]."""
    import torch
    heads, rows, d = x.shape
    px, hs, rs = _rows_view(x, "x")
    if workspace is None:
        workspace = _ws(_size_out("oscar_calib_clip_workspace_bytes", heads, rows, d), x.device)
    _check(load().oscar_calib_clip(heads, rows, d, px, hs, rs, _ptr(r, "r", torch.float32), float(quantile),
                                   _ptr(tau, "tau", torch.float32), _ptr(workspace, "workspace", torch.uint8),
                                   workspace.numel(), _stream(stream)),
           "oscar_calib_clip")
    return tau


def oscar_calib_codebook(x, r, tau, group_size: int, levels=None, workspace=None, stream=None):
    """Fixed-end Lloyd-Max codebook of x [heads, rows, D] rotated by r (or
    None) and clipped to tau [heads]; returns levels, a device fp32 [4]."""
    import torch
    heads, rows, d = x.shape
    px, hs, rs = _rows_view(x, "x")
    if levels is None:
        levels = torch.empty(4, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = _ws(_size_out("oscar_calib_codebook_workspace_bytes", heads, rows, d), x.device)
    _check(load().oscar_calib_codebook(heads, rows, d, int(group_size), px, hs, rs, _ptr(r, "r", torch.float32),
                                       _ptr(tau, "tau", torch.float32), _ptr(levels, "levels", torch.float32),
                                       _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream)),
           "oscar_calib_codebook")
    return levels


def oscar_calibrate(q, k, v, clip_quantile: float = 0.995, sm_scale: float = 0.0, workspace=None, stream=None):
    """The whole calibration of one layer on the GPU.  q [Hkv, g, N, D]
    contiguous fp32; k, v [Hkv, N, D] fp32 views.  Returns a dict of device
    tensors r_k, r_v [Hkv, D, D], tau_k, tau_v [Hkv], c_q, c_s [Hkv, D, D]."""
    import torch
    hkv, g, n, d = q.shape
    pk, hs, ns = _rows_view(k, "k")
    pv, hs2, ns2 = _rows_view(v, "v")
    if (hs, ns) != (hs2, ns2):
        raise ValueError("k and v must have the same strides")
    dev = q.device
    res = {name: torch.empty(hkv, d, d, dtype=torch.float32, device=dev) for name in ("r_k", "r_v", "c_q", "c_s")}
    res["tau_k"] = torch.empty(hkv, dtype=torch.float32, device=dev)
    res["tau_v"] = torch.empty(hkv, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _ws(_size_out("oscar_calib_workspace_bytes", hkv, g, n, d), dev)
    _check(load().oscar_calibrate(
        hkv, g, n, d, float(sm_scale), _ptr(q, "q", torch.float32), pk, pv, hs, ns, float(clip_quantile),
        res["r_k"].data_ptr(), res["r_v"].data_ptr(), res["tau_k"].data_ptr(), res["tau_v"].data_ptr(),
        res["c_q"].data_ptr(), res["c_s"].data_ptr(), _ptr(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream)), "oscar_calibrate")
    return res


def oscar_dequantize(pool: OscarPool, num_tokens: int, page_ids, int2_pool, r_k, r_v, k_out, v_out, stream=None):
    """INT2 history records of tokens 0..num_tokens-1 back to fp32
    [num_tokens, Hkv, D]; r_k / r_v (or None) are the rotations to undo."""
    import torch
    _check(load().oscar_dequantize(
        pool.handle, int(num_tokens), _ptr(page_ids, "page_ids", torch.int32), _pages(int2_pool, pool.int2_page_bytes),
        _ptr(int2_pool, "int2_pool", torch.uint8), _ptr(r_k, "r_k", torch.float32), _ptr(r_v, "r_v", torch.float32),
        _ptr(k_out, "k_out", torch.float32), _ptr(v_out, "v_out", torch.float32), _stream(stream)),
        "oscar_dequantize")


def oscar_attention_error(q, k, v, k_hat, v_hat, stats, sm_scale: float = 0.0, stream=None):
    """Per causal query row of q [Hkv, g, N, D]: {KL(p || p^), summed squared
    logit error, ||o - o^||^2, ||o||^2} into stats [Hkv, g, N, 4]; k, v,
    k_hat, v_hat [Hkv, N, D] views sharing one set of strides."""
    import torch
    hkv, g, n, d = q.shape
    views = [_rows_view(t, name) for t, name in ((k, "k"), (v, "v"), (k_hat, "k_hat"), (v_hat, "v_hat"))]
    if len({(hs, ns) for _, hs, ns in views}) != 1:
        raise ValueError("k, v, k_hat and v_hat must share strides")
    _, hs, ns = views[0]
    _check(load().oscar_attention_error(
        hkv, g, n, d, float(sm_scale), _ptr(q, "q", torch.float32), views[0][0], views[1][0], views[2][0],
        views[3][0], hs, ns, _ptr(stats, "stats", torch.float32), _stream(stream)), "oscar_attention_error")
    return stats
