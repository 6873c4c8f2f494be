"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libpkv.so`` (hand-written HIP kernels behind the
C ABI in ``include/pkv.h``).  The functions below only check tensor
dtypes/devices/shapes and pass raw device pointers plus torch's current HIP
stream; every step of the computation runs in the library's kernels.  There
is no fallback: without the built library (``__graft_entry__.build()``)
importing the functions raises.

Names follow the C ABI without the ``pkv_`` prefix.
"""
from __future__ import annotations

import ctypes
import math
import os
from pathlib import Path

import numpy as np
import torch

_HERE = Path(__file__).resolve().parent
LIB_PATH = _HERE / "libpkv.so"

PKV_OK = 0

_lib = None

# (name, restype, argtypes) for every symbol include/pkv.h declares
_P, _I32, _SZ, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
_I64 = ctypes.c_int64
SIGNATURES = {
    "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_kv_append": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P]),
    "pkv_decode_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_decode_partition_size": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_paged_attention_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                                  _I32, _I32, _I32, _I32, _F, _I32, _P, _P, _SZ,
                                                  _P]),
    "pkv_paged_attention_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32,
                                                          _I32, _I32, _I32, _I32, _I32, _I32,
                                                          _F, _I32, _P, _P]),
    "pkv_paged_attention_prefill": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                                   _I32, _I32, _I32, _I32, _I32, _I32, _I32, _F,
                                                   _P, _SZ, _P]),
    "pkv_prefill_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_validate_slots": (ctypes.c_int, [_P, _I32, _I32, _I32, _P]),
    "pkv_validate_tables": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _I32, _P]),
    "pkv_validate_chunks": (ctypes.c_int, [_P, _P, _I32, _I32, _P]),
    "pkv_bm_create": (_P, [_I32, _I32]),
    "pkv_bm_destroy": (None, [_P]),
    "pkv_bm_num_free": (_I32, [_P]),
    "pkv_bm_allocate": (ctypes.c_int, [_P, _I64, _I32]),
    "pkv_bm_append_token": (ctypes.c_int, [_P, _I64, _P]),
    "pkv_bm_append_tokens": (ctypes.c_int, [_P, _P, _I32, _P]),
    "pkv_bm_fork": (ctypes.c_int, [_P, _I64, _I64, _I32]),
    "pkv_bm_free": (ctypes.c_int, [_P, _I64]),
    "pkv_bm_seq_len": (_I32, [_P, _I64]),
    "pkv_bm_block_table": (_I32, [_P, _I64, _P, _I32]),
    "pkv_bm_build_tables": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, _P]),
    "pkv_bm_slots": (ctypes.c_int, [_P, _I64, _I32, _I32, _P]),
    "pkv_bm_swap": (ctypes.c_int, [_P, _P, _I64, _P, _P, _I32, _P]),
    "pkv_bm_block_size": (_I32, [_P]),
    "pkv_sched_create": (_P, [_P, _I32, _I32, _I32]),
    "pkv_sched_destroy": (None, [_P]),
    "pkv_sched_add_request": (ctypes.c_int, [_P, _I64, _I32, _I32]),
    "pkv_sched_num_waiting": (_I32, [_P]),
    "pkv_sched_num_running": (_I32, [_P]),
    "pkv_sched_step": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                      _P]),
    "pkv_server_create": (_P, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                               _F]),
    "pkv_server_destroy": (None, [_P]),
    "pkv_server_plan": (ctypes.c_int, [_P, _P, _P]),
    "pkv_server_plan_arrays": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P]),
    "pkv_server_execute": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "pkv_copy_blocks": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                       _I32, _P]),
    "pkv_copy_blocks_dma": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                           _I32, _I32, _P]),
}
PKV_ERR_NO_BLOCKS = 4
PKV_ERR_SCRATCH = 5
NOALLOC_SCRATCH_BYTES = 32 << 20   # PKV_NOALLOC_SCRATCH_BYTES


class PkvError(RuntimeError):
    pass


def load_library(path: str | Path = LIB_PATH):
    """Loads libpkv.so and declares its signatures (no GPU needed)."""
    global _lib
    if _lib is not None and Path(path) == LIB_PATH:
        return _lib
    path = Path(path)
    if not path.exists():
        raise PkvError(f"{path} is missing: build it with __graft_entry__.build() "
                       "(hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(str(path))
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


# Host-side functions (plain host code): the block manager, the scheduler,
# the precondition checks and the status strings.
HOST_LIB_ENV = "PKV_HOST_LIB"
_HOST_PREFIXES = ("pkv_bm_", "pkv_sched_", "pkv_validate_", "pkv_status_string")
_host = None


def host_library():
    """The library the host-side functions come from: libpkv.so, or the
    host-only build of the same sources that $PKV_HOST_LIB names (for
    example a sanitizer build).  The step executor (pkv_server_*) takes its
    scheduler and block manager from libpkv.so, so it is not used with such
    a build."""
    global _host
    if _host is None:
        path = os.environ.get(HOST_LIB_ENV)
        if not path:
            _host = load_library()
        else:
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                if name.startswith(_HOST_PREFIXES):
                    fn = getattr(lib, name)
                    fn.restype = res
                    fn.argtypes = args
            _host = lib
    return _host


def _check(rc: int, what: str):
    if rc != PKV_OK:
        msg = host_library().pkv_status_string(rc).decode()
        raise PkvError(f"{what}: {msg} (status {rc})")


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _cache_shape(k_cache, v_cache):
    _dev(k_cache, "k_cache", torch.float16, 4)
    _dev(v_cache, "v_cache", torch.float16, 4)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    return tuple(k_cache.shape)  # NB, Hkv, bs, D


def kv_append(key, value, k_cache, v_cache, slot_mapping, stream=None):
    """Writes key/value [T, Hkv, D] rows into their slots of the caches."""
    NB, Hkv, bs, D = _cache_shape(k_cache, v_cache)
    _dev(key, "key", torch.float16, 3)
    _dev(value, "value", torch.float16, 3)
    _dev(slot_mapping, "slot_mapping", torch.int32, 1)
    T = slot_mapping.shape[0]
    if key.shape != (T, Hkv, D) or value.shape != (T, Hkv, D):
        raise ValueError(f"key/value must be {(T, Hkv, D)}")
    rc = load_library().pkv_kv_append(key.data_ptr(), value.data_ptr(), k_cache.data_ptr(),
                                      v_cache.data_ptr(), slot_mapping.data_ptr(), T, Hkv, D,
                                      bs, NB, _stream(stream))
    _check(rc, "kv_append")


def decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_seq_len, partition_size=0) -> int:
    return int(load_library().pkv_decode_partition_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len, partition_size))


def decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_seq_len, partition_size=0) -> int:
    return int(load_library().pkv_decode_workspace_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len, partition_size))


def paged_attention_decode(q, k_cache, v_cache, block_tables, seq_lens, *, max_seq_len: int,
                           scale: float | None = None, out=None, workspace=None,
                           partition_size: int = 0, seq_order=None, stream=None):
    """out[S, Hq, D] (float32) of one query token per sequence.

    ``workspace`` (uint8, at least ``decode_workspace_size(...)`` bytes) holds
    the split partials; one buffer serves any number of calls on the same
    stream.  Without it a buffer is allocated for the call.  ``seq_order``
    (host int32 permutation of the batch, optional) is the dispatch order,
    e.g. ``longest_first(host_lengths)``; outputs do not depend on it."""
    NB, Hkv, bs, D = _cache_shape(k_cache, v_cache)
    _dev(q, "q", torch.float16, 3)
    _dev(block_tables, "block_tables", torch.int32, 2)
    _dev(seq_lens, "seq_lens", torch.int32, 1)
    S, Hq, Dq = q.shape
    if Dq != D or block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("q / block_tables / seq_lens shapes disagree")
    MB = block_tables.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32, 3)
    if out.shape != (S, Hq, D):
        raise ValueError("out shape")
    need = decode_workspace_size(S, Hq, Hkv, D, bs, max_seq_len, partition_size)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8, 1)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    order_ptr = None
    if seq_order is not None:
        seq_order = _host_i32(seq_order, "seq_order").reshape(-1)
        if seq_order.shape[0] != S:
            raise ValueError("seq_order must have one entry per sequence")
        order_ptr = seq_order.ctypes.data
    rc = load_library().pkv_paged_attention_decode(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), seq_lens.data_ptr(), S, Hq, Hkv, D, bs, NB, MB,
        int(max_seq_len), float(scale), int(partition_size), order_ptr, ws_ptr, ws_bytes,
        _stream(stream))
    _check(rc, "paged_attention_decode")
    return out


def paged_attention_decode_noalloc(q, k_cache, v_cache, block_tables, seq_lens, out, *,
                                   max_seq_len: int, scale: float | None = None,
                                   partition_size: int = 0, seq_order=None, stream=None):
    """The decode of ``paged_attention_decode`` for callers that cannot
    allocate: ``out`` [S, Hq, D] float32 is required, and the split partials
    go to the library's per-GPU device scratch (``NOALLOC_SCRATCH_BYTES``)
    instead of a workspace.  Calls that may overlap on one GPU race on that
    scratch.  Raises PkvError when the partials exceed it."""
    NB, Hkv, bs, D = _cache_shape(k_cache, v_cache)
    _dev(q, "q", torch.float16, 3)
    _dev(block_tables, "block_tables", torch.int32, 2)
    _dev(seq_lens, "seq_lens", torch.int32, 1)
    _dev(out, "out", torch.float32, 3)
    S, Hq, Dq = q.shape
    if Dq != D or block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("q / block_tables / seq_lens shapes disagree")
    if out.shape != (S, Hq, D):
        raise ValueError("out shape")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    order_ptr = None
    if seq_order is not None:
        seq_order = _host_i32(seq_order, "seq_order").reshape(-1)
        if seq_order.shape[0] != S:
            raise ValueError("seq_order must have one entry per sequence")
        order_ptr = seq_order.ctypes.data
    rc = load_library().pkv_paged_attention_decode_noalloc(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), seq_lens.data_ptr(), S, Hq, Hkv, D, bs, NB,
        block_tables.shape[1], int(max_seq_len), float(scale), int(partition_size), order_ptr,
        _stream(stream))
    _check(rc, "paged_attention_decode_noalloc")
    return out


def longest_first(seq_lens) -> np.ndarray:
    """The dispatch order that starts the longest sequences first (host
    int32, ties in batch order) for ``paged_attention_decode(seq_order=)``."""
    L = np.asarray(seq_lens).reshape(-1)
    return np.argsort(-L.astype(np.int64), kind="stable").astype(np.int32)


def prefill_workspace_size(num_chunks, total_q_tokens, max_q_len, num_q_heads, head_dim,
                           max_seq_len) -> int:
    return int(load_library().pkv_prefill_workspace_size(num_chunks, total_q_tokens, max_q_len,
                                                         num_q_heads, head_dim, max_seq_len))


def paged_attention_prefill(q, cu_q_lens, k_cache, v_cache, block_tables, seq_lens, *,
                            max_q_len: int, max_seq_len: int | None = None,
                            scale: float | None = None, out=None, workspace=None, stream=None):
    """out[sum C, Hq, D] (float32) of causal chunks on paged prefixes.

    ``max_seq_len`` bounds seq_lens (default: the block table's capacity).
    ``workspace`` (uint8, at least ``prefill_workspace_size(...)`` bytes)
    holds the partial outputs of split key ranges; without it a buffer is
    allocated for the call."""
    NB, Hkv, bs, D = _cache_shape(k_cache, v_cache)
    _dev(q, "q", torch.float16, 3)
    _dev(cu_q_lens, "cu_q_lens", torch.int32, 1)
    _dev(block_tables, "block_tables", torch.int32, 2)
    _dev(seq_lens, "seq_lens", torch.int32, 1)
    T, Hq, Dq = q.shape
    C = seq_lens.shape[0]
    if Dq != D or cu_q_lens.shape[0] != C + 1 or block_tables.shape[0] != C:
        raise ValueError("q / cu_q_lens / block_tables / seq_lens shapes disagree")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    MB = block_tables.shape[1]
    if max_seq_len is None:
        max_seq_len = MB * bs
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32, 3)
    if out.shape != (T, Hq, D):
        raise ValueError("out shape")
    need = prefill_workspace_size(C, T, int(max_q_len), Hq, D, int(max_seq_len))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8, 1)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    rc = load_library().pkv_paged_attention_prefill(
        out.data_ptr(), q.data_ptr(), cu_q_lens.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), block_tables.data_ptr(), seq_lens.data_ptr(), C, T,
        int(max_q_len), Hq, Hkv, D, bs, NB, MB, int(max_seq_len), float(scale), ws_ptr,
        ws_bytes, _stream(stream))
    _check(rc, "paged_attention_prefill")
    return out


def _pool(t: torch.Tensor, name: str):
    """A KV pool [NB, Hkv, bs, D] fp16 on the GPU or in pinned host memory."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type == "cpu" and not t.is_pinned():
        raise ValueError(f"{name} on the host must be pinned (pin_memory=True)")
    if t.device.type not in ("cpu", "cuda"):
        raise ValueError(f"{name} must be on the GPU or in pinned host memory")
    if t.dtype != torch.float16 or t.dim() != 4 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [NB, Hkv, bs, D] float16 tensor")
    return tuple(t.shape)


def _pools(src_k, src_v, dst_k, dst_v):
    s, sv, d, dv = (_pool(src_k, "src_k"), _pool(src_v, "src_v"), _pool(dst_k, "dst_k"),
                    _pool(dst_v, "dst_v"))
    if s != sv or d != dv or s[1:] != d[1:]:
        raise ValueError("pools must share [Hkv, bs, D] and K/V shapes must match")
    return s[0], d[0], s[1], s[2], s[3]


def _host_i32(a, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.int32:
        raise TypeError(f"{name} must be int32, got {a.dtype}")
    return a


def _validated(rc, bad, what):
    if rc != PKV_OK:
        raise PkvError(f"{what}: precondition violated at index {bad.value}")


def validate_slots(slot_mapping, num_blocks: int, block_size: int) -> None:
    """Host check of a slot mapping (numpy int32): every slot >= 0 inside the
    pool and no slot written twice.  Raises PkvError naming the row."""
    sl = _host_i32(slot_mapping, "slot_mapping").reshape(-1)
    bad = ctypes.c_int64(-1)
    rc = host_library().pkv_validate_slots(sl.ctypes.data, sl.shape[0], int(num_blocks),
                                           int(block_size), ctypes.byref(bad))
    _validated(rc, bad, "validate_slots")


def validate_tables(block_tables, seq_lens, num_blocks: int, block_size: int) -> None:
    """Host check of block tables [S, MB] and lengths [S] (numpy int32):
    1 <= L <= MB * block_size and every live entry inside the pool.  Raises
    PkvError naming the flat table index (s * MB + j)."""
    t = _host_i32(block_tables, "block_tables")
    L = _host_i32(seq_lens, "seq_lens").reshape(-1)
    if t.ndim != 2 or t.shape[0] != L.shape[0]:
        raise ValueError("block_tables must be [S, MB] with S = len(seq_lens)")
    bad = ctypes.c_int64(-1)
    rc = host_library().pkv_validate_tables(t.ctypes.data, L.ctypes.data, L.shape[0],
                                            t.shape[1], int(num_blocks), int(block_size),
                                            ctypes.byref(bad))
    _validated(rc, bad, "validate_tables")


def validate_chunks(cu_q_lens, seq_lens, total_q_tokens: int) -> None:
    """Host check of prefill chunk bounds (numpy int32): cu_q_lens[0] = 0,
    0 <= chunk_len <= seq_len, last entry = total_q_tokens.  Raises PkvError
    naming the chunk."""
    cu = _host_i32(cu_q_lens, "cu_q_lens").reshape(-1)
    L = _host_i32(seq_lens, "seq_lens").reshape(-1)
    if cu.shape[0] != L.shape[0] + 1:
        raise ValueError("cu_q_lens must have len(seq_lens) + 1 entries")
    bad = ctypes.c_int64(-1)
    rc = host_library().pkv_validate_chunks(cu.ctypes.data, L.ctypes.data, L.shape[0],
                                            int(total_q_tokens), ctypes.byref(bad))
    _validated(rc, bad, "validate_chunks")


def copy_blocks(src_k, src_v, dst_k, dst_v, src_blocks, dst_blocks, stream=None):
    """Copies block src_blocks[i] of (src_k, src_v) to block dst_blocks[i] of
    (dst_k, dst_v) in one kernel; pools on the GPU or in pinned host memory,
    block lists int32 on the GPU (or pinned).  Ids outside a pool are
    skipped."""
    sNB, dNB, Hkv, bs, D = _pools(src_k, src_v, dst_k, dst_v)
    for t, n in ((src_blocks, "src_blocks"), (dst_blocks, "dst_blocks")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.dim() != 1 \
                or not t.is_contiguous() or (t.device.type == "cpu" and not t.is_pinned()):
            raise ValueError(f"{n} must be a contiguous int32 vector on the GPU or pinned")
    if src_blocks.shape != dst_blocks.shape:
        raise ValueError("src_blocks and dst_blocks differ in length")
    rc = load_library().pkv_copy_blocks(src_k.data_ptr(), src_v.data_ptr(), dst_k.data_ptr(),
                                        dst_v.data_ptr(), src_blocks.data_ptr(),
                                        dst_blocks.data_ptr(), src_blocks.shape[0], Hkv, D, bs,
                                        sNB, dNB, _stream(stream))
    _check(rc, "copy_blocks")


def copy_blocks_dma(src_k, src_v, dst_k, dst_v, src_blocks, dst_blocks, stream=None):
    """The same copy as ``copy_blocks`` with host-side block lists (any int
    sequence), issued as hipMemcpyAsync per run of consecutive blocks."""
    import numpy as np
    sNB, dNB, Hkv, bs, D = _pools(src_k, src_v, dst_k, dst_v)
    s = np.ascontiguousarray(src_blocks, dtype=np.int32)
    d = np.ascontiguousarray(dst_blocks, dtype=np.int32)
    if s.shape != d.shape or s.ndim != 1:
        raise ValueError("src_blocks and dst_blocks must be 1-D of equal length")
    rc = load_library().pkv_copy_blocks_dma(src_k.data_ptr(), src_v.data_ptr(),
                                            dst_k.data_ptr(), dst_v.data_ptr(), s.ctypes.data,
                                            d.ctypes.data, s.shape[0], Hkv, D, bs, sNB, dNB,
                                            _stream(stream))
    _check(rc, "copy_blocks_dma")


class OutOfBlocks(PkvError):
    """The block manager has too few free blocks (nothing was changed)."""


class BlockManager:
    """Host free-list block manager of libpkv (``pkv_bm_*``): allocates
    ceil(n / block_size) blocks per request from a LIFO free list, appends
    tokens, shares whole prefix blocks with reference counts, and builds the
    block tables and slot mappings the kernels take (as numpy int32 arrays)."""

    def __init__(self, num_blocks: int, block_size: int):
        import numpy as np
        self._np = np
        self._lib = host_library()
        self._h = self._lib.pkv_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise PkvError("pkv_bm_create: invalid arguments")
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def close(self):
        if self._h:
            self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _rc(self, rc, what):
        if rc == PKV_ERR_NO_BLOCKS:
            raise OutOfBlocks(f"{what}: not enough free KV blocks")
        _check(rc, what)

    @property
    def num_free(self) -> int:
        return int(self._lib.pkv_bm_num_free(self._h))

    def allocate(self, request_id: int, num_tokens: int):
        self._rc(self._lib.pkv_bm_allocate(self._h, int(request_id), int(num_tokens)), "allocate")

    def append_token(self, request_id: int) -> int:
        slot = ctypes.c_int32()
        self._rc(self._lib.pkv_bm_append_token(self._h, int(request_id), ctypes.byref(slot)),
                 "append_token")
        return slot.value

    def append_tokens(self, request_ids):
        np = self._np
        ids = np.ascontiguousarray(request_ids, dtype=np.int64)
        slots = np.empty(ids.shape[0], np.int32)
        self._rc(self._lib.pkv_bm_append_tokens(self._h, ids.ctypes.data, ids.shape[0],
                                                slots.ctypes.data), "append_tokens")
        return slots

    def fork(self, parent_id: int, child_id: int, prefix_tokens: int):
        self._rc(self._lib.pkv_bm_fork(self._h, int(parent_id), int(child_id),
                                       int(prefix_tokens)), "fork")

    def free(self, request_id: int):
        self._rc(self._lib.pkv_bm_free(self._h, int(request_id)), "free")

    def seq_len(self, request_id: int) -> int:
        return int(self._lib.pkv_bm_seq_len(self._h, int(request_id)))

    def block_table(self, request_id: int):
        np = self._np
        n = self._lib.pkv_bm_block_table(self._h, int(request_id), None, 0)
        if n < 0:
            raise PkvError("block_table: unknown request")
        out = np.empty(n, np.int32)
        self._lib.pkv_bm_block_table(self._h, int(request_id), out.ctypes.data, n)
        return out

    def build_tables(self, request_ids, max_blocks_per_seq: int, pad_block: int = 0):
        np = self._np
        ids = np.ascontiguousarray(request_ids, dtype=np.int64)
        tab = np.empty((ids.shape[0], max_blocks_per_seq), np.int32)
        lens = np.empty(ids.shape[0], np.int32)
        self._rc(self._lib.pkv_bm_build_tables(self._h, ids.ctypes.data, ids.shape[0],
                                               int(max_blocks_per_seq), int(pad_block),
                                               tab.ctypes.data, lens.ctypes.data),
                 "build_tables")
        return tab, lens

    def slots(self, request_id: int, first_pos: int, count: int):
        np = self._np
        out = np.empty(count, np.int32)
        self._rc(self._lib.pkv_bm_slots(self._h, int(request_id), int(first_pos), int(count),
                                        out.ctypes.data), "slots")
        return out

    def swap_to(self, other: "BlockManager", request_id: int):
        """Moves a request to ``other`` (e.g. the host pool's manager on swap
        out, the device pool's on swap in); returns the (source, target)
        block pairs the caller must copy before reusing the source blocks."""
        np = self._np
        n = max(len(self.block_table(request_id)), 1)
        src, dst = np.empty(n, np.int32), np.empty(n, np.int32)
        cnt = ctypes.c_int32()
        self._rc(self._lib.pkv_bm_swap(self._h, other._h, int(request_id), src.ctypes.data,
                                       dst.ctypes.data, n, ctypes.byref(cnt)), "swap")
        return src[:cnt.value], dst[:cnt.value]


class _StepPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("num_prefill", "num_prefill_tokens",
                                              "num_decode", "num_new_tokens",
                                              "num_finished", "num_preempted")]


class StepPlan:
    """One step of the scheduler: numpy arrays sized to what the step uses.
    prefill_*: chunk rows (cu_q_lens has num_prefill + 1 entries); decode_*:
    decode rows; slot_mapping: the chunks' slots in cu_q_lens order, then one
    per decode row."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


class Scheduler:
    """Iteration-level scheduler of libpkv (``pkv_sched_*``) over a
    ``BlockManager``: admission, chunked prefill within a token budget,
    decode rows, preemption by recompute; ``step()`` closes the previous
    step and plans the next one."""

    def __init__(self, block_manager: BlockManager, max_batch_size: int, max_num_tokens: int,
                 max_seq_len: int):
        import numpy as np
        self._np = np
        self._lib = host_library()
        self.bm = block_manager
        self._h = self._lib.pkv_sched_create(block_manager._h, int(max_batch_size),
                                             int(max_num_tokens), int(max_seq_len))
        if not self._h:
            raise PkvError("pkv_sched_create: invalid arguments")
        self.max_batch_size, self.max_num_tokens = int(max_batch_size), int(max_num_tokens)
        self.max_seq_len = int(max_seq_len)

    def close(self):
        if self._h:
            self._lib.pkv_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_request(self, request_id: int, prompt_len: int, max_new_tokens: int):
        _check(self._lib.pkv_sched_add_request(self._h, int(request_id), int(prompt_len),
                                               int(max_new_tokens)), "add_request")

    @property
    def num_waiting(self) -> int:
        return int(self._lib.pkv_sched_num_waiting(self._h))

    @property
    def num_running(self) -> int:
        return int(self._lib.pkv_sched_num_running(self._h))

    def step(self, max_blocks_per_seq: int, pad_block: int = 0) -> StepPlan:
        np = self._np
        B, T, MB = self.max_batch_size, self.max_num_tokens, int(max_blocks_per_seq)
        a = dict(prefill_ids=np.empty(B, np.int64), cu_q_lens=np.empty(B + 1, np.int32),
                 prefill_tables=np.empty((B, MB), np.int32), prefill_lens=np.empty(B, np.int32),
                 decode_ids=np.empty(B, np.int64), decode_tables=np.empty((B, MB), np.int32),
                 decode_lens=np.empty(B, np.int32), slot_mapping=np.empty(T + B, np.int32),
                 finished=np.empty(B, np.int64), preempted=np.empty(B, np.int64))
        plan = _StepPlan()
        rc = self._lib.pkv_sched_step(
            self._h, MB, int(pad_block), ctypes.byref(plan), a["prefill_ids"].ctypes.data,
            a["cu_q_lens"].ctypes.data, a["prefill_tables"].ctypes.data,
            a["prefill_lens"].ctypes.data, a["decode_ids"].ctypes.data,
            a["decode_tables"].ctypes.data, a["decode_lens"].ctypes.data,
            a["slot_mapping"].ctypes.data, a["finished"].ctypes.data,
            a["preempted"].ctypes.data)
        _check(rc, "sched_step")
        P, D = plan.num_prefill, plan.num_decode
        return StepPlan(
            prefill_ids=a["prefill_ids"][:P], cu_q_lens=a["cu_q_lens"][:P + 1],
            prefill_tables=a["prefill_tables"][:P], prefill_lens=a["prefill_lens"][:P],
            decode_ids=a["decode_ids"][:D], decode_tables=a["decode_tables"][:D],
            decode_lens=a["decode_lens"][:D], slot_mapping=a["slot_mapping"][:plan.num_new_tokens],
            finished=a["finished"][:plan.num_finished],
            preempted=a["preempted"][:plan.num_preempted],
            num_prefill_tokens=plan.num_prefill_tokens)
