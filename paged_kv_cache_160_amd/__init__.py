"""Paged KV cache decode attention for AMD Instinct MI355X (gfx950).

A thin Python binding over libpagedkv.so (include/pagedkv.h): argument
marshalling only.  Every step of the path - block allocation, cache writes,
copy-on-write, decode attention and the partition merge - runs in the native
library (C++ on the host, HIP kernels on the GPU).  PyTorch tensors supply the
device memory and the current stream.  There is no CPU fallback: if the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import _lib

__all__ = [
    "PKV_F32", "PKV_F16", "PKV_BF16", "PKV_FP8_E4M3", "PKV_FP8_E5M2", "PKV_INT8_INT4", "BLOCK_SIZE", "BLOCK_SIZES",
    "PagedKVError", "cache_code", "CACHE_FORMATS",
    "kv_cache_append", "copy_blocks", "paged_attention_decode", "paged_attention_decode_append",
    "paged_attention_decode_append_partials", "paged_attention_merge_partials",
    "paged_attention_decode_append_noalloc", "SCRATCH_BYTES", "MAX_ORDER_SEQS",
    "workspace_size", "WS_COUNTER_BYTES",
    "decode_partition_size", "BlockAllocator", "dtype_code", "abi_version", "gather_blocks", "scatter_blocks",
    "paged_attention_prefill",
]

PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3, PKV_FP8_E5M2, PKV_INT8_INT4 = 0, 1, 2, 3, 4, 5
BLOCK_SIZE = 16
BLOCK_SIZES = (16, 32)         # tokens per block the library takes

_TORCH_TO_CODE = {
    torch.float32: PKV_F32,
    torch.float16: PKV_F16,
    torch.bfloat16: PKV_BF16,
    torch.float8_e4m3fn: PKV_FP8_E4M3,
    torch.uint8: PKV_FP8_E4M3,      # raw e4m3 codes
    torch.float8_e5m2: PKV_FP8_E5M2,
}

# cache format name -> (library code, K pool torch dtype, V pool torch dtype,
# V pool elements per K pool element)
CACHE_FORMATS = {
    "f32": (PKV_F32, torch.float32, torch.float32, 1),
    "f16": (PKV_F16, torch.float16, torch.float16, 1),
    "bf16": (PKV_BF16, torch.bfloat16, torch.bfloat16, 1),
    "fp8_e4m3": (PKV_FP8_E4M3, torch.uint8, torch.uint8, 1),
    "fp8_e5m2": (PKV_FP8_E5M2, torch.float8_e5m2, torch.float8_e5m2, 1),
    "int8_int4": (PKV_INT8_INT4, torch.int8, torch.uint8, 2),   # V: two int4 codes per byte
}


class PagedKVError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = _lib.lib().pkv_strerror(code).decode()
        super().__init__(f"{where}: {msg} ({code})")
        self.code = code


def _check(code: int, where: str) -> None:
    if code != 0:
        raise PagedKVError(code, where)


def dtype_code(t: torch.dtype) -> int:
    try:
        return _TORCH_TO_CODE[t]
    except KeyError:
        raise TypeError(f"unsupported dtype {t}") from None


def cache_code(k_pool: torch.Tensor, v_pool: Optional[torch.Tensor] = None) -> int:
    """Library code of the cache format the pools hold: their dtype, with an
    int8 K pool meaning int8 keys and int4 values (V pool uint8, two codes per
    byte, last dimension head_dim / 2)."""
    if k_pool.dtype == torch.int8:
        if v_pool is not None and (v_pool.dtype != torch.uint8 or v_pool.shape[-1] * 2 != k_pool.shape[-1]):
            raise ValueError("an int8 K pool pairs with a uint8 V pool of head_dim / 2 bytes per row")
        return PKV_INT8_INT4
    if v_pool is not None and v_pool.dtype != k_pool.dtype:
        raise ValueError("K and V pools must share a dtype (except int8 K with int4 V)")
    return dtype_code(k_pool.dtype)


_QUANTISED = (PKV_FP8_E4M3, PKV_FP8_E5M2, PKV_INT8_INT4)


def _pool_code(k_pool: torch.Tensor, v_pool: torch.Tensor, k_scale: Optional[torch.Tensor],
               v_scale: Optional[torch.Tensor]) -> int:
    """cache_code, with the shapes the kernels index checked on the host: the
    V pool matches the K pool's blocks, heads and block size, and a quantised
    format has float32 scales [num_blocks, num_kv_heads, block_size] for K
    and V."""
    code = cache_code(k_pool, v_pool)
    if tuple(v_pool.shape[:3]) != tuple(k_pool.shape[:3]):
        raise ValueError("K and V pools must have the same blocks, heads and block size")
    if code != PKV_INT8_INT4 and v_pool.shape[3] != k_pool.shape[3]:
        raise ValueError("K and V pools must have the same head_dim")
    if code in _QUANTISED:
        for sc in (k_scale, v_scale):
            if sc is None or sc.dtype != torch.float32 or tuple(sc.shape) != tuple(k_pool.shape[:3]):
                raise ValueError("a quantised cache needs float32 K and V scales [num_blocks, num_kv_heads, "
                                 "block_size]")
    return code


def abi_version() -> int:
    return _lib.lib().pkv_abi_version()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    """Device address of a tensor for a device entry point: it must be a
    contiguous GPU tensor (a host address would reach a kernel)."""
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError("tensors passed to libpagedkv's device calls must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libpagedkv must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _workspace_for(need: int, workspace: Optional[torch.Tensor], device, stream) -> Optional[torch.Tensor]:
    """The caller's workspace if it holds ``need`` bytes, else a new one.  A
    new workspace is allocated on the stream the kernels run on, so that
    PyTorch's caching allocator hands its memory to no other stream's
    allocation while those kernels may still use it (the tensor may be
    dropped as soon as the call returns)."""
    if not need or (workspace is not None and workspace.numel() * workspace.element_size() >= need):
        return workspace
    if stream is None:
        return torch.zeros(need, dtype=torch.uint8, device=device)
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream), device=device)
    with torch.cuda.stream(s):
        return torch.zeros(need, dtype=torch.uint8, device=device)


def _pool_geometry(k_pool: torch.Tensor) -> Tuple[int, int, int, int]:
    """(num_blocks, num_kv_heads, head_dim, block_size) of a K pool
    ``[num_blocks, num_kv_heads, block_size, head_dim]``, block_size 16 or 32."""
    if k_pool.dim() != 4 or k_pool.shape[2] not in BLOCK_SIZES:
        raise ValueError("pools are [num_blocks, num_kv_heads, block_size (16 or 32), head_dim]")
    return int(k_pool.shape[0]), int(k_pool.shape[1]), int(k_pool.shape[3]), int(k_pool.shape[2])


def kv_cache_append(k_new: torch.Tensor, v_new: torch.Tensor, k_pool: torch.Tensor,
                    v_pool: torch.Tensor, slot_mapping: torch.Tensor,
                    k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                    stream=None) -> None:
    """Write rows ``k_new, v_new [T, Hkv, D]`` to ``slot_mapping [T]`` (int64) of the pools."""
    nb, hkv, d, bs = _pool_geometry(k_pool)
    if k_new.shape[1:] != (hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [T, Hkv, D] matching the pool")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != k_new.shape[0]:
        raise ValueError("slot_mapping must be int64 [T]")
    _check(_lib.lib().kv_cache_append_bs(
        _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
        _ptr(slot_mapping), int(k_new.shape[0]), hkv, d, nb, bs, dtype_code(k_new.dtype),
        _pool_code(k_pool, v_pool, k_scale, v_scale), _stream(stream)), "kv_cache_append_bs")


def copy_blocks(k_pool: torch.Tensor, v_pool: torch.Tensor, pairs: torch.Tensor,
                k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                stream=None) -> None:
    """Copy whole blocks ``pairs [n, 2] = (src, dst)`` (int32, device)."""
    nb, hkv, d, bs = _pool_geometry(k_pool)
    if pairs.dtype != torch.int32 or (pairs.numel() and pairs.shape[-1] != 2):
        raise ValueError("pairs must be int32 [n, 2]")
    code = _pool_code(k_pool, v_pool, k_scale, v_scale)
    _check(_lib.lib().pkv_copy_blocks_bs(
        _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(pairs),
        int(pairs.numel() // 2), hkv, d, nb, bs, code, _stream(stream)), "pkv_copy_blocks_bs")


def decode_partition_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                          max_context_len: int, cache_dtype: int) -> Tuple[int, int]:
    ps, npart = ctypes.c_int(), ctypes.c_int()
    _check(_lib.lib().pkv_decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                max_context_len, cache_dtype, ctypes.byref(ps),
                                                ctypes.byref(npart)), "pkv_decode_partition_size")
    return ps.value, npart.value


def workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                   max_context_len: int, partition_size: int = 0, cache_dtype: int = PKV_BF16) -> int:
    return int(_lib.lib().paged_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                         max_context_len, partition_size, cache_dtype))


# Bytes at the start of a decode workspace that hold the one-call form's
# counters (PKV_WS_COUNTER_BYTES): zero before a workspace's first use, left
# zero by every call.
WS_COUNTER_BYTES = 32768 * 8
# Largest batch whose single-partition decode launches take sequences
# longest first (PKV_MAX_ORDER_SEQS).
MAX_ORDER_SEQS = 8192
# The library's fixed device scratch per GPU (PKV_SCRATCH_BYTES), used by
# paged_attention_decode_append_noalloc.
SCRATCH_BYTES = 16 * 1024 * 1024


def paged_attention_decode(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                           v_pool: torch.Tensor, block_tables: torch.Tensor,
                           context_lens: torch.Tensor, max_context_len: int,
                           scale: Optional[float] = None, k_scale: Optional[torch.Tensor] = None,
                           v_scale: Optional[torch.Tensor] = None, partition_size: int = 0,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode step: ``out[b, h] = softmax(q[b, h] . K_b^T * scale) V_b`` over
    each sequence's first ``context_lens[b]`` cached tokens."""
    nb, hkv, d, bs = _pool_geometry(k_pool)
    if q.dim() != 3 or q.shape[2] != d or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must be [B, Hq, D] of one dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    B, hq = int(q.shape[0]), int(q.shape[1])
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("block_tables must be [B, max_blocks], context_lens [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cdt = _pool_code(k_pool, v_pool, k_scale, v_scale)
    need = workspace_size(B, hq, hkv, d, max_context_len, partition_size, cdt)
    workspace = _workspace_for(need, workspace, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.lib().paged_attention_decode_bs(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(context_lens), B, hq, hkv, d, nb, bs, int(block_tables.shape[1]),
        int(max_context_len), float(scale), dtype_code(q.dtype), cdt, int(partition_size),
        _ptr(workspace), ws_bytes, _stream(stream)), "paged_attention_decode_bs")
    return out


def paged_attention_prefill(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor, query_start: torch.Tensor,
                            max_context_len: int, max_query_len: int, scale: Optional[float] = None,
                            k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """Chunked prefill: ``out[t, h]`` for chunk row t of sequence b (rows
    ``query_start[b] .. query_start[b+1]-1``) attends over the first
    ``context_lens[b] - n_b + i + 1`` cached tokens, i = t - query_start[b]."""
    nb, hkv, d, bs = _pool_geometry(k_pool)
    if q.dim() != 3 or q.shape[2] != d or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must be [T, Hq, D] of one dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or query_start.dtype != torch.int32:
        raise ValueError("block_tables, context_lens and query_start must be int32")
    B = int(context_lens.numel())
    if block_tables.dim() != 2 or block_tables.shape[0] != B or query_start.numel() != B + 1:
        raise ValueError("block_tables must be [B, max_blocks], query_start [B + 1]")
    T, hq = int(q.shape[0]), int(q.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _pool_code(k_pool, v_pool, k_scale, v_scale)
    _check(_lib.lib().paged_attention_prefill_bs(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
        _ptr(context_lens), _ptr(query_start), B, T, hq, hkv, d, nb, bs, int(block_tables.shape[1]),
        int(max_context_len), int(max_query_len), float(scale), dtype_code(q.dtype), code,
        _stream(stream)), "paged_attention_prefill_bs")
    return out


def _block_bytes(pool: torch.Tensor) -> int:
    return pool[0].numel() * pool.element_size()


def gather_blocks(staging: torch.Tensor, pool: torch.Tensor, blocks: torch.Tensor, stream=None) -> torch.Tensor:
    """staging[i] = pool[blocks[i]] for whole blocks (all heads); ``staging``
    is a device tensor shaped [n, *pool.shape[1:]] of pool's dtype."""
    n = int(blocks.numel())
    if blocks.dtype != torch.int32 or staging.shape != (n,) + tuple(pool.shape[1:]) or staging.dtype != pool.dtype:
        raise ValueError("staging must be [n, *pool.shape[1:]] of the pool's dtype; blocks int32 [n]")
    _check(_lib.lib().pkv_gather_blocks(_ptr(staging), _ptr(pool), _ptr(blocks), n, _block_bytes(pool),
                                        int(pool.shape[0]), _stream(stream)), "pkv_gather_blocks")
    return staging


def scatter_blocks(pool: torch.Tensor, staging: torch.Tensor, blocks: torch.Tensor, stream=None) -> None:
    """pool[blocks[i]] = staging[i] for whole blocks."""
    n = int(blocks.numel())
    if blocks.dtype != torch.int32 or staging.shape != (n,) + tuple(pool.shape[1:]) or staging.dtype != pool.dtype:
        raise ValueError("staging must be [n, *pool.shape[1:]] of the pool's dtype; blocks int32 [n]")
    _check(_lib.lib().pkv_scatter_blocks(_ptr(pool), _ptr(staging), _ptr(blocks), n, _block_bytes(pool),
                                         int(pool.shape[0]), _stream(stream)), "pkv_scatter_blocks")


def _decode_append_call(fn_name, out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables,
                        context_lens, max_context_len, scale, k_scale, v_scale, partition_size, workspace,
                        stream):
    nb, hkv, d, bs = _pool_geometry(k_pool)
    if q.dim() != 3 or q.shape[2] != d or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must be [B, Hq, D] of one dtype")
    B, hq = int(q.shape[0]), int(q.shape[1])
    if slot_mapping is not None:
        if k_new.shape != (B, hkv, d) or v_new.shape != k_new.shape:
            raise ValueError("k_new/v_new must be [B, Hkv, D]")
        if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != B:
            raise ValueError("slot_mapping must be int64 [B]")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cdt = _pool_code(k_pool, v_pool, k_scale, v_scale)
    need = workspace_size(B, hq, hkv, d, max_context_len, partition_size, cdt)
    workspace = _workspace_for(need, workspace, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    src_code = dtype_code(k_new.dtype) if k_new is not None else dtype_code(q.dtype)
    _check(getattr(_lib.lib(), fn_name + "_bs")(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
        _ptr(v_scale), _ptr(slot_mapping), _ptr(block_tables), _ptr(context_lens), B, hq, hkv, d, nb, bs,
        int(block_tables.shape[1]), int(max_context_len), float(scale), dtype_code(q.dtype),
        src_code, cdt, int(partition_size), _ptr(workspace), ws_bytes, _stream(stream)), fn_name)
    return out, workspace


def paged_attention_decode_append(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                                  v_new: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                  slot_mapping: torch.Tensor, block_tables: torch.Tensor,
                                  context_lens: torch.Tensor, max_context_len: int,
                                  scale: Optional[float] = None, k_scale: Optional[torch.Tensor] = None,
                                  v_scale: Optional[torch.Tensor] = None, partition_size: int = 0,
                                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """A decode step with the cache write fused in: row b of ``k_new, v_new
    [B, Hkv, D]`` goes to ``slot_mapping[b]`` (the slot of position
    ``context_lens[b] - 1``), then ``out`` = attention over the whole cache."""
    if slot_mapping is None:
        raise ValueError("slot_mapping is required")
    return _decode_append_call("paged_attention_decode_append", out, q, k_new, v_new, k_pool, v_pool,
                               slot_mapping, block_tables, context_lens, max_context_len, scale, k_scale,
                               v_scale, partition_size, workspace, stream)[0]


def paged_attention_decode_append_noalloc(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                                          v_new: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                          slot_mapping: torch.Tensor, block_tables: torch.Tensor,
                                          context_lens: torch.Tensor, max_context_len: int,
                                          scale: Optional[float] = None, k_scale: Optional[torch.Tensor] = None,
                                          v_scale: Optional[torch.Tensor] = None, partition_size: int = 0,
                                          stream=None) -> torch.Tensor:
    """:func:`paged_attention_decode_append` without a workspace: the library's
    fixed device scratch holds the partition states (nothing is allocated;
    calls that overlap on one GPU must not be issued)."""
    nb, hkv, d, bs = _pool_geometry(k_pool)
    if q.dim() != 3 or q.shape[2] != d or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must be [B, Hq, D] of one dtype")
    B, hq = int(q.shape[0]), int(q.shape[1])
    if k_new.shape != (B, hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [B, Hkv, D]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != B:
        raise ValueError("slot_mapping must be int64 [B]")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cdt = _pool_code(k_pool, v_pool, k_scale, v_scale)
    _check(_lib.lib().paged_attention_decode_append_noalloc(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
        _ptr(v_scale), _ptr(slot_mapping), _ptr(block_tables), _ptr(context_lens), B, hq, hkv, d, nb, bs,
        int(block_tables.shape[1]), int(max_context_len), float(scale), dtype_code(q.dtype),
        dtype_code(k_new.dtype), cdt, int(partition_size), _stream(stream)), "paged_attention_decode_append_noalloc")
    return out


def paged_attention_decode_append_partials(out, q, k_new, v_new, k_pool, v_pool, slot_mapping, block_tables,
                                           context_lens, max_context_len, scale=None, k_scale=None,
                                           v_scale=None, partition_size=0, workspace=None, stream=None):
    """First launch of the split form (attention kernel only); returns
    ``(out, workspace)`` for :func:`paged_attention_merge_partials`.
    ``slot_mapping`` may be None (no cache write)."""
    return _decode_append_call("paged_attention_decode_append_partials", out, q, k_new, v_new, k_pool, v_pool,
                               slot_mapping, block_tables, context_lens, max_context_len, scale, k_scale,
                               v_scale, partition_size, workspace, stream)


def paged_attention_merge_partials(out: torch.Tensor, context_lens: torch.Tensor, num_kv_heads: int,
                                   max_blocks_per_seq: int, max_context_len: int, cache_dtype: int,
                                   partition_size: int = 0, workspace: Optional[torch.Tensor] = None,
                                   stream=None, block_size: int = BLOCK_SIZE) -> torch.Tensor:
    """Second launch of the split form: merge the partition states
    (``block_size`` and ``cache_dtype``, a library format code such as
    :func:`cache_code` returns: those of the pool the first launch read)."""
    B, hq, d = (int(x) for x in out.shape)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.lib().paged_attention_merge_partials_bs(
        _ptr(out), _ptr(context_lens), B, hq, num_kv_heads, d, int(block_size), max_blocks_per_seq,
        int(max_context_len), dtype_code(out.dtype), int(cache_dtype), int(partition_size), _ptr(workspace),
        ws_bytes, _stream(stream)), "paged_attention_merge_partials_bs")
    return out


def _int32_array(tokens) -> np.ndarray:
    arr = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
    return arr if arr.size else np.zeros(1, np.int32)[:0]


class BlockAllocator:
    """Host block allocator (refcounts, fork, copy-on-write planning and,
    once ``enable_prefix_cache`` is called, prefix caching)."""

    def __init__(self, num_blocks: int, max_blocks_per_seq: int, block_size: int = BLOCK_SIZE):
        self._lib = _lib.lib()
        self._h = self._lib.pkv_alloc_create_bs(num_blocks, max_blocks_per_seq, block_size)
        if not self._h:
            raise PagedKVError(-1, "pkv_alloc_create_bs")
        self.num_blocks = num_blocks
        self.max_blocks_per_seq = max_blocks_per_seq
        self.block_size = int(self._lib.pkv_alloc_block_size(self._h))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pkv_alloc_destroy(h)
            self._h = None

    def set_free_order(self, order: Sequence[int]) -> None:
        arr = (ctypes.c_int32 * len(order))(*[int(x) for x in order])
        _check(self._lib.pkv_alloc_set_free_order(self._h, arr, len(order)), "set_free_order")

    def create(self, seq_id: int) -> None:
        _check(self._lib.pkv_seq_create(self._h, seq_id), "pkv_seq_create")

    def fork(self, parent: int, child: int) -> None:
        _check(self._lib.pkv_seq_fork(self._h, parent, child), "pkv_seq_fork")

    def free(self, seq_id: int) -> None:
        _check(self._lib.pkv_seq_free(self._h, seq_id), "pkv_seq_free")

    def seq_len(self, seq_id: int) -> int:
        r = self._lib.pkv_seq_len(self._h, seq_id)
        if r < 0:
            raise PagedKVError(r, "pkv_seq_len")
        return r

    def append_slots(self, seq_id: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        slots = (ctypes.c_int64 * max(n, 1))()
        pair = (ctypes.c_int32 * 2)()
        ncow = ctypes.c_int()
        _check(self._lib.pkv_seq_append_slots(self._h, seq_id, n, slots, pair, ctypes.byref(ncow)),
               "pkv_seq_append_slots")
        return list(slots[:n]), ([(pair[0], pair[1])] if ncow.value else [])

    def batch_append_one(self, seq_ids: Sequence[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        n = len(seq_ids)
        ids = (ctypes.c_int64 * max(n, 1))(*seq_ids)
        slots = (ctypes.c_int64 * max(n, 1))()
        pairs = (ctypes.c_int32 * (2 * max(n, 1)))()
        ncow = ctypes.c_int()
        _check(self._lib.pkv_batch_append_one(self._h, ids, n, slots, pairs, ctypes.byref(ncow)),
               "pkv_batch_append_one")
        return list(slots[:n]), [(pairs[2 * i], pairs[2 * i + 1]) for i in range(ncow.value)]

    # -- swap ------------------------------------------------------------------
    def swap_out(self, seq_id: int) -> List[int]:
        """Release the sequence's (unshared) blocks, keeping its length; returns
        them in logical order for the caller to gather."""
        blocks = (ctypes.c_int32 * max(self.max_blocks_per_seq, 1))()
        n = ctypes.c_int()
        _check(self._lib.pkv_seq_swap_out(self._h, seq_id, blocks, ctypes.byref(n)), "pkv_seq_swap_out")
        return list(blocks[:n.value])

    def swap_in(self, seq_id: int) -> List[int]:
        """Fresh blocks for a swapped sequence, in logical order (to scatter into)."""
        blocks = (ctypes.c_int32 * max(self.max_blocks_per_seq, 1))()
        n = ctypes.c_int()
        _check(self._lib.pkv_seq_swap_in(self._h, seq_id, blocks, ctypes.byref(n)), "pkv_seq_swap_in")
        return list(blocks[:n.value])

    # -- prefix caching --------------------------------------------------------
    def enable_prefix_cache(self, model_key: int = 0, hash_bits: int = 64) -> None:
        _check(self._lib.pkv_prefix_cache_enable(self._h, int(model_key) & (2 ** 64 - 1), hash_bits),
               "pkv_prefix_cache_enable")

    def create_cached(self, seq_id: int, tokens) -> int:
        """New sequence holding the longest cached prefix of ``tokens`` (a
        sequence of ints or an int32 array); returns its length (the number of
        prompt tokens whose K/V is already cached)."""
        toks = _int32_array(tokens)
        got = ctypes.c_int()
        _check(self._lib.pkv_seq_create_cached(self._h, seq_id, toks.ctypes.data_as(_lib.P_i32), toks.size,
                                               ctypes.byref(got)), "pkv_seq_create_cached")
        return got.value

    def append_tokens(self, seq_id: int, tokens) -> Tuple[List[int], List[Tuple[int, int]]]:
        toks = _int32_array(tokens)
        n = int(toks.size)
        slots = (ctypes.c_int64 * max(n, 1))()
        pair = (ctypes.c_int32 * 2)()
        ncow = ctypes.c_int()
        _check(self._lib.pkv_seq_append_tokens(self._h, seq_id, toks.ctypes.data_as(_lib.P_i32), n, slots, pair,
                                               ctypes.byref(ncow)), "pkv_seq_append_tokens")
        return list(slots[:n]), ([(pair[0], pair[1])] if ncow.value else [])

    def batch_append_tokens(self, seq_ids: Sequence[int], tokens: Sequence[int]
                            ) -> Tuple[List[int], List[Tuple[int, int]]]:
        n = len(seq_ids)
        if len(tokens) != n:
            raise ValueError("one token per sequence")
        ids = (ctypes.c_int64 * max(n, 1))(*seq_ids)
        toks = (ctypes.c_int32 * max(n, 1))(*[int(t) for t in tokens])
        slots = (ctypes.c_int64 * max(n, 1))()
        pairs = (ctypes.c_int32 * (2 * max(n, 1)))()
        ncow = ctypes.c_int()
        _check(self._lib.pkv_batch_append_tokens(self._h, ids, toks, n, slots, pairs, ctypes.byref(ncow)),
               "pkv_batch_append_tokens")
        return list(slots[:n]), [(pairs[2 * i], pairs[2 * i + 1]) for i in range(ncow.value)]

    def prefix_stats(self) -> dict:
        st = _lib.PrefixStats()
        _check(self._lib.pkv_prefix_stats(self._h, ctypes.byref(st)), "pkv_prefix_stats")
        return {name: getattr(st, name) for name, _ in _lib.PrefixStats._fields_}

    def block_tables(self, seq_ids: Sequence[int], max_blocks: Optional[int] = None,
                     out_tables: Optional[torch.Tensor] = None, out_lens: Optional[torch.Tensor] = None):
        """(tables int32 [n, max_blocks], lens int32 [n]) as CPU tensors, written
        into ``out_tables`` / ``out_lens`` (for example pinned buffers) when given."""
        n = len(seq_ids)
        mb = self.max_blocks_per_seq if max_blocks is None else max_blocks
        ids = (ctypes.c_int64 * max(n, 1))(*seq_ids)
        tables = torch.zeros((n, mb), dtype=torch.int32) if out_tables is None else out_tables
        lens = torch.zeros(n, dtype=torch.int32) if out_lens is None else out_lens
        if (tables.device.type != "cpu" or lens.device.type != "cpu" or tables.dtype != torch.int32
                or lens.dtype != torch.int32 or tables.shape != (n, mb) or lens.shape != (n,)
                or not tables.is_contiguous()):
            raise ValueError("block table buffers must be contiguous int32 CPU [n, max_blocks] and [n]")
        _check(self._lib.pkv_build_block_tables(
            self._h, ids, n, mb, ctypes.cast(tables.data_ptr(), _lib.P_i32),
            ctypes.cast(lens.data_ptr(), _lib.P_i32)), "pkv_build_block_tables")
        return tables, lens

    def stats(self) -> dict:
        st = _lib.AllocStats()
        _check(self._lib.pkv_alloc_stats(self._h, ctypes.byref(st)), "pkv_alloc_stats")
        return {name: getattr(st, name) for name, _ in _lib.AllocStats._fields_}
