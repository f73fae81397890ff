"""Paged KV cache storage: slot arithmetic and cache writes, in plain numpy.

Storage model ("KV Cache 和 vLLM" §3.1-3.2; "KV Cache优化实战" §4.2): the cache
of one layer is a pool of fixed 16-token physical blocks; a sequence's tokens
are logically contiguous (tokens 0-15 in logical block 0, 16-31 in logical
block 1, ...) and a per-sequence block table maps each logical block to the
physical block that holds it.

In-block layout (a reading; the pages fix only the 16-token block, and 32 as
the larger choice for long traffic, "KV Cache 和 vLLM" §6.3): for each
physical block and each KV head, the block's token rows of head_dim elements
are contiguous, i.e. the pool is ``[num_blocks][num_kv_heads][bs][head_dim]``
with bs = 16 or 32 tokens per block.
Quantised pools carry one float32 scale per (block, head, token) in
``[num_blocks][num_kv_heads][bs]``; an INT4 pool holds two codes per byte,
``[num_blocks][num_kv_heads][bs][head_dim / 2]``.

Test infrastructure: only tests, the smoke check and the CPU baseline leg of
the benchmark use this module.
"""
from __future__ import annotations

import numpy as np

from . import kv_formats

BLOCK_TOKENS = 16


def blocks_for(length: int, block_size: int = BLOCK_TOKENS) -> int:
    """Blocks a sequence of ``length`` tokens owns: ceil(length / block_size)."""
    return -(-int(length) // block_size)


def slot_of(table_row, position: int, block_size: int = BLOCK_TOKENS) -> int:
    """Slot of logical position ``position`` given the sequence's block table
    row: physical block ``table_row[position // bs]``, offset ``position % bs``;
    slot = bs * physical_block + offset (bs = 16, or 32)."""
    return block_size * int(table_row[position // block_size]) + position % block_size


class Pool:
    """One layer's K and V pools.

    Formats (``kv_formats.FORMATS``): unquantised pools keep float64 values
    (exact copies of the written rows); quantised ones keep what the GPU
    pool holds - the codes (int4: two per byte) and one float32 scale per
    (block, head, token).  K and V may use different element formats.  A
    written-mask marks filled slots; unwritten slots are undefined in the GPU
    pool and are never compared."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, cache_dtype: str,
                 block_size: int = BLOCK_TOKENS):
        self.bs = block_size
        self.num_blocks = num_blocks
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.cache_dtype = cache_dtype
        self.k_elem, self.v_elem = kv_formats.FORMATS[cache_dtype]
        shape = (num_blocks, num_kv_heads, self.bs, head_dim)
        self.written = np.zeros((num_blocks, self.bs), dtype=bool)
        self.store = {}
        for name, elem in (("k", self.k_elem), ("v", self.v_elem)):
            if kv_formats.is_quantised(elem):
                width = head_dim // 2 if elem == "i4" else head_dim
                self.store[name] = (np.zeros(shape[:3] + (width,), dtype=np.uint8),
                                    np.zeros(shape[:3], dtype=np.float32))
            else:
                self.store[name] = (np.zeros(shape, dtype=np.float64), None)

    # the e4m3 attribute names used by tests that read codes and scales
    @property
    def k_codes(self):
        return self.store["k"][0]

    @property
    def v_codes(self):
        return self.store["v"][0]

    @property
    def k_scale(self):
        return self.store["k"][1]

    @property
    def v_scale(self):
        return self.store["v"][1]

    @property
    def k(self):
        return self.store["k"][0]

    @property
    def v(self):
        return self.store["v"][0]

    # -- writes -------------------------------------------------------------
    def append(self, k_rows: np.ndarray, v_rows: np.ndarray, slots) -> None:
        """Write token rows ``[n][Hkv][D]`` to their slots (a negative slot means
        "skip this row").  Unquantised: an exact copy of the values.  Quantised:
        each (token, head) row is quantised with its own scale."""
        slots = np.asarray(slots, dtype=np.int64)
        keep = slots >= 0
        slots = slots[keep]
        blk = slots // self.bs
        off = slots % self.bs
        if np.any(blk >= self.num_blocks):
            raise IndexError("slot outside the pool")
        for name, rows, elem in (("k", k_rows, self.k_elem), ("v", v_rows, self.v_elem)):
            rows = np.asarray(rows)[keep]
            data, scales = self.store[name]
            if scales is None:
                data[blk, :, off, :] = rows
            else:
                codes, sc = kv_formats.quantise(rows, elem)
                data[blk, :, off, :] = codes
                scales[blk, :, off] = sc
        self.written[blk, off] = True

    def copy_block(self, src: int, dst: int) -> None:
        """Copy-on-write: the whole block (every head and slot, plus scales)."""
        for data, scales in self.store.values():
            data[dst] = data[src]
            if scales is not None:
                scales[dst] = scales[src]
        self.written[dst] = self.written[src]

    # -- reads --------------------------------------------------------------
    def read_slots(self, blocks, offsets):
        """float64 K and V rows ``[n][Hkv][D]`` stored at the given slots
        (dequantised with their scales for quantised formats)."""
        out = []
        for name, elem in (("k", self.k_elem), ("v", self.v_elem)):
            data, scales = self.store[name]
            if scales is None:
                out.append(data[blocks, :, offsets, :])
            else:
                out.append(kv_formats.dequantise(data[blocks, :, offsets, :], scales[blocks, :, offsets], elem))
        return out[0], out[1]

    def gather(self, table_row, length: int):
        """K, V ``[length][Hkv][D]`` float64 of one sequence, read through its
        block table in logical order: position t lives in physical block
        ``table_row[t // bs]`` at offset ``t % bs``."""
        t = np.arange(int(length))
        blocks = np.asarray(table_row, dtype=np.int64)[t // self.bs]
        if length and (blocks.min() < 0 or blocks.max() >= self.num_blocks):
            raise IndexError("block table entry outside the pool")
        if length and not np.all(self.written[blocks, t % self.bs]):
            raise ValueError("read of an unwritten slot")
        return self.read_slots(blocks, t % self.bs)
