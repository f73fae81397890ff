"""Paged KV cache storage: slot arithmetic and cache writes, in plain numpy.

Storage model ("KV Cache 和 vLLM" §3.1-3.2; "KV Cache优化实战" §4.2): the cache
of one layer is a pool of fixed 16-token physical blocks; a sequence's tokens
are logically contiguous (tokens 0-15 in logical block 0, 16-31 in logical
block 1, ...) and a per-sequence block table maps each logical block to the
physical block that holds it.

In-block layout (a reading; the pages fix only the 16-token block): for each
physical block and each KV head, the 16 token rows of head_dim elements are
contiguous, i.e. the pool is ``[num_blocks][num_kv_heads][16][head_dim]``.
fp8 pools carry one float32 scale per (block, head, token) in
``[num_blocks][num_kv_heads][16]``.

Test infrastructure: only tests, the smoke check and the CPU baseline leg of
the benchmark use this module.
"""
from __future__ import annotations

import numpy as np

from . import fp8_e4m3

BLOCK_TOKENS = 16


def blocks_for(length: int) -> int:
    """Blocks a sequence of ``length`` tokens owns: ceil(length / 16)."""
    return -(-int(length) // BLOCK_TOKENS)


def slot_of(table_row, position: int) -> int:
    """Slot of logical position ``position`` given the sequence's block table
    row: physical block ``table_row[position // 16]``, offset ``position % 16``;
    slot = 16 * physical_block + offset."""
    return BLOCK_TOKENS * int(table_row[position // BLOCK_TOKENS]) + position % BLOCK_TOKENS


class Pool:
    """One layer's K and V pools.

    Same-dtype pools keep float64 values (exact copies of the written rows) and
    a written-mask; fp8 pools keep the e4m3 codes, the float32 scales and the
    written-mask.  Unwritten slots are undefined in the GPU pool and are never
    compared."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, cache_dtype: str):
        self.num_blocks = num_blocks
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.cache_dtype = cache_dtype
        shape = (num_blocks, num_kv_heads, BLOCK_TOKENS, head_dim)
        self.written = np.zeros((num_blocks, BLOCK_TOKENS), dtype=bool)
        if cache_dtype == "fp8_e4m3":
            self.k_codes = np.zeros(shape, dtype=np.uint8)
            self.v_codes = np.zeros(shape, dtype=np.uint8)
            self.k_scale = np.zeros(shape[:3], dtype=np.float32)
            self.v_scale = np.zeros(shape[:3], dtype=np.float32)
        else:
            self.k = np.zeros(shape, dtype=np.float64)
            self.v = np.zeros(shape, dtype=np.float64)

    # -- writes -------------------------------------------------------------
    def append(self, k_rows: np.ndarray, v_rows: np.ndarray, slots) -> None:
        """Write token rows ``[n][Hkv][D]`` to their slots (a negative slot means
        "skip this row").  Same dtype: an exact copy of the values.  fp8: each
        (token, head) row is quantised with its own scale."""
        slots = np.asarray(slots, dtype=np.int64)
        keep = slots >= 0
        slots = slots[keep]
        k_rows = np.asarray(k_rows)[keep]
        v_rows = np.asarray(v_rows)[keep]
        blk = slots // BLOCK_TOKENS
        off = slots % BLOCK_TOKENS
        if np.any(blk >= self.num_blocks):
            raise IndexError("slot outside the pool")
        if self.cache_dtype == "fp8_e4m3":
            kc, ks = fp8_e4m3.quantise_rows(k_rows)
            vc, vs = fp8_e4m3.quantise_rows(v_rows)
            self.k_codes[blk, :, off, :] = kc
            self.v_codes[blk, :, off, :] = vc
            self.k_scale[blk, :, off] = ks
            self.v_scale[blk, :, off] = vs
        else:
            self.k[blk, :, off, :] = k_rows
            self.v[blk, :, off, :] = v_rows
        self.written[blk, off] = True

    def copy_block(self, src: int, dst: int) -> None:
        """Copy-on-write: the whole block (every head and slot, plus fp8 scales)."""
        if self.cache_dtype == "fp8_e4m3":
            self.k_codes[dst] = self.k_codes[src]
            self.v_codes[dst] = self.v_codes[src]
            self.k_scale[dst] = self.k_scale[src]
            self.v_scale[dst] = self.v_scale[src]
        else:
            self.k[dst] = self.k[src]
            self.v[dst] = self.v[src]
        self.written[dst] = self.written[src]

    # -- reads --------------------------------------------------------------
    def read_slots(self, blocks, offsets):
        """float64 K and V rows ``[n][Hkv][D]`` stored at the given slots
        (dequantised with their scales for fp8)."""
        if self.cache_dtype == "fp8_e4m3":
            k = fp8_e4m3.dequantise(self.k_codes[blocks, :, offsets, :], self.k_scale[blocks, :, offsets])
            v = fp8_e4m3.dequantise(self.v_codes[blocks, :, offsets, :], self.v_scale[blocks, :, offsets])
            return k, v
        return self.k[blocks, :, offsets, :], self.v[blocks, :, offsets, :]

    def gather(self, table_row, length: int):
        """K, V ``[length][Hkv][D]`` float64 of one sequence, read through its
        block table in logical order: position t lives in physical block
        ``table_row[t // 16]`` at offset ``t % 16``."""
        t = np.arange(int(length))
        blocks = np.asarray(table_row, dtype=np.int64)[t // BLOCK_TOKENS]
        if length and (blocks.min() < 0 or blocks.max() >= self.num_blocks):
            raise IndexError("block table entry outside the pool")
        if length and not np.all(self.written[blocks, t % BLOCK_TOKENS]):
            raise ValueError("read of an unwritten slot")
        return self.read_slots(blocks, t % BLOCK_TOKENS)
