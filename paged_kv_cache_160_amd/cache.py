"""Per-layer paged K/V pools driven by the native block allocator.

Marshalling only: the allocator decides slots and copy-on-write pairs (C++),
the HIP kernels copy blocks, write rows and run decode attention.  PyTorch
owns the device memory.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Union

import torch

from . import (BLOCK_SIZE, CACHE_FORMATS, PKV_FP8_E4M3, PKV_FP8_E5M2, PKV_INT8_INT4, BlockAllocator, copy_blocks,
               gather_blocks, kv_cache_append, paged_attention_decode, paged_attention_decode_append, scatter_blocks,
               workspace_size)

Rows = Union[torch.Tensor, Sequence[torch.Tensor]]


class PagedKVCache:
    """``num_layers`` pools of ``num_blocks`` blocks of ``block_size`` tokens
    (16 or 32) sharing one block table per sequence (every layer stores a
    token at the same slot)."""

    def __init__(self, num_layers: int, num_blocks: int, num_kv_heads: int, head_dim: int,
                 cache_dtype, max_blocks_per_seq: int, device="cuda", block_size: int = BLOCK_SIZE):
        """``cache_dtype``: a format name of ``CACHE_FORMATS`` ("bf16",
        "fp8_e4m3", "fp8_e5m2", "int8_int4", ...) or a torch dtype (uint8
        and float8_e4m3fn mean fp8 e4m3)."""
        self.num_layers = num_layers
        self.num_blocks = num_blocks
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.max_blocks_per_seq = max_blocks_per_seq
        self.block_size = block_size
        self.device = torch.device(device)
        if not isinstance(cache_dtype, str):
            cache_dtype = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16",
                           torch.uint8: "fp8_e4m3", torch.float8_e4m3fn: "fp8_e4m3",
                           torch.float8_e5m2: "fp8_e5m2"}[cache_dtype]
        self.format = cache_dtype
        self.cache_code, k_dt, v_dt, v_per = CACHE_FORMATS[cache_dtype]
        self.quantised = self.cache_code in (PKV_FP8_E4M3, PKV_FP8_E5M2, PKV_INT8_INT4)
        self.fp8 = self.quantised
        self.cache_dtype = k_dt
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        vshape = (num_blocks, num_kv_heads, block_size, head_dim // v_per)
        self.k = [torch.empty(shape, dtype=k_dt, device=self.device) for _ in range(num_layers)]
        self.v = [torch.empty(vshape, dtype=v_dt, device=self.device) for _ in range(num_layers)]
        if self.quantised:
            sshape = (num_blocks, num_kv_heads, block_size)
            self.k_scale = [torch.empty(sshape, dtype=torch.float32, device=self.device) for _ in range(num_layers)]
            self.v_scale = [torch.empty(sshape, dtype=torch.float32, device=self.device) for _ in range(num_layers)]
        else:
            self.k_scale = [None] * num_layers
            self.v_scale = [None] * num_layers
        self.alloc = BlockAllocator(num_blocks, max_blocks_per_seq, block_size)
        self.cow_pairs_applied: List[tuple] = []
        self._ws: Optional[torch.Tensor] = None

    # -- allocator passthroughs ----------------------------------------------
    def set_free_order(self, order) -> None:
        self.alloc.set_free_order(order)

    def create(self, seq_id: int) -> None:
        self.alloc.create(seq_id)

    def fork(self, parent: int, child: int) -> None:
        self.alloc.fork(parent, child)

    def free(self, seq_id: int) -> None:
        self.alloc.free(seq_id)

    def seq_len(self, seq_id: int) -> int:
        return self.alloc.seq_len(seq_id)

    # -- swap -----------------------------------------------------------------
    def _tensors(self):
        """Every pool tensor, layer by layer (K, V and the scales if any)."""
        out = []
        for l in range(self.num_layers):
            out += [self.k[l], self.v[l]]
            if self.quantised:
                out += [self.k_scale[l], self.v_scale[l]]
        return out

    def swap_out(self, seq_id: int) -> list:
        """Move a sequence's blocks to pinned host memory ("KV Cache 和 vLLM"
        §6.2): the allocator releases them, each pool tensor's blocks are
        gathered into one device staging buffer and copied to the host in one
        transfer.  Returns the host tensors (one per pool tensor); keep them
        for swap_in.  The copies are asynchronous on the current stream."""
        blocks = self.alloc.swap_out(seq_id)
        bt = torch.tensor(blocks, dtype=torch.int32).to(self.device)
        host = []
        for t in self._tensors():
            staging = torch.empty((len(blocks),) + tuple(t.shape[1:]), dtype=t.dtype, device=self.device)
            gather_blocks(staging, t, bt)
            h = torch.empty(staging.shape, dtype=t.dtype, pin_memory=True)
            h.copy_(staging, non_blocking=True)
            host.append(h)
        return host

    def swap_in(self, seq_id: int, host: list) -> List[int]:
        """Bring a swapped sequence back into fresh blocks from the host tensors
        swap_out returned; returns the new blocks."""
        blocks = self.alloc.swap_in(seq_id)
        bt = torch.tensor(blocks, dtype=torch.int32).to(self.device)
        for t, h in zip(self._tensors(), host):
            if h.shape[0] != len(blocks):
                raise ValueError("host copy does not match the sequence's blocks")
            scatter_blocks(t, h.to(self.device, non_blocking=True), bt)
        return blocks

    # -- writes ---------------------------------------------------------------
    def _layer_rows(self, rows: Rows, layer: int) -> torch.Tensor:
        if isinstance(rows, torch.Tensor):
            return rows
        return rows[layer]

    def _apply_cow(self, pairs) -> None:
        if not pairs:
            return
        t = torch.tensor(pairs, dtype=torch.int32).to(self.device)
        for layer in range(self.num_layers):
            copy_blocks(self.k[layer], self.v[layer], t, self.k_scale[layer], self.v_scale[layer])
        self.cow_pairs_applied.extend(pairs)

    def _write(self, slots: torch.Tensor, k_rows: Rows, v_rows: Rows) -> None:
        for layer in range(self.num_layers):
            kv_cache_append(self._layer_rows(k_rows, layer), self._layer_rows(v_rows, layer),
                            self.k[layer], self.v[layer], slots,
                            self.k_scale[layer], self.v_scale[layer])

    def append(self, seq_id: int, k_rows: Rows, v_rows: Rows) -> List[int]:
        """Append n token rows ``[n, Hkv, D]`` (device tensors; one tensor for
        every layer or a list per layer) to one sequence."""
        n = int(self._layer_rows(k_rows, 0).shape[0])
        slots, pairs = self.alloc.append_slots(seq_id, n)
        self._apply_cow(pairs)
        if n:
            self._write(torch.tensor(slots, dtype=torch.int64).to(self.device), k_rows, v_rows)
        return slots

    def append_one_each(self, seq_ids: Sequence[int], k_rows: Rows, v_rows: Rows) -> List[int]:
        """One decode step's append: row i of ``k_rows [B, Hkv, D]`` goes to
        sequence ``seq_ids[i]``."""
        slots, pairs = self.alloc.batch_append_one(list(seq_ids))
        self._apply_cow(pairs)
        self._write(torch.tensor(slots, dtype=torch.int64).to(self.device), k_rows, v_rows)
        return slots

    # -- reads ----------------------------------------------------------------
    def block_tables(self, seq_ids: Sequence[int]):
        """Device (tables int32 [B, max_blocks_per_seq], lens int32 [B]) and the
        host max context length."""
        tables, lens = self.alloc.block_tables(list(seq_ids), self.max_blocks_per_seq)
        max_len = int(lens.max()) if len(seq_ids) else 0
        return tables.to(self.device), lens.to(self.device), max_len

    def decode(self, q: torch.Tensor, layer: int, seq_ids: Optional[Sequence[int]] = None,
               tables=None, partition_size: int = 0, out: Optional[torch.Tensor] = None,
               max_context_len: Optional[int] = None) -> torch.Tensor:
        if tables is None:
            tables = self.block_tables(seq_ids)
        bt, lens, max_len = tables
        if max_context_len is not None:
            max_len = max_context_len
        if out is None:
            out = torch.empty_like(q)
        need = workspace_size(q.shape[0], q.shape[1], self.num_kv_heads, self.head_dim, max_len,
                              partition_size, self.cache_code)
        if need and (self._ws is None or self._ws.numel() < need):
            self._ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
        return paged_attention_decode(out, q, self.k[layer], self.v[layer], bt, lens, max_len,
                                      k_scale=self.k_scale[layer], v_scale=self.v_scale[layer],
                                      partition_size=partition_size, workspace=self._ws)

    def decode_step(self, q: Rows, seq_ids: Sequence[int], k_rows: Rows, v_rows: Rows,
                    partition_size: int = 0, out: Optional[List[torch.Tensor]] = None) -> List[torch.Tensor]:
        """One decode step over every layer: the allocator reserves one slot
        per sequence (copy-on-write pairs applied first), then per layer one
        fused launch writes the step's K/V rows and attends over the cache.
        ``q``, ``k_rows``, ``v_rows``: one tensor for every layer or a list."""
        seq_ids = list(seq_ids)
        slots, pairs = self.alloc.batch_append_one(seq_ids)
        self._apply_cow(pairs)
        slot_t = torch.tensor(slots, dtype=torch.int64).to(self.device)
        bt, lens, max_len = self.block_tables(seq_ids)
        outs = []
        for layer in range(self.num_layers):
            ql = self._layer_rows(q, layer)
            o = out[layer] if out is not None else torch.empty_like(ql)
            need = workspace_size(ql.shape[0], ql.shape[1], self.num_kv_heads, self.head_dim, max_len,
                                  partition_size, self.cache_code)
            if need and (self._ws is None or self._ws.numel() < need):
                self._ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
            paged_attention_decode_append(o, ql, self._layer_rows(k_rows, layer), self._layer_rows(v_rows, layer),
                                          self.k[layer], self.v[layer], slot_t, bt, lens, max_len,
                                          k_scale=self.k_scale[layer], v_scale=self.v_scale[layer],
                                          partition_size=partition_size, workspace=self._ws)
            outs.append(o)
        return outs
