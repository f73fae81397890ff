"""Per-layer paged K/V pools driven by the native block allocator.

Marshalling only: the allocator decides slots and copy-on-write pairs (C++),
the HIP kernels copy blocks, write rows and run decode attention.  PyTorch
owns the device memory.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Union

import torch

from . import (BLOCK_SIZE, CACHE_FORMATS, PKV_FP8_E4M3, PKV_FP8_E5M2, PKV_INT8_INT4, BlockAllocator, PagedKVError,
               _lib, copy_blocks, gather_blocks, kv_cache_append, paged_attention_decode, paged_attention_decode_append,
               scatter_blocks, workspace_size)

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

    def swap(self, out_seqs: Sequence[int], back_in: Optional[dict] = None, out_host: Optional[dict] = None) -> dict:
        """Swap ``out_seqs`` out and the sequences of ``back_in`` in, with the
        two directions of the host link overlapped ("KV Cache 和 vLLM" §6.2:
        the link is what swapping costs; it carries both directions at once).

        ``back_in`` maps each sequence to the buffer an earlier ``swap`` call
        returned for it.  The allocator releases the blocks of ``out_seqs``
        first and then gives each ``back_in`` sequence fresh blocks, which may
        be blocks just released: their scatters wait for the gathers.  A
        sequence travels as one pinned host buffer: every pool tensor's blocks
        are gathered into one device staging buffer and copied at once.
        Device -> host copies run on the current stream, host -> device copies
        on a second stream; the current stream waits for both before this
        returns (nothing here synchronises the host).  The device staging
        buffers stay allocated between calls (per direction, one per
        sequence of the largest call so far).  Returns
        ``{seq: (pinned uint8 buffer, n_blocks)}`` for ``out_seqs``.
        ``out_host`` may map outgoing sequences to pinned uint8 buffers to
        fill (large enough; reusing them avoids pinning new memory on every
        call, which costs more than the copies): a buffer handed back in
        through ``back_in`` may be reused by a later call, since the current
        stream has waited for its copy.  Host buffers (type, pinning, size,
        block count) are checked before anything changes; an allocator error
        raises after the swaps already made."""
        back_in = back_in or {}
        out_host = out_host or {}
        tensors = self._tensors()
        bb = [t[0].numel() * t.element_size() for t in tensors]      # bytes of one block of each tensor

        # host buffers are checked before the allocator changes anything
        def check_host(s_, host, n):
            if host.dtype != torch.uint8 or not host.is_pinned() or host.numel() < n * sum(bb):
                raise ValueError(f"host buffer of sequence {s_} must be pinned uint8 of >= {n * sum(bb)} bytes")

        for s_, (host, n) in back_in.items():
            if n != -(-self.alloc.seq_len(s_) // self.block_size):
                raise ValueError(f"host buffer of sequence {s_} does not match its length")
            check_host(s_, host, n)
        for s_, host in out_host.items():
            if s_ in out_seqs:
                check_host(s_, host, -(-self.alloc.seq_len(s_) // self.block_size))
        outs = {s_: self.alloc.swap_out(s_) for s_ in out_seqs}
        ins = {s_: self.alloc.swap_in(s_) for s_ in back_in}
        lib = _lib.lib()
        cur = torch.cuda.current_stream(self.device)
        if getattr(self, "_side", None) is None:
            self._side = torch.cuda.Stream(self.device)
        side = self._side
        if getattr(self, "_swap_done", None) is not None:
            cur.wait_event(self._swap_done)      # the staging buffers' last use, whatever stream that was on

        def move(staging, blocks_t, n, gather, stream):
            off = 0
            for t, b_ in zip(tensors, bb):
                fn = lib.pkv_gather_blocks if gather else lib.pkv_scatter_blocks
                args = ((staging.data_ptr() + off, t.data_ptr()) if gather else (t.data_ptr(), staging.data_ptr() + off))
                rc = fn(*args, blocks_t.data_ptr(), n, b_, self.num_blocks, stream.cuda_stream)
                if rc:
                    raise PagedKVError(rc, "pkv_gather_blocks" if gather else "pkv_scatter_blocks")
                off += n * b_

        def ids_on_device(blocks):
            # block ids go up from pinned memory: an asynchronous copy from
            # pageable memory is staged by the runtime, which blocks the caller
            # once its staging buffers are taken by copies still queued
            return torch.tensor(blocks, dtype=torch.int32).pin_memory().to(self.device, non_blocking=True)

        # device staging buffers are kept between calls; each is used on one
        # stream only, so that stream orders its reuse
        if getattr(self, "_stage", None) is None:
            self._stage = {"out": [], "in": []}

        def stage(kind, i, nbytes, stream):
            bufs = self._stage[kind]
            while len(bufs) <= i:
                bufs.append(None)
            if bufs[i] is None or bufs[i].numel() < nbytes:
                with torch.cuda.stream(stream):
                    bufs[i] = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            return bufs[i][:nbytes]

        result, staged = {}, []
        for i, (s_, blocks) in enumerate(outs.items()):
            n = len(blocks)
            staging = stage("out", i, n * sum(bb), cur)
            bt = ids_on_device(blocks)
            if n:
                move(staging, bt, n, True, cur)
            staged.append((s_, staging, n))
        gathered = torch.cuda.Event()
        gathered.record(cur)
        for s_, staging, n in staged:
            host = out_host.get(s_)
            if host is None:
                host = torch.empty(staging.numel(), dtype=torch.uint8, pin_memory=True)
            host[:staging.numel()].copy_(staging, non_blocking=True)
            result[s_] = (host, n)
        with torch.cuda.stream(side):
            pending = []
            for i, (s_, blocks) in enumerate(ins.items()):
                host, n = back_in[s_]
                staging = stage("in", i, n * sum(bb), side)
                staging.copy_(host[:staging.numel()], non_blocking=True)
                bt = ids_on_device(blocks)
                pending.append((staging, bt, n))
            side.wait_event(gathered)            # reused blocks are read before they are written
            for staging, bt, n in pending:
                if n:
                    move(staging, bt, n, False, side)
        cur.wait_stream(side)
        self._swap_done = torch.cuda.Event()
        self._swap_done.record(cur)
        return result

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
