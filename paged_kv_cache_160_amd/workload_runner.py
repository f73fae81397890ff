"""Build a workload's cache state on the GPU by running its setup script
(``workloads.setup_ops``) through the native allocator and HIP kernels.

Rows come from the seeded generators in ``workloads`` and are uploaded once
per append; every slot, copy and write is decided and done by the library.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np
import torch

import workloads as wl

from .cache import PagedKVCache

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
                "fp8_e4m3": torch.uint8}      # dtypes of rows and queries (cache formats: CACHE_FORMATS)


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Values already representable in ``dtype``: the cast is exact."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device).to(TORCH_DTYPES[dtype])


class GpuWorkload:
    def __init__(self, w: wl.Workload, num_layers: int = 1, num_blocks: Optional[int] = None,
                 device="cuda"):
        self.w = w
        self.cache = PagedKVCache(num_layers, num_blocks or w.num_blocks, w.num_kv_heads, w.head_dim,
                                  w.cache_dtype, w.max_blocks_per_seq, device=device, block_size=w.block_size)
        self.device = device
        self.trace: List[tuple] = []
        self._rows: Dict[int, tuple] = {}

    def rows(self, seq: int):
        if seq not in self._rows:
            self._rows[seq] = (wl.kv_rows(self.w, seq, "k"), wl.kv_rows(self.w, seq, "v"))
        return self._rows[seq]

    def drop_rows(self, seq: int) -> None:
        self._rows.pop(seq, None)

    def apply(self, op) -> None:
        kind = op[0]
        c = self.cache
        if kind == "free_order":
            c.set_free_order(op[1])
        elif kind == "create":
            c.create(op[1])
        elif kind == "fork":
            c.fork(op[1], op[2])
        elif kind == "free":
            c.free(op[1])
        elif kind == "append":
            seq, n = op[1], op[2]
            start = c.seq_len(seq)
            if seq >= wl.CHURN_ID_BASE:
                # churn sequences only shape the free list: no rows are written
                slots, pairs = c.alloc.append_slots(seq, n)
                self.trace.append((seq, slots, pairs))
                return
            k, v = self.rows(seq)
            kd = to_device(k[start:start + n], self.w.src_dtype, self.device)
            vd = to_device(v[start:start + n], self.w.src_dtype, self.device)
            before = len(c.cow_pairs_applied)
            slots = c.append(seq, kd, vd)
            self.trace.append((seq, slots, c.cow_pairs_applied[before:]))
        else:
            raise ValueError(kind)

    def run(self, ops, release_rows: bool = False) -> "GpuWorkload":
        for op in ops:
            self.apply(op)
            if release_rows and op[0] == "append" and op[1] < wl.CHURN_ID_BASE:
                self.drop_rows(op[1])
        return self

    def append_one_each(self, seqs) -> List[int]:
        """One more position for each sequence, rows from each stream."""
        c = self.cache
        ks, vs = [], []
        for s in seqs:
            k, v = self.rows(s)
            L = c.seq_len(s)
            ks.append(k[L])
            vs.append(v[L])
        kd = to_device(np.stack(ks), self.w.src_dtype, self.device)
        vd = to_device(np.stack(vs), self.w.src_dtype, self.device)
        return c.append_one_each(list(seqs), kd, vd)

    def step_rows(self, seqs):
        """Each sequence's next K/V row (position = its current length)."""
        c = self.cache
        ks, vs = [], []
        for s in seqs:
            k, v = self.rows(s)
            L = c.seq_len(s)
            ks.append(k[L])
            vs.append(v[L])
        return (to_device(np.stack(ks), self.w.src_dtype, self.device),
                to_device(np.stack(vs), self.w.src_dtype, self.device))

    def decode_step(self, seqs, step: int, partition_size: int = 0) -> torch.Tensor:
        """Fused decode step (append the next row of each sequence, attend)."""
        kd, vd = self.step_rows(seqs)
        return self.cache.decode_step(self.queries(step), list(seqs), kd, vd, partition_size=partition_size)[0]

    def queries(self, step: int = 0) -> torch.Tensor:
        return to_device(wl.queries(self.w, step), self.w.q_dtype, self.device)
