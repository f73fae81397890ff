"""Run a workload's setup script through the oracle's allocator model and
cache pool, and compute expected decode outputs.

Test infrastructure: only tests, the smoke check and the CPU baseline leg of
the benchmark use this module.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

import workloads as wl

from . import attention
from .allocator import BlockAllocatorModel
from .cache import Pool


class OracleState:
    def __init__(self, w: wl.Workload, build_pool: bool = True, num_blocks: Optional[int] = None,
                 pool_seqs: Optional[set] = None):
        """``pool_seqs``: write rows into the pool for these sequences only
        (None: all); the allocator still runs every operation."""
        self.w = w
        self.pool_seqs = pool_seqs
        nb = num_blocks or w.num_blocks
        self.alloc = BlockAllocatorModel(nb, w.max_blocks_per_seq, w.block_size)
        self.pool = Pool(nb, w.num_kv_heads, w.head_dim, w.cache_dtype, w.block_size) if build_pool else None
        self.trace: List[tuple] = []          # (seq, slots, pairs) of every append
        self._rows: Dict[int, tuple] = {}

    def rows(self, seq: int):
        if seq not in self._rows:
            self._rows[seq] = (wl.kv_rows(self.w, seq, "k"), wl.kv_rows(self.w, seq, "v"))
        return self._rows[seq]

    def apply(self, op) -> None:
        kind = op[0]
        if kind == "free_order":
            self.alloc.set_free_order(op[1])
        elif kind == "create":
            self.alloc.create(op[1])
        elif kind == "fork":
            self.alloc.fork(op[1], op[2])
        elif kind == "free":
            self.alloc.free_seq(op[1])
        elif kind == "append":
            seq, n = op[1], op[2]
            start = self.alloc.seq_len(seq)
            slots, pairs = self.alloc.append_slots(seq, n)
            self.trace.append((seq, slots, pairs))
            if self.pool is not None:
                for src, dst in pairs:
                    self.pool.copy_block(src, dst)
                if seq < wl.CHURN_ID_BASE and n and (self.pool_seqs is None or seq in self.pool_seqs):
                    k, v = self.rows(seq)
                    self.pool.append(k[start:start + n], v[start:start + n], slots)
        else:
            raise ValueError(kind)

    def run(self, ops) -> "OracleState":
        for op in ops:
            self.apply(op)
        return self

    def append_one_each(self, seqs) -> List[int]:
        """One more position for each sequence (a decode step's append)."""
        out = []
        for s in seqs:
            self.apply(("append", s, 1))
            out.extend(self.trace[-1][1])
        return out

    def tables(self, seqs):
        t, lens = self.alloc.block_tables(seqs, self.w.max_blocks_per_seq)
        return np.array(t, dtype=np.int32), np.array(lens, dtype=np.int32)


def expected_decode_paged(st: OracleState, q: np.ndarray, seqs) -> np.ndarray:
    """Decode through the oracle's own tables and pool (the paged form)."""
    tables, lens = st.tables(seqs)
    return attention.decode_paged(q, st.pool, tables, lens, 1.0 / math.sqrt(st.w.head_dim))


def expected_decode_rows(w: wl.Workload, q: np.ndarray, seqs, lengths) -> np.ndarray:
    """Decode straight from each sequence's generated rows (never through a
    pool): out[b] = attend(q[b], cached values of rows 0..L_b-1)."""
    out = np.zeros((len(seqs),) + q.shape[1:], dtype=np.float64)
    for i, (s, L) in enumerate(zip(seqs, lengths)):
        k = wl.kv_rows(w, s, "k", L)
        v = wl.kv_rows(w, s, "v", L)
        K, V = attention.rows_as_cached(k, v, w.cache_dtype)
        out[i] = attention.attend(q[i], K, V, 1.0 / math.sqrt(w.head_dim))
    return out
