"""Chunked prefill attention over a paged cache, fp64, from its definition.

Pages: in the prefill stage every prompt token is processed at once, each
position attending to the positions before it and to itself ("KV Cache 和
vLLM" §1.1; "企业官网建设流程全解析" §3.1-3.2, where the causal mask keeps a
token from seeing later ones); the K/V of earlier tokens is reused from the
cache instead of recomputed ("KV Cache优化实战" §5.2).

Reading: a chunk of n new tokens of a sequence whose cache holds L tokens
after the chunk's own rows were appended occupies positions L-n .. L-1; the
chunk's query i, at position p = L - n + i, attends to cached positions
0 .. p (the cached context and the chunk's earlier tokens and itself), with
the same softmax(q K^T * scale) V as a decode step and the same GQA mapping.
So each row is exactly a decode at its own position, which is how it is
written here.

Test infrastructure: only tests, the smoke check and the CPU baseline leg of
the benchmark use this module.
"""
from __future__ import annotations

import numpy as np

from .attention import attend
from .cache import Pool


def prefill_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """One sequence: chunk queries q ``[n][Hq][D]``, all cached rows K, V
    ``[L][Hkv][D]`` (the chunk's own rows last) -> out ``[n][Hq][D]`` fp64."""
    q = np.asarray(q, dtype=np.float64)
    n = q.shape[0]
    L = K.shape[0]
    if n > L:
        raise ValueError("the chunk's rows must already be in the cache (n <= L)")
    out = np.zeros(q.shape, dtype=np.float64)
    for i in range(n):
        p = L - n + i
        out[i] = attend(q[i], K[:p + 1], V[:p + 1], scale)
    return out


def prefill_paged(q: np.ndarray, query_start, pool: Pool, block_tables, context_lens,
                  scale: float) -> np.ndarray:
    """Batch form: q ``[T][Hq][D]`` holds the chunks back to back, sequence
    b's in rows query_start[b] .. query_start[b+1]-1; K/V come through the
    block tables.  Returns out ``[T][Hq][D]`` fp64."""
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(len(context_lens)):
        s0, s1 = int(query_start[b]), int(query_start[b + 1])
        if s1 == s0:
            continue
        K, V = pool.gather(block_tables[b], int(context_lens[b]))
        out[s0:s1] = prefill_rows(q[s0:s1], K, V, scale)
    return out
