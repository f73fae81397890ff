"""Single-token decode attention, fp64, written out from its definition.

Definition ("企业官网建设流程全解析" §1.2): Attention(Q, K, V) =
softmax(Q K^T / sqrt(d_k)) V.  At a decode step the only query is the newest
token's; its K and V were appended to the cache first, so it attends to every
cached token including itself ("企业官网建设流程全解析" §3.2-3.3) and no mask
applies.  The softmax subtracts the row maximum before exponentiating, as the
page's NumPy demonstration does (§5.2).

Grouped-query attention ("企业官网建设流程全解析" §2.2; "KV Cache优化实战" §2.1):
several query heads share one KV head.  Reading: query head h uses KV head
h // (Hq / Hkv), i.e. consecutive query heads form a group.

Reading for an empty context (L = 0): the output is all zeros.

Test infrastructure: only tests, the smoke check and the CPU baseline leg of
the benchmark use this module.
"""
from __future__ import annotations

import math

import numpy as np

from . import kv_formats
from .cache import Pool


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """One sequence: q ``[Hq][D]``, K and V ``[L][Hkv][D]`` -> out ``[Hq][D]``, fp64.

    For query head h with KV head g = h // (Hq/Hkv):
      sigma_t = scale * sum_d q[h, d] * K[t, g, d]
      m = max_t sigma_t;  w_t = exp(sigma_t - m)
      out[h] = sum_t w_t V[t, g] / sum_t w_t
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, D = q.shape
    L, Hkv, _ = K.shape
    group = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    if L == 0:
        return out
    for h in range(Hq):
        g = h // group
        sigma = (K[:, g, :] @ q[h]) * scale
        m = np.max(sigma)
        w = np.exp(sigma - m)
        out[h] = (w @ V[:, g, :]) / np.sum(w)
    return out


def decode_paged(q: np.ndarray, pool: Pool, block_tables, context_lens, scale: float) -> np.ndarray:
    """Batch decode reading K/V through the block tables (the paged form).

    q ``[B][Hq][D]``; block_tables ``[B][max_blocks]``; context_lens ``[B]``.
    Returns out ``[B][Hq][D]`` fp64."""
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(q.shape[0]):
        K, V = pool.gather(block_tables[b], int(context_lens[b]))
        out[b] = attend(q[b], K, V, scale)
    return out


def rows_as_cached(k_rows: np.ndarray, v_rows: np.ndarray, cache_dtype: str):
    """The float64 values a cache of ``cache_dtype`` holds for token rows
    ``[L][Hkv][D]``: the rows themselves, or for a quantised format the
    dequantised codes (each (token, head) row quantised with its own scale)."""
    k_elem, v_elem = kv_formats.FORMATS[cache_dtype]
    return kv_formats.values_as_cached(k_rows, k_elem), kv_formats.values_as_cached(v_rows, v_elem)


def partition_state(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                    start: int, stop: int):
    """Softmax state of one partition of logical positions [start, stop):
    per query head m_p = max sigma, l_p = sum exp(sigma - m_p),
    acc_p = sum exp(sigma - m_p) V  (unnormalised).  Empty partitions give
    m_p = -inf, l_p = 0, acc_p = 0."""
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    Hkv = K.shape[1]
    group = Hq // Hkv
    m = np.full(Hq, -np.inf)
    l = np.zeros(Hq)
    acc = np.zeros((Hq, D))
    if stop <= start:
        return m, l, acc
    for h in range(Hq):
        g = h // group
        sigma = (np.asarray(K[start:stop, g, :], dtype=np.float64) @ q[h]) * scale
        m[h] = np.max(sigma)
        w = np.exp(sigma - m[h])
        l[h] = np.sum(w)
        acc[h] = w @ np.asarray(V[start:stop, g, :], dtype=np.float64)
    return m, l, acc


def combine_partitions(ms, ls, accs) -> np.ndarray:
    """Log-sum-exp merge of partition states (exact algebra of the softmax):
    M = max_p m_p;  w_p = exp(m_p - M);  out = sum_p w_p acc_p / sum_p w_p l_p.
    If every partition is empty the result is zeros."""
    ms = np.asarray(ms, dtype=np.float64)        # [P][Hq]
    ls = np.asarray(ls, dtype=np.float64)        # [P][Hq]
    accs = np.asarray(accs, dtype=np.float64)    # [P][Hq][D]
    M = np.max(ms, axis=0)
    out = np.zeros(accs.shape[1:])
    for h in range(ms.shape[1]):
        if not np.isfinite(M[h]):
            continue
        w = np.exp(ms[:, h] - M[h])
        out[h] = (w @ accs[:, h, :]) / (w @ ls[:, h])
    return out


def attend_partitioned(q, K, V, scale: float, partition_tokens: int) -> np.ndarray:
    """The same output computed as independent partitions of
    ``partition_tokens`` logical positions, merged with ``combine_partitions``."""
    L = K.shape[0]
    n_part = max(1, math.ceil(L / partition_tokens))
    states = [partition_state(q, K, V, scale, p * partition_tokens,
                              min(L, (p + 1) * partition_tokens)) for p in range(n_part)]
    ms, ls, accs = zip(*states)
    return combine_partitions(ms, ls, accs)
