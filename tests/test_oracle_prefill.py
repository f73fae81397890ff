"""Pins for the oracle's chunked prefill attention.

Library routine: torch's scaled_dot_product_attention in fp64 on the CPU,
with GQA, given the causal mask shifted by the cached length as an explicit
boolean mask (and, with no cached context, its own is_causal=True).  Closed
form: with no context the first query sees only itself, so its output is its
own V row.  Invariant: a query's output does not depend on rows after its
position and does depend on the row at it.
"""
import math

import numpy as np
import pytest
import torch

from oracle import cache, prefill
from oracle.allocator import BlockAllocatorModel


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa(q, K, V, mask=None, causal=False):
    tq = torch.from_numpy(q).permute(1, 0, 2)[None].contiguous()   # [1, Hq, n, D]
    tk = torch.from_numpy(K).permute(1, 0, 2)[None].contiguous()   # [1, Hkv, L, D]
    tv = torch.from_numpy(V).permute(1, 0, 2)[None].contiguous()
    m = None if mask is None else torch.from_numpy(mask)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal,
                                                           enable_gqa=True)
    return ref[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("Hq,Hkv,D,L,n", [(4, 2, 64, 40, 7), (32, 8, 128, 300, 64), (8, 8, 64, 17, 17),
                                          (16, 1, 128, 90, 1), (6, 3, 64, 50, 33)])
def test_matches_torch_sdpa_with_shifted_causal_mask(Hq, Hkv, D, L, n):
    rng = np.random.default_rng(Hq * 1000 + L + n)
    q = _rand(rng, n, Hq, D)
    K = _rand(rng, L, Hkv, D)
    V = _rand(rng, L, Hkv, D)
    ours = prefill.prefill_rows(q, K, V, 1.0 / math.sqrt(D))
    ctx = L - n
    mask = np.arange(L)[None, :] <= (ctx + np.arange(n))[:, None]      # [n, L]
    assert np.max(np.abs(ours - _sdpa(q, K, V, mask=mask))) < 1e-12


def test_no_context_matches_is_causal():
    rng = np.random.default_rng(5)
    n, Hq, Hkv, D = 29, 8, 2, 64
    q, K, V = _rand(rng, n, Hq, D), _rand(rng, n, Hkv, D), _rand(rng, n, Hkv, D)
    ours = prefill.prefill_rows(q, K, V, 1.0 / math.sqrt(D))
    assert np.max(np.abs(ours - _sdpa(q, K, V, causal=True))) < 1e-12
    # the first query sees only itself: its output is its own V row
    G = Hq // Hkv
    for h in range(Hq):
        assert np.array_equal(ours[0, h], V[0, h // G])


def test_causality():
    rng = np.random.default_rng(6)
    L, n, Hq, Hkv, D = 40, 10, 4, 2, 64
    q, K, V = _rand(rng, n, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    base = prefill.prefill_rows(q, K, V, 0.125)
    i = 4
    p = L - n + i
    K2, V2 = K.copy(), V.copy()
    K2[p + 1:] += 5.0
    V2[p + 1:] -= 3.0
    moved = prefill.prefill_rows(q, K2, V2, 0.125)
    assert np.array_equal(moved[:i + 1], base[:i + 1])
    assert np.all(np.abs(moved[i + 1:] - base[i + 1:]) > 0)
    V3 = V.copy()
    V3[p] += 1.0
    assert np.all(np.abs(prefill.prefill_rows(q, K, V3, 0.125)[i] - base[i]) > 0)


def test_paged_batch_equals_contiguous():
    rng = np.random.default_rng(7)
    Hq, Hkv, D = 8, 2, 64
    lens, chunks = [45, 16, 70], [5, 16, 1]
    a = BlockAllocatorModel(32, 8)
    a.set_free_order(rng.permutation(32))
    pool = cache.Pool(32, Hkv, D, "f32")
    rows = {}
    for b, L in enumerate(lens):
        a.create(b)
        slots, _ = a.append_slots(b, L)
        K, V = _rand(rng, L, Hkv, D).astype(np.float32), _rand(rng, L, Hkv, D).astype(np.float32)
        pool.append(K, V, np.asarray(slots))
        rows[b] = (K, V)
    tables, clens = a.block_tables(range(3), 8)
    qs = np.concatenate([[0], np.cumsum(chunks)])
    q = _rand(rng, int(qs[-1]), Hq, D)
    got = prefill.prefill_paged(q, qs, pool, tables, clens, 0.125)
    for b in range(3):
        exp = prefill.prefill_rows(q[qs[b]:qs[b + 1]], rows[b][0], rows[b][1], 0.125)
        assert np.array_equal(got[qs[b]:qs[b + 1]], exp)


def test_chunk_longer_than_cache_is_refused():
    with pytest.raises(ValueError):
        prefill.prefill_rows(np.zeros((3, 2, 4)), np.zeros((2, 1, 4)), np.zeros((2, 1, 4)), 0.5)
