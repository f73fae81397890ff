"""Pins for the oracle's decode attention.

Library routines: torch's scaled_dot_product_attention (fp64, CPU, GQA) and
scipy's softmax on contiguous rows that never pass through the pool.  Closed
forms: all-equal keys give the mean of V; a one-token context gives V0; two
tokens give a logistic weighting with the 1/sqrt(d) factor written out; the
GQA head mapping is visible with constant V per KV head.  Invariants: block
placement does not change the output; partitioned evaluation merged with the
log-sum-exp formula equals the plain form.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention, cache
from oracle.allocator import BlockAllocatorModel


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("Hq,Hkv,D,L", [(4, 2, 64, 40), (32, 8, 128, 300), (8, 8, 64, 17),
                                        (16, 1, 128, 33), (6, 3, 64, 1)])
def test_matches_torch_sdpa(Hq, Hkv, D, L):
    rng = np.random.default_rng(Hq * 1000 + L)
    q = _rand(rng, Hq, D)
    K = _rand(rng, L, Hkv, D)
    V = _rand(rng, L, Hkv, D)
    ours = attention.attend(q, K, V, 1.0 / math.sqrt(D))
    tq = torch.from_numpy(q)[None, :, None, :]                   # [1, Hq, 1, D]
    tk = torch.from_numpy(K).permute(1, 0, 2)[None].contiguous()  # [1, Hkv, L, D]
    tv = torch.from_numpy(V).permute(1, 0, 2)[None].contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, enable_gqa=True)
    ref = ref[0, :, 0, :].numpy()
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_matches_scipy_softmax_bruteforce():
    rng = np.random.default_rng(11)
    Hq, Hkv, D, L = 8, 2, 128, 123
    q, K, V = _rand(rng, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    ours = attention.attend(q, K, V, 1.0 / math.sqrt(D))
    G = Hq // Hkv
    for h in range(Hq):
        Kc = np.ascontiguousarray(K[:, h // G, :])
        Vc = np.ascontiguousarray(V[:, h // G, :])
        p = scipy.special.softmax(Kc @ q[h] / np.sqrt(D))
        assert np.max(np.abs(p @ Vc - ours[h])) < 1e-12


def test_all_equal_keys_give_mean_of_v():
    rng = np.random.default_rng(12)
    Hq, Hkv, D, L = 4, 2, 64, 37
    q = _rand(rng, Hq, D)
    K = np.broadcast_to(_rand(rng, 1, Hkv, D), (L, Hkv, D))
    V = _rand(rng, L, Hkv, D)
    out = attention.attend(q, K, V, 1.0 / math.sqrt(D))
    for h in range(Hq):
        assert np.max(np.abs(out[h] - V[:, h // 2, :].mean(axis=0))) < 1e-13


def test_single_token_gives_v0_exactly():
    rng = np.random.default_rng(13)
    q, K, V = _rand(rng, 4, 64), _rand(rng, 1, 2, 64), _rand(rng, 1, 2, 64)
    out = attention.attend(q, K, V, 0.125)
    for h in range(4):
        assert np.array_equal(out[h], V[0, h // 2])


def test_two_tokens_closed_form_with_sqrt_d():
    # key 0 = c * q, key 1 = 0: sigma0 = c |q|^2 / sqrt(D), sigma1 = 0, so
    # out = (e^sigma0 V0 + V1) / (e^sigma0 + 1)
    rng = np.random.default_rng(14)
    D = 128
    q = _rand(rng, 1, D)
    c = 0.3
    K = np.zeros((2, 1, D))
    K[0, 0] = c * q[0]
    V = _rand(rng, 2, 1, D)
    s0 = c * float(q[0] @ q[0]) / math.sqrt(D)
    expect = (math.exp(s0) * V[0, 0] + V[1, 0]) / (math.exp(s0) + 1.0)
    out = attention.attend(q, K, V, 1.0 / math.sqrt(D))
    assert np.max(np.abs(out[0] - expect)) < 1e-13


def test_gqa_mapping_consecutive_groups():
    # V constant per KV head: out[h] must be that constant of KV head h // G
    rng = np.random.default_rng(15)
    Hq, Hkv, D, L = 8, 4, 64, 20
    q, K = _rand(rng, Hq, D), _rand(rng, L, Hkv, D)
    V = np.zeros((L, Hkv, D))
    for g in range(Hkv):
        V[:, g, :] = 10.0 * (g + 1)
    out = attention.attend(q, K, V, 1.0 / math.sqrt(D))
    for h in range(Hq):
        assert np.allclose(out[h], 10.0 * (h // 2 + 1), atol=1e-12, rtol=0)


def test_one_hot_key_dominates():
    rng = np.random.default_rng(16)
    D, L = 128, 50
    q = _rand(rng, 1, D)
    K = 0.01 * _rand(rng, L, 1, D)
    K[17, 0] = 50.0 * q[0] / np.linalg.norm(q[0])
    V = _rand(rng, L, 1, D)
    out = attention.attend(q, K, V, 1.0 / math.sqrt(D))
    assert np.max(np.abs(out[0] - V[17, 0])) < 1e-6


def test_empty_context_is_zero():
    out = attention.attend(np.ones((4, 64)), np.zeros((0, 2, 64)), np.zeros((0, 2, 64)), 0.125)
    assert out.shape == (4, 64) and not out.any()


def _build_paged(lengths, Hkv, D, num_blocks, order, seed, cache_dtype="f32", block_size=16):
    rng = np.random.default_rng(seed)
    alloc = BlockAllocatorModel(num_blocks, 64, block_size)
    alloc.set_free_order(order)
    pool = cache.Pool(num_blocks, Hkv, D, cache_dtype, block_size)
    rows = []
    for b, L in enumerate(lengths):
        alloc.create(b)
        slots, pairs = alloc.append_slots(b, L)
        assert not pairs
        K = rng.standard_normal((L, Hkv, D)).astype(np.float32)
        V = rng.standard_normal((L, Hkv, D)).astype(np.float32)
        pool.append(K, V, slots)
        rows.append((K, V))
    tables, lens = alloc.block_tables(range(len(lengths)), 64)
    return pool, np.array(tables), np.array(lens), rows


@pytest.mark.parametrize("cache_dtype", ["f32", "fp8_e4m3"])
def test_paged_equals_contiguous_and_placement_invariant(cache_dtype):
    lengths = [1, 16, 17, 40, 75]
    Hq, Hkv, D = 4, 2, 64
    q = np.random.default_rng(21).standard_normal((len(lengths), Hq, D))
    nb = 40
    outs = []
    for perm_seed in (0, 1, 2):
        order = np.random.default_rng(perm_seed).permutation(nb)
        pool, tables, lens, rows = _build_paged(lengths, Hkv, D, nb, order, seed=5,
                                                cache_dtype=cache_dtype)
        out = attention.decode_paged(q, pool, tables, lens, 1 / math.sqrt(D))
        for b, (K, V) in enumerate(rows):
            Kc, Vc = attention.rows_as_cached(K, V, cache_dtype)
            assert np.array_equal(out[b], attention.attend(q[b], Kc, Vc, 1 / math.sqrt(D)))
        outs.append(out)
    # different physical placement, identical output (bitwise in fp64)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("cache_dtype", ["f32", "int8_int4"])
def test_block_size_does_not_change_the_output(cache_dtype):
    # the same rows in 16-token and in 32-token blocks, placed at random:
    # reading through the tables gives the rows in logical order, so the
    # outputs agree bit for bit, and each row sits at slot bs*table[p//bs] + p%bs
    lengths = [1, 31, 32, 33, 64, 97]
    Hq, Hkv, D = 4, 2, 64
    q = np.random.default_rng(22).standard_normal((len(lengths), Hq, D))
    outs = []
    for bs, nb in ((16, 60), (32, 30)):
        order = np.random.default_rng(bs).permutation(nb)
        pool, tables, lens, rows = _build_paged(lengths, Hkv, D, nb, order, seed=6,
                                                cache_dtype=cache_dtype, block_size=bs)
        assert pool.k.shape[2] == bs
        for b, (K, V) in enumerate(rows):
            Kc, _ = attention.rows_as_cached(K, V, cache_dtype)
            for p in (0, lengths[b] - 1):
                sl = cache.slot_of(tables[b], p, bs)
                assert sl == bs * tables[b][p // bs] + p % bs
                assert np.array_equal(pool.read_slots([sl // bs], [sl % bs])[0][0], Kc[p])
        outs.append(attention.decode_paged(q, pool, tables, lens, 1 / math.sqrt(D)))
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("P", [16, 64, 512, 4096])
def test_partitioned_merge_equals_plain(P):
    rng = np.random.default_rng(31)
    Hq, Hkv, D, L = 8, 2, 128, 1000
    q, K, V = _rand(rng, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    plain = attention.attend(q, K, V, 1 / math.sqrt(D))
    part = attention.attend_partitioned(q, K, V, 1 / math.sqrt(D), P)
    assert np.max(np.abs(plain - part)) < 1e-12


def test_combine_ignores_empty_partitions():
    rng = np.random.default_rng(32)
    Hq, Hkv, D, L = 4, 1, 64, 30
    q, K, V = _rand(rng, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    s0 = attention.partition_state(q, K, V, 0.125, 0, 16)
    s1 = attention.partition_state(q, K, V, 0.125, 16, 30)
    s2 = attention.partition_state(q, K, V, 0.125, 30, 30)       # empty
    assert np.all(np.isneginf(s2[0])) and not s2[1].any()
    merged = attention.combine_partitions(*zip(s0, s1, s2))
    assert np.max(np.abs(merged - attention.attend(q, K, V, 0.125))) < 1e-13
    assert not attention.combine_partitions(*zip(s2, s2)).any()
