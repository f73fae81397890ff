"""Host-side checks of libpagedkv.so that need no GPU: every declared symbol
is exported, the C++ allocator matches the oracle's allocator model
bit-exactly on every workload's setup and on random operation streams, and
invalid arguments are rejected on the host before anything is enqueued."""
import ctypes
import math
import os
import re

import numpy as np
import pytest
import torch

import paged_kv_cache_160_amd as pkv
from paged_kv_cache_160_amd import _lib
import workloads as wl
from oracle.allocator import AllocError, BlockAllocatorModel

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pagedkv.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("kv_cache_append", "paged_attention_decode", "paged_attention_workspace_size",
                     "pkv_copy_blocks", "pkv_alloc_create", "pkv_seq_append_slots"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding declares a signature for each of them
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_strerror_and_version():
    lib = _lib.lib()
    assert lib.pkv_abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert lib.pkv_strerror(code)
    assert lib.pkv_strerror(-99) == b"unknown error code"


# ---- allocator: C++ vs the oracle model ------------------------------------------

def _run_both(w, ops):
    model = BlockAllocatorModel(w.num_blocks, w.max_blocks_per_seq, w.block_size)
    native = pkv.BlockAllocator(w.num_blocks, w.max_blocks_per_seq, w.block_size)
    for op in ops:
        kind = op[0]
        if kind == "free_order":
            model.set_free_order(op[1])
            native.set_free_order(op[1])
        elif kind == "create":
            model.create(op[1]); native.create(op[1])
        elif kind == "fork":
            model.fork(op[1], op[2]); native.fork(op[1], op[2])
        elif kind == "free":
            model.free_seq(op[1]); native.free(op[1])
        elif kind == "append":
            a = model.append_slots(op[1], op[2])
            b = native.append_slots(op[1], op[2])
            assert a == b, op
    return model, native


@pytest.mark.parametrize("cid,bs", [(c, 16) for c in (1, 2, 3, 4, 5)] + [(c, 32) for c in (1, 2, 4, 5)])
def test_allocator_matches_model_on_workload_setup(cid, bs):
    w = wl.with_block_size(wl.make_workload(cid), bs)
    model, native = _run_both(w, wl.setup_ops(w))
    seqs = list(range(w.num_seqs))
    mt, ml = model.block_tables(seqs, w.max_blocks_per_seq)
    nt, nl = native.block_tables(seqs)
    assert np.array_equal(np.array(mt, dtype=np.int32), nt.numpy())
    assert ml == nl.tolist() == w.context_lens
    ms, ns = model.stats(), native.stats()
    for k in ms:
        assert ms[k] == pytest.approx(ns[k]), k
    # with long sequences the last-block waste is small: utilisation > 90%
    # ("KV Cache 和 vLLM" §3.1 reports above 90% for paged storage)
    if cid >= 2:
        assert ns["utilisation"] > 0.9


def test_workload4_copy_on_write_pairs():
    w = wl.make_workload(4)
    model, native = _run_both(w, wl.setup_ops(w))
    st = native.stats()
    # 8 holders of the partial prefix block: the first 7 appenders copy it
    assert st["cow_copies"] == 7
    assert st["shared_blocks"] == 1500 // 16


def test_batch_append_matches_sequential_model():
    w = wl.make_workload(4)
    model, native = _run_both(w, wl.setup_ops(w))
    seqs = list(range(w.num_seqs))
    for _ in range(40):
        exp_slots, exp_pairs = [], []
        for s in seqs:
            sl, pr = model.append_slots(s, 1)
            exp_slots += sl
            exp_pairs += pr
        got_slots, got_pairs = native.batch_append_one(seqs)
        assert got_slots == exp_slots and got_pairs == exp_pairs


def test_batch_append_shared_block_counts_exact():
    # 3 forks of a 5-token sequence share its partial block: a batch step
    # copies for the first three holders and writes in place for the last,
    # so exactly 3 fresh blocks are needed: a pool of 4 is just enough.
    native = pkv.BlockAllocator(4, 4)
    native.create(0)
    native.append_slots(0, 5)
    for c in (1, 2, 3):
        native.fork(0, c)
    slots, pairs = native.batch_append_one([0, 1, 2, 3])
    assert len(pairs) == 3 and native.stats()["free_blocks"] == 0
    assert [s % 16 for s in slots] == [5, 5, 5, 5]


@pytest.mark.parametrize("seed,bs", [(s, 16) for s in range(4)] + [(s, 32) for s in range(3)])
def test_allocator_random_streams_match_model(seed, bs):
    rng = np.random.default_rng(100 + seed + bs)
    nb, mb = 48 * 16 // bs, 12 * 16 // bs
    model = BlockAllocatorModel(nb, mb, bs)
    native = pkv.BlockAllocator(nb, mb, bs)
    assert native.block_size == bs
    order = rng.permutation(nb)
    model.set_free_order(order)
    native.set_free_order(order)
    live, nxt = [], 0
    swapped = set()
    for _ in range(2000):
        r = rng.random()
        if r < 0.15 or not live:
            model.create(nxt); native.create(nxt); live.append(nxt); nxt += 1
        elif r < 0.3:
            s = live.pop(int(rng.integers(len(live))))
            model.free_seq(s); native.free(s)
            swapped.discard(s)
        elif r < 0.4:
            p = live[int(rng.integers(len(live)))]
            if p in swapped:
                continue
            model.fork(p, nxt); native.fork(p, nxt); live.append(nxt); nxt += 1
        elif r < 0.47:
            s = live[int(rng.integers(len(live)))]
            op = "swap_in" if s in swapped else "swap_out"
            try:
                exp = getattr(model, op)(s)
            except AllocError as e:
                with pytest.raises(pkv.PagedKVError) as got:
                    getattr(native, op)(s)
                assert got.value.code == {"no_free_blocks": -5, "invalid_arg": -1}[e.kind]
                continue
            assert getattr(native, op)(s) == exp
            swapped.symmetric_difference_update({s})
        else:
            s = live[int(rng.integers(len(live)))]
            n = int(rng.integers(0, 40))
            if s in swapped:
                with pytest.raises(pkv.PagedKVError) as got:
                    native.append_slots(s, n)
                assert got.value.code == -1
                continue
            try:
                exp = model.append_slots(s, n)
            except AllocError as e:
                with pytest.raises(pkv.PagedKVError) as got:
                    native.append_slots(s, n)
                assert got.value.code == {"no_free_blocks": -5, "invalid_arg": -1}[e.kind]
                continue
            assert native.append_slots(s, n) == exp
        assert model.stats() == pytest.approx(native.stats())


def test_allocator_errors_leave_state_unchanged():
    a = pkv.BlockAllocator(2, 8)
    a.create(1)
    a.append_slots(1, 20)
    before = (a.block_tables([1]), a.stats())
    with pytest.raises(pkv.PagedKVError) as e:
        a.append_slots(1, 13)           # needs a third block
    assert e.value.code == -5
    after = (a.block_tables([1]), a.stats())
    assert before[1] == after[1] and np.array_equal(before[0][0], after[0][0])
    with pytest.raises(pkv.PagedKVError) as e:
        a.append_slots(7, 1)
    assert e.value.code == -6
    with pytest.raises(pkv.PagedKVError) as e:
        a.create(1)
    assert e.value.code == -1
    with pytest.raises(pkv.PagedKVError):
        a.batch_append_one([1, 1])
    assert _lib.lib().pkv_alloc_create(0, 4) is None


# ---- argument validation of the device calls (host side only) ---------------------

FAKE = 1 << 20          # an aligned non-null address; never dereferenced here


def _decode(**kw):
    args = dict(out=FAKE, q=FAKE, k_pool=FAKE, v_pool=FAKE, k_scale=None, v_scale=None,
                block_tables=FAKE, context_lens=FAKE, num_seqs=4, num_q_heads=32, num_kv_heads=8,
                head_dim=128, num_blocks=64, max_blocks_per_seq=8, max_context_len=128, scale=0.1,
                q_dtype=pkv.PKV_BF16, cache_dtype=pkv.PKV_BF16, partition_size=0,
                workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    return _lib.lib().paged_attention_decode(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), -2),
    (dict(num_q_heads=30), -1),
    (dict(num_q_heads=8 * 17), -2),
    (dict(q_dtype=pkv.PKV_F16), -2),
    (dict(q_dtype=pkv.PKV_F32, cache_dtype=pkv.PKV_FP8_E4M3), -2),
    (dict(cache_dtype=pkv.PKV_FP8_E4M3), -1),             # fp8 without scales
    (dict(max_context_len=8 * 16 + 1), -1),
    (dict(partition_size=24), -1),
    (dict(q=FAKE + 4), -1),
    (dict(q=None), -1),
    (dict(q_dtype=7), -1),
    (dict(max_context_len=4096, max_blocks_per_seq=256, partition_size=512), -3),
])
def test_decode_rejects_bad_arguments(kw, code):
    assert _decode(**kw) == code


def test_decode_empty_batch_is_noop():
    assert _decode(num_seqs=0) == 0


def test_append_and_copy_reject_bad_arguments():
    L = _lib.lib()
    # dtype mismatch, unsupported head_dim, fp8 without scales
    assert L.kv_cache_append(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 4, 8, 128, 64,
                             pkv.PKV_F16, pkv.PKV_BF16, None) == -2
    assert L.kv_cache_append(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 4, 8, 80, 64,
                             pkv.PKV_BF16, pkv.PKV_BF16, None) == -2
    assert L.kv_cache_append(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 4, 8, 128, 64,
                             pkv.PKV_F32, pkv.PKV_FP8_E4M3, None) == -1
    assert L.kv_cache_append(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 0, 8, 128, 64,
                             pkv.PKV_BF16, pkv.PKV_BF16, None) == 0
    assert L.pkv_copy_blocks(FAKE, FAKE, None, None, FAKE, 2, 8, 128, 64,
                             pkv.PKV_FP8_E4M3, None) == -1
    assert L.pkv_copy_blocks(FAKE, FAKE, None, None, FAKE, 0, 8, 128, 64,
                             pkv.PKV_BF16, None) == 0


def test_partition_plan_and_workspace():
    for (B, hq, hkv, L) in [(16, 32, 8, 4096), (32, 32, 8, 32768), (64, 32, 32, 2048), (4, 4, 2, 41)]:
        ps, npart = pkv.decode_partition_size(B, hq, hkv, 128, L, pkv.PKV_BF16)
        assert ps % 16 == 0 and ps > 0 and npart == -(-L // ps)
        ws = pkv.workspace_size(B, hq, hkv, 128, L, 0, pkv.PKV_BF16)
        if npart == 1:
            # a workspace only for the longest-first order of launches of
            # >= 1024 workgroups over more than 256 sequences: after the
            # counter area, one int32 per sequence
            ordered = 256 < B <= pkv.MAX_ORDER_SEQS and B * hkv >= 1024
            assert ws == (pkv.WS_COUNTER_BYTES + -(-4 * B // 256) * 256 if ordered else 0), (B, hkv, L, ws)
        else:
            assert ws >= pkv.WS_COUNTER_BYTES + B * hq * npart * (128 + 2) * 4
    assert pkv.workspace_size(16, 32, 8, 128, 4096, 16, pkv.PKV_BF16) >= 16 * 32 * 256 * 130 * 4


def test_partition_plan_of_the_benched_workloads():
    # the Llama-3-8B layer shape after the bench's first appends: two
    # partitions, 256 workgroups; 32 x 32768 tokens: eight partitions of
    # 4112 tokens (65 blocks per wave, 2048 workgroups) in every cache format
    assert pkv.decode_partition_size(16, 32, 8, 128, 4100, pkv.PKV_BF16) == (2064, 2)
    for cache in (pkv.PKV_BF16, pkv.PKV_FP8_E4M3, pkv.PKV_INT8_INT4):
        assert pkv.decode_partition_size(32, 32, 8, 128, 32769, cache) == (4112, 8)
    # int8 K + int4 V asks for two workgroups per CU: four partitions here
    assert pkv.decode_partition_size(16, 32, 8, 128, 4100, pkv.PKV_INT8_INT4) == (1040, 4)


def test_counter_area_size_matches_header():
    # the binding's constant is the header's PKV_WS_COUNTER_BYTES
    with open(HEADER, encoding="utf-8") as f:
        text = f.read()
    units = int(re.search(r"#define PKV_WS_COUNTER_UNITS (\d+)", text).group(1))
    assert re.search(r"#define PKV_WS_COUNTER_BYTES \(PKV_WS_COUNTER_UNITS \* 8\)", text)
    assert pkv.WS_COUNTER_BYTES == units * 8
    assert pkv.MAX_ORDER_SEQS == int(re.search(r"#define PKV_MAX_ORDER_SEQS (\d+)", text).group(1))


def test_swap_hand_worked_matches_model():
    # the same sequence as the model's hand-worked swap pin
    a = pkv.BlockAllocator(6, 8)
    a.create(0)
    a.append_slots(0, 40)
    a.create(1)
    a.append_slots(1, 20)
    assert a.swap_out(0) == [0, 1, 2]
    assert a.seq_len(0) == 40 and a.stats()["cached_tokens"] == 20
    for bad in (lambda: a.append_slots(0, 1), lambda: a.block_tables([0]), lambda: a.fork(0, 9),
                lambda: a.swap_out(0), lambda: a.create(0), lambda: a.batch_append_one([1, 0])):
        with pytest.raises(pkv.PagedKVError) as e:
            bad()
        assert e.value.code == -1
    a.create(2)
    a.append_slots(2, 33)
    assert a.block_tables([2])[0][0, :3].tolist() == [2, 1, 0]
    with pytest.raises(pkv.PagedKVError) as e:
        a.swap_in(0)
    assert e.value.code == -5
    a.free(2)
    assert a.swap_in(0) == [0, 1, 2]
    assert a.block_tables([0])[1].tolist() == [40]
    a.fork(0, 3)
    with pytest.raises(pkv.PagedKVError) as e:
        a.swap_out(0)                    # shared blocks stay
    assert e.value.code == -1


def test_block_size_is_16_or_32():
    for bad in (0, 8, 24, 64):
        with pytest.raises(pkv.PagedKVError):
            pkv.BlockAllocator(4, 4, block_size=bad)
    lib = pkv._lib.lib()
    assert lib.pkv_alloc_block_size(None) == -1
    # device calls check the block size on the host before anything else runs
    assert lib.kv_cache_append_bs(None, None, None, None, None, None, None, 1, 1, 64, 4, 24,
                                  pkv.PKV_BF16, pkv.PKV_BF16, None) == -1
    assert lib.pkv_copy_blocks_bs(None, None, None, None, None, 1, 1, 64, 4, 64, pkv.PKV_BF16, None) == -1
    assert lib.paged_attention_decode_bs(None, None, None, None, None, None, None, None, 1, 4, 1, 64, 4, 8,
                                         4, 64, 0.125, pkv.PKV_BF16, pkv.PKV_BF16, 0, None, 0, None) == -1
    assert lib.paged_attention_merge_partials_bs(None, None, 1, 4, 1, 64, 48, 4, 64, pkv.PKV_BF16, pkv.PKV_BF16, 0,
                                                 None, 0, None) == -1
    assert lib.paged_attention_prefill_bs(None, None, None, None, None, None, None, None, None, 1, 1, 4, 1, 64, 4,
                                          8, 4, 64, 1, 0.125, pkv.PKV_BF16, pkv.PKV_BF16, None) == -1
    # 32-token blocks: max_context_len may reach 32 * max_blocks_per_seq, not more
    assert lib.paged_attention_decode_bs(None, None, None, None, None, None, None, None, 0, 4, 1, 64, 4, 32,
                                         4, 128, 0.125, pkv.PKV_BF16, pkv.PKV_BF16, 0, None, 0, None) == 0
    assert lib.paged_attention_decode_bs(None, None, None, None, None, None, None, None, 0, 4, 1, 64, 4, 32,
                                         4, 129, 0.125, pkv.PKV_BF16, pkv.PKV_BF16, 0, None, 0, None) == -1


def test_prefill_refuses_non_positive_scale():
    # the prefill kernel compares raw scores against a threshold scaled by
    # 1/scale, so the host refuses a scale that is not positive and finite
    # (a valid call with no tokens returns 0 before any launch)
    lib = pkv._lib.lib()
    args = lambda scale: (None, None, None, None, None, None, None, None, None, 0, 0, 4, 1, 64, 4, 16, 4, 64, 0,
                          scale, pkv.PKV_BF16, pkv.PKV_BF16, None)
    assert lib.paged_attention_prefill_bs(*args(0.125)) == 0
    for bad in (0.0, -0.125, float("inf"), float("nan")):
        assert lib.paged_attention_prefill_bs(*args(bad)) == -1


def test_device_calls_refuse_host_tensors():
    # a host tensor's address must never reach a kernel: the binding refuses
    # it before calling the library
    pool = torch.zeros((8, 2, 16, 64), dtype=torch.bfloat16)
    rows = torch.zeros((1, 2, 64), dtype=torch.bfloat16)
    slots = torch.zeros(1, dtype=torch.int64)
    with pytest.raises(ValueError, match="GPU"):
        pkv.kv_cache_append(rows, rows, pool, pool, slots)
    q = torch.zeros((1, 4, 64), dtype=torch.bfloat16)
    tables = torch.zeros((1, 4), dtype=torch.int32)
    lens = torch.ones(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        pkv.paged_attention_decode(torch.empty_like(q), q, pool, pool, tables, lens, 1, partition_size=16)


def test_binding_checks_pool_shapes_and_scales_on_the_host():
    # shapes the kernels index are checked before any call: V pool against K
    # pool, and float32 scales [num_blocks, num_kv_heads, block_size] for a
    # quantised cache (the checks come before the device checks, so host
    # tensors suffice here)
    k = torch.zeros((8, 2, 16, 64), dtype=torch.uint8)
    sc = torch.ones((8, 2, 16), dtype=torch.float32)
    assert pkv._pool_code(k, k, sc, sc) == pkv.PKV_FP8_E4M3
    with pytest.raises(ValueError, match="scales"):
        pkv._pool_code(k, k, None, sc)
    with pytest.raises(ValueError, match="scales"):
        pkv._pool_code(k, k, sc, sc.reshape(-1))
    with pytest.raises(ValueError, match="scales"):
        pkv._pool_code(k, k, sc, sc.double())
    with pytest.raises(ValueError, match="blocks"):
        pkv._pool_code(k, k[:4], sc, sc)
    b = torch.zeros((8, 2, 16, 64), dtype=torch.bfloat16)
    assert pkv._pool_code(b, b, None, None) == pkv.PKV_BF16
    with pytest.raises(ValueError, match="head_dim"):
        pkv._pool_code(b, torch.zeros((8, 2, 16, 32), dtype=torch.bfloat16), None, None)
    k8 = torch.zeros((8, 2, 16, 64), dtype=torch.int8)
    v4 = torch.zeros((8, 2, 16, 32), dtype=torch.uint8)
    assert pkv._pool_code(k8, v4, sc, sc) == pkv.PKV_INT8_INT4


def test_sizes_past_the_grid_limit_are_refused():
    # (sequence, query head) rows beyond 2^31 - 1 would overflow the merge
    # grid and the workspace size: refused on the host
    lib = pkv._lib.lib()
    assert lib.paged_attention_workspace_size(1 << 20, 1 << 12, 1 << 8, 128, 4096, 0, pkv.PKV_BF16) == 0
    assert lib.paged_attention_decode_bs(None, None, None, None, None, None, None, None, 1 << 20, 1 << 12, 1 << 8,
                                         128, 4, 16, 256, 4096, 0.125, pkv.PKV_BF16, pkv.PKV_BF16, 0, None, 0,
                                         None) == -1


def test_noalloc_decode_refuses_sizes_beyond_its_scratch():
    # the decode step without a workspace checks its scratch need on the host
    # before any device call (no GPU here: a device call would fail with a
    # HIP error instead)
    lib = pkv._lib.lib()
    B, hq, hkv, D, L, ps = 2, 8, 2, 128, 32768 * 4, 16
    need = pkv.workspace_size(B, hq, hkv, D, L, ps, pkv.PKV_BF16)
    assert need > pkv.SCRATCH_BYTES
    fake = 1 << 20          # never dereferenced
    rc = lib.paged_attention_decode_append_noalloc(fake, fake, fake, fake, fake, fake, None, None, fake, fake, fake,
                                                   B, hq, hkv, D, 64, 16, L // 16, L, 1.0 / math.sqrt(D),
                                                   pkv.PKV_BF16, pkv.PKV_BF16, pkv.PKV_BF16, ps, None)
    assert rc == -8
    assert "scratch" in lib.pkv_strerror(rc).decode()
