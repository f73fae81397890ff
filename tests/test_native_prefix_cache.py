"""The library's prefix cache against the model (CPU only, no GPU calls):
bit-exact slots, copy pairs, hit lengths, errors and statistics over the
hand-worked example and random request streams under pool pressure, also
with the hash cut to a few bits so that most lookups meet colliding
entries ("KV Cache优化实战" §5.2-5.3)."""
import pytest

import paged_kv_cache_160_amd as pkv
from oracle.allocator import PrefixCachingAllocatorModel
from tests.test_oracle_prefix_cache import EXPECTED_HAND, _stream, expected_hand, hand_worked, replay


def _native(nb, mb, model_key=0, hash_bits=64, bs=16):
    a = pkv.BlockAllocator(nb, mb, bs)
    a.enable_prefix_cache(model_key, hash_bits)
    return a


def test_hand_worked_example():
    a = _native(5, 8)
    seen = hand_worked(a)
    for k, v in EXPECTED_HAND.items():
        assert seen[k] == v, k
    assert seen["r3_refused"] == -5
    tables, lens = a.block_tables([3, 4])
    assert tables[0, :3].tolist() == [4, 2, 3] and tables[1, :2].tolist() == [0, 1]
    assert seen["prefix"] == {"cached_blocks": 4, "evictable_blocks": 0, "lookup_blocks": 11,
                              "hit_blocks": 4, "evictions": 2}


def test_hand_worked_example_32_token_blocks():
    a = _native(5, 8, bs=32)
    seen = hand_worked(a, 32)
    for k, v in expected_hand(32).items():
        assert seen[k] == v, k
    assert seen["r3_refused"] == -5


@pytest.mark.parametrize("seed,hash_bits,bs", [(s, h, 16) for s in range(6) for h in (64, 2)] +
                         [(s, h, 32) for s in (0, 1, 4) for h in (64, 2)])
def test_random_streams_match_model(seed, hash_bits, bs):
    ops = list(_stream(seed, n_ops=800, shared=seed < 4))
    nb, mb = 40 * 16 // bs, 12 * 16 // bs
    m = PrefixCachingAllocatorModel(nb, mb, model_key=99, block_size=bs)
    a = _native(nb, mb, model_key=99, hash_bits=hash_bits, bs=bs)
    got, exp = [], []
    for i in range(0, len(ops), 50):
        chunk = ops[i:i + 50]
        exp += replay(m, chunk)
        got += replay(a, chunk)
        assert got == exp, i
        assert a.prefix_stats() == m.prefix_stats()
        assert a.stats() == pytest.approx(m.stats())
    if seed < 4:
        assert m.prefix_stats()["evictions"] > 20 * 16 // bs // (bs // 16) and m.prefix_stats()["hit_blocks"] > 20
    else:
        assert sum(1 for r in exp if r[0] == "swap" and r[1] != "error") > 5


def test_disabled_cache_keeps_plain_behaviour():
    a = pkv.BlockAllocator(4, 4)
    a.create(0)
    a.append_tokens(0, [1] * 16)
    a.free(0)
    assert a.stats()["free_blocks"] == 4                # nothing kept
    assert a.prefix_stats()["cached_blocks"] == 0
    with pytest.raises(pkv.PagedKVError) as e:
        a.create_cached(1, [1] * 17)                    # caching is off
    assert e.value.code == -1


def test_enable_rules():
    a = pkv.BlockAllocator(4, 4)
    for bits in (0, 65):
        with pytest.raises(pkv.PagedKVError):
            a.enable_prefix_cache(0, bits)
    a.create(0)
    with pytest.raises(pkv.PagedKVError):
        a.enable_prefix_cache(0)                        # not idle
    a.free(0)
    a.enable_prefix_cache(0)
    with pytest.raises(pkv.PagedKVError):
        a.enable_prefix_cache(0)                        # twice
    a.create(1)
    with pytest.raises(pkv.PagedKVError) as e:
        a.create_cached(1, [1])                         # live id
    assert e.value.code == -1


def test_batch_error_precedence_matches_model():
    # a failing batch decode-step append reports the error of the first
    # sequence (in the order the batch names them) that is unknown, swapped
    # out or named again, and changes nothing
    from oracle.allocator import AllocError
    codes = {"unknown_seq": -6, "invalid_arg": -1}
    for batch in ([1, 1, 99], [1, 99, 1], [99, 1, 1], [1, 2, 2], [2, 3, 1, 3, 99]):
        for lib_like in (True, False):
            a = _native(16, 8) if lib_like else PrefixCachingAllocatorModel(16, 8)
            for s in (1, 2, 3):
                a.create(s)
                a.append_tokens(s, list(range(20)))
            if lib_like:
                with pytest.raises(pkv.PagedKVError) as e:
                    a.batch_append_tokens(batch, [7] * len(batch))
                got_lib = e.value.code
                assert a.stats()["used_blocks"] == 6 and [a.seq_len(s) for s in (1, 2, 3)] == [20] * 3
            else:
                with pytest.raises(AllocError) as e:
                    a.batch_append_tokens(batch, [7] * len(batch))
                got_model = codes[e.value.kind]
        first_bad = next(s for i, s in enumerate(batch) if s == 99 or s in batch[:i])
        assert got_lib == got_model == (codes["unknown_seq"] if first_bad == 99 else codes["invalid_arg"]), batch
