"""Pins for the oracle's allocator model: hand-worked examples (tables and
slots worked out by hand from the stated rules) and invariants checked after
every operation of long seeded random operation streams."""
import numpy as np
import pytest

from oracle.allocator import AllocError, BlockAllocatorModel


def test_hand_worked_four_sequences():
    a = BlockAllocatorModel(8, 4)
    a.set_free_order([5, 3, 6, 0, 7, 1, 2, 4])
    for s in range(4):
        a.create(s)
    assert a.append_slots(0, 1) == ([80], [])
    assert a.append_slots(1, 16) == (list(range(48, 64)), [])
    assert a.append_slots(2, 17) == (list(range(96, 112)) + [0], [])
    assert a.append_slots(3, 40) == (list(range(112, 128)) + list(range(16, 32)) + list(range(32, 40)), [])
    tables, lens = a.block_tables(range(4), 4)
    assert tables == [[5, 0, 0, 0], [3, 0, 0, 0], [6, 0, 0, 0], [7, 1, 2, 0]]
    assert lens == [1, 16, 17, 40]
    # one appended token each; only sequence 1 crosses into a new block
    assert a.append_slots(0, 1) == ([81], [])
    assert a.append_slots(1, 1) == ([64], [])          # takes block 4, the last free one
    assert a.append_slots(2, 1) == ([1], [])
    assert a.append_slots(3, 1) == ([40], [])
    assert a.stats()["free_blocks"] == 0
    # a block-crossing append with no free block fails and changes nothing
    before = (dict(a.tables), dict(a.lens), list(a.free), list(a.ref))
    with pytest.raises(AllocError) as e:
        a.append_slots(0, 15)
    assert e.value.kind == "no_free_blocks"
    assert before == (dict(a.tables), dict(a.lens), list(a.free), list(a.ref))
    # freeing sequence 2 releases blocks 6 then 0: block 0 is reused first
    a.free_seq(2)
    assert a.append_slots(0, 15) == (list(range(82, 96)) + [0], [])
    assert a.tables[0] == [5, 0]


def test_hand_worked_fork_and_copy_on_write():
    a = BlockAllocatorModel(6, 8)
    a.create(0)
    assert a.append_slots(0, 20) == (list(range(0, 20)), [])
    a.fork(0, 1)
    assert a.ref[:2] == [2, 2]
    # seq 1 writes into the shared partial block 1: copy to block 2 first
    assert a.append_slots(1, 1) == ([36], [(1, 2)])
    assert a.tables[1] == [0, 2] and a.ref[1] == 1
    # seq 0 is now the only holder of block 1: written in place
    assert a.append_slots(0, 1) == ([20], [])
    a.fork(0, 2)
    assert a.ref[0] == 3 and a.ref[1] == 2
    assert a.append_slots(2, 12) == (list(range(53, 64)) + [64], [(1, 3)])
    assert a.tables[2] == [0, 3, 4]
    st = a.stats()
    assert st["used_blocks"] == 5 and st["free_blocks"] == 1 and st["shared_blocks"] == 1
    assert st["cow_copies"] == 2 and st["cached_tokens"] == 21 + 21 + 33
    assert st["stored_tokens"] == 16 + 5 + 5 + 16 + 1
    assert st["utilisation"] == pytest.approx(43 / 80)


def test_full_shared_block_is_never_copied():
    a = BlockAllocatorModel(5, 8)
    a.create(0)
    a.append_slots(0, 32)
    a.fork(0, 1)
    slots, pairs = a.append_slots(1, 1)
    assert pairs == [] and slots == [32] and a.tables[1] == [0, 1, 2]
    assert a.ref[:3] == [2, 2, 1]


def test_errors():
    a = BlockAllocatorModel(4, 2)
    a.create(0)
    with pytest.raises(AllocError) as e:
        a.append_slots(0, 33)                         # needs 3 > max_blocks_per_seq
    assert e.value.kind == "invalid_arg"
    with pytest.raises(AllocError) as e:
        a.append_slots(9, 1)
    assert e.value.kind == "unknown_seq"
    with pytest.raises(AllocError):
        a.create(0)
    with pytest.raises(AllocError):
        a.set_free_order([0, 1, 2, 2])
    a.append_slots(0, 1)
    with pytest.raises(AllocError):
        a.set_free_order([0, 1, 2, 3])                # pool not idle


def _check_invariants(a: BlockAllocatorModel):
    # reference counts equal the number of table entries naming each block
    counts = [0] * a.num_blocks
    for t in a.tables.values():
        for blk in t:
            counts[blk] += 1
    assert counts == a.ref
    # sum of counts = sum over sequences of ceil(L/16)
    assert sum(a.ref) == sum(-(-L // 16) for L in a.lens.values())
    # free + distinct used = pool, and the free list holds no duplicates
    assert len(set(a.free)) == len(a.free)
    used = {b for b in range(a.num_blocks) if a.ref[b] > 0}
    assert used.isdisjoint(a.free) and len(used) + len(a.free) == a.num_blocks
    for s, t in a.tables.items():
        assert len(t) == -(-a.lens[s] // 16)


@pytest.mark.parametrize("seed", range(6))
def test_random_streams_keep_invariants(seed):
    rng = np.random.default_rng(seed)
    a = BlockAllocatorModel(64, 16)
    a.set_free_order(rng.permutation(64))
    live, next_id = [], 0
    for _ in range(1500):
        r = rng.random()
        if r < 0.15 or not live:
            a.create(next_id)
            live.append(next_id)
            next_id += 1
        elif r < 0.30:
            a.free_seq(live.pop(int(rng.integers(len(live)))))
        elif r < 0.40:
            parent = live[int(rng.integers(len(live)))]
            a.fork(parent, next_id)
            live.append(next_id)
            next_id += 1
        else:
            s = live[int(rng.integers(len(live)))]
            n = int(rng.integers(0, 40))
            snapshot = (dict((k, list(v)) for k, v in a.tables.items()), dict(a.lens), list(a.free), list(a.ref))
            try:
                slots, pairs = a.append_slots(s, n)
            except AllocError as e:
                assert e.kind in ("no_free_blocks", "invalid_arg")
                assert snapshot == (dict((k, list(v)) for k, v in a.tables.items()), dict(a.lens), list(a.free), list(a.ref))
                continue
            assert len(slots) == n and len(pairs) <= 1
            # every written slot belongs to a block this sequence alone holds
            for sl in slots:
                assert a.ref[sl // 16] == 1
            # slots are the sequence's positions L-n..L-1 through its table
            L = a.lens[s]
            for i, sl in enumerate(slots):
                p = L - n + i
                assert sl == 16 * a.tables[s][p // 16] + p % 16
            for old, new in pairs:
                assert a.ref[old] >= 1 and a.ref[new] == 1
        _check_invariants(a)


# ---- swap ("KV Cache 和 vLLM" §6.2) ------------------------------------------------

def test_hand_worked_swap_out_and_in():
    # pool of 6, block 0 handed out first.  A = 40 tokens -> blocks 0,1,2;
    # B = 20 tokens -> 3,4; free stack (top last) [5].  Swapping A out
    # releases 0,1,2 in order -> [5,0,1,2]; C (33 tokens) takes 2,1,0.
    # A cannot come back (3 needed, 1 free) until C is freed (released in
    # logical order 2,1,0 -> [5,2,1,0]); then A takes 0,1,2 again.
    m = BlockAllocatorModel(6, 8)
    m.create(0)
    m.append_slots(0, 40)
    m.create(1)
    m.append_slots(1, 20)
    assert m.swap_out(0) == [0, 1, 2]
    assert m.seq_len(0) == 40 and m.free == [5, 0, 1, 2]
    for bad in (lambda: m.append_slots(0, 1), lambda: m.block_tables([0], 8), lambda: m.fork(0, 9),
                lambda: m.swap_out(0), lambda: m.create(0)):
        with pytest.raises(AllocError) as e:
            bad()
        assert e.value.kind == "invalid_arg"
    m.create(2)
    assert m.append_slots(2, 33)[0][:1] == [32] and m.tables[2] == [2, 1, 0]
    with pytest.raises(AllocError) as e:
        m.swap_in(0)
    assert e.value.kind == "no_free_blocks" and m.seq_len(0) == 40
    m.free_seq(2)
    assert m.swap_in(0) == [0, 1, 2]
    assert m.block_tables([0], 8)[1] == [40]
    assert m.stats()["used_blocks"] == 5


def test_swap_out_refuses_shared_blocks():
    m = BlockAllocatorModel(8, 8)
    m.create(0)
    m.append_slots(0, 20)
    m.fork(0, 1)
    before = (dict(m.tables), list(m.free), list(m.ref))
    with pytest.raises(AllocError):
        m.swap_out(0)
    assert (dict(m.tables), list(m.free), list(m.ref)) == before
    m.free_seq(1)
    assert m.swap_out(0) == [0, 1]
    m.free_seq(0)                       # a swapped sequence can be dropped
    assert m.swapped == {} and len(m.free) == 8


# ---- 32-token blocks ("KV Cache 和 vLLM" §6.3) -----------------------------------------

def test_hand_worked_32_token_blocks():
    # free order 4,1,5,0,2,3.  s0: 1 token -> block 4; s1: 33 tokens -> 1, 5;
    # s2: 32 tokens -> 0, then one more -> 2; fork s1 as s3 and append one
    # token: 33 % 32 != 0 and block 5 is shared, so it is copied into 3.
    a = BlockAllocatorModel(6, 4, block_size=32)
    a.set_free_order([4, 1, 5, 0, 2, 3])
    for s in range(3):
        a.create(s)
    assert a.append_slots(0, 1) == ([128], [])
    assert a.append_slots(1, 33) == (list(range(32, 64)) + [160], [])
    assert a.append_slots(2, 32) == (list(range(0, 32)), [])
    assert a.append_slots(2, 1) == ([64], [])
    assert a.block_tables(range(3), 4) == ([[4, 0, 0, 0], [1, 5, 0, 0], [0, 2, 0, 0]], [1, 33, 33])
    a.fork(1, 3)
    assert a.append_slots(3, 1) == ([97], [(5, 3)])
    assert a.tables[3] == [1, 3] and a.ref[5] == 1 and a.ref[1] == 2
    assert a.append_slots(0, 31) == (list(range(129, 160)), [])
    with pytest.raises(AllocError) as e:
        a.append_slots(0, 1)                          # position 32 needs a block; none free
    assert e.value.kind == "no_free_blocks"
    with pytest.raises(AllocError) as e:
        a.append_slots(2, 100)                        # 133 tokens = 5 blocks > 4
    assert e.value.kind == "invalid_arg"
    assert a.append_slots(1, 31) == (list(range(161, 192)), [])   # block 5 is private again
    st = a.stats()
    assert st["used_blocks"] == 6 and st["shared_blocks"] == 1 and st["cow_copies"] == 1
    assert st["cached_tokens"] == 32 + 64 + 33 + 34
    assert st["stored_tokens"] == 32 + 32 + 32 + 32 + 1 + 2
    assert st["utilisation"] == pytest.approx(131 / 192)
    a.free_seq(1)                                     # block 1 -> count 1; block 5 freed
    assert a.append_slots(0, 1) == ([160], []) and a.tables[0] == [4, 5]
    assert a.swap_out(2) == [0, 2] and a.free == [0, 2]
    assert a.swap_in(2) == [2, 0]


def test_block_size_must_be_16_or_32():
    for bad in (8, 24, 64):
        with pytest.raises(AllocError):
            BlockAllocatorModel(4, 4, block_size=bad)


@pytest.mark.parametrize("seed", range(3))
def test_random_streams_with_32_token_blocks(seed):
    rng = np.random.default_rng(100 + seed)
    a = BlockAllocatorModel(40, 10, block_size=32)
    a.set_free_order(rng.permutation(40))
    live, nxt = [], 0
    for _ in range(1200):
        r = rng.random()
        if r < 0.15 or not live:
            a.create(nxt)
            live.append(nxt)
            nxt += 1
        elif r < 0.3:
            a.free_seq(live.pop(int(rng.integers(len(live)))))
        elif r < 0.4:
            a.fork(live[int(rng.integers(len(live)))], nxt)
            live.append(nxt)
            nxt += 1
        else:
            s = live[int(rng.integers(len(live)))]
            n = int(rng.integers(0, 70))
            try:
                slots, pairs = a.append_slots(s, n)
            except AllocError:
                continue
            L = a.lens[s]
            for i, sl in enumerate(slots):
                p = L - n + i
                assert sl == 32 * a.tables[s][p // 32] + p % 32 and a.ref[sl // 32] == 1
        counts = [0] * a.num_blocks
        for t in a.tables.values():
            for b in t:
                counts[b] += 1
        assert counts == a.ref
        for s, t in a.tables.items():
            assert len(t) == -(-a.lens[s] // 32)
        assert len(a.free) + sum(1 for r in a.ref if r > 0) == a.num_blocks
