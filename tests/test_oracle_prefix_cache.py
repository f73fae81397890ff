"""Pins of the prefix-caching allocator model (CPU only).

The model keys blocks by whole token prefixes ("KV Cache优化实战" §5.2-5.3;
"企业官网建设流程全解析" §6.2-6.3).  These tests pin it to things other
than itself:
  * a hand-worked request sequence whose tables, hits and evictions were
    worked out on paper, in which leaf-first eviction and plain
    least-recently-used eviction pick different blocks;
  * a shadow of every physical slot holding the prefix its K/V row stands
    for: a cache hit must hand out only slots whose shadow equals the new
    prompt's prefix (a key that forgot the earlier blocks, or eviction of a
    block still in use, breaks this);
  * brute force: with no eviction and requests served one at a time, the hit
    count is the longest run of leading full blocks shared with any earlier
    request's token stream;
  * the structural invariants the eviction rule guarantees.
"""
import numpy as np
import pytest

from oracle.allocator import BLOCK_TOKENS, AllocError, PrefixCachingAllocatorModel

B = BLOCK_TOKENS


def blk(v, bs=B):
    return [v] * bs


# ---- hand-worked example ------------------------------------------------------

def hand_worked(alloc, bs=B):
    """Runs the paper example on ``alloc`` (model or native, blocks of ``bs``
    tokens) and returns what each step observed.  Pool of 5 blocks, block 0
    handed out first; a, b, ... are blocks of bs equal tokens.

    r1 = a b c x: no hit; blocks 0,1,2 indexed (a, ab, abc), 3 partial.
    free r1: 0,1,2 evictable with stamps 1,2,3; 3 back on the free list.
    r2 = a b d y: hits blocks 0,1; takes 3 (free) for d and 4 for y; 3 is
    indexed as abd.  Free list now empty, evictable {2}.
    r3 = e f z while r2 lives: needs 3 blocks, 1 available -> refused.
    free r2: 0,1,3 evictable with stamps 4,5,6; 4 free.  Leaves: 2 (abc,
    stamp 3) and 3 (abd, stamp 6); 0 and 1 have indexed children.
    r3 again: takes 4 (free), then evicts 2, then 3 - plain LRU would have
    evicted 2 and then 0, the root both chains hang from.
    r4 = a b c w: abc is gone, a and ab remain -> 2 blocks hit.
    """
    a, b, c, d, e, f = (blk(v, bs) for v in (11, 12, 13, 14, 15, 16))
    seen = {}
    p1 = a + b + c + [1]
    seen["r1_hit"] = alloc.create_cached(1, p1)
    seen["r1_slots"] = alloc.append_tokens(1, p1)[0]
    alloc.free_seq(1) if hasattr(alloc, "free_seq") else alloc.free(1)
    p2 = a + b + d + [2]
    seen["r2_hit"] = alloc.create_cached(2, p2)
    seen["r2_slots"] = alloc.append_tokens(2, p2[seen["r2_hit"]:])[0]
    p3 = e + f + [3]
    assert alloc.create_cached(3, p3) == 0
    try:
        alloc.append_tokens(3, p3)
        seen["r3_refused"] = False
    except Exception as err:          # AllocError or PagedKVError
        seen["r3_refused"] = getattr(err, "kind", getattr(err, "code", None))
    alloc.free_seq(2) if hasattr(alloc, "free_seq") else alloc.free(2)
    seen["r3_slots"] = alloc.append_tokens(3, p3)[0]
    p4 = a + b + c + [4]
    seen["r4_hit"] = alloc.create_cached(4, p4)
    seen["prefix"] = alloc.prefix_stats()
    return seen


def expected_hand(bs=B):
    return {
        "r1_hit": 0,
        "r1_slots": list(range(0, 3 * bs + 1)),                              # blocks 0,1,2,3
        "r2_hit": 2 * bs,
        "r2_slots": list(range(3 * bs, 4 * bs)) + [4 * bs],                  # block 3 then block 4
        "r3_slots": list(range(4 * bs, 5 * bs)) + list(range(2 * bs, 3 * bs)) + [3 * bs],   # blocks 4, 2, 3
        "r4_hit": 2 * bs,
    }


EXPECTED_HAND = expected_hand()


@pytest.mark.parametrize("bs", [16, 32])
def test_hand_worked_leaf_first_eviction(bs):
    m = PrefixCachingAllocatorModel(5, 8, block_size=bs)
    seen = hand_worked(m, bs)
    for k, v in expected_hand(bs).items():
        assert seen[k] == v, k
    assert seen["r3_refused"] == "no_free_blocks"
    assert m.tables[3] == [4, 2, 3] and m.tables[4] == [0, 1]
    assert seen["prefix"] == {"cached_blocks": 4, "evictable_blocks": 0, "lookup_blocks": 3 + 3 + 2 + 3,
                              "hit_blocks": 4, "evictions": 2}


def test_lookup_never_covers_the_last_prompt_token():
    m = PrefixCachingAllocatorModel(8, 8)
    p = blk(1) + blk(2)
    m.create_cached(0, p)
    m.append_tokens(0, p)
    assert m.create_cached(1, p) == 16           # (32 - 1) // 16 = 1 block
    assert m.create_cached(2, p + [5]) == 32
    assert m.create_cached(3, blk(1)) == 0       # a one-block prompt never hits
    assert m.create_cached(4, []) == 0


def test_lookup_bound_with_32_token_blocks():
    # the same two 16-token runs form one 32-token block: a 32-token prompt
    # never hits, a 33-token one hits the whole block
    m = PrefixCachingAllocatorModel(8, 8, block_size=32)
    p = blk(1) + blk(2)
    m.create_cached(0, p + [3])
    m.append_tokens(0, p + [3])
    assert m.create_cached(1, p) == 0            # (32 - 1) // 32 = 0 blocks
    assert m.create_cached(2, p + [5]) == 32
    assert m.create_cached(3, blk(1) + blk(9) + [5]) == 0
    assert len(m.index) == 1


def test_model_key_separates_caches():
    # same tokens under a different key is a different prefix
    m = PrefixCachingAllocatorModel(8, 8, model_key=7)
    p = blk(1) + blk(2) + [3]
    m.create_cached(0, p)
    m.append_tokens(0, p)
    assert m.create_cached(1, p) == 32
    assert all(k[0] == 7 for k in m.index)


def test_append_without_tokens_stops_indexing():
    m = PrefixCachingAllocatorModel(8, 8)
    m.create(0)
    m.append_tokens(0, blk(1))
    m.append_slots(0, 20)                        # untracked from here on
    m.append_tokens(0, [9] * 12)
    assert len(m.index) == 1


# ---- shadow content over random streams -------------------------------------------

def _stream(seed, n_ops=600, pool=40, sys_prompts=3, vocab=3, shared=True):
    """Random request stream: prompts start with one of a few system prompts
    and go on with tokens from a tiny vocabulary, so equal blocks at
    different depths are common; sequences grow, fork and finish under pool
    pressure.  Yields ops; the model and the native allocator replay them."""
    rng = np.random.default_rng(seed)
    systems = [list(rng.integers(100, 100 + vocab, size=int(rng.integers(20, 70)))) for _ in range(sys_prompts)]
    live, nxt = [], 0
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.3 or not live:
            if shared:
                sysp = systems[int(rng.integers(sys_prompts))]
            else:                                           # private prompts: blocks rarely shared
                sysp = list(rng.integers(1000, 100000, size=int(rng.integers(20, 70))))
            prompt = sysp + list(rng.integers(0, vocab, size=int(rng.integers(1, 40))))
            yield ("request", nxt, [int(t) for t in prompt])
            live.append(nxt)
            nxt += 1
        elif r < 0.5:
            yield ("free", live.pop(int(rng.integers(len(live)))))
        elif r < 0.56:
            p = live[int(rng.integers(len(live)))]
            yield ("fork", p, nxt)
            live.append(nxt)
            nxt += 1
        elif r < 0.62:
            s = live[int(rng.integers(len(live)))]
            yield ("append_slots", s, int(rng.integers(1, 20)))
        elif r < 0.66:
            yield ("swap", live[int(rng.integers(len(live)))])
        elif r < 0.8:
            ids = [live[i] for i in rng.permutation(len(live))[:int(rng.integers(1, len(live) + 1))]]
            yield ("batch", ids, [int(t) for t in rng.integers(0, vocab, size=len(ids))])
        else:
            s = live[int(rng.integers(len(live)))]
            yield ("generate", s, [int(t) for t in rng.integers(0, vocab, size=int(rng.integers(1, 24)))])


class Shadow:
    """slot -> the token prefix whose last position's K/V the slot holds."""

    def __init__(self, bs=B):
        self.bs = bs
        self.slot = {}
        self.stream = {}

    def wrote(self, seq, slots):
        toks = self.stream[seq]
        base = len(toks) - len(slots)
        for i, s in enumerate(slots):
            self.slot[s] = tuple(toks[:base + i + 1])

    def copied(self, pairs):
        bs = self.bs
        for src, dst in pairs:
            for o in range(bs):
                if bs * src + o in self.slot:
                    self.slot[bs * dst + o] = self.slot[bs * src + o]


_CODES = {-1: "invalid_arg", -5: "no_free_blocks", -6: "unknown_seq"}


def error_kind(e):
    if isinstance(e, AllocError):
        return e.kind
    code = getattr(e, "code", None)
    if code in _CODES:
        return _CODES[code]
    raise e


def replay(alloc, ops, shadow=None, check=None):
    """Applies ops to ``alloc``; returns the observed results (for comparing
    the model and the native allocator) and keeps ``shadow`` up to date."""
    out = []
    free = alloc.free_seq if hasattr(alloc, "free_seq") else alloc.free
    for op in ops:
        kind = op[0]
        try:
            if kind == "request":
                _, s, prompt = op
                n = alloc.create_cached(s, prompt)
                if shadow is not None:
                    shadow.stream[s] = list(prompt[:n])
                    if check:
                        check(alloc, s, prompt, n)
                slots, pairs = alloc.append_tokens(s, prompt[n:])
                if shadow is not None:
                    shadow.stream[s] = list(prompt)
                    shadow.copied(pairs)
                    shadow.wrote(s, slots)
                out.append((kind, n, slots, pairs))
            elif kind == "free":
                free(op[1])
                out.append((kind,))
            elif kind == "fork":
                alloc.fork(op[1], op[2])
                if shadow is not None:
                    shadow.stream[op[2]] = list(shadow.stream[op[1]])
                out.append((kind,))
            elif kind == "append_slots":
                slots, pairs = alloc.append_slots(op[1], op[2])
                if shadow is not None:
                    shadow.copied(pairs)
                    shadow.stream[op[1]] += [None] * op[2]
                    shadow.wrote(op[1], slots)
                out.append((kind, slots, pairs))
            elif kind == "batch":
                ids, toks = op[1], op[2]
                slots, pairs = alloc.batch_append_tokens(ids, toks)
                if shadow is not None:
                    shadow.copied(pairs)
                    for s, t, sl in zip(ids, toks, slots):
                        shadow.stream[s].append(t)
                        shadow.wrote(s, [sl])
                out.append((kind, slots, pairs))
            elif kind == "swap":
                s = op[1]
                out_set = alloc.__dict__.setdefault("_test_swapped", set())
                if s in out_set:
                    blocks = alloc.swap_in(s)
                    out_set.discard(s)
                    if shadow is not None:
                        toks, bs = shadow.stream[s], shadow.bs
                        for p in range(len(toks)):
                            shadow.slot[bs * blocks[p // bs] + p % bs] = tuple(toks[:p + 1])
                else:
                    blocks = alloc.swap_out(s)
                    out_set.add(s)
                out.append((kind, blocks))
            elif kind == "generate":
                slots, pairs = alloc.append_tokens(op[1], op[2])
                if shadow is not None:
                    shadow.copied(pairs)
                    shadow.stream[op[1]] += op[2]
                    shadow.wrote(op[1], slots)
                out.append((kind, slots, pairs))
        except Exception as e:             # the model's AllocError or the library's error
            out.append((kind, "error", error_kind(e)))
        if kind == "free":
            alloc.__dict__.setdefault("_test_swapped", set()).discard(op[1])
        if kind == "free" and shadow is not None:
            shadow.stream.pop(op[1], None)
    return out


def _hit_check(shadow):
    bs = shadow.bs

    def check(m, s, prompt, n):
        assert n % bs == 0 and n <= max(len(prompt) - 1, 0)
        for p in range(n):
            slot = bs * m.tables[s][p // bs] + p % bs
            assert shadow.slot.get(slot) == tuple(prompt[:p + 1]), (s, p)
    return check


def _invariants(m):
    for key, b in m.index.items():
        assert m.key_of[b] == key
        if len(key) > 1 + m.bs:
            assert key[:-m.bs] in m.index                          # parents stay indexed
    for b in m.evictable:
        assert m.ref[b] == 0 and b in m.key_of
    assert len(m.free) + len(m.evictable) + sum(1 for r in m.ref if r > 0) == m.num_blocks


@pytest.mark.parametrize("seed,bs", [(s, 16) for s in range(6)] + [(s, 32) for s in (0, 1, 4)])
def test_hits_hold_the_right_content_under_pressure(seed, bs):
    m = PrefixCachingAllocatorModel(40 * 16 // bs, 12 * 16 // bs, block_size=bs)
    shadow = Shadow(bs)
    ops = list(_stream(seed, shared=seed < 4))
    res = replay(m, ops, shadow, _hit_check(shadow))
    _invariants(m)
    st = m.prefix_stats()
    if seed < 4:
        assert st["hit_blocks"] > 20 and st["evictions"] > 320 // bs // (bs // 16), st   # exercises both
    else:
        assert sum(1 for r in res if r[0] == "swap" and r[1] != "error") > 5   # swaps go through
    assert any(r[1:2] == ("error",) for r in res)


# ---- brute force with no eviction ---------------------------------------------------

@pytest.mark.parametrize("seed,B", [(s, 16) for s in range(4)] + [(s, 32) for s in range(2)])
def test_hits_equal_brute_force_longest_shared_prefix(seed, B):
    rng = np.random.default_rng(50 + seed)
    m = PrefixCachingAllocatorModel(4096, 64, block_size=B)
    systems = [list(rng.integers(0, 4, size=int(rng.integers(10, 60)))) for _ in range(4)]
    done = []                                    # full token streams of finished requests
    for r in range(120):
        prompt = systems[int(rng.integers(4))] + list(rng.integers(0, 4, size=int(rng.integers(1, 50))))
        if len(prompt) % B == 0:
            prompt.append(1)                     # keep the bound from cutting a cached block
        prompt = [int(t) for t in prompt]
        best = 0
        for stream in done:
            full = len(stream) // B
            k = 0
            while k < min(full, (len(prompt) - 1) // B) and stream[B * k:B * k + B] == prompt[B * k:B * k + B]:
                k += 1
            best = max(best, k)
        n = m.create_cached(r, prompt)
        assert n == B * best, r
        m.append_tokens(r, prompt[n:])
        gen = [int(t) for t in rng.integers(0, 4, size=int(rng.integers(0, 40)))]
        m.append_tokens(r, gen)
        done.append(prompt + gen)
        m.free_seq(r)
    assert m.evictions == 0


def test_refused_batch_changes_nothing():
    # pool of 2: sequence 0 holds both blocks; in the batch its token fits
    # in place but sequence 1 needs a block, so the whole batch is refused
    m = PrefixCachingAllocatorModel(2, 8)
    m.create(0)
    m.create(1)
    m.append_tokens(0, blk(1) + [2])
    before = (dict(m.lens), m.prefix_stats(), m.stats(), list(m.tokens[0]))
    with pytest.raises(AllocError) as e:
        m.batch_append_tokens([0, 1], [4, 5])
    assert e.value.kind == "no_free_blocks"
    assert (dict(m.lens), m.prefix_stats(), m.stats(), list(m.tokens[0])) == before
