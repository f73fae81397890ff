"""Reference model of the paged block allocator (host-side, integer only).

What the pages fix:
  * fixed 16-token blocks, allocated on demand: a sequence takes a new
    physical block only when its current one is full, and appends it to the
    end of its block table ("KV Cache 和 vLLM" §3.1; "KV Cache优化实战" §4.2);
  * a finished request returns its blocks, which later requests reuse
    wherever they lie ("KV Cache优化实战" §4.2);
  * requests with a common prefix point their block tables at the same
    physical blocks, stored once; when contents diverge each request gets new
    blocks, and copy-on-write handles writes into shared blocks ("KV Cache 和
    vLLM" §3.3);
  * running out of cache memory must degrade (queue or recompute) rather than
    crash ("企业官网建设流程全解析" §6.4).

Block size: 16 tokens, or 32 ("KV Cache 和 vLLM" §6.3: larger blocks shrink the
block tables of long sequences at the cost of more internal fragmentation for
short ones); every rule below counts positions in blocks of that size.

Readings (the pages leave these open):
  * blocks carry a reference count; fork shares every block of the parent and
    increments each count; free decrements and returns a block at zero;
  * the free list is a stack: ``set_free_order(order)`` makes ``order[0]`` the
    next block handed out; a freed block goes on top (so it is reused first);
    a sequence's blocks are released in logical order 0, 1, 2, ...;
  * an append of n tokens to a sequence of length L: if L % bs != 0 and the
    last block is shared (count > 1) that block is copied first - one fresh
    block is taken, the pair (old, new) is reported for copying, the old count
    is decremented and the table entry repointed; then one fresh block is
    taken for each position p in [L, L+n) with p % bs == 0, in position order;
  * a full shared block is never written and so never copied;
  * an append that needs more fresh blocks than are free, or that would
    exceed ``max_blocks_per_seq``, changes nothing and reports an error;
  * swap ("KV Cache 和 vLLM" §6.2: under memory pressure blocks move out to
    CPU memory and back): ``swap_out`` needs every block of the sequence
    unshared (count 1), reports its blocks in logical order, releases them
    in that order and keeps only the length; ``swap_in`` takes
    ceil(length / bs) fresh blocks in order, all or nothing.  A swapped
    sequence can only be swapped in, freed or asked its length.

Test infrastructure: only tests, the smoke check and the CPU baseline leg of
the benchmark use this module.
"""
from __future__ import annotations

import copy
from typing import Dict, List, Tuple

BLOCK_TOKENS = 16


class AllocError(Exception):
    def __init__(self, kind: str):
        super().__init__(kind)
        self.kind = kind          # "no_free_blocks" | "unknown_seq" | "invalid_arg"


class BlockAllocatorModel:
    def __init__(self, num_blocks: int, max_blocks_per_seq: int, block_size: int = BLOCK_TOKENS):
        if num_blocks <= 0 or max_blocks_per_seq <= 0 or block_size not in (16, 32):
            raise AllocError("invalid_arg")
        self.bs = block_size
        self.num_blocks = num_blocks
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free: List[int] = list(range(num_blocks - 1, -1, -1))   # top = end; block 0 first
        self.ref = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.swapped: Dict[int, int] = {}          # swapped-out sequence -> length
        self.cow_copies = 0

    # -- free list ----------------------------------------------------------
    def set_free_order(self, order) -> None:
        order = [int(x) for x in order]
        if len(self.free) != self.num_blocks:
            raise AllocError("invalid_arg")          # only on an idle pool
        if sorted(order) != list(range(self.num_blocks)):
            raise AllocError("invalid_arg")
        self.free = order[::-1]

    def _available(self) -> int:
        return len(self.free)

    def _take(self) -> int:
        blk = self.free.pop()
        self.ref[blk] = 1
        return blk

    def _release(self, blk: int) -> None:
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            self.free.append(blk)

    # -- sequences ----------------------------------------------------------
    def _live(self, seq: int) -> bool:
        return seq in self.tables or seq in self.swapped

    def _resident(self, seq: int) -> None:
        if seq in self.swapped:
            raise AllocError("invalid_arg")
        if seq not in self.tables:
            raise AllocError("unknown_seq")

    def create(self, seq: int) -> None:
        if self._live(seq):
            raise AllocError("invalid_arg")
        self.tables[seq] = []
        self.lens[seq] = 0

    def fork(self, parent: int, child: int) -> None:
        self._resident(parent)
        if self._live(child):
            raise AllocError("invalid_arg")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for blk in self.tables[child]:
            self.ref[blk] += 1

    def free_seq(self, seq: int) -> None:
        if seq in self.swapped:
            del self.swapped[seq]
            return
        if seq not in self.tables:
            raise AllocError("unknown_seq")
        for blk in self.tables.pop(seq):
            self._release(blk)
        del self.lens[seq]

    def swap_out(self, seq: int) -> List[int]:
        """Blocks of ``seq`` in logical order, released; the sequence keeps
        only its length until ``swap_in``."""
        self._resident(seq)
        table = self.tables[seq]
        if any(self.ref[b] != 1 for b in table):
            raise AllocError("invalid_arg")
        for blk in table:
            self._release(blk)
        del self.tables[seq]
        self.swapped[seq] = self.lens.pop(seq)
        return list(table)

    def swap_in(self, seq: int) -> List[int]:
        """Fresh blocks, in logical order, for the swapped sequence's length."""
        if seq not in self.swapped:
            raise AllocError("unknown_seq" if seq not in self.tables else "invalid_arg")
        L = self.swapped[seq]
        need = -(-L // self.bs)
        if need > self._available():
            raise AllocError("no_free_blocks")
        blocks = [self._take() for _ in range(need)]
        del self.swapped[seq]
        self.tables[seq] = blocks
        self.lens[seq] = L
        return list(blocks)

    def append_slots(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Slots for the next n positions of ``seq`` and the copy pairs the
        caller must apply (before writing) to keep shared blocks intact."""
        self._resident(seq)
        if n < 0:
            raise AllocError("invalid_arg")
        table = self.tables[seq]
        L = self.lens[seq]
        needs_cow = (n > 0 and L % self.bs != 0 and self.ref[table[-1]] > 1)
        new_blocks = -(-(L + n) // self.bs) - -(-L // self.bs)
        if len(table) + new_blocks > self.max_blocks_per_seq:
            raise AllocError("invalid_arg")
        if int(needs_cow) + new_blocks > self._available():
            raise AllocError("no_free_blocks")
        pairs: List[Tuple[int, int]] = []
        if needs_cow:
            old = table[-1]
            new = self._take()
            pairs.append((old, new))
            self.ref[old] -= 1          # still > 0: another sequence holds it
            table[-1] = new
            self.cow_copies += 1
        slots = []
        for p in range(L, L + n):
            if p % self.bs == 0:
                table.append(self._take())
            slots.append(self.bs * table[p // self.bs] + p % self.bs)
        self.lens[seq] = L + n
        return slots, pairs

    def seq_len(self, seq: int) -> int:
        if seq in self.swapped:
            return self.swapped[seq]
        if seq not in self.lens:
            raise AllocError("unknown_seq")
        return self.lens[seq]

    def block_tables(self, seqs, max_blocks: int):
        """Tables ``[n][max_blocks]`` (unused entries 0) and lengths ``[n]``."""
        tables, lens = [], []
        for s in seqs:
            self._resident(s)
            t = self.tables[s]
            if len(t) > max_blocks:
                raise AllocError("invalid_arg")
            tables.append(t + [0] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return tables, lens

    # -- statistics ---------------------------------------------------------
    def stats(self) -> dict:
        """Counts and KV memory utilisation.

        stored_tokens counts every filled physical slot once (a shared block's
        slot is filled if any holder has reached it); utilisation =
        stored_tokens / (bs * used_blocks).  cached_tokens is the logical
        total sum_b L_b."""
        filled: Dict[int, int] = {}
        for s, t in self.tables.items():
            L = self.lens[s]
            for i, blk in enumerate(t):
                f = min(self.bs, L - self.bs * i)
                filled[blk] = max(filled.get(blk, 0), f)
        used = sum(1 for r in self.ref if r > 0)
        stored = sum(filled.values())
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self.free),
            "used_blocks": used,
            "shared_blocks": sum(1 for r in self.ref if r > 1),
            "cow_copies": self.cow_copies,
            "cached_tokens": sum(self.lens.values()),
            "stored_tokens": stored,
            "utilisation": (stored / (self.bs * used)) if used else 0.0,
        }


class PrefixCachingAllocatorModel(BlockAllocatorModel):
    """The allocator with prefix caching; keys are whole token prefixes.

    What the pages fix ("KV Cache优化实战" §5.2-5.3; "企业官网建设流程全解析"
    §6.2-6.3): cached KV blocks are found by their content, keyed by the
    model identity together with the token ids; a new request walks its
    prefix block by block, reuses every block that matches exactly and stops
    at the first that does not; the cache is finite, and what is evicted
    must follow the prefix tree (a block whose prefix is gone is useless), not
    plain access order.

    Readings (the pages leave these open):
      * only full blocks are indexed; the key of a sequence's block i is
        (model key, tokens 0 .. bs*i+bs-1), the whole prefix it ends;
      * a block is indexed when an append that names its tokens fills it,
        unless its key is indexed already (the block then stays private), and
        for i > 0 only if the sequence's block i-1 is the one indexed under
        the shorter key - so whoever holds an indexed block holds its parent;
      * ``create``, ``create_cached`` and ``fork`` of a tracked sequence give
        tracked sequences; an append without tokens (``append_slots``) stops
        tracking the sequence, since the keys of its later blocks are unknown;
      * a lookup matches at most (n_tokens - 1) // bs blocks, so the last
        prompt token is always computed, and takes a reference on each match;
      * an indexed block whose count drops to zero stays indexed and becomes
        evictable, stamped with a counter that rises at each such release;
      * a fresh block comes from the free list while it has any; otherwise
        the evictable block with the smallest stamp among those with no
        indexed child is evicted and reused (leaf first: a chain shrinks from
        its tail, and its head, shared by the most requests, goes last);
      * capacity for an append counts free and evictable blocks.
    """

    def __init__(self, num_blocks: int, max_blocks_per_seq: int, model_key: int = 0,
                 block_size: int = BLOCK_TOKENS):
        super().__init__(num_blocks, max_blocks_per_seq, block_size)
        self.model_key = int(model_key)
        self.index: Dict[tuple, int] = {}          # prefix key -> block
        self.key_of: Dict[int, tuple] = {}         # indexed block -> its key
        self.evictable: Dict[int, int] = {}        # block (count 0, indexed) -> stamp
        self.clock = 0
        self.tokens: Dict[int, List[int]] = {}     # tracked sequences' tokens
        self.lookup_blocks = self.hit_blocks = self.evictions = 0

    def _key(self, toks, nblocks: int) -> tuple:
        return (self.model_key,) + tuple(toks[:self.bs * nblocks])

    def _children(self, blk: int) -> int:
        key = self.key_of[blk]
        return sum(1 for k in self.index if len(k) == len(key) + self.bs and k[:len(key)] == key)

    # -- free list with eviction --------------------------------------------
    def _available(self) -> int:
        return len(self.free) + len(self.evictable)

    def _take(self) -> int:
        if self.free:
            return super()._take()
        _, blk = min((st, b) for b, st in self.evictable.items() if self._children(b) == 0)
        del self.evictable[blk]
        del self.index[self.key_of.pop(blk)]
        self.evictions += 1
        self.ref[blk] = 1
        return blk

    def _release(self, blk: int) -> None:
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            if blk in self.key_of:
                self.clock += 1
                self.evictable[blk] = self.clock
            else:
                self.free.append(blk)

    # -- sequences ----------------------------------------------------------
    def create(self, seq: int) -> None:
        super().create(seq)
        self.tokens[seq] = []

    def create_cached(self, seq: int, tokens) -> int:
        """New tracked sequence holding the longest indexed prefix of
        ``tokens``; returns its length (a multiple of bs)."""
        if self._live(seq):
            raise AllocError("invalid_arg")
        tokens = [int(t) for t in tokens]
        most = min(max(len(tokens) - 1, 0) // self.bs, self.max_blocks_per_seq)
        hits = []
        for i in range(most):
            blk = self.index.get(self._key(tokens, i + 1))
            if blk is None:
                break
            hits.append(blk)
        self.lookup_blocks += most
        self.hit_blocks += len(hits)
        for blk in hits:
            if self.ref[blk] == 0:
                del self.evictable[blk]
            self.ref[blk] += 1
        n = self.bs * len(hits)
        self.tables[seq] = hits
        self.lens[seq] = n
        self.tokens[seq] = tokens[:n]
        return n

    def fork(self, parent: int, child: int) -> None:
        super().fork(parent, child)
        if parent in self.tokens:
            self.tokens[child] = list(self.tokens[parent])

    def free_seq(self, seq: int) -> None:
        super().free_seq(seq)
        self.tokens.pop(seq, None)

    def append_slots(self, seq: int, n: int):
        slots, pairs = super().append_slots(seq, n)
        if n > 0:
            self.tokens.pop(seq, None)
        return slots, pairs

    def swap_out(self, seq: int):
        blocks = super().swap_out(seq)
        self.tokens.pop(seq, None)          # swapped-in copies are private: indexing stops
        return blocks

    def append_tokens(self, seq: int, tokens):
        tokens = [int(t) for t in tokens]
        slots, pairs = super().append_slots(seq, len(tokens))
        if seq in self.tokens:
            toks = self.tokens[seq]
            done = len(toks) // self.bs
            toks.extend(tokens)
            for i in range(done, len(toks) // self.bs):
                self._index_block(seq, i)
        return slots, pairs

    def batch_append_tokens(self, seqs, tokens):
        """One token for each sequence, in order; all or nothing."""
        seqs = [int(s) for s in seqs]
        # the batch is checked in order before any block is taken: the first
        # sequence that is unknown, swapped out or named again decides the error
        seen = set()
        for s in seqs:
            self._resident(s)
            if s in seen:
                raise AllocError("invalid_arg")
            seen.add(s)
        saved = copy.deepcopy(self.__dict__)
        slots, pairs = [], []
        try:
            for s, t in zip(seqs, tokens):
                sl, pr = self.append_tokens(s, [t])
                slots += sl
                pairs += pr
        except AllocError:
            self.__dict__.update(saved)
            raise
        return slots, pairs

    def _index_block(self, seq: int, i: int) -> None:
        key = self._key(self.tokens[seq], i + 1)
        if key in self.index:
            return
        table = self.tables[seq]
        if i > 0 and self.index.get(key[:-self.bs]) != table[i - 1]:
            return
        self.index[key] = table[i]
        self.key_of[table[i]] = key

    def prefix_stats(self) -> dict:
        return {"cached_blocks": len(self.index), "evictable_blocks": len(self.evictable),
                "lookup_blocks": self.lookup_blocks, "hit_blocks": self.hit_blocks,
                "evictions": self.evictions}
