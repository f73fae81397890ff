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

Readings (the pages leave these open):
  * blocks carry a reference count; fork shares every block of the parent and
    increments each count; free decrements and returns a block at zero;
  * the free list is a stack: ``set_free_order(order)`` makes ``order[0]`` the
    next block handed out; a freed block goes on top (so it is reused first);
    a sequence's blocks are released in logical order 0, 1, 2, ...;
  * an append of n tokens to a sequence of length L: if L % 16 != 0 and the
    last block is shared (count > 1) that block is copied first - one fresh
    block is taken, the pair (old, new) is reported for copying, the old count
    is decremented and the table entry repointed; then one fresh block is
    taken for each position p in [L, L+n) with p % 16 == 0, in position order;
  * a full shared block is never written and so never copied;
  * an append that needs more fresh blocks than are free, or that would
    exceed ``max_blocks_per_seq``, changes nothing and reports an error.

Test infrastructure: only tests, the smoke check and the CPU baseline leg of
the benchmark use this module.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

BLOCK_TOKENS = 16


class AllocError(Exception):
    def __init__(self, kind: str):
        super().__init__(kind)
        self.kind = kind          # "no_free_blocks" | "unknown_seq" | "invalid_arg"


class BlockAllocatorModel:
    def __init__(self, num_blocks: int, max_blocks_per_seq: int):
        if num_blocks <= 0 or max_blocks_per_seq <= 0:
            raise AllocError("invalid_arg")
        self.num_blocks = num_blocks
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free: List[int] = list(range(num_blocks - 1, -1, -1))   # top = end; block 0 first
        self.ref = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.cow_copies = 0

    # -- free list ----------------------------------------------------------
    def set_free_order(self, order) -> None:
        order = [int(x) for x in order]
        if len(self.free) != self.num_blocks:
            raise AllocError("invalid_arg")          # only on an idle pool
        if sorted(order) != list(range(self.num_blocks)):
            raise AllocError("invalid_arg")
        self.free = order[::-1]

    def _take(self) -> int:
        blk = self.free.pop()
        self.ref[blk] = 1
        return blk

    def _release(self, blk: int) -> None:
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            self.free.append(blk)

    # -- sequences ----------------------------------------------------------
    def create(self, seq: int) -> None:
        if seq in self.tables:
            raise AllocError("invalid_arg")
        self.tables[seq] = []
        self.lens[seq] = 0

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.tables:
            raise AllocError("unknown_seq")
        if child in self.tables:
            raise AllocError("invalid_arg")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for blk in self.tables[child]:
            self.ref[blk] += 1

    def free_seq(self, seq: int) -> None:
        if seq not in self.tables:
            raise AllocError("unknown_seq")
        for blk in self.tables.pop(seq):
            self._release(blk)
        del self.lens[seq]

    def append_slots(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Slots for the next n positions of ``seq`` and the copy pairs the
        caller must apply (before writing) to keep shared blocks intact."""
        if seq not in self.tables:
            raise AllocError("unknown_seq")
        if n < 0:
            raise AllocError("invalid_arg")
        table = self.tables[seq]
        L = self.lens[seq]
        needs_cow = (n > 0 and L % BLOCK_TOKENS != 0 and self.ref[table[-1]] > 1)
        new_blocks = -(-(L + n) // BLOCK_TOKENS) - -(-L // BLOCK_TOKENS)
        if len(table) + new_blocks > self.max_blocks_per_seq:
            raise AllocError("invalid_arg")
        if int(needs_cow) + new_blocks > len(self.free):
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
            if p % BLOCK_TOKENS == 0:
                table.append(self._take())
            slots.append(BLOCK_TOKENS * table[p // BLOCK_TOKENS] + p % BLOCK_TOKENS)
        self.lens[seq] = L + n
        return slots, pairs

    def seq_len(self, seq: int) -> int:
        if seq not in self.lens:
            raise AllocError("unknown_seq")
        return self.lens[seq]

    def block_tables(self, seqs, max_blocks: int):
        """Tables ``[n][max_blocks]`` (unused entries 0) and lengths ``[n]``."""
        tables, lens = [], []
        for s in seqs:
            if s not in self.tables:
                raise AllocError("unknown_seq")
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
        stored_tokens / (16 * used_blocks).  cached_tokens is the logical
        total sum_b L_b."""
        filled: Dict[int, int] = {}
        for s, t in self.tables.items():
            L = self.lens[s]
            for i, blk in enumerate(t):
                f = min(BLOCK_TOKENS, L - BLOCK_TOKENS * i)
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
            "utilisation": (stored / (BLOCK_TOKENS * used)) if used else 0.0,
        }
