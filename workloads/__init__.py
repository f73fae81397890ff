"""Seeded synthetic inputs for paged decode attention.

This module is shared by the fp64 oracle (``oracle/``) and the GPU path
(``paged_kv_cache_160_amd``).  It holds only random draws, sizes and operation
scripts: no attention arithmetic, no slot or block-table arithmetic and no
quantisation.  Every array it returns is a float32 array whose values are
already exactly representable in the named dtype, so the GPU side can cast it
to that dtype losslessly and the oracle can widen it to float64 losslessly.

Each random stream is keyed by ``(seed, tag, index)`` through
``numpy.random.default_rng``, so either side can regenerate any one sequence
(or any one step's queries) on its own without drawing the others.

The five workloads follow the shapes of the pages' examples:
  1 tiny      - B=4, L={1,16,17,40} then one append each, Hq=4, Hkv=2, D=64, fp32
  2 8b-shape  - B=16, L=4096, Hq=32, Hkv=8, D=128, bf16 (the Llama-3-8B head
                shape of "企业官网建设流程全解析" §2.1-2.2)
  3 7b-mha    - B=64, L~U{1..2048}, Hq=Hkv=32, D=128, fp16, churned free list
  4 prefix    - 8 sequences sharing a 1500-token prefix (the 1500-token
                system prompt of "KV Cache 和 vLLM" §3.3), suffix ~U{64..512}
  5 long-fp8  - B=32, L=32768, Hq=32, Hkv=8, D=128, fp32 rows stored as fp8
                e4m3 with per-token, per-head scales ("KV Cache优化实战" §3.2-3.3),
                query bf16
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

BLOCK_TOKENS = 16

# Stream tags: one random stream per (seed, tag, index).
_TAG_K = 1
_TAG_V = 2
_TAG_Q = 3
_TAG_LENS = 4
_TAG_PLACE = 5
_TAG_CHURN = 6
_TAG_PREFIX_K = 7
_TAG_PREFIX_V = 8
_TAG_TOKENS = 9
_TAG_CTX_K = 10
_TAG_CTX_V = 11
_TAG_CHUNK = 12

DTYPES = ("f32", "f16", "bf16", "fp8_e4m3")


@dataclass
class Workload:
    config_id: int
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str                # dtype of q and of the output
    src_dtype: str              # dtype of the K/V rows handed to the cache write
    cache_dtype: str            # dtype of the pool
    context_lens: List[int]     # per-sequence length after setup (before any decode step)
    num_blocks: int             # physical blocks in one layer's pool
    max_blocks_per_seq: int
    free_order: Optional[np.ndarray] = None   # initial free-list order (a permutation)
    churn_ops: Optional[list] = None          # alloc/free script run before setup
    churn_release: Optional[np.ndarray] = None  # order in which churn survivors are freed
    prefix_len: int = 0                       # shared-prefix length (workload 4)
    decode_appends: int = 0                   # extra single-token appends per sequence
    extra: dict = field(default_factory=dict)
    block_size: int = BLOCK_TOKENS            # tokens per physical block (16 or 32)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tag), int(index)])


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the nearest value of ``dtype`` (RNE, via torch's
    casts) and return them as float32.  fp8 rows are not rounded here: the
    cache write quantises them."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype in ("f32", "fp8_e4m3"):
        return x
    import torch
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return torch.from_numpy(x).to(tdt).to(torch.float32).numpy()


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


# ----------------------------------------------------------------------------
# Workload definitions
# ----------------------------------------------------------------------------

def _pool_for(lens: List[int], factor: float = 1.1, block_size: int = BLOCK_TOKENS) -> int:
    demand = sum(-(-L // block_size) for L in lens)
    return int(math.ceil(factor * demand))


def _churn_script(seed: int, num_blocks: int, n_ops: int = 20000,
                  max_seq_blocks: int = 128) -> Tuple[list, np.ndarray]:
    """Alloc/free script for a fragmented free list.

    Each op is ("alloc", n_blocks) or ("free", k) where k indexes the list of
    live churn sequences in creation order.  Only block *counts* are tracked
    here (to keep every alloc within capacity); which physical blocks are
    handed out is decided by whichever allocator runs the script."""
    rng = _rng(seed, _TAG_CHURN)
    ops = []
    live: List[int] = []          # sizes of live sequences, creation order
    used = 0
    for _ in range(n_ops):
        want_alloc = (not live) or rng.random() < 0.5
        size = int(rng.integers(1, max_seq_blocks + 1))
        if want_alloc and used + size <= num_blocks:
            ops.append(("alloc", size))
            live.append(size)
            used += size
        elif live:
            k = int(rng.integers(0, len(live)))
            ops.append(("free", k))
            used -= live.pop(k)
    release = rng.permutation(len(live)).astype(np.int64)
    return ops, release


def make_workload(config_id: int, seed: Optional[int] = None) -> Workload:
    """Return workload ``config_id`` (1..5) with its seed (default 1000 + id)."""
    if seed is None:
        seed = 1000 + config_id
    if config_id == 1:
        lens = [1, 16, 17, 40]
        nb = 64
        return Workload(1, "tiny-fp32", seed, 4, 4, 2, 64, "f32", "f32", "f32",
                        lens, nb, max_blocks_per_seq=4,
                        free_order=_rng(seed, _TAG_PLACE).permutation(nb).astype(np.int32),
                        decode_appends=1)
    if config_id == 2:
        lens = [4096] * 16
        nb = _pool_for(lens)
        return Workload(2, "llama3-8b-shape-bf16", seed, 16, 32, 8, 128, "bf16", "bf16", "bf16",
                        lens, nb, max_blocks_per_seq=4096 // BLOCK_TOKENS + 8,
                        free_order=_rng(seed, _TAG_PLACE).permutation(nb).astype(np.int32))
    if config_id == 3:
        lens = [int(x) for x in _rng(seed, _TAG_LENS).integers(1, 2049, size=64)]
        nb = _pool_for(lens)
        ops, release = _churn_script(seed, nb)
        return Workload(3, "7b-mha-fp16-ragged", seed, 64, 32, 32, 128, "f16", "f16", "f16",
                        lens, nb, max_blocks_per_seq=2048 // BLOCK_TOKENS + 8,
                        free_order=np.arange(nb, dtype=np.int32),
                        churn_ops=ops, churn_release=release)
    if config_id == 4:
        prefix = 1500
        suff = [int(x) for x in _rng(seed, _TAG_LENS).integers(64, 513, size=8)]
        lens = [prefix + s for s in suff]
        # distinct blocks: the full prefix blocks once, and every sequence's own
        # blocks from the partial prefix block onwards
        full_prefix = prefix // BLOCK_TOKENS
        demand = full_prefix + sum(-(-L // BLOCK_TOKENS) - full_prefix for L in lens)
        nb = int(math.ceil(1.1 * demand))
        return Workload(4, "shared-prefix-bf16", seed, 8, 32, 8, 128, "bf16", "bf16", "bf16",
                        lens, nb, max_blocks_per_seq=(prefix + 512) // BLOCK_TOKENS + 8,
                        free_order=_rng(seed, _TAG_PLACE).permutation(nb).astype(np.int32),
                        prefix_len=prefix, extra={"suffix_lens": suff})
    if config_id == 5:
        lens = [32768] * 32
        nb = _pool_for(lens)
        return Workload(5, "long-fp8-e4m3", seed, 32, 32, 8, 128, "bf16", "f32", "fp8_e4m3",
                        lens, nb, max_blocks_per_seq=32768 // BLOCK_TOKENS + 8,
                        free_order=_rng(seed, _TAG_PLACE).permutation(nb).astype(np.int32))
    raise ValueError(f"unknown workload {config_id}")


def custom_workload(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    context_lens: List[int], dtype: str = "bf16", cache_dtype: Optional[str] = None,
                    q_dtype: Optional[str] = None, seed: int = 7, pool_factor: float = 1.25,
                    extra_blocks: int = 4, block_size: int = BLOCK_TOKENS) -> Workload:
    """A free-form workload (edge cases and small parity sweeps)."""
    cache_dtype = cache_dtype or dtype
    q_dtype = q_dtype or ("bf16" if dtype == "f32" and cache_dtype == "fp8_e4m3" else dtype)
    nb = max(1, _pool_for(context_lens, pool_factor, block_size) + extra_blocks)
    mb = max(1, max([-(-L // block_size) for L in context_lens] + [1]) + 2)
    return Workload(0, "custom", seed, num_seqs, num_q_heads, num_kv_heads, head_dim,
                    q_dtype, dtype, cache_dtype, list(context_lens), nb, mb,
                    free_order=_rng(seed, _TAG_PLACE).permutation(nb).astype(np.int32), block_size=block_size)


def with_block_size(w: Workload, block_size: int) -> Workload:
    """The same workload (same rows, lengths and placement seed) on a pool of
    ``block_size``-token blocks sized by the same rule."""
    import dataclasses
    if block_size == w.block_size:
        return w
    ratio = w.block_size / block_size
    nb = max(1, int(math.ceil(w.num_blocks * ratio)) + 2)
    mb = max(1, int(math.ceil(w.max_blocks_per_seq * ratio)) + 1)
    out = dataclasses.replace(w, block_size=block_size, num_blocks=nb, max_blocks_per_seq=mb,
                              free_order=_rng(w.seed, _TAG_PLACE, block_size).permutation(nb).astype(np.int32),
                              churn_ops=None, churn_release=None, name=f"{w.name}-bs{block_size}")
    return out


# ----------------------------------------------------------------------------
# Value streams
# ----------------------------------------------------------------------------

def kv_rows(w: Workload, seq: int, which: str, n_tokens: Optional[int] = None) -> np.ndarray:
    """K or V rows [n_tokens][Hkv][D] (float32, values in ``w.src_dtype``) for
    positions 0..n_tokens-1 of sequence ``seq``.  For workload 4 the first
    ``prefix_len`` rows are the shared prefix, identical for every sequence."""
    if n_tokens is None:
        n_tokens = w.context_lens[seq] + w.decode_appends
    tag = _TAG_K if which == "k" else _TAG_V
    shape_tail = (w.num_kv_heads, w.head_dim)
    if w.prefix_len:
        ptag = _TAG_PREFIX_K if which == "k" else _TAG_PREFIX_V
        pre = _normal(_rng(w.seed, ptag), (w.prefix_len,) + shape_tail)
        rest = _normal(_rng(w.seed, tag, seq), (max(0, n_tokens - w.prefix_len),) + shape_tail)
        rows = np.concatenate([pre, rest], axis=0)[:n_tokens]
    else:
        rows = _normal(_rng(w.seed, tag, seq), (n_tokens,) + shape_tail)
    return round_to_dtype(rows, w.src_dtype)


def queries(w: Workload, step: int = 0) -> np.ndarray:
    """q [B][Hq][D] for decode step ``step`` (float32, values in ``w.q_dtype``)."""
    q = _normal(_rng(w.seed, _TAG_Q, step), (w.num_seqs, w.num_q_heads, w.head_dim))
    return round_to_dtype(q, w.q_dtype)


def random_rows(seed: int, tag: int, shape, dtype: str) -> np.ndarray:
    """Free-form N(0,1) rows rounded to ``dtype`` (tests that build their own cases)."""
    return round_to_dtype(_normal(_rng(seed, 100 + tag), shape), dtype)


# ----------------------------------------------------------------------------
# Setup scripts
# ----------------------------------------------------------------------------

CHURN_ID_BASE = 1_000_000


def setup_ops(w: Workload, share_prefix: bool = True) -> list:
    """The allocator operations that build the workload's cache state, as a
    list of tuples for whichever allocator runs them:

      ("free_order", order)   reorder the free list of the idle pool
      ("create", seq)         new empty sequence
      ("append", seq, n)      next n positions of seq (rows: the next n rows
                              of seq's stream, see kv_rows)
      ("fork", parent, child) child shares parent's blocks
      ("free", seq)           drop a sequence

    Churn sequences (workload 3) use ids from CHURN_ID_BASE and write no rows.
    With share_prefix=False, workload 4's sequences each append the prefix
    privately instead of forking it (the unshared twin of the same values)."""
    ops: list = [("free_order", w.free_order)]
    if w.churn_ops:
        live: List[int] = []
        nxt = CHURN_ID_BASE
        for op, arg in w.churn_ops:
            if op == "alloc":
                ops.append(("create", nxt))
                ops.append(("append", nxt, w.block_size * arg))
                live.append(nxt)
                nxt += 1
            else:
                ops.append(("free", live.pop(arg)))
        for k in w.churn_release:
            ops.append(("free", live[int(k)]))
    if w.prefix_len and share_prefix:
        ops.append(("create", 0))
        ops.append(("append", 0, w.prefix_len))
        for b in range(1, w.num_seqs):
            ops.append(("fork", 0, b))
        for b in range(w.num_seqs):
            ops.append(("append", b, w.context_lens[b] - w.prefix_len))
        return ops
    for b in range(w.num_seqs):
        ops.append(("create", b))
    for b in range(w.num_seqs):
        ops.append(("append", b, w.context_lens[b]))
    return ops


def chunk_workload(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int, cached: List[int],
                   chunk: List[int], dtype: str = "bf16", cache_dtype: Optional[str] = None,
                   q_dtype: Optional[str] = None, seed: int = 0, extra_blocks: int = 0,
                   block_size: int = BLOCK_TOKENS) -> Workload:
    """A chunked-prefill batch: sequence b holds ``cached[b]`` tokens and
    appends a chunk of ``chunk[b]`` more; context_lens are the totals."""
    lens = [int(c) + int(n) for c, n in zip(cached, chunk)]
    w = custom_workload(num_seqs, num_q_heads, num_kv_heads, head_dim, lens, dtype=dtype,
                        cache_dtype=cache_dtype, q_dtype=q_dtype, seed=seed, extra_blocks=extra_blocks,
                        block_size=block_size)
    w.extra["chunk"] = [int(n) for n in chunk]
    return w


def chunk_queries(w: Workload, step: int = 0) -> np.ndarray:
    """q [T][Hq][D] for the chunks back to back (float32, values in ``w.q_dtype``)."""
    T = int(sum(w.extra["chunk"]))
    q = _normal(_rng(w.seed, _TAG_CHUNK, step), (T, w.num_q_heads, w.head_dim))
    return round_to_dtype(q, w.q_dtype)


# ----------------------------------------------------------------------------
# Token streams (prefix caching)
# ----------------------------------------------------------------------------

def token_digests(seed: int, tokens) -> List[int]:
    """One 63-bit digest per position: position t's digest stands for tokens
    0..t, chained (blake2b of the previous digest and the token).  Used only
    to seed per-position rows, so that equal prefixes get equal K/V rows the
    way a model's would; it is not the cache's own hash."""
    out = []
    h = hashlib.blake2b(f"{int(seed)}".encode(), digest_size=8).digest()
    for t in tokens:
        h = hashlib.blake2b(h + int(t).to_bytes(4, "little", signed=True), digest_size=8).digest()
        out.append(int.from_bytes(h, "little") >> 1)
    return out


def context_rows(seed: int, tokens, start: int, stop: int, num_kv_heads: int, head_dim: int,
                 which: str, dtype: str) -> np.ndarray:
    """K or V rows [stop-start][Hkv][D] (float32, values in ``dtype``) for
    positions start..stop-1 of a token stream: each position's row is drawn
    from a stream keyed by the digest of the prefix it ends."""
    tag = _TAG_CTX_K if which == "k" else _TAG_CTX_V
    digs = token_digests(seed, list(tokens)[:stop])
    rows = np.empty((max(stop - start, 0), num_kv_heads, head_dim), np.float32)
    for i, t in enumerate(range(start, stop)):
        rows[i] = _normal(_rng(seed, tag, digs[t]), (num_kv_heads, head_dim))
    return round_to_dtype(rows, dtype)


@dataclass
class Turn:
    session: int
    turn: int
    prompt: List[int]          # the request's full prompt
    output: List[int]          # the tokens the turn generates


def agent_sessions(seed: int, n_sessions: int, turns: int, system_len: int, user_len: int,
                   output_len: int, vocab: int = 32000, dynamic_head: int = 0) -> List[Turn]:
    """Multi-turn sessions in the shape of "KV Cache优化实战" §5.1: every
    session starts from one fixed system prompt; each turn's prompt is the
    previous turn's prompt and output plus ``user_len`` new tokens, so
    almost all of a late turn's prompt was seen before.  ``dynamic_head``
    tokens of per-request content (a time stamp, a user id) placed right
    after the first system block reproduce the unstable template of
    §5.3.  Turns are listed round-robin over sessions, turn by turn."""
    rng = _rng(seed, _TAG_TOKENS)
    system = [int(t) for t in rng.integers(0, vocab, size=system_len)]
    history = [list(system) for _ in range(n_sessions)]
    out: List[Turn] = []
    for turn in range(turns):
        for s in range(n_sessions):
            user = [int(t) for t in rng.integers(0, vocab, size=user_len)]
            prompt = history[s] + user
            if dynamic_head:
                head = [int(t) for t in rng.integers(0, vocab, size=dynamic_head)]
                cut = min(BLOCK_TOKENS, len(prompt))
                prompt = prompt[:cut] + head + prompt[cut:]
            gen = [int(t) for t in rng.integers(0, vocab, size=output_len)]
            out.append(Turn(s, turn, prompt, gen))
            history[s] = history[s] + user + gen
    return out
