"""Planted mistakes in the oracle (CPU only): each plausible error - a dropped
or halved 1/sqrt(d), a wrong GQA index, K and V swapped, a partition merge
without the exp(m_p - M) rescale, round-half-up instead of ties-to-even, a
wrong fp8 exponent bias, a scale from the mean instead of the max, an
off-by-one position, a reversed free order, a copy-on-write that skips the
copy, a prefix cache that evicts by plain recency, keys a block by its own
tokens only, lets a lookup cover the last prompt token or forgets released
blocks, a prefill mask that hides the diagonal or a chunk placed at the
start of the sequence, a wrong e5m2 bias, swapped int4 nibbles, integer
rounding with ties up, or an allocator or pool that ignores the block size - must make at least one of the pins fail.  This shows the pins are
sharp enough to catch the mistakes they are meant to catch."""
import numpy as np
import pytest

from oracle import allocator as alloc_mod
from oracle import attention, cache, fp8_e4m3, kv_formats, prefill
from oracle.allocator import BLOCK_TOKENS as BLOCK
from tests import test_oracle_allocator as pins_alloc
from tests import test_oracle_attention as pins_attn
from tests import test_oracle_fp8 as pins_fp8
from tests import test_oracle_kv_formats as pins_formats
from tests import test_oracle_prefill as pins_prefill
from tests import test_oracle_prefix_cache as pins_prefix


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


# ---- attention mutants --------------------------------------------------------

def _attend_no_scale(q, K, V, scale):
    return _attend_ref(q, K, V, 1.0)


def _attend_ref(q, K, V, scale, group_fn=lambda h, G, Hkv: h // G):
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    Hq, D = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D))
    if L == 0:
        return out
    for h in range(Hq):
        g = group_fn(h, G, Hkv)
        s = (K[:, g, :] @ q[h]) * scale
        w = np.exp(s - np.max(s))
        out[h] = (w @ V[:, g, :]) / np.sum(w)
    return out


@pytest.mark.parametrize("mutant", [
    _attend_no_scale,
    lambda q, K, V, s: _attend_ref(q, K, V, s, group_fn=lambda h, G, Hkv: h % Hkv),
    lambda q, K, V, s: _attend_ref(q, K, V, s * 0.5),
    lambda q, K, V, s: _attend_ref(q, V, K, s),
], ids=["no-sqrt-d", "gqa-modulo", "half-scale", "k-v-swapped"])
def test_attention_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(attention, "attend", mutant)
    _fails(pins_attn.test_matches_torch_sdpa, 8, 2, 64, 40)


def test_gqa_mutant_caught_by_closed_form(monkeypatch):
    monkeypatch.setattr(attention, "attend",
                        lambda q, K, V, s: _attend_ref(q, K, V, s, group_fn=lambda h, G, Hkv: h % Hkv))
    _fails(pins_attn.test_gqa_mapping_consecutive_groups)


def test_missing_scale_caught_by_closed_form(monkeypatch):
    monkeypatch.setattr(attention, "attend", _attend_no_scale)
    _fails(pins_attn.test_two_tokens_closed_form_with_sqrt_d)


def test_partition_merge_mutant_is_caught(monkeypatch):
    # forgetting to rescale each partition by exp(m_p - M)
    def bad_combine(ms, ls, accs):
        accs = np.asarray(accs, np.float64)
        return accs.sum(axis=0) / np.asarray(ls, np.float64).sum(axis=0)[:, None]
    monkeypatch.setattr(attention, "combine_partitions", bad_combine)
    _fails(pins_attn.test_partitioned_merge_equals_plain, 64)


# ---- fp8 mutants ------------------------------------------------------------------

def test_round_half_up_is_caught(monkeypatch):
    pos = fp8_e4m3.decode_table()[:0x7F]

    def half_up(y):
        y = np.asarray(y, np.float64)
        a = np.abs(y)
        hi = np.minimum(np.searchsorted(pos, a, side="left"), len(pos) - 1)
        lo = np.maximum(hi - 1, 0)
        pick_hi = (pos[hi] - a) <= (a - pos[lo])          # ties go up
        code = np.where(pick_hi, hi, lo).astype(np.uint8)
        return (code | (np.signbit(y).astype(np.uint8) << 7)).astype(np.uint8)

    monkeypatch.setattr(fp8_e4m3, "encode_rne", half_up)
    _fails(pins_fp8.test_encode_matches_torch_on_grid_with_ties)


def test_wrong_bias_is_caught(monkeypatch):
    monkeypatch.setattr(fp8_e4m3, "_BIAS", 8)
    _fails(pins_fp8.test_decode_all_codes_match_torch)


def test_scale_from_mean_is_caught(monkeypatch):
    def bad_quantise(x):
        x = np.asarray(x, np.float32)
        s = (np.mean(np.abs(x), axis=-1) / np.float32(448)).astype(np.float32)
        s = np.where(s == 0, np.float32(1), s).astype(np.float32)
        y = np.clip(x / s[..., None], -448, 448).astype(np.float32)
        return fp8_e4m3.encode_rne(y), s
    monkeypatch.setattr(fp8_e4m3, "quantise_rows", bad_quantise)
    _fails(pins_fp8.test_quantise_rows_scale_and_extremes)


# ---- cache / allocator mutants ------------------------------------------------------

def test_off_by_one_gather_is_caught(monkeypatch):
    orig = cache.Pool.gather

    def shifted(self, table_row, length):
        K, V = orig(self, table_row, length)
        return np.roll(K, 1, axis=0), V
    monkeypatch.setattr(cache.Pool, "gather", shifted)
    _fails(pins_attn.test_paged_equals_contiguous_and_placement_invariant, "f32")


def test_reversed_free_order_is_caught(monkeypatch):
    def set_free_order(self, order):
        self.free = [int(x) for x in order]             # hands out order[-1] first
    monkeypatch.setattr(alloc_mod.BlockAllocatorModel, "set_free_order", set_free_order)
    _fails(pins_alloc.test_hand_worked_four_sequences)


def test_cow_without_copy_is_caught(monkeypatch):
    orig = alloc_mod.BlockAllocatorModel.append_slots

    def no_cow(self, seq, n):
        # write into the shared block in place (no copy pair)
        for blk in self.tables.get(seq, [])[-1:]:
            if self.ref[blk] > 1:
                self.ref[blk] = 1
        return orig(self, seq, n)
    monkeypatch.setattr(alloc_mod.BlockAllocatorModel, "append_slots", no_cow)
    _fails(pins_alloc.test_hand_worked_fork_and_copy_on_write)


# ---- prefix-cache mutants -------------------------------------------------------------

PCM = alloc_mod.PrefixCachingAllocatorModel


def test_plain_lru_eviction_is_caught(monkeypatch):
    def lru_take(self):
        if self.free:
            return alloc_mod.BlockAllocatorModel._take(self)
        _, blk = min((st, b) for b, st in self.evictable.items())     # ignores children
        del self.evictable[blk]
        del self.index[self.key_of.pop(blk)]
        self.evictions += 1
        self.ref[blk] = 1
        return blk
    monkeypatch.setattr(PCM, "_take", lru_take)
    _fails(pins_prefix.test_hand_worked_leaf_first_eviction, 16)


def test_block_only_key_is_caught(monkeypatch):
    # keying a block by its own 16 tokens, forgetting the prefix before it
    monkeypatch.setattr(PCM, "_key", lambda self, toks, nb: (self.model_key,) + tuple(
        toks[self.bs * (nb - 1):self.bs * nb]))
    _fails(pins_prefix.test_hits_hold_the_right_content_under_pressure, 0, 16)


def test_lookup_bound_off_by_one_is_caught(monkeypatch):
    orig = PCM.create_cached

    def greedy(self, seq, tokens):
        return orig(self, seq, list(tokens) + [0])      # as if the bound were n // 16
    monkeypatch.setattr(PCM, "create_cached", greedy)
    _fails(pins_prefix.test_lookup_never_covers_the_last_prompt_token)


def test_forgetting_released_blocks_is_caught(monkeypatch):
    def forget(self, blk):
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            if blk in self.key_of:                      # dropped from the index at once
                del self.index[self.key_of.pop(blk)]
            self.free.append(blk)
    monkeypatch.setattr(PCM, "_release", forget)
    _fails(pins_prefix.test_hits_equal_brute_force_longest_shared_prefix, 0, 16)


# ---- prefill mutants --------------------------------------------------------------------

def _prefill_with(q, K, V, scale, first_key_hidden=False, chunk_at_start=False):
    q = np.asarray(q, np.float64)
    n, L = q.shape[0], K.shape[0]
    out = np.zeros(q.shape)
    for i in range(n):
        p = i if chunk_at_start else L - n + i
        stop = p if first_key_hidden and p > 0 else p + 1       # k < p instead of k <= p
        out[i] = attention.attend(q[i], K[:stop], V[:stop], scale)
    return out


@pytest.mark.parametrize("kw", [{"first_key_hidden": True}, {"chunk_at_start": True}],
                         ids=["mask-hides-diagonal", "chunk-at-start"])
def test_prefill_mutants_are_caught(monkeypatch, kw):
    monkeypatch.setattr(prefill, "prefill_rows", lambda q, K, V, s: _prefill_with(q, K, V, s, **kw))
    _fails(pins_prefill.test_matches_torch_sdpa_with_shifted_causal_mask, 4, 2, 64, 40, 7)


# ---- cache-format mutants -------------------------------------------------------------------

def test_wrong_e5m2_bias_is_caught(monkeypatch):
    monkeypatch.setattr(kv_formats, "_E5M2_BIAS", 16)
    _fails(pins_formats.test_e5m2_decode_matches_torch)


def test_swapped_nibbles_are_caught(monkeypatch):
    def swapped(codes):
        c = np.asarray(codes, dtype=np.int16)
        u = (c & 0xF).astype(np.uint8)
        return (u[..., 1::2] | (u[..., 0::2] << 4)).astype(np.uint8)
    monkeypatch.setattr(kv_formats, "pack_int4", swapped)
    _fails(pins_formats.test_int4_packing_bytes)


def test_int_ties_up_are_caught(monkeypatch):
    def half_up(x, qmax):
        x = np.asarray(x, dtype=np.float32)
        s = kv_formats._row_scales(x, qmax)
        y = np.clip((x / s[..., None]).astype(np.float32), -qmax, qmax)
        return np.floor(y + np.float32(0.5)).astype(np.int8), s
    monkeypatch.setattr(kv_formats, "quantise_int_rows", half_up)
    _fails(pins_formats.test_int_codes_are_nearest_with_ties_to_even, 7)


# ---- block-size mutants -------------------------------------------------------------------

def test_allocator_ignoring_block_size_is_caught(monkeypatch):
    init = alloc_mod.BlockAllocatorModel.__init__

    def sixteen(self, *a, **kw):
        init(self, *a, **kw)
        self.bs = BLOCK
    monkeypatch.setattr(alloc_mod.BlockAllocatorModel, "__init__", sixteen)
    _fails(pins_alloc.test_hand_worked_32_token_blocks)


def test_pool_ignoring_block_size_is_caught(monkeypatch):
    init = cache.Pool.__init__

    def sixteen(self, num_blocks, num_kv_heads, head_dim, cache_dtype, block_size=BLOCK):
        init(self, num_blocks * block_size // BLOCK, num_kv_heads, head_dim, cache_dtype, BLOCK)
    monkeypatch.setattr(cache.Pool, "__init__", sixteen)
    _fails(pins_attn.test_block_size_does_not_change_the_output, "f32")
