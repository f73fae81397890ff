// Host block allocator for the paged KV cache: free list, per-sequence block
// tables, reference counts, fork and copy-on-write planning.
//
// Pages: blocks of 16 (or 32) tokens are taken on demand when a sequence's current
// block is full ("KV Cache 和 vLLM" §3.1); finished sequences return their
// blocks and later sequences reuse them wherever they lie ("KV Cache优化实战"
// §4.2); sequences with a common prefix share physical blocks, and
// copy-on-write covers writes into shared blocks ("KV Cache 和 vLLM" §3.3);
// running out of cache degrades instead of crashing ("企业官网建设流程全解析"
// §6.4), so every failing call here leaves the state untouched.
//
// The rules the pages leave open (reference counts, a stack-ordered free
// list, release order, which writer copies) are stated in include/pagedkv.h.
//
// Prefix caching ("KV Cache优化实战" §5.2-5.3; "企业官网建设流程全解析"
// §6.2-6.3): full blocks are indexed by their content - a hash chained from
// the model key through every earlier block's tokens - and a new request
// reuses the longest run of indexed blocks matching its prompt.  An index
// entry is the exact pair (parent block, the block's token ids); the hash only picks
// the bucket and every candidate is compared in full, so a hash collision
// costs a comparison, never a wrong match.  Because leaf-first eviction
// never drops a block while an indexed child points at it, the pair names a
// whole prefix: matching pairs down the chain is matching the prefix.  A
// sequence keeps only the tokens of its unfinished last block.

#include <algorithm>
#include <array>
#include <cstdint>
#include <new>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pagedkv.h"

namespace {

constexpr int kMaxBlock = 32;       // block sizes: 16 or 32 tokens
constexpr int32_t kNoToken = 0;      // non-null stand-in for an empty token list

struct Seq {
  std::vector<int32_t> table;
  int64_t len = 0;
  bool tracked = false;              // token ids known for every position
  bool swapped = false;              // blocks moved out: only len is kept
  std::vector<int32_t> pending;      // tokens of the unfinished last block
};

using BlockTokens = std::array<int32_t, kMaxBlock>;   // first bs entries used

// 64-bit FNV-1a over the parent's hash (8 bytes, little-endian) and the
// block's bs token ids (4 bytes each, little-endian).
uint64_t chain_hash(uint64_t parent_hash, const int32_t* toks, int bs) {
  uint64_t h = 0xcbf29ce484222325ull;
  auto mix = [&h](uint8_t byte) {
    h ^= byte;
    h *= 0x100000001b3ull;
  };
  for (int i = 0; i < 8; ++i) mix(static_cast<uint8_t>(parent_hash >> (8 * i)));
  for (int t = 0; t < bs; ++t) {
    uint32_t u = static_cast<uint32_t>(toks[t]);
    for (int i = 0; i < 4; ++i) mix(static_cast<uint8_t>(u >> (8 * i)));
  }
  return h;
}

struct CacheEntry {
  bool indexed = false;
  int32_t parent = -1;               // indexed parent block, -1 at the root
  int32_t children = 0;              // indexed blocks whose parent this is
  uint64_t hash = 0;
  uint64_t stamp = 0;                // release order while evictable
  BlockTokens tokens{};
};

struct PrefixCache {
  bool enabled = false;
  int bs = PKV_BLOCK_SIZE;
  uint64_t model_key = 0;
  uint64_t mask = ~0ull;
  std::vector<CacheEntry> entry;                      // per physical block
  std::unordered_multimap<uint64_t, int32_t> index;   // masked hash -> block
  std::set<std::pair<uint64_t, int32_t>> leaves;      // evictable, no children
  int64_t evictable = 0;
  int64_t cached = 0;
  uint64_t clock = 0;
  int64_t lookup_blocks = 0, hit_blocks = 0, evictions = 0;

  uint64_t hash_of(int32_t parent, const int32_t* toks) const {
    return chain_hash(parent < 0 ? model_key : entry[parent].hash, toks, bs);
  }
  // The indexed block with this parent and these tokens, or -1.
  int32_t find(int32_t parent, const int32_t* toks, uint64_t h) const {
    auto range = index.equal_range(h & mask);
    for (auto it = range.first; it != range.second; ++it) {
      const CacheEntry& e = entry[it->second];
      if (e.parent == parent && std::equal(toks, toks + bs, e.tokens.begin())) return it->second;
    }
    return -1;
  }
};

}  // namespace

struct pkv_alloc {
  int32_t num_blocks = 0;
  int32_t max_blocks_per_seq = 0;
  int32_t bs = PKV_BLOCK_SIZE;       // tokens per block: 16 or 32
  std::vector<int32_t> free_stack;   // back() is handed out next
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<int64_t> seq_order;    // creation order, for deterministic stats walks
  int64_t cow_copies = 0;
  PrefixCache pc;

  int64_t blocks_for(int64_t len) const { return (len + bs - 1) / bs; }

  // Blocks an append may take: free ones and, with prefix caching, the
  // evictable ones (indexed, no holder).
  int64_t available() const { return static_cast<int64_t>(free_stack.size()) + pc.evictable; }

  int32_t take() {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
    } else {
      b = pc.leaves.begin()->second;   // oldest released leaf
      evict(b);
    }
    ref[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[b] != 0) return;
    if (!pc.enabled || !pc.entry[b].indexed) {
      free_stack.push_back(b);
      return;
    }
    CacheEntry& e = pc.entry[b];
    e.stamp = ++pc.clock;
    ++pc.evictable;
    if (e.children == 0) pc.leaves.emplace(e.stamp, b);
  }
  void evict(int32_t b) {
    CacheEntry& e = pc.entry[b];
    pc.leaves.erase({e.stamp, b});
    --pc.evictable;
    auto range = pc.index.equal_range(e.hash & pc.mask);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == b) {
        pc.index.erase(it);
        break;
      }
    if (e.parent >= 0) {
      CacheEntry& p = pc.entry[e.parent];
      if (--p.children == 0 && ref[e.parent] == 0) pc.leaves.emplace(p.stamp, e.parent);
    }
    e = CacheEntry{};
    --pc.cached;
    ++pc.evictions;
  }

  // A lookup hit on block b: take a reference, leaving the evictable set.
  void hold(int32_t b) {
    if (ref[b]++ == 0) {
      --pc.evictable;
      pc.leaves.erase({pc.entry[b].stamp, b});
    }
  }

  // After an append of n positions: record its tokens on a tracked sequence
  // (toks null: untrack it, the keys of its later blocks are unknown).
  void after_append(Seq& s, const int32_t* toks, int64_t n) {
    if (!s.tracked || n == 0) return;
    if (!toks) {
      s.tracked = false;
      s.pending.clear();
      return;
    }
    record_tokens(s, toks, n);
  }

  // Record the tokens of an append on a tracked sequence, indexing every
  // block they fill (the append's slots were already reserved).
  void record_tokens(Seq& s, const int32_t* toks, int64_t n) {
    int64_t first = s.len - n;                 // position of toks[0]
    for (int64_t i = 0; i < n; ++i) {
      s.pending.push_back(toks[i]);
      int64_t p = first + i;
      if (p % bs == bs - 1) {
        index_block(s, p / bs);
        s.pending.clear();
      }
    }
  }

  void index_block(const Seq& s, int64_t i) {
    int32_t parent = -1;
    if (i > 0) {
      parent = s.table[i - 1];
      if (!pc.entry[parent].indexed) return;   // chain not this sequence's
    }
    uint64_t h = pc.hash_of(parent, s.pending.data());
    if (pc.find(parent, s.pending.data(), h) >= 0) return;   // indexed already
    int32_t b = s.table[i];
    CacheEntry& e = pc.entry[b];
    e.indexed = true;
    e.parent = parent;
    e.children = 0;
    e.hash = h;
    std::copy(s.pending.begin(), s.pending.end(), e.tokens.begin());
    if (parent >= 0) ++pc.entry[parent].children;
    pc.index.emplace(h & pc.mask, b);
    ++pc.cached;
  }

  // Fresh blocks an append of n tokens needs, and whether it copies first.
  void plan(const Seq& s, int64_t n, bool* cow, int64_t* fresh) const {
    *cow = n > 0 && (s.len % bs) != 0 && ref[s.table.back()] > 1;
    *fresh = blocks_for(s.len + n) - blocks_for(s.len);
  }

  // Apply a planned append; capacity was checked by the caller.
  void apply(Seq& s, int64_t n, int64_t* slots, int32_t* pair, int* n_cow) {
    *n_cow = 0;
    if (n > 0 && (s.len % bs) != 0 && ref[s.table.back()] > 1) {
      int32_t old_b = s.table.back();
      int32_t new_b = take();
      --ref[old_b];                    // another sequence still holds it
      s.table.back() = new_b;
      pair[0] = old_b;
      pair[1] = new_b;
      *n_cow = 1;
      ++cow_copies;
    }
    for (int64_t i = 0; i < n; ++i) {
      int64_t p = s.len + i;
      if (p % bs == 0) s.table.push_back(take());
      slots[i] = static_cast<int64_t>(s.table[p / bs]) * bs + p % bs;
    }
    s.len += n;
  }
};

// Exported calls that may allocate host memory catch what the standard
// containers throw: no exception crosses the C boundary.
extern "C" {

pkv_alloc* pkv_alloc_create_bs(int num_blocks, int max_blocks_per_seq, int block_size) {
  if (num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      (block_size != PKV_BLOCK_SIZE && block_size != PKV_BLOCK_SIZE_LARGE))
    return nullptr;
  pkv_alloc* a = new (std::nothrow) pkv_alloc();
  if (!a) return nullptr;
  try {
      a->bs = block_size;
      a->pc.bs = block_size;
      a->num_blocks = num_blocks;
      a->max_blocks_per_seq = max_blocks_per_seq;
      a->ref.assign(num_blocks, 0);
      a->free_stack.resize(num_blocks);
      for (int i = 0; i < num_blocks; ++i) a->free_stack[i] = num_blocks - 1 - i;
  } catch (...) {
    delete a;
    return nullptr;
  }
  return a;
}

pkv_alloc* pkv_alloc_create(int num_blocks, int max_blocks_per_seq) {
  return pkv_alloc_create_bs(num_blocks, max_blocks_per_seq, PKV_BLOCK_SIZE);
}

int pkv_alloc_block_size(const pkv_alloc* a) { return a ? a->bs : PKV_ERR_INVALID_ARG; }

void pkv_alloc_destroy(pkv_alloc* a) { delete a; }

int pkv_alloc_set_free_order(pkv_alloc* a, const int32_t* order, int n) {
  try {
    if (!a || !order || n != a->num_blocks) return PKV_ERR_INVALID_ARG;
    if (!a->seqs.empty() || static_cast<int>(a->free_stack.size()) != a->num_blocks)
      return PKV_ERR_INVALID_ARG;
    std::vector<char> seen(n, 0);
    for (int i = 0; i < n; ++i) {
      if (order[i] < 0 || order[i] >= n || seen[order[i]]) return PKV_ERR_INVALID_ARG;
      seen[order[i]] = 1;
    }
    for (int i = 0; i < n; ++i) a->free_stack[i] = order[n - 1 - i];
    return PKV_OK;
  } catch (...) {
    return PKV_ERR_HOST_MEMORY;
  }
}

int pkv_seq_create(pkv_alloc* a, int64_t seq_id) {
  try {
    if (!a) return PKV_ERR_INVALID_ARG;
    if (a->seqs.count(seq_id)) return PKV_ERR_INVALID_ARG;
    Seq s;
    s.tracked = a->pc.enabled;
    a->seqs.emplace(seq_id, std::move(s));
    a->seq_order.push_back(seq_id);
    return PKV_OK;
  } catch (...) {
    return PKV_ERR_HOST_MEMORY;
  }
}

int pkv_seq_fork(pkv_alloc* a, int64_t parent, int64_t child) {
  try {
    if (!a) return PKV_ERR_INVALID_ARG;
    auto it = a->seqs.find(parent);
    if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    if (it->second.swapped) return PKV_ERR_INVALID_ARG;
    if (a->seqs.count(child)) return PKV_ERR_INVALID_ARG;
    Seq c = it->second;
    for (int32_t b : c.table) ++a->ref[b];
    a->seqs.emplace(child, std::move(c));
    a->seq_order.push_back(child);
    return PKV_OK;
  } catch (...) {
    return PKV_ERR_HOST_MEMORY;
  }
}

int pkv_seq_free(pkv_alloc* a, int64_t seq_id) {
  try {
    if (!a) return PKV_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    for (int32_t b : it->second.table) a->release(b);
    a->seqs.erase(it);
    a->seq_order.erase(std::find(a->seq_order.begin(), a->seq_order.end(), seq_id));
    return PKV_OK;
  } catch (...) {
    return PKV_ERR_HOST_MEMORY;
  }
}

int pkv_seq_len(pkv_alloc* a, int64_t seq_id) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  return static_cast<int>(it->second.len);
}

}  // extern "C"

namespace {

// One append of n positions; toks (n ids) or null for an append without
// tokens, which stops the sequence being tracked.
int append_impl(pkv_alloc* a, int64_t seq_id, int n, const int32_t* toks, int64_t* slots_out,
                int32_t* cow_pairs_out, int* n_cow_out) {
  if (!a || n < 0 || !n_cow_out || !cow_pairs_out || (n > 0 && !slots_out))
    return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  if (it->second.swapped) return PKV_ERR_INVALID_ARG;
  Seq& s = it->second;
  bool cow;
  int64_t fresh;
  a->plan(s, n, &cow, &fresh);
  if (static_cast<int64_t>(s.table.size()) + fresh > a->max_blocks_per_seq)
    return PKV_ERR_INVALID_ARG;
  if ((cow ? 1 : 0) + fresh > a->available()) return PKV_ERR_NO_FREE_BLOCKS;
  a->apply(s, n, slots_out, cow_pairs_out, n_cow_out);
  a->after_append(s, toks, n);
  return PKV_OK;
}

// One position for each of n distinct sequences, all or nothing.
int batch_impl(pkv_alloc* a, const int64_t* seq_ids, const int32_t* toks, int n, int64_t* slots_out,
               int32_t* cow_pairs_out, int* n_cow_out) {
  if (!a || n < 0 || !n_cow_out || (n > 0 && (!seq_ids || !slots_out || !cow_pairs_out)))
    return PKV_ERR_INVALID_ARG;
  // Check the whole batch first.  Each sequence gets one position; a
  // sequence named twice would see its own first append, so reject repeats.
  // Copies earlier in the batch lower the count of a shared block, so a
  // later holder of the same block may write it in place: track that.
  int64_t need = 0;
  std::unordered_map<int64_t, int> seen;
  std::unordered_map<int32_t, int32_t> dropped;   // block -> copies planned so far
  for (int i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    if (it->second.swapped) return PKV_ERR_INVALID_ARG;
    if (seen[seq_ids[i]]++) return PKV_ERR_INVALID_ARG;
    const Seq& s = it->second;
    int64_t fresh = a->blocks_for(s.len + 1) - a->blocks_for(s.len);
    bool cow = false;
    if (s.len % a->bs != 0) {
      int32_t last = s.table.back();
      cow = a->ref[last] - dropped[last] > 1;
      if (cow) ++dropped[last];
    }
    if (static_cast<int64_t>(s.table.size()) + fresh > a->max_blocks_per_seq)
      return PKV_ERR_INVALID_ARG;
    need += (cow ? 1 : 0) + fresh;
  }
  if (need > a->available()) return PKV_ERR_NO_FREE_BLOCKS;
  int n_cow = 0;
  for (int i = 0; i < n; ++i) {
    int c = 0;
    Seq& s = a->seqs[seq_ids[i]];
    a->apply(s, 1, slots_out + i, cow_pairs_out + 2 * n_cow, &c);
    a->after_append(s, toks ? toks + i : nullptr, 1);
    n_cow += c;
  }
  *n_cow_out = n_cow;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_seq_append_slots(pkv_alloc* a, int64_t seq_id, int n_tokens, int64_t* slots_out,
                         int32_t* cow_pairs_out, int* n_cow_out) {
  try {
    return append_impl(a, seq_id, n_tokens, nullptr, slots_out, cow_pairs_out, n_cow_out);
  } catch (...) {
    return PKV_ERR_HOST_MEMORY;
  }
}

int pkv_seq_append_tokens(pkv_alloc* a, int64_t seq_id, const int32_t* tokens, int n_tokens,
                          int64_t* slots_out, int32_t* cow_pairs_out, int* n_cow_out) {
  try {
    if (n_tokens > 0 && !tokens) return PKV_ERR_INVALID_ARG;
    return append_impl(a, seq_id, n_tokens, tokens ? tokens : &kNoToken, slots_out, cow_pairs_out,
                       n_cow_out);
  } catch (...) {
    return PKV_ERR_HOST_MEMORY;
  }
}

int pkv_batch_append_one(pkv_alloc* a, const int64_t* seq_ids, int n, int64_t* slots_out,
                         int32_t* cow_pairs_out, int* n_cow_out) {
  try {
    return batch_impl(a, seq_ids, nullptr, n, slots_out, cow_pairs_out, n_cow_out);
  } catch (...) {
    return PKV_ERR_HOST_MEMORY;
  }
}

int pkv_batch_append_tokens(pkv_alloc* a, const int64_t* seq_ids, const int32_t* tokens, int n,
                            int64_t* slots_out, int32_t* cow_pairs_out, int* n_cow_out) {
  try {
    if (n > 0 && !tokens) return PKV_ERR_INVALID_ARG;
    return batch_impl(a, seq_ids, tokens ? tokens : &kNoToken, n, slots_out, cow_pairs_out, n_cow_out);
  } catch (...) {
    return PKV_ERR_HOST_MEMORY;
  }
}

int pkv_prefix_cache_enable(pkv_alloc* a, uint64_t model_key, int hash_bits) {
  try {
    if (!a || hash_bits < 1 || hash_bits > 64 || a->pc.enabled) return PKV_ERR_INVALID_ARG;
    if (!a->seqs.empty() || static_cast<int>(a->free_stack.size()) != a->num_blocks)
      return PKV_ERR_INVALID_ARG;
    a->pc.enabled = true;
    a->pc.model_key = model_key;
    a->pc.mask = hash_bits == 64 ? ~0ull : ((1ull << hash_bits) - 1);
    a->pc.entry.assign(a->num_blocks, CacheEntry{});
    return PKV_OK;
  } catch (...) {
    return PKV_ERR_HOST_MEMORY;
  }
}

int pkv_seq_create_cached(pkv_alloc* a, int64_t seq_id, const int32_t* tokens, int n_tokens,
                          int* n_cached_out) {
  try {
    if (!a || !a->pc.enabled || n_tokens < 0 || !n_cached_out || (n_tokens > 0 && !tokens))
      return PKV_ERR_INVALID_ARG;
    if (a->seqs.count(seq_id)) return PKV_ERR_INVALID_ARG;
    PrefixCache& pc = a->pc;
    // at most (n - 1) / bs blocks, so the last prompt token is always computed
    const int bs = a->bs;
    int64_t most = std::min<int64_t>(n_tokens > 0 ? (n_tokens - 1) / bs : 0, a->max_blocks_per_seq);
    Seq s;
    s.tracked = true;
    int32_t parent = -1;
    for (int64_t i = 0; i < most; ++i) {
      const int32_t* t = tokens + i * bs;
      int32_t b = pc.find(parent, t, pc.hash_of(parent, t));
      if (b < 0) break;
      s.table.push_back(b);
      parent = b;
    }
    for (int32_t b : s.table) a->hold(b);
    s.len = static_cast<int64_t>(s.table.size()) * bs;
    pc.lookup_blocks += most;
    pc.hit_blocks += static_cast<int64_t>(s.table.size());
    *n_cached_out = static_cast<int>(s.len);
    a->seqs.emplace(seq_id, std::move(s));
    a->seq_order.push_back(seq_id);
    return PKV_OK;
  } catch (...) {
    return PKV_ERR_HOST_MEMORY;
  }
}

int pkv_prefix_stats(pkv_alloc* a, pkv_prefix_stats_t* out) {
  if (!a || !out) return PKV_ERR_INVALID_ARG;
  out->cached_blocks = a->pc.cached;
  out->evictable_blocks = a->pc.evictable;
  out->lookup_blocks = a->pc.lookup_blocks;
  out->hit_blocks = a->pc.hit_blocks;
  out->evictions = a->pc.evictions;
  return PKV_OK;
}

int pkv_build_block_tables(pkv_alloc* a, const int64_t* seq_ids, int n, int max_blocks_per_seq,
                           int32_t* tables_out, int32_t* lens_out) {
  try {
    if (!a || n < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
    if (n > 0 && (!seq_ids || !tables_out || !lens_out)) return PKV_ERR_INVALID_ARG;
    for (int i = 0; i < n; ++i) {
      auto it = a->seqs.find(seq_ids[i]);
      if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
      if (it->second.swapped) return PKV_ERR_INVALID_ARG;
      if (static_cast<int64_t>(it->second.table.size()) > max_blocks_per_seq)
        return PKV_ERR_INVALID_ARG;
    }
    for (int i = 0; i < n; ++i) {
      const Seq& s = a->seqs[seq_ids[i]];
      int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks_per_seq;
      std::fill(row, row + max_blocks_per_seq, 0);
      std::copy(s.table.begin(), s.table.end(), row);
      lens_out[i] = static_cast<int32_t>(s.len);
    }
    return PKV_OK;
  } catch (...) {
    return PKV_ERR_HOST_MEMORY;
  }
}

int pkv_alloc_stats(pkv_alloc* a, pkv_alloc_stats_t* out) {
  if (!a || !out) return PKV_ERR_INVALID_ARG;
  std::vector<int32_t> filled(a->num_blocks, 0);
  int64_t cached = 0;
  for (int64_t id : a->seq_order) {
    const Seq& s = a->seqs[id];
    if (s.swapped) continue;
    cached += s.len;
    for (size_t i = 0; i < s.table.size(); ++i) {
      int64_t f = std::min<int64_t>(a->bs, s.len - static_cast<int64_t>(i) * a->bs);
      filled[s.table[i]] = std::max<int32_t>(filled[s.table[i]], static_cast<int32_t>(f));
    }
  }
  int64_t used = 0, shared = 0, stored = 0;
  for (int b = 0; b < a->num_blocks; ++b) {
    if (a->ref[b] > 0) ++used;
    if (a->ref[b] > 1) ++shared;
    stored += filled[b];
  }
  out->num_blocks = a->num_blocks;
  out->free_blocks = static_cast<int64_t>(a->free_stack.size());
  out->used_blocks = used;
  out->shared_blocks = shared;
  out->cow_copies = a->cow_copies;
  out->cached_tokens = cached;
  out->stored_tokens = stored;
  out->utilisation = used ? static_cast<double>(stored) / (static_cast<double>(a->bs) * used) : 0.0;
  return PKV_OK;
}

int pkv_seq_swap_out(pkv_alloc* a, int64_t seq_id, int32_t* blocks_out, int* n_out) {
  try {
    if (!a || !n_out) return PKV_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    Seq& s = it->second;
    if (s.swapped) return PKV_ERR_INVALID_ARG;
    if (!s.table.empty() && !blocks_out) return PKV_ERR_INVALID_ARG;
    for (int32_t b : s.table)
      if (a->ref[b] != 1) return PKV_ERR_INVALID_ARG;       // shared: its holders would lose it
    std::copy(s.table.begin(), s.table.end(), blocks_out);
    *n_out = static_cast<int>(s.table.size());
    for (int32_t b : s.table) a->release(b);
    s.table.clear();
    s.swapped = true;
    s.tracked = false;                                      // swapped-in copies are private
    s.pending.clear();
    return PKV_OK;
  } catch (...) {
    return PKV_ERR_HOST_MEMORY;
  }
}

int pkv_seq_swap_in(pkv_alloc* a, int64_t seq_id, int32_t* blocks_out, int* n_out) {
  try {
    if (!a || !n_out) return PKV_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    Seq& s = it->second;
    if (!s.swapped) return PKV_ERR_INVALID_ARG;
    const int64_t need = a->blocks_for(s.len);
    if (need > 0 && !blocks_out) return PKV_ERR_INVALID_ARG;
    if (need > a->available()) return PKV_ERR_NO_FREE_BLOCKS;
    for (int64_t i = 0; i < need; ++i) s.table.push_back(a->take());
    std::copy(s.table.begin(), s.table.end(), blocks_out);
    *n_out = static_cast<int>(need);
    s.swapped = false;
    return PKV_OK;
  } catch (...) {
    return PKV_ERR_HOST_MEMORY;
  }
}

}  // extern "C"
