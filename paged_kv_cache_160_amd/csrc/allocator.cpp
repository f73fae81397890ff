// Host block allocator for the paged KV cache: free list, per-sequence block
// tables, reference counts, fork and copy-on-write planning.
//
// Pages: blocks of 16 tokens are taken on demand when a sequence's current
// block is full ("KV Cache 和 vLLM" §3.1); finished sequences return their
// blocks and later sequences reuse them wherever they lie ("KV Cache优化实战"
// §4.2); sequences with a common prefix share physical blocks, and
// copy-on-write covers writes into shared blocks ("KV Cache 和 vLLM" §3.3);
// running out of cache degrades instead of crashing ("企业官网建设流程全解析"
// §6.4), so every failing call here leaves the state untouched.
//
// The rules the pages leave open (reference counts, a stack-ordered free
// list, release order, which writer copies) are stated in include/pagedkv.h.

#include <algorithm>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

namespace {

constexpr int kBlock = PKV_BLOCK_SIZE;

inline int64_t blocks_for(int64_t len) { return (len + kBlock - 1) / kBlock; }

struct Seq {
  std::vector<int32_t> table;
  int64_t len = 0;
};

}  // namespace

struct pkv_alloc {
  int32_t num_blocks = 0;
  int32_t max_blocks_per_seq = 0;
  std::vector<int32_t> free_stack;   // back() is handed out next
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<int64_t> seq_order;    // creation order, for deterministic stats walks
  int64_t cow_copies = 0;

  int32_t take() {
    int32_t b = free_stack.back();
    free_stack.pop_back();
    ref[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) free_stack.push_back(b);
  }

  // Fresh blocks an append of n tokens needs, and whether it copies first.
  void plan(const Seq& s, int64_t n, bool* cow, int64_t* fresh) const {
    *cow = n > 0 && (s.len % kBlock) != 0 && ref[s.table.back()] > 1;
    *fresh = blocks_for(s.len + n) - blocks_for(s.len);
  }

  // Apply a planned append; capacity was checked by the caller.
  void apply(Seq& s, int64_t n, int64_t* slots, int32_t* pair, int* n_cow) {
    *n_cow = 0;
    if (n > 0 && (s.len % kBlock) != 0 && ref[s.table.back()] > 1) {
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
      if (p % kBlock == 0) s.table.push_back(take());
      slots[i] = static_cast<int64_t>(s.table[p / kBlock]) * kBlock + p % kBlock;
    }
    s.len += n;
  }
};

extern "C" {

pkv_alloc* pkv_alloc_create(int num_blocks, int max_blocks_per_seq) {
  if (num_blocks <= 0 || max_blocks_per_seq <= 0) return nullptr;
  pkv_alloc* a = new (std::nothrow) pkv_alloc();
  if (!a) return nullptr;
  a->num_blocks = num_blocks;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->ref.assign(num_blocks, 0);
  a->free_stack.resize(num_blocks);
  for (int i = 0; i < num_blocks; ++i) a->free_stack[i] = num_blocks - 1 - i;
  return a;
}

void pkv_alloc_destroy(pkv_alloc* a) { delete a; }

int pkv_alloc_set_free_order(pkv_alloc* a, const int32_t* order, int n) {
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
}

int pkv_seq_create(pkv_alloc* a, int64_t seq_id) {
  if (!a) return PKV_ERR_INVALID_ARG;
  if (a->seqs.count(seq_id)) return PKV_ERR_INVALID_ARG;
  a->seqs.emplace(seq_id, Seq{});
  a->seq_order.push_back(seq_id);
  return PKV_OK;
}

int pkv_seq_fork(pkv_alloc* a, int64_t parent, int64_t child) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  if (a->seqs.count(child)) return PKV_ERR_INVALID_ARG;
  Seq c = it->second;
  for (int32_t b : c.table) ++a->ref[b];
  a->seqs.emplace(child, std::move(c));
  a->seq_order.push_back(child);
  return PKV_OK;
}

int pkv_seq_free(pkv_alloc* a, int64_t seq_id) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  for (int32_t b : it->second.table) a->release(b);
  a->seqs.erase(it);
  a->seq_order.erase(std::find(a->seq_order.begin(), a->seq_order.end(), seq_id));
  return PKV_OK;
}

int pkv_seq_len(pkv_alloc* a, int64_t seq_id) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  return static_cast<int>(it->second.len);
}

int pkv_seq_append_slots(pkv_alloc* a, int64_t seq_id, int n_tokens, int64_t* slots_out,
                         int32_t* cow_pairs_out, int* n_cow_out) {
  if (!a || n_tokens < 0 || !n_cow_out || !cow_pairs_out || (n_tokens > 0 && !slots_out))
    return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  Seq& s = it->second;
  bool cow;
  int64_t fresh;
  a->plan(s, n_tokens, &cow, &fresh);
  if (static_cast<int64_t>(s.table.size()) + fresh > a->max_blocks_per_seq)
    return PKV_ERR_INVALID_ARG;
  if ((cow ? 1 : 0) + fresh > static_cast<int64_t>(a->free_stack.size()))
    return PKV_ERR_NO_FREE_BLOCKS;
  a->apply(s, n_tokens, slots_out, cow_pairs_out, n_cow_out);
  return PKV_OK;
}

int pkv_batch_append_one(pkv_alloc* a, const int64_t* seq_ids, int n, int64_t* slots_out,
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
    if (seen[seq_ids[i]]++) return PKV_ERR_INVALID_ARG;
    const Seq& s = it->second;
    int64_t fresh = blocks_for(s.len + 1) - blocks_for(s.len);
    bool cow = false;
    if (s.len % kBlock != 0) {
      int32_t last = s.table.back();
      cow = a->ref[last] - dropped[last] > 1;
      if (cow) ++dropped[last];
    }
    if (static_cast<int64_t>(s.table.size()) + fresh > a->max_blocks_per_seq)
      return PKV_ERR_INVALID_ARG;
    need += (cow ? 1 : 0) + fresh;
  }
  if (need > static_cast<int64_t>(a->free_stack.size())) return PKV_ERR_NO_FREE_BLOCKS;
  int n_cow = 0;
  for (int i = 0; i < n; ++i) {
    int c = 0;
    a->apply(a->seqs[seq_ids[i]], 1, slots_out + i, cow_pairs_out + 2 * n_cow, &c);
    n_cow += c;
  }
  *n_cow_out = n_cow;
  return PKV_OK;
}

int pkv_build_block_tables(pkv_alloc* a, const int64_t* seq_ids, int n, int max_blocks_per_seq,
                           int32_t* tables_out, int32_t* lens_out) {
  if (!a || n < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
  if (n > 0 && (!seq_ids || !tables_out || !lens_out)) return PKV_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
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
}

int pkv_alloc_stats(pkv_alloc* a, pkv_alloc_stats_t* out) {
  if (!a || !out) return PKV_ERR_INVALID_ARG;
  std::vector<int32_t> filled(a->num_blocks, 0);
  int64_t cached = 0;
  for (int64_t id : a->seq_order) {
    const Seq& s = a->seqs[id];
    cached += s.len;
    for (size_t i = 0; i < s.table.size(); ++i) {
      int64_t f = std::min<int64_t>(kBlock, s.len - static_cast<int64_t>(i) * kBlock);
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
  out->utilisation = used ? static_cast<double>(stored) / (static_cast<double>(kBlock) * used) : 0.0;
  return PKV_OK;
}

}  // extern "C"
