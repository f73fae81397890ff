// Host-side declarations shared by the C-ABI shim and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include "pagedkv.h"

#ifndef PKV_DECODE_ORDER
#define PKV_DECODE_ORDER 1     // longest-first order for many single-partition workgroups
#endif

namespace pkv {

// Map the runtime's last error after a launch to a return code.
inline int check_launch() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int launch_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                  float* k_scale, float* v_scale, const int64_t* slot_mapping, int num_tokens,
                  int num_kv_heads, int head_dim, int num_blocks, int block_size, pkv_dtype src_dtype,
                  pkv_dtype cache_dtype, hipStream_t stream);

int launch_copy_blocks(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                       const int32_t* pairs, int n_pairs, int num_kv_heads, int head_dim,
                       int num_blocks, int block_size, pkv_dtype cache_dtype, hipStream_t stream);

int launch_swap_blocks(void* staging, void* pool, const int32_t* blocks, int n_blocks, int64_t block_bytes,
                       int num_blocks, bool to_staging, hipStream_t stream);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int num_seqs, num_q_heads, num_kv_heads, head_dim;
  int num_blocks, max_blocks_per_seq, max_context_len;
  int block_size;          // tokens per block: 16 or 32
  float scale;
  pkv_dtype q_dtype, cache_dtype;
  int partition_size;      // tokens, multiple of 16 (resolved, never 0)
  int num_partitions;      // ceil(max_context_len / partition_size), >= 1
  // fused cache write of this step's token (slot_mapping == nullptr: none)
  const void* k_new;       // [num_seqs][num_kv_heads][head_dim] of src_dtype
  const void* v_new;
  const int64_t* slot_mapping;   // [num_seqs]: slot of position context_lens[b] - 1
  pkv_dtype src_dtype;
  // One-call form: per (sequence, KV head) two words, zero between calls;
  // the first counts arrivals (low 16 bits) and published states (above),
  // the second is unused.  The last partition of a sequence to finish merges.
  // nullptr: the attention kernel writes every partition state and a merge
  // kernel combines them (split form).
  int* counters;           // [num_seqs][num_kv_heads][2]
  // Longest-first order (single-partition launches of many workgroups,
  // decode_uses_order): workgroup r takes sequence seq_order[r], which an
  // order kernel launched just before writes; nullptr: index order.
  const int32_t* seq_order;   // [num_seqs]
  float* part_ml;          // [num_seqs][num_q_heads][num_partitions][2]  (m, l)
  float* part_acc;         // [num_seqs][num_q_heads][num_partitions][head_dim]
};

// What a decode call launches: the attention kernel and, when sequences are
// split into partitions, the merge kernel after it (or only one of them).
enum DecodeStages { kStageAttend = 1, kStageMerge = 2, kStageBoth = 3 };

int launch_decode(const DecodeArgs& a, hipStream_t stream, int stages);

struct PrefillArgs {
  void* out;                   // [num_tokens][num_q_heads][head_dim], q dtype
  const void* q;               // [num_tokens][num_q_heads][head_dim]
  const void* k_pool;
  const void* v_pool;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens; // [num_seqs]: cached length after the chunk's append
  const int32_t* query_start;  // [num_seqs + 1]: chunk b = q rows query_start[b] .. query_start[b+1]-1
  int num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim;
  int num_blocks, max_blocks_per_seq, max_context_len, max_query_len;
  int block_size;              // tokens per block: 16 or 32
  float scale;
  pkv_dtype q_dtype, cache_dtype;
  int tiles_per_seq;           // set by the launcher
};

int launch_prefill(const PrefillArgs& a, hipStream_t stream);

// The library's fixed device scratch on the current GPU (PKV_SCRATCH_BYTES,
// counters cleared on first use on the given stream).
int scratch_workspace(hipStream_t stream, void** ptr);

// Whether a decode launch takes sequences longest first: single-partition
// launches of at least four workgroups per CU (the dispatcher then hands
// them out in turns; split sequences already have workgroups of at most one
// partition each, and the order measured no faster there), for batches of
// 2 .. PKV_MAX_ORDER_SEQS sequences.
inline bool decode_uses_order(int num_seqs, int num_kv_heads, int num_partitions) {
  return PKV_DECODE_ORDER && num_partitions == 1 && num_seqs >= 2 && num_seqs <= PKV_MAX_ORDER_SEQS &&
         static_cast<int64_t>(num_seqs) * num_kv_heads >= 4 * 256;
}

// Up to this many sequences every workgroup of an ordered launch ranks the
// batch itself; larger batches are sorted once per call into the workspace.
constexpr int kMaxRankSeqs = 256;
inline bool decode_order_in_workspace(int num_seqs, int num_kv_heads, int num_partitions) {
  return decode_uses_order(num_seqs, num_kv_heads, num_partitions) && num_seqs > kMaxRankSeqs;
}

// Automatic partition length for a decode launch (tokens, multiple of 16).
int choose_partition_size(int num_seqs, int num_kv_heads, int max_context_len, pkv_dtype cache_dtype);

}  // namespace pkv
