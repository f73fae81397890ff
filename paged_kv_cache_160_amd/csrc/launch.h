// Host-side declarations shared by the C-ABI shim and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include "pagedkv.h"

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
  // One-call form: per (sequence, KV head) an arrival and a published count,
  // zero between calls; the last partition of a sequence to finish merges.
  // nullptr: the attention kernel writes every partition state and a merge
  // kernel combines them (split form).
  int* counters;           // [num_seqs][num_kv_heads][2]
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

// Automatic partition length for a decode launch (tokens, multiple of 16).
int choose_partition_size(int num_seqs, int num_kv_heads, int max_context_len, pkv_dtype cache_dtype);

}  // namespace pkv
