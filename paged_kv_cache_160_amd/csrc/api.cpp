// C-ABI shim: host-side argument checks, workspace sizing and kernel
// dispatch.  Nothing here allocates device memory or synchronises.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "launch.h"
#include "pagedkv.h"

#ifndef PKV_DECODE_MERGE_HERE_MAX
#define PKV_DECODE_MERGE_HERE_MAX 4   // most partitions a one-call decode merges inside its attention kernel
#endif
#ifndef PKV_DECODE_MERGE_HERE_WGS
#define PKV_DECODE_MERGE_HERE_WGS 512 // ... more than two only in launches of at most this many workgroups
#endif

namespace {

constexpr int kTile = 16;     // partitions are whole 16-token tiles

bool block_size_ok(int bs) { return bs == PKV_BLOCK_SIZE || bs == PKV_BLOCK_SIZE_LARGE; }

// Kernels index 16-row tiles with int32: (num_blocks * num_kv_heads) tiles
// per 16 tokens of block must fit.
bool tiles_fit(int num_blocks, int num_kv_heads, int block_size) {
  return static_cast<int64_t>(num_blocks) * num_kv_heads * (block_size / kTile) < (static_cast<int64_t>(1) << 31);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int d) { return d >= PKV_F32 && d <= PKV_INT8_INT4; }

// Caches holding codes plus a float32 scale per (token, head).
bool quantised(pkv_dtype c) { return c == PKV_FP8_E4M3 || c == PKV_FP8_E5M2 || c == PKV_INT8_INT4; }

// dtypes K/V rows may arrive in (the cache write quantises them if needed).
bool source_dtype(pkv_dtype d) { return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16; }

bool supported_head_dim(int d) { return d == 64 || d == 128; }

// (q dtype, cache dtype) pairs the decode kernels are built for.
bool decode_pair_ok(pkv_dtype q, pkv_dtype c) {
  if (quantised(c)) return q == PKV_BF16 || q == PKV_F16;
  return q == c && source_dtype(q);
}

int resolve_partitions(int num_seqs, int num_kv_heads, int max_context_len, int partition_size,
                       pkv_dtype cache_dtype, int* ps_out, int* np_out) {
  int ps = partition_size;
  if (ps == 0) ps = pkv::choose_partition_size(num_seqs, num_kv_heads, max_context_len, cache_dtype);
  if (ps <= 0 || ps % kTile != 0 || ps > PKV_MAX_PARTITION_TOKENS) return PKV_ERR_INVALID_ARG;
  int64_t np = (static_cast<int64_t>(max_context_len) + ps - 1) / ps;
  if (np < 1) np = 1;
  if (np > (1 << 20)) return PKV_ERR_UNSUPPORTED;
  *ps_out = ps;
  *np_out = static_cast<int>(np);
  return PKV_OK;
}

// Workspace layout: the one-call form's counters (two int32 for each of up
// to PKV_WS_COUNTER_UNITS (sequence, KV head) pairs, zero between calls; a
// fixed size, so that no call of any size ever writes states where another
// call keeps counters), then per (sequence, query head, partition) (m, l)
// pairs, then the unnormalised partition outputs; each part 256-byte
// aligned.
struct WorkspaceLayout {
  size_t counters = 0, order = 0, ml = 0, acc = 0, total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

constexpr size_t kCounterBytes = static_cast<size_t>(PKV_WS_COUNTER_UNITS) * 2 * sizeof(int32_t);

WorkspaceLayout workspace_layout(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int np) {
  WorkspaceLayout w;
  if (np <= 1) {
    // a single-partition launch needs a workspace only for the longest-first
    // order (kept after the counter area, which it leaves untouched)
    if (pkv::decode_order_in_workspace(num_seqs, num_kv_heads, np)) {
      w.order = kCounterBytes;
      w.total = w.order + align256(static_cast<size_t>(num_seqs) * sizeof(int32_t));
    }
    return w;
  }
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * np;
  w.counters = 0;
  w.ml = kCounterBytes;
  w.acc = w.ml + align256(rows * 2 * sizeof(float));
  w.total = w.acc + rows * head_dim * sizeof(float);
  return w;
}

bool decode_sizes_ok(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                     int max_context_len) {
  // (sequence, query head) rows index the merge grid and the workspace
  return num_seqs >= 0 && num_kv_heads > 0 && num_q_heads > 0 && num_q_heads % num_kv_heads == 0 &&
         max_context_len >= 0 && head_dim > 0 && static_cast<int64_t>(num_seqs) * num_q_heads <= 0x7fffffff;
}

}  // namespace

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_strerror(int code) {
  switch (code) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported dtype, head_dim or group size";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_NO_FREE_BLOCKS: return "no free blocks";
    case PKV_ERR_UNKNOWN_SEQ: return "unknown sequence id";
    case PKV_ERR_HOST_MEMORY: return "host memory exhausted (allocator state may be partly updated)";
    case PKV_ERR_SCRATCH: return "decode sizes need more than the library's fixed scratch (PKV_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

int kv_cache_append_bs(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                       float* k_scale, float* v_scale, const int64_t* slot_mapping, int num_tokens,
                       int num_kv_heads, int head_dim, int num_blocks, int block_size, pkv_dtype src_dtype,
                       pkv_dtype cache_dtype, void* stream) {
  if (!valid_dtype(src_dtype) || !valid_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0 || !block_size_ok(block_size))
    return PKV_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (!source_dtype(src_dtype)) return PKV_ERR_UNSUPPORTED;
  if (!quantised(cache_dtype) && src_dtype != cache_dtype) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (quantised(cache_dtype) && (!k_scale || !v_scale)) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return PKV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(num_tokens) * num_kv_heads > (static_cast<int64_t>(1) << 31))
    return PKV_ERR_UNSUPPORTED;
  return pkv::launch_append(k_new, v_new, k_pool, v_pool, k_scale, v_scale, slot_mapping, num_tokens,
                            num_kv_heads, head_dim, num_blocks, block_size, src_dtype, cache_dtype,
                            static_cast<hipStream_t>(stream));
}

int kv_cache_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                    float* k_scale, float* v_scale, const int64_t* slot_mapping, int num_tokens,
                    int num_kv_heads, int head_dim, int num_blocks, pkv_dtype src_dtype,
                    pkv_dtype cache_dtype, void* stream) {
  return kv_cache_append_bs(k_new, v_new, k_pool, v_pool, k_scale, v_scale, slot_mapping, num_tokens,
                            num_kv_heads, head_dim, num_blocks, PKV_BLOCK_SIZE, src_dtype, cache_dtype, stream);
}

int pkv_copy_blocks_bs(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                       const int32_t* pairs, int n_pairs, int num_kv_heads, int head_dim,
                       int num_blocks, int block_size, pkv_dtype cache_dtype, void* stream) {
  if (!valid_dtype(cache_dtype) || n_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      !block_size_ok(block_size))
    return PKV_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (n_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !pairs) return PKV_ERR_INVALID_ARG;
  if (quantised(cache_dtype) && (!k_scale || !v_scale)) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_pool) || !aligned16(v_pool)) return PKV_ERR_INVALID_ARG;
  if (n_pairs > 65535 || num_kv_heads > 65535) return PKV_ERR_UNSUPPORTED;
  return pkv::launch_copy_blocks(k_pool, v_pool, k_scale, v_scale, pairs, n_pairs, num_kv_heads,
                                 head_dim, num_blocks, block_size, cache_dtype, static_cast<hipStream_t>(stream));
}

int pkv_copy_blocks(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                    const int32_t* pairs, int n_pairs, int num_kv_heads, int head_dim,
                    int num_blocks, pkv_dtype cache_dtype, void* stream) {
  return pkv_copy_blocks_bs(k_pool, v_pool, k_scale, v_scale, pairs, n_pairs, num_kv_heads, head_dim,
                            num_blocks, PKV_BLOCK_SIZE, cache_dtype, stream);
}

int pkv_decode_partition_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                              int max_context_len, pkv_dtype cache_dtype, int* partition_size_out,
                              int* num_partitions_out) {
  (void)head_dim;
  if (!partition_size_out || !num_partitions_out || !valid_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
  if (!decode_sizes_ok(num_seqs, num_q_heads, num_kv_heads, 64, max_context_len))
    return PKV_ERR_INVALID_ARG;
  return resolve_partitions(num_seqs, num_kv_heads, max_context_len, 0, cache_dtype, partition_size_out,
                            num_partitions_out);
}


size_t paged_attention_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                      int head_dim, int max_context_len, int partition_size,
                                      pkv_dtype cache_dtype) {
  if (!valid_dtype(cache_dtype)) return 0;
  if (!decode_sizes_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len)) return 0;
  int ps, np;
  if (resolve_partitions(num_seqs, num_kv_heads, max_context_len, partition_size, cache_dtype, &ps, &np) !=
      PKV_OK)
    return 0;
  return workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, np).total;
}

}  // extern "C"

namespace {

int decode_impl(void* out, const void* q, const void* k_new, const void* v_new, const void* k_pool,
                const void* v_pool, const float* k_scale, const float* v_scale, const int64_t* slot_mapping,
                const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int num_q_heads,
                int num_kv_heads, int head_dim, int num_blocks, int block_size, int max_blocks_per_seq,
                int max_context_len, float scale, pkv_dtype q_dtype, pkv_dtype src_dtype, pkv_dtype cache_dtype,
                int partition_size, void* workspace, size_t workspace_bytes, void* stream, int stages) {
  if (!valid_dtype(q_dtype) || !valid_dtype(cache_dtype) || !valid_dtype(src_dtype)) return PKV_ERR_INVALID_ARG;
  if (!decode_sizes_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len))
    return PKV_ERR_INVALID_ARG;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0 || !block_size_ok(block_size)) return PKV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PKV_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (!decode_pair_ok(q_dtype, cache_dtype)) return PKV_ERR_UNSUPPORTED;
  if (!tiles_fit(num_blocks, num_kv_heads, block_size)) return PKV_ERR_UNSUPPORTED;
  if (slot_mapping) {
    if (!source_dtype(src_dtype)) return PKV_ERR_UNSUPPORTED;
    if (!quantised(cache_dtype) && src_dtype != cache_dtype) return PKV_ERR_UNSUPPORTED;
  }
  if (num_q_heads / num_kv_heads > 16) return PKV_ERR_UNSUPPORTED;
  if (partition_size < 0 || partition_size % kTile != 0 || partition_size > PKV_MAX_PARTITION_TOKENS)
    return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PKV_ERR_INVALID_ARG;
  if (quantised(cache_dtype) && (!k_scale || !v_scale)) return PKV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return PKV_ERR_INVALID_ARG;
  if (quantised(cache_dtype) && (!aligned16(k_scale) || !aligned16(v_scale)))
    return PKV_ERR_INVALID_ARG;
  if (slot_mapping && (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))) return PKV_ERR_INVALID_ARG;

  int ps, np;
  int rc = resolve_partitions(num_seqs, num_kv_heads, max_context_len, partition_size, cache_dtype, &ps, &np);
  if (rc != PKV_OK) return rc;
  const WorkspaceLayout ws = workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, np);
  // a single-partition launch without room for the order runs in index order
  const bool room = workspace && workspace_bytes >= ws.total && aligned16(workspace);
  if (np > 1 && !room) return PKV_ERR_WORKSPACE;

  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.scale = scale;
  a.q_dtype = q_dtype;
  a.cache_dtype = cache_dtype;
  a.partition_size = ps;
  a.num_partitions = np;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot_mapping = slot_mapping;
  a.src_dtype = src_dtype;
  if (np == 1 && ws.total > 0 && room)
    a.seq_order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + ws.order);
  if (np > 1) {
    char* base = static_cast<char*>(workspace);
    a.part_ml = reinterpret_cast<float*>(base + ws.ml);
    a.part_acc = reinterpret_cast<float*>(base + ws.acc);
    // the one-call form merges inside the attention kernel for up to two
    // partitions, and for three or four when the launch has at most
    // PKV_DECODE_MERGE_HERE_WGS workgroups, with at most PKV_WS_COUNTER_UNITS
    // (sequence, KV head) pairs; otherwise a merge kernel follows, as in the
    // split form (same bits).  Interleaved A/B: the shared-prefix batch (4
    // partitions, 256 workgroups) 13.95 against 14.25 us, int8 K + int4 V on
    // the Llama-3-8B shape (4 partitions, 512 workgroups) 26.9 against
    // 27.45 us; 32 x 32768 fp8 tokens in 8 partitions (2048 workgroups)
    // 389 against 377 us - there the last partition to finish reads many
    // states back while other workgroups wait for its CU slot, and the
    // merging instance's registers cost the long launch.
    const int64_t wgs = static_cast<int64_t>(num_seqs) * num_kv_heads * np;
    const bool here = np <= 2 || (np <= PKV_DECODE_MERGE_HERE_MAX && wgs <= PKV_DECODE_MERGE_HERE_WGS);
    if (stages == pkv::kStageBoth && here &&
        static_cast<int64_t>(num_seqs) * num_kv_heads <= static_cast<int64_t>(PKV_WS_COUNTER_UNITS)) {
      a.counters = reinterpret_cast<int*>(base + ws.counters);
    }
  }
  return pkv::launch_decode(a, static_cast<hipStream_t>(stream), stages);
}

}  // namespace

extern "C" {

int paged_attention_decode_bs(void* out, const void* q, const void* k_pool, const void* v_pool,
                              const float* k_scale, const float* v_scale, const int32_t* block_tables,
                              const int32_t* context_lens, int num_seqs, int num_q_heads,
                              int num_kv_heads, int head_dim, int num_blocks, int block_size,
                              int max_blocks_per_seq, int max_context_len, float scale, pkv_dtype q_dtype,
                              pkv_dtype cache_dtype, int partition_size, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, nullptr, nullptr, k_pool, v_pool, k_scale, v_scale, nullptr, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                     max_blocks_per_seq, max_context_len, scale, q_dtype, q_dtype, cache_dtype,
                     partition_size, workspace, workspace_bytes, stream, pkv::kStageBoth);
}

int paged_attention_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                           const float* k_scale, const float* v_scale, const int32_t* block_tables,
                           const int32_t* context_lens, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_dim, int num_blocks, int max_blocks_per_seq,
                           int max_context_len, float scale, pkv_dtype q_dtype,
                           pkv_dtype cache_dtype, int partition_size, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return paged_attention_decode_bs(out, q, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens,
                                   num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, PKV_BLOCK_SIZE,
                                   max_blocks_per_seq, max_context_len, scale, q_dtype, cache_dtype,
                                   partition_size, workspace, workspace_bytes, stream);
}

int paged_attention_decode_append_bs(void* out, const void* q, const void* k_new, const void* v_new,
                                     void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                     const int64_t* slot_mapping, const int32_t* block_tables,
                                     const int32_t* context_lens, int num_seqs, int num_q_heads,
                                     int num_kv_heads, int head_dim, int num_blocks, int block_size,
                                     int max_blocks_per_seq, int max_context_len, float scale, pkv_dtype q_dtype,
                                     pkv_dtype src_dtype, pkv_dtype cache_dtype, int partition_size,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!slot_mapping) return PKV_ERR_INVALID_ARG;
  return decode_impl(out, q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, slot_mapping, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                     max_blocks_per_seq, max_context_len, scale, q_dtype, src_dtype, cache_dtype,
                     partition_size, workspace, workspace_bytes, stream, pkv::kStageBoth);
}

int paged_attention_decode_append_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                                          void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                          const int64_t* slot_mapping, const int32_t* block_tables,
                                          const int32_t* context_lens, int num_seqs, int num_q_heads,
                                          int num_kv_heads, int head_dim, int num_blocks, int block_size,
                                          int max_blocks_per_seq, int max_context_len, float scale,
                                          pkv_dtype q_dtype, pkv_dtype src_dtype, pkv_dtype cache_dtype,
                                          int partition_size, void* stream) {
  if (!slot_mapping) return PKV_ERR_INVALID_ARG;
  // invalid sizes give 0 here and are reported by decode_impl
  const size_t need = paged_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                     max_context_len, partition_size, cache_dtype);
  if (need > static_cast<size_t>(PKV_SCRATCH_BYTES)) return PKV_ERR_SCRATCH;
  void* scratch = nullptr;
  if (need > 0) {
    const int rc = pkv::scratch_workspace(static_cast<hipStream_t>(stream), &scratch);
    if (rc != PKV_OK) return rc;
  }
  return decode_impl(out, q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, slot_mapping, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                     max_blocks_per_seq, max_context_len, scale, q_dtype, src_dtype, cache_dtype,
                     partition_size, scratch, need > 0 ? static_cast<size_t>(PKV_SCRATCH_BYTES) : 0, stream,
                     pkv::kStageBoth);
}

int paged_attention_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                                  void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                  const int64_t* slot_mapping, const int32_t* block_tables,
                                  const int32_t* context_lens, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int num_blocks, int max_blocks_per_seq,
                                  int max_context_len, float scale, pkv_dtype q_dtype, pkv_dtype src_dtype,
                                  pkv_dtype cache_dtype, int partition_size, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return paged_attention_decode_append_bs(out, q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, slot_mapping,
                                          block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
                                          head_dim, num_blocks, PKV_BLOCK_SIZE, max_blocks_per_seq,
                                          max_context_len, scale, q_dtype, src_dtype, cache_dtype, partition_size,
                                          workspace, workspace_bytes, stream);
}

int paged_attention_decode_append_partials_bs(void* out, const void* q, const void* k_new, const void* v_new,
                                              void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                              const int64_t* slot_mapping, const int32_t* block_tables,
                                              const int32_t* context_lens, int num_seqs, int num_q_heads,
                                              int num_kv_heads, int head_dim, int num_blocks, int block_size,
                                              int max_blocks_per_seq, int max_context_len, float scale,
                                              pkv_dtype q_dtype, pkv_dtype src_dtype, pkv_dtype cache_dtype,
                                              int partition_size, void* workspace, size_t workspace_bytes,
                                              void* stream) {
  return decode_impl(out, q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, slot_mapping, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                     max_blocks_per_seq, max_context_len, scale, q_dtype, src_dtype, cache_dtype,
                     partition_size, workspace, workspace_bytes, stream, pkv::kStageAttend);
}

int paged_attention_decode_append_partials(void* out, const void* q, const void* k_new, const void* v_new,
                                           void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                           const int64_t* slot_mapping, const int32_t* block_tables,
                                           const int32_t* context_lens, int num_seqs, int num_q_heads,
                                           int num_kv_heads, int head_dim, int num_blocks,
                                           int max_blocks_per_seq, int max_context_len, float scale,
                                           pkv_dtype q_dtype, pkv_dtype src_dtype, pkv_dtype cache_dtype,
                                           int partition_size, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  return paged_attention_decode_append_partials_bs(
      out, q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, slot_mapping, block_tables, context_lens, num_seqs,
      num_q_heads, num_kv_heads, head_dim, num_blocks, PKV_BLOCK_SIZE, max_blocks_per_seq, max_context_len, scale,
      q_dtype, src_dtype, cache_dtype, partition_size, workspace, workspace_bytes, stream);
}

int paged_attention_merge_partials_bs(void* out, const int32_t* context_lens, int num_seqs, int num_q_heads,
                                      int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                                      int max_context_len, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                      int partition_size, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (!valid_dtype(q_dtype) || !source_dtype(q_dtype) || !valid_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
  if (!decode_sizes_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len))
    return PKV_ERR_INVALID_ARG;
  if (max_blocks_per_seq <= 0 || !block_size_ok(block_size) ||
      static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PKV_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (partition_size < 0 || partition_size % kTile != 0 || partition_size > PKV_MAX_PARTITION_TOKENS)
    return PKV_ERR_INVALID_ARG;
  int ps, np;
  int rc = resolve_partitions(num_seqs, num_kv_heads, max_context_len, partition_size, cache_dtype, &ps, &np);
  if (rc != PKV_OK) return rc;
  if (num_seqs == 0 || np == 1) return PKV_OK;       // nothing was split
  if (!out || !context_lens || !aligned16(out)) return PKV_ERR_INVALID_ARG;
  const WorkspaceLayout ws = workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, np);
  if (!workspace || workspace_bytes < ws.total || !aligned16(workspace)) return PKV_ERR_WORKSPACE;
  pkv::DecodeArgs a{};
  a.out = out;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.q_dtype = q_dtype;
  // the merge kernel is instantiated per output dtype; any cache dtype that
  // pairs with q_dtype selects the same one
  a.cache_dtype = q_dtype;
  a.partition_size = ps;
  a.num_partitions = np;
  char* base = static_cast<char*>(workspace);
  a.part_ml = reinterpret_cast<float*>(base + ws.ml);
  a.part_acc = reinterpret_cast<float*>(base + ws.acc);
  return pkv::launch_decode(a, static_cast<hipStream_t>(stream), pkv::kStageMerge);
}

int paged_attention_merge_partials(void* out, const int32_t* context_lens, int num_seqs, int num_q_heads,
                                   int num_kv_heads, int head_dim, int max_blocks_per_seq, int max_context_len,
                                   pkv_dtype q_dtype, pkv_dtype cache_dtype, int partition_size, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return paged_attention_merge_partials_bs(out, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           PKV_BLOCK_SIZE, max_blocks_per_seq, max_context_len, q_dtype,
                                           cache_dtype, partition_size, workspace, workspace_bytes, stream);
}

int paged_attention_prefill_bs(void* out, const void* q, const void* k_pool, const void* v_pool,
                               const float* k_scale, const float* v_scale, const int32_t* block_tables,
                               const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                               int num_tokens, int num_q_heads, int num_kv_heads, int head_dim, int num_blocks,
                               int block_size, int max_blocks_per_seq, int max_context_len, int max_query_len,
                               float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, void* stream) {
  if (!valid_dtype(q_dtype) || !valid_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
  if (!decode_sizes_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len))
    return PKV_ERR_INVALID_ARG;
  if (num_tokens < 0 || max_query_len < 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      !block_size_ok(block_size))
    return PKV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PKV_ERR_INVALID_ARG;
  if (max_query_len > max_context_len || max_query_len > num_tokens) return PKV_ERR_INVALID_ARG;
  // the kernel takes row maxima of raw scores: the scale must be positive
  if (!(scale > 0.0f) || !std::isfinite(scale)) return PKV_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (q_dtype == PKV_F32 || !decode_pair_ok(q_dtype, cache_dtype)) return PKV_ERR_UNSUPPORTED;
  if (max_context_len > PKV_MAX_PREFILL_CONTEXT) return PKV_ERR_UNSUPPORTED;
  if (!tiles_fit(num_blocks, num_kv_heads, block_size)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return PKV_ERR_INVALID_ARG;
  if (quantised(cache_dtype) && (!k_scale || !v_scale)) return PKV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out)) return PKV_ERR_INVALID_ARG;

  pkv::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.max_query_len = max_query_len;
  a.scale = scale;
  a.q_dtype = q_dtype;
  a.cache_dtype = cache_dtype;
  return pkv::launch_prefill(a, static_cast<hipStream_t>(stream));
}

int paged_attention_prefill(void* out, const void* q, const void* k_pool, const void* v_pool,
                            const float* k_scale, const float* v_scale, const int32_t* block_tables,
                            const int32_t* context_lens, const int32_t* query_start, int num_seqs, int num_tokens,
                            int num_q_heads, int num_kv_heads, int head_dim, int num_blocks, int max_blocks_per_seq,
                            int max_context_len, int max_query_len, float scale, pkv_dtype q_dtype,
                            pkv_dtype cache_dtype, void* stream) {
  return paged_attention_prefill_bs(out, q, k_pool, v_pool, k_scale, v_scale, block_tables, context_lens,
                                    query_start, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                                    num_blocks, PKV_BLOCK_SIZE, max_blocks_per_seq, max_context_len, max_query_len,
                                    scale, q_dtype, cache_dtype, stream);
}

}  // extern "C"

namespace {

int swap_impl(void* staging, void* pool, const int32_t* blocks, int n_blocks, int64_t block_bytes, int num_blocks,
              bool to_staging, void* stream) {
  if (n_blocks < 0 || num_blocks <= 0 || block_bytes <= 0 || block_bytes % 16 != 0) return PKV_ERR_INVALID_ARG;
  if (n_blocks == 0) return PKV_OK;
  if (!staging || !pool || !blocks || !aligned16(staging) || !aligned16(pool)) return PKV_ERR_INVALID_ARG;
  if (n_blocks > 0x7fffffff / 2) return PKV_ERR_UNSUPPORTED;
  return pkv::launch_swap_blocks(staging, pool, blocks, n_blocks, block_bytes, num_blocks, to_staging,
                                 static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int pkv_gather_blocks(void* staging, const void* pool, const int32_t* blocks, int n_blocks, int64_t block_bytes,
                      int num_blocks, void* stream) {
  return swap_impl(staging, const_cast<void*>(pool), blocks, n_blocks, block_bytes, num_blocks, true, stream);
}

int pkv_scatter_blocks(void* pool, const void* staging, const int32_t* blocks, int n_blocks, int64_t block_bytes,
                       int num_blocks, void* stream) {
  return swap_impl(const_cast<void*>(staging), pool, blocks, n_blocks, block_bytes, num_blocks, false, stream);
}

}  // extern "C"
