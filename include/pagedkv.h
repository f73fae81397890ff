/*
 * pagedkv.h - C ABI of libpagedkv.so: single-token decode attention over a
 * paged KV cache on AMD Instinct MI355X (gfx950).
 *
 * The method (pages: "KV Cache 和 vLLM" §1.2-1.3, §3.1-3.3; "KV Cache优化实战"
 * §2.1, §3.2-3.3, §4.2; "企业官网建设流程全解析" §1.2-1.3, §2.2, §3.2):
 *   - each layer keeps its K and V in a pool of fixed 16-token physical blocks
 *     (or 32-token ones, "KV Cache 和 vLLM" §6.3: fewer table entries for long
 *     sequences, more unused slots for short ones);
 *   - each sequence has a block table mapping logical block i (tokens
 *     bs*i..bs*i+bs-1, bs the block size) to a physical block, so a sequence is logically contiguous
 *     and physically scattered;
 *   - a decode step appends the new token's K and V to the cache, then the new
 *     query attends over every cached token, itself included:
 *       out[h] = softmax(q[h] . K^T * scale) V,  scale = 1/sqrt(head_dim),
 *     with query head h reading KV head h / (Hq/Hkv) (grouped-query attention);
 *   - KV may be stored quantised (fp8 e4m3 or e5m2, or int8 keys with int4
 *     values) with one scale per token and per head.
 *
 * Conventions for every call:
 *   - Return value: PKV_OK (0) or a negative PKV_ERR_* code; pkv_strerror()
 *     names it.  No C++ exception crosses this interface.
 *   - Device pointers are owned by the caller (for example PyTorch tensors).
 *     The library never allocates, frees or keeps device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every device call only enqueues work on it and returns; none
 *     synchronises.  Argument checks are done on the host before anything is
 *     enqueued; a failed check enqueues nothing.  A launch failure reported by
 *     the HIP runtime is returned as PKV_ERR_HIP.
 *   - Kernels never read or write outside the buffers described below, for
 *     any contents of slot_mapping, block_tables, context_lens or pairs:
 *     out-of-range entries are skipped.  Outputs are defined only when those
 *     contents meet the stated preconditions.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_BLOCK_SIZE 16         /* tokens per physical block ("KV Cache 和 vLLM" §3.1) */
#define PKV_BLOCK_SIZE_LARGE 32   /* the other block size the _bs calls take (§6.3 there) */
#define PKV_ABI_VERSION 1
#define PKV_MAX_PARTITION_TOKENS 32768   /* largest decode partition (tokens) */
/* A decode workspace (when one is needed) starts with PKV_WS_COUNTER_BYTES of
   counters: two int32 for each of up to PKV_WS_COUNTER_UNITS (sequence, KV
   head) pairs, used by the one-call decode forms to find the last partition
   of a sequence to finish.  They must be zero before a workspace's first
   use (a zero-filled workspace is) and every call leaves them zero; the
   area's size does not depend on the call, so a workspace may serve calls
   of any size.  The rest of a workspace needs no initialisation. */
/* Single-partition decode launches of at least 1024 workgroups over batches
   of 2 .. PKV_MAX_ORDER_SEQS sequences take the sequences longest first.  For
   more than 256 sequences the order (one int32 per sequence) is computed by
   the call into its workspace, after the counter area (without a workspace of
   paged_attention_workspace_size() bytes such a launch runs in index order). */
#define PKV_MAX_ORDER_SEQS 8192
#define PKV_WS_COUNTER_UNITS 32768
#define PKV_WS_COUNTER_BYTES (PKV_WS_COUNTER_UNITS * 8)
/* Device scratch the library keeps per GPU for paged_attention_decode_append_noalloc. */
#define PKV_SCRATCH_BYTES (16 * 1024 * 1024)
#define PKV_MAX_PREFILL_CONTEXT 32768    /* longest context a prefill call reads (tokens) */

typedef enum {
  PKV_F32 = 0,
  PKV_F16 = 1,
  PKV_BF16 = 2,
  PKV_FP8_E4M3 = 3,  /* OCP E4M3FN: bias 7, max 448, no infinities */
  PKV_FP8_E5M2 = 4,  /* OCP E5M2: bias 15, max 57344; stored codes are finite */
  PKV_INT8_INT4 = 5  /* cache only: K int8 codes, V int4 codes (two per byte) */
} pkv_dtype;

enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,    /* null pointer, bad size, Hq % Hkv != 0, ... */
  PKV_ERR_UNSUPPORTED = -2,    /* dtype pair, head_dim or group size not built */
  PKV_ERR_WORKSPACE = -3,      /* workspace missing or smaller than required */
  PKV_ERR_HIP = -4,            /* the HIP runtime reported an error */
  PKV_ERR_NO_FREE_BLOCKS = -5, /* allocator: not enough free blocks; nothing changed */
  PKV_ERR_UNKNOWN_SEQ = -6,    /* allocator: no such sequence id */
  PKV_ERR_HOST_MEMORY = -7,    /* allocator: host memory ran out during the call; its state
                                  may be partly updated, so destroy it */
  PKV_ERR_SCRATCH = -8         /* the call needs more than the library's fixed scratch
                                  (PKV_SCRATCH_BYTES); use the form that takes a workspace */
};

/* Library ABI version (PKV_ABI_VERSION). */
int pkv_abi_version(void);

/* Static text for a return code. */
const char* pkv_strerror(int code);

/* ------------------------------------------------------------------------ */
/* Device layouts (row-major, contiguous), bs = block size (tokens):         */
/*   k_pool, v_pool   [num_blocks][num_kv_heads][bs][head_dim] of cache dtype */
/*                    (one byte per code for fp8 and int8; PKV_INT8_INT4's V */
/*                    pool is [num_blocks][num_kv_heads][bs][head_dim / 2]   */
/*                    bytes, element 2i in the low nibble of byte i)         */
/*   k_scale, v_scale [num_blocks][num_kv_heads][bs] float32 (quantised      */
/*                    caches only: fp8 e4m3 / e5m2, int8 + int4)             */
/*   slot = physical_block * bs + (position % bs)                            */
/* The plain calls use bs = PKV_BLOCK_SIZE (16).  Each call named _bs takes  */
/* the same arguments plus `block_size` (16 or 32; anything else gives      */
/* PKV_ERR_INVALID_ARG) right after num_blocks (after head_dim for the      */
/* merge), and reads every "16" of the plain call's description as that     */
/* block size - except partition sizes, which stay multiples of 16 tokens.  */
/* A pool of 32-token blocks also needs num_blocks * num_kv_heads * 2 <     */
/* 2^31 (else PKV_ERR_UNSUPPORTED from the decode and prefill calls).       */
/* ------------------------------------------------------------------------ */

/*
 * kv_cache_append - write new K/V token rows into their slots.
 * Pages: "KV Cache 和 vLLM" §1.3 (each step computes the new token's K and V
 * and appends them to the layer's cache) and §3.1 (16-token blocks);
 * "KV Cache优化实战" §3.2-3.3 (fp8 KV with per-token / per-head scales;
 * K and V tolerate quantisation differently, so K at int8 and V at int4).
 *
 *   k_new, v_new  device, [num_tokens][num_kv_heads][head_dim] of src_dtype
 *   k_pool, v_pool device pools (layout above) of cache_dtype
 *   k_scale, v_scale device [num_blocks][num_kv_heads][16] float32; required
 *                 for a quantised cache (PKV_FP8_E4M3, PKV_FP8_E5M2,
 *                 PKV_INT8_INT4), ignored (may be NULL) otherwise
 *   slot_mapping  device int64 [num_tokens]: row i goes to slot_mapping[i];
 *                 a negative entry skips the row; entries >= 16*num_blocks
 *                 are skipped as well
 * Same dtype (f32/f16/bf16): an exact bit copy of each row.
 * fp8 (src f32, f16 or bf16): per (token, head) row, a = max|x| (fp32),
 *   s = a / 448 (fp32, correctly rounded; s = 1 when a == 0), code =
 *   e4m3 round-to-nearest-even of clamp(x / s, -448, 448) with x / s a
 *   correctly rounded fp32 division; codes go to the pool and s to the scale
 *   array at the same (block, head, offset).
 * fp8 e5m2: the same with 57344 in place of 448 and e5m2 codes.
 * int8 + int4: the same per row with 127 (K, int8 codes) and 7 (V, int4
 *   codes), the nearest integer with ties to even; codes are two's
 *   complement, int4 packed two per byte (even element in the low nibble).
 * Slots must be distinct within one call.  num_tokens == 0 is a no-op.
 * head_dim: 64 or 128.
 */
int kv_cache_append(const void* k_new, const void* v_new,
                    void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                    const int64_t* slot_mapping,
                    int num_tokens, int num_kv_heads, int head_dim, int num_blocks,
                    pkv_dtype src_dtype, pkv_dtype cache_dtype, void* stream);

int kv_cache_append_bs(const void* k_new, const void* v_new,
                       void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                       const int64_t* slot_mapping,
                       int num_tokens, int num_kv_heads, int head_dim, int num_blocks, int block_size,
                       pkv_dtype src_dtype, pkv_dtype cache_dtype, void* stream);

/*
 * pkv_copy_blocks - copy whole physical blocks (K, V and, for a quantised
 * cache, the scales) from src to dst, for the copy-on-write of a shared block that one
 * sequence is about to write ("KV Cache 和 vLLM" §3.3).
 *   pairs  device int32 [n_pairs][2] = {src, dst}; pairs with an entry
 *          outside [0, num_blocks) are skipped.  dst blocks must be distinct
 *          and no dst may be a src of the same call.
 */
int pkv_copy_blocks(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                    const int32_t* pairs, int n_pairs,
                    int num_kv_heads, int head_dim, int num_blocks, pkv_dtype cache_dtype,
                    void* stream);

int pkv_copy_blocks_bs(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                       const int32_t* pairs, int n_pairs,
                       int num_kv_heads, int head_dim, int num_blocks, int block_size,
                       pkv_dtype cache_dtype, void* stream);

/*
 * pkv_decode_partition_size - the partition length (tokens, a multiple of 16)
 * paged_attention_decode uses when called with partition_size == 0, and the
 * resulting partitions per sequence for max_context_len.  The plan fills
 * the 256 CUs with at least one workgroup each (two for int8 K + int4 V
 * caches, whose decoding is heaviest per byte) and at most 72 blocks per
 * wave.  Host only.
 */
int pkv_decode_partition_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                              int max_context_len, pkv_dtype cache_dtype,
                              int* partition_size_out, int* num_partitions_out);

/*
 * paged_attention_workspace_size - bytes of device workspace
 * paged_attention_decode needs for these sizes (0 when every sequence fits
 * in one partition).  partition_size: 0 = automatic, else a multiple of 16
 * no larger than PKV_MAX_PARTITION_TOKENS.
 * Returns 0 as well for invalid sizes (the decode call then reports them).
 */
size_t paged_attention_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                      int head_dim, int max_context_len, int partition_size,
                                      pkv_dtype cache_dtype);


/*
 * paged_attention_decode - one decode step of attention for a batch.
 * Pages: "企业官网建设流程全解析" §1.2 (softmax(Q K^T / sqrt(d_k)) V), §2.2
 * (several query heads share one KV head), §3.2 (the query attends to the
 * whole cache, its own token included); "KV Cache 和 vLLM" §3.2 (block-table
 * translation: only the sequence's own blocks are read).
 *
 *   out           device [num_seqs][num_q_heads][head_dim] of q_dtype (written)
 *   q             device [num_seqs][num_q_heads][head_dim] of q_dtype
 *   k_pool, v_pool, k_scale, v_scale  as for kv_cache_append (scales: quantised
 *                 caches only)
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]; entry i of row
 *                 b is the physical block of sequence b's logical block i
 *   context_lens  device int32 [num_seqs]; L_b, the tokens sequence b attends
 *                 to (positions 0..L_b-1)
 *   max_context_len  host bound with L_b <= max_context_len <=
 *                 16 * max_blocks_per_seq; it sizes the launch
 *   scale         the caller passes 1/sqrt(head_dim)
 *   partition_size 0 = automatic; else tokens per partition, a multiple of 16
 *                 and at most PKV_MAX_PARTITION_TOKENS.
 *                 When a sequence is longer than one partition, its
 *                 partitions' states are merged exactly (log-sum-exp) into
 *                 the output: for up to two partitions per sequence (up to
 *                 four when the launch has at most 512 workgroups, i.e.
 *                 num_seqs * num_kv_heads * partitions <= 512) inside the
 *                 same launch (the workgroup of the sequence's last
 *                 partition to finish reads the others' states from the
 *                 workspace and writes the output row), for more by a second
 *                 kernel of the call; the bits are the same either way.
 *   workspace     device scratch of at least paged_attention_workspace_size()
 *                 bytes (may be NULL when that is 0): arrival counters (the
 *                 first PKV_WS_COUNTER_BYTES: zero before the workspace's
 *                 first use, left zero by every call), then the call's
 *                 longest-first order or its partition states, which need
 *                 no initialisation.  With
 *                 more than PKV_WS_COUNTER_UNITS (sequence, KV head) pairs
 *                 the merge runs as a second kernel of the same call instead
 *                 (same bits).  Calls that may run concurrently must not
 *                 share a workspace.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).  L_b == 0 gives
 * an all-zero output row.  Entries of the used part of a block-table row must
 * lie in [0, num_blocks); a block outside that range contributes no tokens.
 * Tokens at or beyond max_context_len (or 16*max_blocks_per_seq) are ignored.
 * dtype pairs (q / cache): f32/f32, f16/f16, bf16/bf16, and bf16 or f16 with
 * fp8_e4m3, fp8_e5m2 or int8_int4.  head_dim: 64 or 128.  num_q_heads/num_kv_heads: 1..16.
 * Accumulation is fp32; the output is rounded to q_dtype (round to nearest
 * even).  The result for a given (sequence, head) depends only on the values
 * at its logical positions, not on where the blocks lie or who shares them.
 */
int paged_attention_decode(void* out, const void* q,
                           const void* k_pool, const void* v_pool,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int num_blocks, int max_blocks_per_seq, int max_context_len,
                           float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                           int partition_size, void* workspace, size_t workspace_bytes,
                           void* stream);

int paged_attention_decode_bs(void* out, const void* q,
                              const void* k_pool, const void* v_pool,
                              const float* k_scale, const float* v_scale,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                              int num_blocks, int block_size, int max_blocks_per_seq, int max_context_len,
                              float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                              int partition_size, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * paged_attention_decode_append - one decode step with its cache write fused
 * in: the same result, pool bytes and scales as kv_cache_append(k_new, v_new,
 * ..., slot_mapping, num_tokens = num_seqs) followed by
 * paged_attention_decode(...), in one launch (partition states merged in it
 * as in paged_attention_decode).  Pages: the new token's K and V are
 * appended to the cache and the new query then attends over the whole cache,
 * itself included ("KV Cache 和 vLLM" §1.2-1.3; "企业官网建设流程全解析" §3.2).
 *
 *   k_new, v_new  device [num_seqs][num_kv_heads][head_dim] of src_dtype: the
 *                 step's K and V row of each sequence
 *   slot_mapping  device int64 [num_seqs]: slot of sequence b's newest
 *                 position context_lens[b] - 1 (the slot the allocator handed
 *                 out for it); a negative entry writes nothing for b
 *   all other arguments as for paged_attention_decode; src_dtype as for
 *   kv_cache_append (equal to cache_dtype, or f32/f16/bf16 for a quantised
 *   cache).
 * The row of sequence b is written by the workgroup whose partition holds
 * position context_lens[b] - 1, before any K/V is read, so sequences with
 * context_lens[b] == 0 write nothing.
 */
int paged_attention_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                                  void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                  const int64_t* slot_mapping,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                  int num_blocks, int max_blocks_per_seq, int max_context_len,
                                  float scale, pkv_dtype q_dtype, pkv_dtype src_dtype,
                                  pkv_dtype cache_dtype, int partition_size, void* workspace,
                                  size_t workspace_bytes, void* stream);

int paged_attention_decode_append_bs(void* out, const void* q, const void* k_new, const void* v_new,
                                     void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                     const int64_t* slot_mapping,
                                     const int32_t* block_tables, const int32_t* context_lens,
                                     int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                     int num_blocks, int block_size, int max_blocks_per_seq,
                                     int max_context_len, float scale, pkv_dtype q_dtype,
                                     pkv_dtype src_dtype, pkv_dtype cache_dtype, int partition_size,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode_append_noalloc - paged_attention_decode_append
 * (block_size 16 or 32, as the _bs form) that allocates nothing and takes no
 * workspace, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The partition states and counters a split sequence needs live in a
 * device array of PKV_SCRATCH_BYTES (16 MiB) that the library holds on
 * each GPU it runs on until the process ends; the first call on a device
 * looks up the array's address and clears its counters (a fill kernel on the
 * call's stream).  Every call on a GPU shares that GPU's array, so calls
 * that may overlap on one GPU (other streams, other threads) race and must
 * not be issued.  Same arguments, result and bytes as
 * paged_attention_decode_append_bs without workspace and workspace_bytes.
 * Returns PKV_ERR_SCRATCH, before touching the device, when the call would
 * need more than PKV_SCRATCH_BYTES (paged_attention_workspace_size() of its
 * sizes); calls no hipMalloc, hipFree or allocating library routine.
 */
int paged_attention_decode_append_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                                          void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                          const int64_t* slot_mapping,
                                          const int32_t* block_tables, const int32_t* context_lens,
                                          int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                          int num_blocks, int block_size, int max_blocks_per_seq,
                                          int max_context_len, float scale, pkv_dtype q_dtype,
                                          pkv_dtype src_dtype, pkv_dtype cache_dtype, int partition_size,
                                          void* stream);

/*
 * Split form of paged_attention_decode_append, in two launches, for callers
 * that schedule or time the merge separately.
 * paged_attention_decode_append_partials takes the same arguments
 * (slot_mapping may be NULL: no cache write, as in paged_attention_decode)
 * and launches only the attention kernel: when some sequence is longer than
 * one partition it writes every sequence's partition states (empty
 * partitions included) into the workspace, else the output rows; it does not
 * use the workspace's counters.  paged_attention_merge_partials then merges
 * those states into the output rows (log-sum-exp, the same arithmetic in the
 * same order as the one-call form, so the output bits are equal); it
 * must get the same num_seqs, head counts, head_dim, max_context_len,
 * cache_dtype, partition_size and workspace, on the same stream (the
 * automatic partition plan depends on the cache format).  The pair gives exactly
 * the bytes of the one-call form.  When nothing is split, the merge call
 * does nothing.
 */
int paged_attention_decode_append_partials(void* out, const void* q, const void* k_new, const void* v_new,
                                           void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                           const int64_t* slot_mapping,
                                           const int32_t* block_tables, const int32_t* context_lens,
                                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                           int num_blocks, int max_blocks_per_seq, int max_context_len,
                                           float scale, pkv_dtype q_dtype, pkv_dtype src_dtype,
                                           pkv_dtype cache_dtype, int partition_size, void* workspace,
                                           size_t workspace_bytes, void* stream);

int paged_attention_merge_partials(void* out, const int32_t* context_lens,
                                   int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                   int max_blocks_per_seq, int max_context_len, pkv_dtype q_dtype,
                                   pkv_dtype cache_dtype, int partition_size, void* workspace,
                                   size_t workspace_bytes, void* stream);

int paged_attention_decode_append_partials_bs(void* out, const void* q, const void* k_new, const void* v_new,
                                              void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                              const int64_t* slot_mapping,
                                              const int32_t* block_tables, const int32_t* context_lens,
                                              int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                              int num_blocks, int block_size, int max_blocks_per_seq,
                                              int max_context_len, float scale, pkv_dtype q_dtype,
                                              pkv_dtype src_dtype, pkv_dtype cache_dtype, int partition_size,
                                              void* workspace, size_t workspace_bytes, void* stream);

int paged_attention_merge_partials_bs(void* out, const int32_t* context_lens,
                                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                      int block_size, int max_blocks_per_seq, int max_context_len,
                                      pkv_dtype q_dtype, pkv_dtype cache_dtype, int partition_size,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attention_prefill - chunked prefill: each sequence's chunk of new
 * tokens attends over the sequence's cached K/V and causally over itself.
 *
 * Pages: in prefill every prompt token is processed at once and attends to
 * the positions before it and to itself ("KV Cache 和 vLLM" §1.1;
 * "企业官网建设流程全解析" §3.1-3.2); K/V of tokens already cached is reused
 * rather than recomputed ("KV Cache优化实战" §5.2).
 *
 * The chunk's own K/V rows must already be in the pool (kv_cache_append
 * takes any number of tokens; the allocator's append gives their slots).
 *   out            device [num_tokens][num_q_heads][head_dim], q dtype
 *   q              device [num_tokens][num_q_heads][head_dim]: the chunks back
 *                  to back
 *   query_start    device int32 [num_seqs + 1], query_start[0] = 0,
 *                  non-decreasing, query_start[num_seqs] <= num_tokens:
 *                  sequence b's chunk is q rows query_start[b] .. [b+1]-1
 *   context_lens   device int32 [num_seqs]: cached tokens including the
 *                  chunk, so chunk row i sits at position
 *                  context_lens[b] - n_b + i and attends to positions 0 .. it
 *   block_tables, pools, scales, scale: as paged_attention_decode; scale
 *                  must be positive and finite (else PKV_ERR_INVALID_ARG)
 *   max_query_len  host: >= every chunk length (sizes the launch; a longer
 *                  chunk, or one outside q, is skipped and its rows untouched)
 *   max_context_len host: >= every context length, at most
 *                  PKV_MAX_PREFILL_CONTEXT
 * Dtype pairs (q / cache): f16/f16, bf16/bf16, and bf16 or f16 with
 * fp8_e4m3, fp8_e5m2 or int8_int4 (codes converted exactly to 16-bit values
 * on their way into LDS, scales applied to scores and probabilities); f32
 * and other head dims give PKV_ERR_UNSUPPORTED.  A sequence with an empty
 * chunk is skipped; with context_lens[b] = 0 its chunk rows are zero.  No
 * workspace; nothing is allocated; asynchronous on stream.
 */
int paged_attention_prefill(void* out, const void* q, const void* k_pool, const void* v_pool,
                            const float* k_scale, const float* v_scale, const int32_t* block_tables,
                            const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                            int num_tokens, int num_q_heads, int num_kv_heads, int head_dim, int num_blocks,
                            int max_blocks_per_seq, int max_context_len, int max_query_len, float scale,
                            pkv_dtype q_dtype, pkv_dtype cache_dtype, void* stream);

int paged_attention_prefill_bs(void* out, const void* q, const void* k_pool, const void* v_pool,
                               const float* k_scale, const float* v_scale, const int32_t* block_tables,
                               const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                               int num_tokens, int num_q_heads, int num_kv_heads, int head_dim, int num_blocks,
                               int block_size, int max_blocks_per_seq, int max_context_len, int max_query_len,
                               float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, void* stream);

/*
 * pkv_gather_blocks / pkv_scatter_blocks - move whole physical blocks between
 * one pool tensor and a contiguous staging buffer, for swapping sequences out
 * to host memory and back ("KV Cache 和 vLLM" §6.2: under memory pressure
 * blocks move out to CPU memory; the host link is slow, so one large copy
 * of a contiguous staging buffer replaces per-block copies).
 *   staging      device, n_blocks * block_bytes bytes; slot i holds blocks[i]
 *   pool         a device pool tensor (K, V, or a scale array): block b is the
 *                block_bytes bytes at b * block_bytes (all heads of it)
 *   blocks       device int32 [n_blocks]; ids outside [0, num_blocks) are
 *                skipped (their staging slot is not touched)
 *   block_bytes  bytes of one block of this tensor, a multiple of 16:
 *                num_kv_heads * bs * head_dim * element size (int4 V: half a
 *                byte per element; scales: num_kv_heads * bs * 4), bs the
 *                pool's block size
 * The caller moves the staging buffer to or from pinned host memory; nothing
 * here touches host memory.  Asynchronous on stream.
 */
int pkv_gather_blocks(void* staging, const void* pool, const int32_t* blocks, int n_blocks,
                      int64_t block_bytes, int num_blocks, void* stream);
int pkv_scatter_blocks(void* pool, const void* staging, const int32_t* blocks, int n_blocks,
                       int64_t block_bytes, int num_blocks, void* stream);

/* ------------------------------------------------------------------------ */
/* Host block allocator.  Opaque handle, not thread-safe, no device memory.  */
/*                                                                          */
/* Pages: blocks are taken on demand when a sequence's current block is full */
/* and appended to its block table ("KV Cache 和 vLLM" §3.1); finished        */
/* sequences return their blocks for reuse ("KV Cache优化实战" §4.2);          */
/* sequences with a common prefix point at the same physical blocks, and      */
/* copy-on-write handles writes to shared blocks ("KV Cache 和 vLLM" §3.3);   */
/* running out of cache must degrade rather than crash ("企业官网建设流程全解析" */
/* §6.4): every failing call leaves the allocator unchanged.                  */
/*                                                                          */
/* Rules: blocks carry reference counts.  The free list is a stack:          */
/* pkv_alloc_set_free_order(order) makes order[0] the next block handed out,  */
/* and a released block goes on top.  A sequence's blocks are released in     */
/* logical order.  Appending n tokens to a sequence of length L: if L % 16 != */
/* 0 and its last block is shared, that block is copied first (one fresh      */
/* block, one {old, new} pair reported, old count decremented, table entry    */
/* repointed); then a fresh block is taken for each position p in [L, L+n)    */
/* with p % 16 == 0.  A full shared block is never written, never copied.     */
/* ------------------------------------------------------------------------ */

typedef struct pkv_alloc pkv_alloc;

typedef struct {
  int64_t num_blocks;
  int64_t free_blocks;
  int64_t used_blocks;     /* blocks with reference count > 0 */
  int64_t shared_blocks;   /* blocks with reference count > 1 */
  int64_t cow_copies;      /* copy pairs reported so far */
  int64_t cached_tokens;   /* sum over live sequences of their length */
  int64_t stored_tokens;   /* filled physical slots, a shared slot counted once */
  double utilisation;      /* stored_tokens / (bs * used_blocks), 0 if none used */
} pkv_alloc_stats_t;

/* New allocator of 16-token blocks with every block free (block 0 handed
   out first).  Returns NULL if num_blocks <= 0 or max_blocks_per_seq <= 0. */
pkv_alloc* pkv_alloc_create(int num_blocks, int max_blocks_per_seq);
/* The same with block_size tokens per block (16 or 32, else NULL): every
   rule below counts positions in blocks of that size, and slots are
   block * block_size + offset ("KV Cache 和 vLLM" §6.3). */
pkv_alloc* pkv_alloc_create_bs(int num_blocks, int max_blocks_per_seq, int block_size);
/* Tokens per block of an allocator (16 or 32), or PKV_ERR_INVALID_ARG. */
int pkv_alloc_block_size(const pkv_alloc* a);
void pkv_alloc_destroy(pkv_alloc* a);

/* Reorder the free list of an idle allocator (no live sequence): order is a
   host permutation of 0..num_blocks-1 and order[0] is handed out first. */
int pkv_alloc_set_free_order(pkv_alloc* a, const int32_t* order, int n);

int pkv_seq_create(pkv_alloc* a, int64_t seq_id);
/* child shares every block of parent (counts incremented) and its length. */
int pkv_seq_fork(pkv_alloc* a, int64_t parent, int64_t child);
/* Drop a sequence: counts decremented, blocks at zero return to the list. */
int pkv_seq_free(pkv_alloc* a, int64_t seq_id);
/* Length of a sequence (>= 0) or a negative error code. */
int pkv_seq_len(pkv_alloc* a, int64_t seq_id);

/*
 * pkv_seq_append_slots - reserve the next n_tokens positions of a sequence.
 *   slots_out      host int64 [n_tokens]: the slot of each new position
 *   cow_pairs_out  host int32 [2]: the {src, dst} copy to apply before
 *                  writing, when *n_cow_out == 1
 *   n_cow_out      host: 0 or 1
 * Fails with PKV_ERR_NO_FREE_BLOCKS when the free list (with prefix caching:
 * free plus evictable blocks) is too short and with
 * PKV_ERR_INVALID_ARG when the table would exceed max_blocks_per_seq; then
 * nothing changes.
 */
int pkv_seq_append_slots(pkv_alloc* a, int64_t seq_id, int n_tokens,
                         int64_t* slots_out, int32_t* cow_pairs_out, int* n_cow_out);

/*
 * pkv_batch_append_one - one new position for each of n sequences (a decode
 * step), in the given order, all or nothing.
 *   slots_out      host int64 [n]
 *   cow_pairs_out  host int32 [n][2]; the first *n_cow_out rows are filled
 */
int pkv_batch_append_one(pkv_alloc* a, const int64_t* seq_ids, int n,
                         int64_t* slots_out, int32_t* cow_pairs_out, int* n_cow_out);

/*
 * pkv_build_block_tables - host int32 tables [n][max_blocks_per_seq] (unused
 * entries 0) and lengths [n] for the given sequences.
 */
int pkv_build_block_tables(pkv_alloc* a, const int64_t* seq_ids, int n, int max_blocks_per_seq,
                           int32_t* tables_out, int32_t* lens_out);

int pkv_alloc_stats(pkv_alloc* a, pkv_alloc_stats_t* out);

/*
 * pkv_seq_swap_out - move a sequence out of the pool ("KV Cache 和 vLLM"
 * §6.2).  Every block of the sequence must be unshared (count 1), else
 * PKV_ERR_INVALID_ARG and nothing changes.  Writes its blocks in logical
 * order to blocks_out (host int32, room for max_blocks_per_seq entries),
 * their count to *n_out, and releases them in that order (prefix-indexed
 * blocks stay cached and evictable).  The sequence keeps only its length;
 * it stops being prefix-indexed.  The caller gathers those blocks (stream
 * order keeps later writes to them behind the gather).
 * pkv_seq_swap_in - bring a swapped sequence back: takes ceil(len / bs)
 * fresh blocks, all or nothing (PKV_ERR_NO_FREE_BLOCKS), writes them in
 * logical order to blocks_out for the caller to scatter into.
 * A swapped sequence can only be swapped in, freed or asked its length;
 * other calls naming it give PKV_ERR_INVALID_ARG.  Allocator statistics
 * count resident sequences only.
 */
int pkv_seq_swap_out(pkv_alloc* a, int64_t seq_id, int32_t* blocks_out, int* n_out);
int pkv_seq_swap_in(pkv_alloc* a, int64_t seq_id, int32_t* blocks_out, int* n_out);

/* ------------------------------------------------------------------------ */
/* Prefix caching.                                                          */
/*                                                                          */
/* Pages: cached KV is looked up by its content - the token ids together    */
/* with a model identifier - block by block from the start of the prompt,   */
/* reusing every block that matches exactly and stopping at the first that  */
/* does not ("KV Cache优化实战" §5.2-5.3; "企业官网建设流程全解析" §6.2);     */
/* the cache is finite and eviction follows the prefix tree, not plain       */
/* access order ("KV Cache优化实战" §5.3; "企业官网建设流程全解析" §6.3).     */
/*                                                                          */
/* Rules: only full blocks are indexed.  Block i of a tracked sequence is    */
/* indexed when an append that names its tokens fills it, unless the same   */
/* prefix (model key and tokens 0 .. 16i+15) is indexed already, and for    */
/* i > 0 only if block i-1 of the sequence is the indexed block of the      */
/* shorter prefix.  Sequences made by pkv_seq_create (with caching on),     */
/* pkv_seq_create_cached or a fork of a tracked sequence are tracked; an    */
/* append without tokens (pkv_seq_append_slots, pkv_batch_append_one)      */
/* untracks a sequence for good.  An indexed block whose count drops to     */
/* zero stays indexed and becomes evictable, stamped in release order.  A   */
/* fresh block comes from the free list while it is not empty, otherwise   */
/* the evictable block with the smallest stamp among those with no indexed  */
/* child is evicted and reused.  Appends count free plus evictable blocks   */
/* as capacity.  Block contents are the caller's: a hit means the K/V rows  */
/* written for those positions are still in the pool.                       */
/* ------------------------------------------------------------------------ */

typedef struct {
  int64_t cached_blocks;     /* indexed blocks (in use or evictable) */
  int64_t evictable_blocks;  /* indexed blocks with count 0 */
  int64_t lookup_blocks;     /* full blocks offered to lookups so far */
  int64_t hit_blocks;        /* of those, blocks found in the cache */
  int64_t evictions;         /* evictable blocks reused so far */
} pkv_prefix_stats_t;

/*
 * pkv_prefix_cache_enable - turn prefix caching on for an idle allocator
 * (no sequence, every block free).  model_key seeds the content hash, so
 * caches of different models never match.  hash_bits (1..64) is how many
 * bits of the hash pick a bucket: 64 in use; fewer force collisions, which
 * cost comparisons but never a wrong match (entries are compared in full).
 * PKV_ERR_INVALID_ARG if already enabled, not idle or hash_bits is out of
 * range.
 */
int pkv_prefix_cache_enable(pkv_alloc* a, uint64_t model_key, int hash_bits);

/*
 * pkv_seq_create_cached - new tracked sequence that starts with the longest
 * run of indexed blocks matching tokens[0 .. n_tokens) from the start, at
 * most (n_tokens - 1) / 16 blocks (the last prompt token is always
 * computed).  Each matched block gains a reference.
 *   tokens        host int32 [n_tokens]: the prompt's token ids
 *   n_cached_out  host: the new sequence's length, 16 x matched blocks; the
 *                 caller appends tokens[*n_cached_out ..] with
 *                 pkv_seq_append_tokens and writes their K/V rows
 * PKV_ERR_INVALID_ARG if caching is off or the id is live.
 */
int pkv_seq_create_cached(pkv_alloc* a, int64_t seq_id, const int32_t* tokens, int n_tokens,
                          int* n_cached_out);

/*
 * pkv_seq_append_tokens - pkv_seq_append_slots for positions whose token ids
 * are known (tokens: host int32 [n_tokens]); on a tracked sequence, indexes
 * every block the append fills.  Same outputs and errors.
 */
int pkv_seq_append_tokens(pkv_alloc* a, int64_t seq_id, const int32_t* tokens, int n_tokens,
                          int64_t* slots_out, int32_t* cow_pairs_out, int* n_cow_out);

/*
 * pkv_batch_append_tokens - pkv_batch_append_one with the new token of each
 * sequence (tokens: host int32 [n]), indexing the blocks it fills; in order,
 * all or nothing.
 */
int pkv_batch_append_tokens(pkv_alloc* a, const int64_t* seq_ids, const int32_t* tokens, int n,
                            int64_t* slots_out, int32_t* cow_pairs_out, int* n_cow_out);

int pkv_prefix_stats(pkv_alloc* a, pkv_prefix_stats_t* out);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
