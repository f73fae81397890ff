// Cache writes: scatter new K/V token rows into their paged slots (with
// quantisation on the way in for fp8 e4m3 / e5m2 and int8-K / int4-V caches)
// and copy whole blocks for copy-on-write.
//
// Pages: each decode step appends the new token's K and V to the layer's
// cache ("KV Cache 和 vLLM" §1.3; "企业官网建设流程全解析" §3.2) into fixed
// 16-token blocks (§3.1 of the first; 32-token blocks, §6.3); quantised KV with a scale per token
// and per head, K kept at higher precision than V ("KV Cache优化实战"
// §3.2-3.3); copy-on-write of shared blocks ("KV Cache 和 vLLM" §3.3).
//
// These kernels move at most a few hundred KiB per decode step and are
// launch-bound; they are written for exactness (bit copies, a bit-exact
// quantiser) and coalesced 16-byte accesses, not for peak bandwidth.

#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace pkv {

// One 16-byte chunk per thread.  A (token, head) row of head_dim elements is
// `chunks_per_row` chunks; a pool row lives at
// ((slot / bs) * Hkv + head) * bs + slot % bs in units of rows (bs = 16, 32).
__global__ void __launch_bounds__(256) append_copy_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
    const int64_t* __restrict__ slot_mapping, int num_tokens, int num_kv_heads,
    int chunks_per_row, int64_t num_slots, int block_size) {
  int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t rows = static_cast<int64_t>(num_tokens) * num_kv_heads;
  int64_t row = gid / chunks_per_row;
  int chunk = static_cast<int>(gid % chunks_per_row);
  if (row >= rows) return;
  int64_t tok = row / num_kv_heads;
  int head = static_cast<int>(row % num_kv_heads);
  int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;
  int64_t dst_row = slot_row(slot, block_size, num_kv_heads, head);
  k_pool[dst_row * chunks_per_row + chunk] = k_new[row * chunks_per_row + chunk];
  v_pool[dst_row * chunks_per_row + chunk] = v_new[row * chunks_per_row + chunk];
}

// Quantised caches: one wave per (token, head) row and per tensor (K rows in
// waves with blockIdx.y == 0 in format KQ, V rows with blockIdx.y == 1 in
// format VQ).  Each lane holds head_dim/64 elements.
template <typename Src, int D, typename KQ, typename VQ>
__global__ void __launch_bounds__(256) append_quant_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    float* __restrict__ k_scale, float* __restrict__ v_scale,
    const int64_t* __restrict__ slot_mapping, int num_tokens, int num_kv_heads,
    int64_t num_slots, int block_size) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t rows = static_cast<int64_t>(num_tokens) * num_kv_heads;
  if (row >= rows) return;
  const bool is_v = blockIdx.y != 0;
  const int64_t tok = row / num_kv_heads;
  const int head = static_cast<int>(row % num_kv_heads);
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;

  const int64_t dst_row = slot_row(slot, block_size, num_kv_heads, head);
  if (is_v) write_row_quant<Src, D, VQ>(v_new, row, v_pool, v_scale, dst_row, lane);
  else write_row_quant<Src, D, KQ>(k_new, row, k_pool, k_scale, dst_row, lane);
}

// Copy-on-write: one workgroup per (pair, head, tensor); 16-byte chunks of
// the (block, head) slab of block_size rows (a K slab and a V slab may differ
// in size: int4 V rows are half as long), plus its block_size scales.
__global__ void __launch_bounds__(256) copy_blocks_kernel(
    uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
    float* __restrict__ k_scale, float* __restrict__ v_scale,
    const int32_t* __restrict__ pairs, int num_kv_heads, int k_chunks_per_tile, int v_chunks_per_tile,
    int num_blocks, int block_size) {
  const int pair = blockIdx.x;
  const int head = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint4* pool = is_v ? v_pool : k_pool;
  const int chunks_per_tile = is_v ? v_chunks_per_tile : k_chunks_per_tile;
  const int64_t s_tile = static_cast<int64_t>(src) * num_kv_heads + head;
  const int64_t d_tile = static_cast<int64_t>(dst) * num_kv_heads + head;
  for (int c = threadIdx.x; c < chunks_per_tile; c += blockDim.x)
    pool[d_tile * chunks_per_tile + c] = pool[s_tile * chunks_per_tile + c];
  float* scales = is_v ? v_scale : k_scale;
  if (scales != nullptr && threadIdx.x < block_size)
    scales[d_tile * block_size + threadIdx.x] = scales[s_tile * block_size + threadIdx.x];
}

// Swap staging: whole blocks (block_chunks 16-byte chunks each, every head)
// between a pool and a contiguous staging buffer, slot i of the staging
// buffer holding blocks[i].  to_staging: pool -> staging, else staging ->
// pool.  Block ids outside [0, num_blocks) are skipped.
__global__ void __launch_bounds__(256) swap_blocks_kernel(uint4* __restrict__ staging, uint4* __restrict__ pool,
                                                          const int32_t* __restrict__ blocks, int64_t block_chunks,
                                                          int num_blocks, int to_staging) {
  const int i = blockIdx.x;
  const int32_t blk = blocks[i];
  if (blk < 0 || blk >= num_blocks) return;
  uint4* p = pool + static_cast<int64_t>(blk) * block_chunks;
  uint4* st = staging + static_cast<int64_t>(i) * block_chunks;
  const int64_t step = static_cast<int64_t>(gridDim.y) * blockDim.x;
  for (int64_t c = static_cast<int64_t>(blockIdx.y) * blockDim.x + threadIdx.x; c < block_chunks; c += step) {
    if (to_staging) st[c] = p[c];
    else p[c] = st[c];
  }
}

// ---- launchers -------------------------------------------------------------------

int launch_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                  float* k_scale, float* v_scale, const int64_t* slot_mapping, int num_tokens,
                  int num_kv_heads, int head_dim, int num_blocks, int block_size, pkv_dtype src_dtype,
                  pkv_dtype cache_dtype, hipStream_t stream) {
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  const int64_t rows = static_cast<int64_t>(num_tokens) * num_kv_heads;
  const bool quant = cache_dtype == PKV_FP8_E4M3 || cache_dtype == PKV_FP8_E5M2 || cache_dtype == PKV_INT8_INT4;
  if (!quant) {
    const int es = cache_dtype == PKV_F32 ? 4 : 2;
    const int chunks = head_dim * es / 16;
    const int64_t threads = rows * chunks;
    const int64_t grid = (threads + 255) / 256;
    hipLaunchKernelGGL(append_copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                       static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                       static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), slot_mapping,
                       num_tokens, num_kv_heads, chunks, num_slots, block_size);
    return check_launch();
  }
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4), 2);
  auto* kp = static_cast<uint8_t*>(k_pool);
  auto* vp = static_cast<uint8_t*>(v_pool);
  auto launch = [&](auto src_tag, auto kq, auto vq) {
    using S = decltype(src_tag);
    using KQ = decltype(kq);
    using VQ = decltype(vq);
    if (head_dim == 128)
      hipLaunchKernelGGL((append_quant_kernel<S, 128, KQ, VQ>), grid, dim3(256), 0, stream, k_new, v_new, kp, vp,
                         k_scale, v_scale, slot_mapping, num_tokens, num_kv_heads, num_slots, block_size);
    else
      hipLaunchKernelGGL((append_quant_kernel<S, 64, KQ, VQ>), grid, dim3(256), 0, stream, k_new, v_new, kp, vp,
                         k_scale, v_scale, slot_mapping, num_tokens, num_kv_heads, num_slots, block_size);
  };
  auto by_format = [&](auto src_tag) {
    if (cache_dtype == PKV_FP8_E4M3) launch(src_tag, FP8{}, FP8{});
    else if (cache_dtype == PKV_FP8_E5M2) launch(src_tag, BF8{}, BF8{});
    else launch(src_tag, I8{}, I4{});
  };
  if (src_dtype == PKV_F32) by_format(F32{});
  else if (src_dtype == PKV_F16) by_format(F16{});
  else by_format(BF16{});
  return check_launch();
}

int launch_copy_blocks(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                       const int32_t* pairs, int n_pairs, int num_kv_heads, int head_dim,
                       int num_blocks, int block_size, pkv_dtype cache_dtype, hipStream_t stream) {
  // bits per element of the K and the V pool
  int k_bits = 16, v_bits = 16;
  if (cache_dtype == PKV_F32) k_bits = v_bits = 32;
  else if (cache_dtype == PKV_FP8_E4M3 || cache_dtype == PKV_FP8_E5M2) k_bits = v_bits = 8;
  else if (cache_dtype == PKV_INT8_INT4) k_bits = 8, v_bits = 4;
  const bool quant = cache_dtype == PKV_FP8_E4M3 || cache_dtype == PKV_FP8_E5M2 || cache_dtype == PKV_INT8_INT4;
  const int k_chunks = block_size * head_dim * k_bits / 8 / 16;
  const int v_chunks = block_size * head_dim * v_bits / 8 / 16;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n_pairs, num_kv_heads, 2), dim3(256), 0, stream,
                     static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool),
                     quant ? k_scale : nullptr, quant ? v_scale : nullptr, pairs, num_kv_heads,
                     k_chunks, v_chunks, num_blocks, block_size);
  return check_launch();
}

int launch_swap_blocks(void* staging, void* pool, const int32_t* blocks, int n_blocks, int64_t block_bytes,
                       int num_blocks, bool to_staging, hipStream_t stream) {
  const int64_t chunks = block_bytes / 16;
  const int64_t per_wg = 256 * 8;                 // 8 chunks per thread per workgroup pass
  const int64_t gy = std::min<int64_t>((chunks + per_wg - 1) / per_wg, 65535);
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(n_blocks, static_cast<unsigned>(gy)), dim3(256), 0, stream,
                     static_cast<uint4*>(staging), static_cast<uint4*>(pool), blocks, chunks, num_blocks,
                     to_staging ? 1 : 0);
  return check_launch();
}

}  // namespace pkv
