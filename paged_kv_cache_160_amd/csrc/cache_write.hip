// Cache writes: scatter new K/V token rows into their paged slots (with fp8
// e4m3 quantisation on the way in) and copy whole blocks for copy-on-write.
//
// Pages: each decode step appends the new token's K and V to the layer's
// cache ("KV Cache 和 vLLM" §1.3; "企业官网建设流程全解析" §3.2) into fixed
// 16-token blocks (§3.1 of the first); fp8 KV with a scale per token and per
// head ("KV Cache优化实战" §3.2-3.3); copy-on-write of shared blocks ("KV Cache
// 和 vLLM" §3.3).
//
// These kernels move at most a few hundred KiB per decode step and are
// launch-bound; they are written for exactness (bit copies, a bit-exact
// quantiser) and coalesced 16-byte accesses, not for peak bandwidth.

#include "device_common.h"
#include "launch.h"

namespace pkv {

// One 16-byte chunk per thread.  A (token, head) row of head_dim elements is
// `chunks_per_row` chunks; a pool row lives at
// ((slot / 16) * Hkv + head) * 16 + slot % 16 in units of rows.
__global__ void __launch_bounds__(256) append_copy_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
    const int64_t* __restrict__ slot_mapping, int num_tokens, int num_kv_heads,
    int chunks_per_row, int64_t num_slots) {
  int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t rows = static_cast<int64_t>(num_tokens) * num_kv_heads;
  int64_t row = gid / chunks_per_row;
  int chunk = static_cast<int>(gid % chunks_per_row);
  if (row >= rows) return;
  int64_t tok = row / num_kv_heads;
  int head = static_cast<int>(row % num_kv_heads);
  int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;
  int64_t blk = slot / kBlockTokens;
  int64_t off = slot % kBlockTokens;
  int64_t dst_row = (blk * num_kv_heads + head) * kBlockTokens + off;
  k_pool[dst_row * chunks_per_row + chunk] = k_new[row * chunks_per_row + chunk];
  v_pool[dst_row * chunks_per_row + chunk] = v_new[row * chunks_per_row + chunk];
}

// fp8: one wave per (token, head) row and per tensor (K rows in waves with
// blockIdx.y == 0, V rows with blockIdx.y == 1).  Each lane holds head_dim/64
// elements.
template <typename Src, int D>
__global__ void __launch_bounds__(256) append_fp8_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    float* __restrict__ k_scale, float* __restrict__ v_scale,
    const int64_t* __restrict__ slot_mapping, int num_tokens, int num_kv_heads,
    int64_t num_slots) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t rows = static_cast<int64_t>(num_tokens) * num_kv_heads;
  if (row >= rows) return;
  const bool is_v = blockIdx.y != 0;
  const void* src = is_v ? v_new : k_new;
  uint8_t* pool = is_v ? v_pool : k_pool;
  float* scales = is_v ? v_scale : k_scale;
  const int64_t tok = row / num_kv_heads;
  const int head = static_cast<int>(row % num_kv_heads);
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;

  const int64_t blk = slot / kBlockTokens;
  const int64_t off = slot % kBlockTokens;
  const int64_t dst_row = (blk * num_kv_heads + head) * kBlockTokens + off;
  write_row_fp8<Src, D>(src, row, pool, scales, dst_row, lane);
}

// Copy-on-write: one workgroup per (pair, head, tensor); 16-byte chunks.
__global__ void __launch_bounds__(256) copy_blocks_kernel(
    uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
    float* __restrict__ k_scale, float* __restrict__ v_scale,
    const int32_t* __restrict__ pairs, int num_kv_heads, int chunks_per_tile, int num_blocks) {
  const int pair = blockIdx.x;
  const int head = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint4* pool = is_v ? v_pool : k_pool;
  const int64_t s_tile = static_cast<int64_t>(src) * num_kv_heads + head;
  const int64_t d_tile = static_cast<int64_t>(dst) * num_kv_heads + head;
  for (int c = threadIdx.x; c < chunks_per_tile; c += blockDim.x)
    pool[d_tile * chunks_per_tile + c] = pool[s_tile * chunks_per_tile + c];
  float* scales = is_v ? v_scale : k_scale;
  if (scales != nullptr && threadIdx.x < kBlockTokens)
    scales[d_tile * kBlockTokens + threadIdx.x] = scales[s_tile * kBlockTokens + threadIdx.x];
}

// ---- launchers -------------------------------------------------------------------

int launch_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                  float* k_scale, float* v_scale, const int64_t* slot_mapping, int num_tokens,
                  int num_kv_heads, int head_dim, int num_blocks, pkv_dtype src_dtype,
                  pkv_dtype cache_dtype, hipStream_t stream) {
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * kBlockTokens;
  const int64_t rows = static_cast<int64_t>(num_tokens) * num_kv_heads;
  if (cache_dtype != PKV_FP8_E4M3) {
    const int es = cache_dtype == PKV_F32 ? 4 : 2;
    const int chunks = head_dim * es / 16;
    const int64_t threads = rows * chunks;
    const int64_t grid = (threads + 255) / 256;
    hipLaunchKernelGGL(append_copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                       static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                       static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), slot_mapping,
                       num_tokens, num_kv_heads, chunks, num_slots);
    return check_launch();
  }
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4), 2);
  auto* kp = static_cast<uint8_t*>(k_pool);
  auto* vp = static_cast<uint8_t*>(v_pool);
#define PKV_APPEND_FP8(SRC, DD)                                                                  \
  hipLaunchKernelGGL((append_fp8_kernel<SRC, DD>), grid, dim3(256), 0, stream, k_new, v_new, kp, \
                     vp, k_scale, v_scale, slot_mapping, num_tokens, num_kv_heads, num_slots)
  if (head_dim == 128) {
    if (src_dtype == PKV_F32) PKV_APPEND_FP8(F32, 128);
    else if (src_dtype == PKV_F16) PKV_APPEND_FP8(F16, 128);
    else PKV_APPEND_FP8(BF16, 128);
  } else {
    if (src_dtype == PKV_F32) PKV_APPEND_FP8(F32, 64);
    else if (src_dtype == PKV_F16) PKV_APPEND_FP8(F16, 64);
    else PKV_APPEND_FP8(BF16, 64);
  }
#undef PKV_APPEND_FP8
  return check_launch();
}

int launch_copy_blocks(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                       const int32_t* pairs, int n_pairs, int num_kv_heads, int head_dim,
                       int num_blocks, pkv_dtype cache_dtype, hipStream_t stream) {
  const int es = cache_dtype == PKV_F32 ? 4 : (cache_dtype == PKV_FP8_E4M3 ? 1 : 2);
  const int chunks_per_tile = kBlockTokens * head_dim * es / 16;
  const bool fp8 = cache_dtype == PKV_FP8_E4M3;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n_pairs, num_kv_heads, 2), dim3(256), 0, stream,
                     static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool),
                     fp8 ? k_scale : nullptr, fp8 ? v_scale : nullptr, pairs, num_kv_heads,
                     chunks_per_tile, num_blocks);
  return check_launch();
}

}  // namespace pkv
