// Chunked prefill attention over the paged cache for gfx950: a chunk of new
// tokens of each sequence attends over the sequence's cached K/V (read
// through the block table) and causally over its own tokens.
//
// Pages: in prefill every prompt token is processed at once, each position
// attending to itself and the positions before it ("KV Cache 和 vLLM" §1.1;
// "企业官网建设流程全解析" §3.1-3.2); the K/V of tokens already cached is
// reused rather than recomputed ("KV Cache优化实战" §5.2); logical blocks map
// to physical blocks through the block table ("KV Cache 和 vLLM" §3.2);
// several query heads share one KV head ("企业官网建设流程全解析" §2.2).
//
// Unlike decode this is a dense contraction (each K/V element meets many
// queries), so it is built for the matrix cores:
//  * Workgroup = W waves owning W * 16 * CTILES query rows of one (sequence,
//    KV head): 8 waves (256 rows) for 16-bit caches, 4 (128 rows) for
//    quantised ones; a row is a (chunk position, head of the GQA group)
//    pair, so the whole group shares every K/V tile.  Each wave owns CTILES
//    tiles of 16 rows.
//  * K and V stream through LDS in stages of 64 keys (4 tiles of 16).  For
//    16-bit caches each wave moves its share of the next stage straight from
//    HBM into the second of two LDS buffers (global_load_lds, no registers)
//    while the workgroup computes the current one; rows are unpadded and
//    their 16-byte chunks XOR-swizzled by row, so the K operand reads meet
//    no bank conflicts (the transposed V reads meet two-way ones, which
//    cost nothing measurable, while a map free of both needed registers
//    the stage loop does not have).  Quantised codes (e4m3, e5m2, int8 K, int4 V) take a
//    register path instead: they become 16-bit values exactly on the way
//    into a padded buffer, and their per-token scales go to LDS beside them.
//      S^T = K (16 keys x D) * Q^T (D x 16 rows)       [16x16x32 MFMA]
//      O  += P (16 rows x 32 keys) * V (32 keys x 16 d) [16x16x32 MFMA]
//    The S^T accumulator (lane = row + 16*(key/4), reg = key%4) already is
//    the P operand: the contraction index of an MFMA may be permuted freely
//    when both operands use the same permutation, so each lane's 8 P values
//    (keys 4j..4j+3 of two 16-key tiles) meet the V values of the same keys.
//  * Online softmax in log2 units per row; the running maximum moves only
//    when a row's maximum grows by more than 2^8.  Each lane compares its own
//    raw scores with a raw threshold, so the cross-lane maximum is only taken
//    when some score passes it.  The stage loop runs in a fast form that
//    never rescales the output (a row's first maximum is set while its output
//    is still zero); a wave whose row maximum grows past the threshold
//    leaves it and finishes its keys in a second form that rescales.  The
//    fast loop then carries no conditional update of the accumulators, which
//    the register allocator otherwise pays for with copies on every stage.
//  * Row sums of P (16-bit caches) come from the matrix cores: one extra
//    MFMA per half-stage multiplies P by a column of ones.
//  * The matrix phases run at raised wave priority, and each issues all of
//    its LDS operand reads before its first MFMA (a scheduling hint): one
//    LDS round trip per phase instead of one per group of four reads.
//  * The causal diagonal bounds each workgroup's key loop; stages entirely
//    below it need no mask.
//  * Workgroups of one (sequence, KV head) are placed on one XCD so they
//    share its L2.

#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace pkv {
namespace {

// Waves per workgroup (4 or 8): 16-bit caches stage K/V straight into LDS
// and share each stage among 8 waves (256 query rows); quantised caches,
// which convert the codes on their way into LDS, run 4.
#ifndef PKV_PREFILL_WAVES_16
#define PKV_PREFILL_WAVES_16 8
#endif
#ifndef PKV_PREFILL_WAVES_Q
#define PKV_PREFILL_WAVES_Q 4
#endif
#ifndef PKV_PREFILL_BUFFERS
#define PKV_PREFILL_BUFFERS 2   // K/V stage buffers (16-bit caches)
#endif
constexpr int kPfBufs = PKV_PREFILL_BUFFERS;
#ifndef PKV_PREFILL_KEYS
#define PKV_PREFILL_KEYS 64    // keys per stage (32 or 64)
#endif
constexpr int kPfKeys = PKV_PREFILL_KEYS;
constexpr int kPfStageTiles = kPfKeys / kTileTokens;          // 16-token units per stage
constexpr int kPfMaxBlocks = PKV_MAX_PREFILL_CONTEXT / kTileTokens;
constexpr int kXcds = 8;

// s_waitcnt on vector memory only: at most N of this wave's loads in flight
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
constexpr float kLog2eP = 1.4426950408889634f;

#ifndef PKV_PREFILL_BUFLDS
#define PKV_PREFILL_BUFLDS 0   // stage loads as buffer loads into LDS
#endif
#ifndef PKV_PREFILL_CTILES
#define PKV_PREFILL_CTILES 2   // 16-row query tiles per wave
#endif

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
constexpr float kRebase = 8.0f;     // log2 headroom before the running max moves

template <int CTILES, int W>
struct PfShape {
  static constexpr int rows_per_wave = 16 * CTILES;
  static constexpr int rows = W * rows_per_wave;            // query rows per workgroup
};

// 16-bit element type of the MFMA operands for query type QT.
template <typename QT>
__device__ __forceinline__ float4_t mfma32(u32x4 a, u32x4 b, float4_t c) {
  if constexpr (std::is_same<QT, BF16>::value)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                  0, 0, 0);
}

template <typename QT>
__device__ __forceinline__ uint32_t pack_pair(float a, float b) {
  if constexpr (std::is_same<QT, BF16>::value) {
    bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    half2_t v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// Four 8-bit codes (one word) of format ET -> four 16-bit values of QT's
// type (two words), exactly, in element order: e4m3, e5m2 and int8 values
// all fit.
template <typename QT, typename ET>
__device__ __forceinline__ u32x2_t codes8_to_16(uint32_t w) {
  constexpr bool kBf = std::is_same<QT, BF16>::value;
  u32x2_t r;
  if constexpr (std::is_same<ET, FP8>::value) {
    if constexpr (kBf) {
      r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
      r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
    } else {
      r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
      r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
    }
  } else if constexpr (std::is_same<ET, BF8>::value) {
    if constexpr (kBf) {
      r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false));
      r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true));
    } else {
      r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, false));
      r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, true));
    }
  } else {
    static_assert(std::is_same<ET, I8>::value, "8-bit format");
    r[0] = pack_pair<QT>(static_cast<float>(static_cast<int8_t>(w & 0xffu)),
                         static_cast<float>(static_cast<int8_t>((w >> 8) & 0xffu)));
    r[1] = pack_pair<QT>(static_cast<float>(static_cast<int8_t>((w >> 16) & 0xffu)),
                         static_cast<float>(static_cast<int8_t>(w >> 24)));
  }
  return r;
}

// 16 bytes of codes of format ET -> their values as 16-bit elements of QT's
// type at dst (16 values for 8-bit codes, 32 for 4-bit ones), exactly.
// INT4: two's complement nibbles, element 2i in the low nibble of byte i.
template <typename QT, typename ET>
__device__ __forceinline__ void codes_to_lds(const u32x4& src, uint16_t* dst) {
  if constexpr (ET::bits == 8) {
    const u32x2_t w0 = codes8_to_16<QT, ET>(src[0]);
    const u32x2_t w1 = codes8_to_16<QT, ET>(src[1]);
    const u32x2_t w2 = codes8_to_16<QT, ET>(src[2]);
    const u32x2_t w3 = codes8_to_16<QT, ET>(src[3]);
    reinterpret_cast<u32x4*>(dst)[0] = u32x4{w0[0], w0[1], w1[0], w1[1]};
    reinterpret_cast<u32x4*>(dst)[1] = u32x4{w2[0], w2[1], w3[0], w3[1]};
  } else {
    static_assert(std::is_same<ET, I4>::value, "4-bit format");
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      u32x4 r;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int32_t x = static_cast<int32_t>(src[wd]);
        const float e0 = static_cast<float>((x << (28 - 8 * k)) >> 28);
        const float e1 = static_cast<float>((x << (24 - 8 * k)) >> 28);
        r[k] = pack_pair<QT>(e0, e1);
      }
      reinterpret_cast<u32x4*>(dst)[wd] = r;
    }
  }
}

__device__ __forceinline__ float cmax4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float csum4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Value of x held by lane src (0..63).
__device__ __forceinline__ float lane_value(float x, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

// 16 bytes of a K/V tile (at byte lane_off of it) for each lane of the wave,
// into LDS at lds + 16 * lane, by a buffer load through a descriptor of the
// tile (so the hardware also bounds every lane's offset by the tile).
__device__ __forceinline__ void tile_chunk_to_lds(const uint8_t* tile, int tile_bytes, uint8_t* lds, int lane_off) {
  constexpr int kRaw32 = 0x00020000;   // descriptor word 3: 32-bit data, untyped
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(tile), 0, tile_bytes, kRaw32);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, lane_off, 0, 0, 0);
}

// One stage's global -> LDS traffic.  16-bit pools (KT = VT = the query
// type) go straight to LDS by row (row_bytes, tile_bytes).  Quantised pools
// go through registers: thread t, round r moves the 16-byte chunk r*256 + t
// of the stage's K rows (and of its V rows, which are shorter for INT4), and
// the chunks are converted to 16-bit values on the way into LDS.
template <typename KT, typename VT, int D, int W>
struct StageIO {
  static constexpr int threads = W * kWave;
  static constexpr int k_row_bytes = D * KT::bits / 8;
  static constexpr int v_row_bytes = D * VT::bits / 8;
  static constexpr int row_bytes = k_row_bytes;              // 16-bit pools: K and V alike
  static constexpr int tile_bytes = kTileTokens * row_bytes;
  static constexpr int k_tile_bytes = kTileTokens * k_row_bytes;
  static constexpr int v_tile_bytes = kTileTokens * v_row_bytes;
  static constexpr int k_chunks = kPfKeys * k_row_bytes / 16;
  static constexpr int v_chunks = kPfKeys * v_row_bytes / 16;
  static constexpr int k_rounds = (k_chunks + threads - 1) / threads;
  static constexpr int v_rounds = (v_chunks + threads - 1) / threads;
  // 16-bit elements per LDS row: D + 16 puts consecutive rows 32 bytes apart
  // in bank space, so the 16 rows a transpose read or a K-operand read
  // touches spread evenly over the banks
  static constexpr int lds_row = D + 16;
  u32x4 k[k_rounds], v[v_rounds];
  float ks;                                                  // thread t < 64 -> a K scale, < 128 -> a V scale
};

// Swizzle of 16-byte chunk positions in an unpadded LDS row of D 16-bit
// elements: consecutive rows (D = 128) or row pairs (D = 64, two rows per
// 256-byte bank line) rotate their chunks, so the 16 rows of one K operand
// read land on distinct banks (the LDS serves 16 lanes of a 16-byte read
// per pass).
template <int D>
struct LdsSwz {
  static __device__ __forceinline__ int of(int r) {
    if constexpr (D == 128) return r & 15;
    else return (r >> 1) & 7;
  }
};

template <typename QT, typename KT, typename VT, int D, int CTILES, int W>
__global__ void __launch_bounds__(W * kWave, (CTILES <= 2 && W == 4) ? 2 : 1)
    paged_prefill_kernel(PrefillArgs a) {
  constexpr int kPfWaves = W;
  constexpr int kPfThreads = W * kWave;
  using IO = StageIO<KT, VT, D, W>;
  using SH = PfShape<CTILES, W>;
  constexpr bool kConv = KT::quantised;      // codes converted on the way into LDS
  constexpr int DCH = D / 32;        // QK MFMAs per 16-key tile
  constexpr int DT = D / 16;         // output column tiles
  constexpr float kNegInf = -INFINITY;

  // quantised caches: one padded 16-bit stage buffer per tensor (and the
  // scales); 16-bit caches: two unpadded, swizzled stage buffers per tensor
  constexpr int kPadElems = kConv ? kPfKeys * IO::lds_row : 8;
  constexpr int kDmaChunks = kConv ? 1 : kPfKeys * IO::row_bytes / 16;
  __shared__ __attribute__((aligned(16))) uint16_t sm_k[kPadElems];
  __shared__ __attribute__((aligned(16))) uint16_t sm_v[kPadElems];
  // one variable per stage buffer: the compiler gives each its own alias
  // scope, so it can tell that the reads of one buffer do not touch another
  // that direct loads are filling
  constexpr int kDma3 = kPfBufs > 2 ? kDmaChunks : 1;
  __shared__ u32x4 sm_k0[kDmaChunks], sm_k1[kDmaChunks], sm_k2[kDma3];
  __shared__ u32x4 sm_v0[kDmaChunks], sm_v1[kDmaChunks], sm_v2[kDma3];
  __shared__ float sm_ks[kPfKeys];
  __shared__ float sm_vs[kPfKeys];
  __shared__ int sm_ids[kPfMaxBlocks];

  // ---- which (sequence, KV head, row tile) this workgroup owns -------------
  const int total = a.num_seqs * a.num_kv_heads * a.tiles_per_seq;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (logical >= total) return;
  const int tile = logical % a.tiles_per_seq;
  const int g = (logical / a.tiles_per_seq) % a.num_kv_heads;
  const int b = logical / (a.tiles_per_seq * a.num_kv_heads);
  const int group = a.num_q_heads / a.num_kv_heads;

  const int qs = a.query_start[b];
  const int n = a.query_start[b + 1] - qs;
  int L = a.context_lens[b];
  // a chunk outside q, or longer than the launch was sized for, is skipped
  if (qs < 0 || n <= 0 || n > a.max_query_len || qs + n > a.num_tokens) return;
  const int rows_b = n * group;
  const int r0 = tile * SH::rows;
  if (r0 >= rows_b) return;
  L = max(0, min(L, min(a.max_context_len, a.max_blocks_per_seq * a.block_size)));
  const int ctx = L - n;             // positions of the chunk: ctx .. L-1

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int c = lane & 15;
  const int j = lane >> 4;

  if (L == 0) {
    // nothing cached: the chunk's rows are zero
    const int r1 = min(rows_b, r0 + SH::rows);
    for (int idx = tid; idx < (r1 - r0) * D; idx += kPfThreads) {
      const int r = r0 + idx / D;
      const int64_t o = (static_cast<int64_t>(qs + r / group) * a.num_q_heads + g * group + r % group) * D + idx % D;
      store_from_f32<QT>(a.out, o, 0.0f);
    }
    return;
  }

  // key range: every row of the tile sees keys <= ctx + (its position)
  const int i_first = r0 / group;
  const int i_last = (min(rows_b, r0 + SH::rows) - 1) / group;
  const int key_end = min(L, max(1, ctx + i_last + 1));       // exclusive
  const int free_end = max(0, ctx + i_first + 1);             // keys < free_end are seen by every row
  const int nstages = (key_end + kPfKeys - 1) / kPfKeys;
  const int nblk = (key_end + kTileTokens - 1) / kTileTokens;

  // ---- query operands and per-row limits -------------------------------------
  // Wave w, tile ct, column c: row r0 + w*16*CTILES + ct*16 + c.  Rows past
  // the chunk take a copy of its last row (their output is never stored):
  // no register a load still fills is overwritten, so the query loads and
  // the block-table loads below are in flight together.
  u32x4 qop[CTILES][DCH];
  int lim[CTILES];
  const uint8_t* qbase = static_cast<const uint8_t*>(a.q);
#pragma unroll
  for (int ct = 0; ct < CTILES; ++ct) {
    const int r = r0 + wave * SH::rows_per_wave + ct * 16 + c;
    const bool valid = r < rows_b;
    const int i = valid ? r / group : n - 1;
    const int head = g * group + (valid ? r % group : 0);
    lim[ct] = max(0, min(ctx + i, L - 1));
    const uint8_t* qp = qbase + ((static_cast<int64_t>(qs + i) * a.num_q_heads + head) * D + 8 * j) * 2;
#pragma unroll
    for (int dc = 0; dc < DCH; ++dc) qop[ct][dc] = *reinterpret_cast<const u32x4*>(qp + 64 * dc);
  }
  // Unit u (tokens 16u .. 16u+15) staged as its tile index at KV head 0,
  // ((phys * Hkv) << rs) + (u & (2^rs - 1)); the table entry is clamped into
  // the pool (the positions it stands for are the caller's to keep valid).
  const int32_t* table = a.block_tables + static_cast<int64_t>(b) * a.max_blocks_per_seq;
  const int rs = block_shift(a.block_size);
  for (int u = tid; u < nblk; u += kPfThreads)
    sm_ids[u] = ((min(max(table[u >> rs], 0), a.num_blocks - 1) * a.num_kv_heads) << rs) + (u & ((1 << rs) - 1));
  const int g_tile = g << rs;

  __syncthreads();   // block ids staged

  // ---- output state ----------------------------------------------------------------
  float4_t o[CTILES][DT];
  // Row sums of P: 16-bit caches add them on the matrix cores, as P times a
  // column of ones (osum: lane (c, j) register rr holds row 4j + rr, as in o,
  // and sums the 16-bit P that meets V); quantised caches, whose P operand
  // carries the V scales, add the fp32 values in lsum (a lane's share of row c).
  float4_t osum[CTILES];
  float m[CTILES], lsum[CTILES], rt[CTILES];
#pragma unroll
  for (int ct = 0; ct < CTILES; ++ct) {
    m[ct] = kNegInf;
    rt[ct] = kNegInf;
    lsum[ct] = 0.0f;
    osum[ct] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[ct][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float sl = a.scale * kLog2eP;       // > 0: the host refuses other scales
  const float inv_sl = 1.0f / sl;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_pool);
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_pool);

  // Byte offset in a stage buffer of 16-byte chunk q (8 elements) of row r,
  // and of its half h.  16-bit caches: unpadded rows whose chunk q sits at
  // position q ^ swz(r); quantised caches (converted on the way in): padded rows.
  auto kaddr = [&](int r, int q) -> int {
    if constexpr (kConv) return (r * IO::lds_row + 8 * q) * 2;
    else return r * IO::row_bytes + 16 * (q ^ LdsSwz<D>::of(r));
  };
  auto vaddr = [&](int r, int q, int h) -> int { return kaddr(r, q) + 8 * h; };

  // One stage (kPfKeys keys from s * kPfKeys) held in LDS at kbuf / vbuf.
  // One stage from half hv0 on.  The fast form (kSlow false) never rescales
  // the output: when a row that already holds output needs a new maximum it
  // returns the half it stopped at, before changing anything for that half,
  // and the caller finishes the work with the slow form, which rescales.
  // Returns -1 when the stage is done.
  auto compute = [&](auto slow_tag, const uint8_t* kbuf, const uint8_t* vbuf, int s, int hv0)
                     __attribute__((always_inline)) -> int {
      constexpr bool kSlow = decltype(slow_tag)::value;
      // the stage in halves of 32 keys: S^T, softmax, then P V for each
#pragma unroll
      for (int hv = 0; hv < kPfKeys / 32; ++hv) {
        if (hv < hv0) continue;
        const int kb = s * kPfKeys + 32 * hv;
        const bool masked = kb + 32 > free_end;

        // S^T tiles: [key tile of the half][row tile]
        float4_t st[2][CTILES];
        // matrix phases run at raised wave priority: of the two waves sharing
        // a SIMD, the one with MFMA work issues first and the other's softmax
        // fills the gaps
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
          for (int ct = 0; ct < CTILES; ++ct) st[kt][ct] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int dc = 0; dc < DCH; ++dc) {
            const u32x4 kop = *reinterpret_cast<const u32x4*>(kbuf + kaddr(32 * hv + kt * 16 + c, 4 * dc + j));
#pragma unroll
            for (int ct = 0; ct < CTILES; ++ct) st[kt][ct] = mfma32<QT>(kop, qop[ct][dc], st[kt][ct]);
          }
        }
        // every operand read of the phase goes out before its first MFMA
        // (left to itself the scheduler splits them into groups, each a full
        // LDS round trip in front of its MFMAs)
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * DCH, 0);          // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * DCH * CTILES, 0);  // MFMA
        __builtin_amdgcn_s_setprio(0);
        if constexpr (kConv) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const float4 ksc = *reinterpret_cast<const float4*>(sm_ks + 32 * hv + kt * 16 + 4 * j);
#pragma unroll
            for (int ct = 0; ct < CTILES; ++ct) {
              st[kt][ct][0] *= ksc.x;
              st[kt][ct][1] *= ksc.y;
              st[kt][ct][2] *= ksc.z;
              st[kt][ct][3] *= ksc.w;
            }
          }
        }
        if (masked) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ct = 0; ct < CTILES; ++ct)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr)
                if (kb + kt * 16 + 4 * j + rr > lim[ct]) st[kt][ct][rr] = kNegInf;
        }

        // online softmax per row (column c of each row tile), in log2 units.
        // The running maximum m only moves when a row's new maximum exceeds it
        // by more than kRebase: probabilities exp2(s*sl - m) stay below
        // 2^kRebase and the output and sum are rescaled far less often (the
        // final division uses the same m for both, so the result is the same).
        // A row's scores are spread over 4 lanes; each lane compares its own
        // raw scores with rt = (m + kRebase) / sl (sl > 0), and only when one
        // of them is above it does the wave take row maxima across lanes.
        float mxr[CTILES];
        bool need = false;
#pragma unroll
        for (int ct = 0; ct < CTILES; ++ct) {
          float mx = kNegInf;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) mx = fmaxf(mx, st[kt][ct][rr]);
          mxr[ct] = mx;
          need |= mx > rt[ct];
        }
        if (__any(need)) {
          if constexpr (!kSlow) {
            // a row with a finite maximum holds output: that needs a rescale
            bool held = false;
#pragma unroll
            for (int ct = 0; ct < CTILES; ++ct) held |= mxr[ct] > rt[ct] && m[ct] != kNegInf;
            if (__any(held)) return hv;
            // first keys of rows with nothing yet (output and sum are zero):
            // only the maximum is set
#pragma unroll
            for (int ct = 0; ct < CTILES; ++ct) {
              const float mxs = cmax4(mxr[ct]) * sl;
              const float mnew = mxs > m[ct] + kRebase ? mxs : m[ct];
              m[ct] = mnew;
              rt[ct] = (mnew + kRebase) * inv_sl;
            }
          } else {
#pragma unroll
            for (int ct = 0; ct < CTILES; ++ct) {
              const float mxs = cmax4(mxr[ct]) * sl;
              const float mnew = mxs > m[ct] + kRebase ? mxs : m[ct];
              const float alpha = mnew == m[ct] ? 1.0f : __builtin_amdgcn_exp2f(m[ct] - mnew);
              m[ct] = mnew;
              rt[ct] = (mnew + kRebase) * inv_sl;
              lsum[ct] *= alpha;
              float ar[4];
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) ar[rr] = lane_value(alpha, 4 * j + rr);
#pragma unroll
              for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) o[ct][dt][rr] *= ar[rr];
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) osum[ct][rr] *= ar[rr];
            }
          }
        }
        u32x4 pop[CTILES];
#pragma unroll
        for (int ct = 0; ct < CTILES; ++ct) {
          float p[2][4];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) p[kt][rr] = __builtin_amdgcn_exp2f(fmaf(st[kt][ct][rr], sl, -m[ct]));
          if constexpr (kConv) {
            lsum[ct] += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
              const float4 vsc = *reinterpret_cast<const float4*>(sm_vs + 32 * hv + kt * 16 + 4 * j);
              p[kt][0] *= vsc.x;
              p[kt][1] *= vsc.y;
              p[kt][2] *= vsc.z;
              p[kt][3] *= vsc.w;
            }
          }
          pop[ct][0] = pack_pair<QT>(p[0][0], p[0][1]);
          pop[ct][1] = pack_pair<QT>(p[0][2], p[0][3]);
          pop[ct][2] = pack_pair<QT>(p[1][0], p[1][1]);
          pop[ct][3] = pack_pair<QT>(p[1][2], p[1][3]);
        }

        // O += P V.  B operand (32 keys x 16 d) by transpose reads: lane c of
        // group j points at V[key 4j + c/4 (+16)][d0 + 4(c%4) ..+3] and
        // receives V[key 4j + e (+16)][d0 + c] for e = 0..3, the keys of its P
        // slots.
        const int vr0 = 32 * hv + 4 * j + (c >> 2);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int vq = 2 * dt + ((c & 3) >> 1);
          const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4_t*)(vbuf + vaddr(vr0, vq, c & 1)));
          const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4_t*)(vbuf + vaddr(vr0 + 16, vq, c & 1)));
          const u32x2_t wlo = __builtin_bit_cast(u32x2_t, lo);
          const u32x2_t whi = __builtin_bit_cast(u32x2_t, hi);
          const u32x4 vop = {wlo[0], wlo[1], whi[0], whi[1]};
#pragma unroll
          for (int ct = 0; ct < CTILES; ++ct) o[ct][dt] = mfma32<QT>(pop[ct], vop, o[ct][dt]);
        }
        if constexpr (!kConv) {
          constexpr uint32_t kOnes = std::is_same<QT, BF16>::value ? 0x3F803F80u : 0x3C003C00u;   // 1.0, 1.0
#pragma unroll
          for (int ct = 0; ct < CTILES; ++ct) osum[ct] = mfma32<QT>(pop[ct], u32x4{kOnes, kOnes, kOnes, kOnes}, osum[ct]);
        }
        // as for S^T: every V operand read, then the MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * DT, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, DT * CTILES + (kConv ? 0 : CTILES), 0);
        __builtin_amdgcn_s_setprio(0);
      }
      return -1;
  };

  if constexpr (kConv) {
    // ---- quantised: global -> registers -> (convert) -> LDS, one buffer ---------
    IO io;
    // round r of thread t moves the stage's 16-byte chunk r*256 + t of K and
    // of V: a fixed row of the stage (so a fixed tile of its 4 and row within
    // it) and column
    auto load_rows = [&](u32x4* dst, const uint8_t* pool, int row_bytes, int tile_bytes, int chunks, int rounds,
                         int s) {
      const int kb = s * kPfKeys;
      for (int r = 0; r < rounds; ++r) {
        const int chunk = r * kPfThreads + tid;
        const int row = chunk * 16 / row_bytes;
        dst[r] = u32x4{0u, 0u, 0u, 0u};
        if (chunk < chunks && kb + row < key_end) {
          const int id = sm_ids[kPfStageTiles * s + row / kTileTokens];
          const int64_t off = static_cast<int64_t>(id + g_tile) * tile_bytes +
                              (row % kTileTokens) * row_bytes + (chunk * 16) % row_bytes;
          dst[r] = *reinterpret_cast<const u32x4*>(pool + off);
        }
      }
    };
    auto load_stage = [&](int s) {
      load_rows(io.k, kpool, IO::k_row_bytes, IO::k_tile_bytes, IO::k_chunks, IO::k_rounds, s);
      load_rows(io.v, vpool, IO::v_row_bytes, IO::v_tile_bytes, IO::v_chunks, IO::v_rounds, s);
      io.ks = 0.0f;
      const int kb = s * kPfKeys;
      if (tid < 2 * kPfKeys) {
        const int key = kb + (tid % kPfKeys);
        if (key < key_end) {
          const int id = sm_ids[key / kTileTokens];
          const int64_t si = static_cast<int64_t>(id + g_tile) * kTileTokens + key % kTileTokens;
          io.ks = tid < kPfKeys ? a.k_scale[si] : a.v_scale[si];
        }
      }
    };
    auto store_stage = [&]() {
#pragma unroll
      for (int r = 0; r < IO::k_rounds; ++r) {
        const int chunk = r * kPfThreads + tid;
        if (chunk < IO::k_chunks) {
          const int row = chunk * 16 / IO::k_row_bytes;
          const int e = (chunk * 16) % IO::k_row_bytes * 8 / KT::bits;   // first element of the chunk
          codes_to_lds<QT, KT>(io.k[r], sm_k + row * IO::lds_row + e);
        }
      }
#pragma unroll
      for (int r = 0; r < IO::v_rounds; ++r) {
        const int chunk = r * kPfThreads + tid;
        if (chunk < IO::v_chunks) {
          const int row = chunk * 16 / IO::v_row_bytes;
          const int e = (chunk * 16) % IO::v_row_bytes * 8 / VT::bits;
          codes_to_lds<QT, VT>(io.v[r], sm_v + row * IO::lds_row + e);
        }
      }
      if (tid < kPfKeys) sm_ks[tid] = io.ks;
      else if (tid < 2 * kPfKeys) sm_vs[tid - kPfKeys] = io.ks;
    };
    const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(sm_k);
    const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(sm_v);
    load_stage(0);
    int s = 0, hv = -1;
    for (; s < nstages; ++s) {
      store_stage();
      __syncthreads();
      if (s + 1 < nstages) load_stage(s + 1);
      hv = compute(std::false_type{}, kb8, vb8, s, 0);
      if (hv >= 0) break;
      __syncthreads();   // every wave is done with this stage's LDS
    }
    if (hv >= 0) {
      // a row's maximum grew: the rest of the keys with rescaling
      compute(std::true_type{}, kb8, vb8, s, hv);
      __syncthreads();
      for (++s; s < nstages; ++s) {
        store_stage();
        __syncthreads();
        if (s + 1 < nstages) load_stage(s + 1);
        compute(std::true_type{}, kb8, vb8, s, 0);
        __syncthreads();
      }
    }
  } else {
    // ---- 16-bit caches: global -> LDS directly, two buffers ----------------------
    // Wave w moves rows kPfKeys/kPfWaves * w ... of each stage (a whole
    // block with 4 waves, half a block with 8): kInsts instructions per
    // tensor, lane i of instruction n filling stage chunk 64n + i, i.e. row
    // (64n+i)/CH at swizzled position (64n+i)%CH.
    constexpr int CH = IO::row_bytes / 16;                  // chunks per row
    constexpr int kInsts = kPfKeys * CH / (kPfWaves * kWave);
    static_assert(kPfKeys * CH == kPfWaves * kInsts * kWave, "a stage splits evenly over the waves");
    int lane_off[kInsts];
#pragma unroll
    for (int k = 0; k < kInsts; ++k) {
      const int slot = (wave * kInsts + k) * kWave + lane;
      const int r = slot / CH;
      const int q = (slot % CH) ^ LdsSwz<D>::of(r);
      lane_off[k] = (r % kTileTokens) * IO::row_bytes + 16 * q;
    }
    auto dma = [&](const uint8_t* kp, const uint8_t* vp, uint8_t* kdst, uint8_t* vdst, int s)
                   __attribute__((always_inline)) {
      // rows past the context (last stage) read the sequence's last block
      // and are zeroed after they land
      const int id = sm_ids[min(kPfStageTiles * s + wave * kPfStageTiles / kPfWaves, nblk - 1)];
      const int64_t base = static_cast<int64_t>(id + g_tile) * IO::tile_bytes;
#if PKV_PREFILL_BUFLDS
      // buffer loads into LDS (not the flat-encoded global form: while one of
      // those is in flight the compiler makes every LDS read wait for all
      // earlier ones)
#pragma unroll
      for (int k = 0; k < kInsts; ++k) {
        const int dst = (wave * kInsts + k) * kWave * 16;
        tile_chunk_to_lds(kp + base, IO::tile_bytes, kdst + dst, lane_off[k]);
        tile_chunk_to_lds(vp + base, IO::tile_bytes, vdst + dst, lane_off[k]);
      }
#else
#pragma unroll
      for (int k = 0; k < kInsts; ++k) {
        const int dst = (wave * kInsts + k) * kWave * 16;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kp + base + lane_off[k]),
                                         (__attribute__((address_space(3))) void*)(kdst + dst), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vp + base + lane_off[k]),
                                         (__attribute__((address_space(3))) void*)(vdst + dst), 16, 0, 0);
      }
#endif
    };
    // A stage's compute and the loads that fill a later stage's buffers go
    // through the restrict-qualified pointers of one inlined call.  The
    // compiler then knows that the operand reads of the current buffers do
    // not touch the buffers being filled, and does not wait for those loads
    // before each read (which would expose their whole latency in every
    // stage); the waits for the current stage's own loads are explicit.
    auto run = [&](auto slow_tag, const uint8_t* __restrict__ ck, const uint8_t* __restrict__ cv,
                   uint8_t* __restrict__ nk, uint8_t* __restrict__ nv, const uint8_t* __restrict__ kp,
                   const uint8_t* __restrict__ vp, int s, bool issue) __attribute__((always_inline)) -> int {
      if (issue) dma(kp, vp, nk, nv, s + kPfBufs - 1);
      return compute(slow_tag, ck, cv, s, 0);
    };
    // V rows at or past key_end of the last stage are zeroed by the wave that
    // loaded them (after its own loads landed): P is 0 there, and 0 times a
    // stale NaN would still be NaN.  K needs no care: those keys are masked.
    auto zero_tail = [&](uint8_t* vdst, int s) {
      constexpr int kRowsPerWave = kPfKeys / kPfWaves;        // stage rows this wave loaded
      const int first = max(key_end - s * kPfKeys, kRowsPerWave * wave);
      const int rows = kRowsPerWave * wave + kRowsPerWave - first;
      for (int idx = lane; idx < max(rows, 0) * CH; idx += kWave)
        *reinterpret_cast<u32x4*>(vdst + (first + idx / CH) * IO::row_bytes + 16 * (idx % CH)) = u32x4{0u, 0u, 0u, 0u};
    };
    // kPfBufs stage buffers: the loads of stage s + kPfBufs - 1 go out after
    // the barrier that ends stage s - 1, into the buffer that stage used.
    constexpr int kLoads = 2 * kInsts;                      // this wave's loads per stage
    static_assert(kPfBufs <= 3, "three stage buffers at most");
    auto kbuf = [&](int i) { return reinterpret_cast<uint8_t*>(i == 0 ? sm_k0 : i == 1 ? sm_k1 : sm_k2); };
    auto vbuf = [&](int i) { return reinterpret_cast<uint8_t*>(i == 0 ? sm_v0 : i == 1 ? sm_v1 : sm_v2); };
    auto step = [&](auto slow_tag, int s, int cur) __attribute__((always_inline)) -> int {
      // this wave's loads of stage s landed (those of the kPfBufs - 2 later
      // stages already issued may fly; near the end, wait for all)
      if (kPfBufs > 2 && s + kPfBufs - 2 < nstages) wait_vmcnt<(kPfBufs - 2) * kLoads>();
      else wait_vmcnt<0>();
      if (s == nstages - 1) zero_tail(vbuf(cur), s);
      __syncthreads();                                      // all of stage s is in LDS; stage s-1 is done
      const int nb = (cur + kPfBufs - 1) % kPfBufs;
      return run(slow_tag, kbuf(cur), vbuf(cur), kbuf(nb), vbuf(nb), kpool, vpool, s, s + kPfBufs - 1 < nstages);
    };
#pragma unroll
    for (int i = 0; i + 1 < kPfBufs; ++i)
      if (i < nstages) dma(kpool, vpool, kbuf(i), vbuf(i), i);
    int s = 0, hv = -1;
    while (s < nstages) {
#pragma unroll
      for (int u = 0; u < kPfBufs; ++u) {                   // stage s uses buffer u = s % kPfBufs
        if (s < nstages) {
          hv = step(std::false_type{}, s, u);
          if (hv >= 0) break;
          ++s;
        }
      }
      if (hv >= 0) break;
    }
    if (hv >= 0) {
      // a row's maximum grew: finish stage s from half hv, then the rest of
      // the keys with rescaling (same barriers per stage as above)
      compute(std::true_type{}, kbuf(s % kPfBufs), vbuf(s % kPfBufs), s, hv);
      for (++s; s < nstages; ++s) step(std::true_type{}, s, s % kPfBufs);
    }
  }

  // ---- normalise and store -------------------------------------------------------
#pragma unroll
  for (int ct = 0; ct < CTILES; ++ct) {
    float ir[4];
    if constexpr (kConv) {
      const float l = csum4(lsum[ct]);
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) ir[rr] = lane_value(inv, 4 * j + rr);
    } else {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) ir[rr] = osum[ct][rr] > 0.0f ? 1.0f / osum[ct][rr] : 0.0f;
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = r0 + wave * SH::rows_per_wave + ct * 16 + 4 * j + rr;
      if (r >= rows_b) continue;
      const int64_t orow = (static_cast<int64_t>(qs + r / group) * a.num_q_heads + g * group + r % group) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) store_from_f32<QT>(a.out, orow + 16 * dt + c, o[ct][dt][rr] * ir[rr]);
    }
  }
}

template <typename QT, typename KT, typename VT, int D>
int launch_prefill_typed(const PrefillArgs& a, hipStream_t stream) {
  constexpr int kCt = PKV_PREFILL_CTILES;
  constexpr int kW = KT::quantised ? PKV_PREFILL_WAVES_Q : PKV_PREFILL_WAVES_16;
  using SH = PfShape<kCt, kW>;
  PrefillArgs b = a;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int64_t rows = static_cast<int64_t>(a.max_query_len) * group;
  b.tiles_per_seq = static_cast<int>((rows + SH::rows - 1) / SH::rows);
  const int64_t total = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * b.tiles_per_seq;
  if (total == 0) return PKV_OK;
  if (total > (int64_t{1} << 30)) return PKV_ERR_UNSUPPORTED;
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  hipLaunchKernelGGL((paged_prefill_kernel<QT, KT, VT, D, kCt, kW>), dim3(static_cast<unsigned>(per_xcd * kXcds)),
                     dim3(kW * kWave), 0, stream, b);
  return check_launch();
}

template <typename QT, typename KT, typename VT>
int launch_prefill_dim(const PrefillArgs& a, hipStream_t stream) {
  if (a.head_dim == 64) return launch_prefill_typed<QT, KT, VT, 64>(a, stream);
  if (a.head_dim == 128) return launch_prefill_typed<QT, KT, VT, 128>(a, stream);
  return PKV_ERR_UNSUPPORTED;
}

template <typename KT, typename VT>
int launch_prefill_quantised(const PrefillArgs& a, hipStream_t stream) {
  if (a.q_dtype == PKV_BF16) return launch_prefill_dim<BF16, KT, VT>(a, stream);
  if (a.q_dtype == PKV_F16) return launch_prefill_dim<F16, KT, VT>(a, stream);
  return PKV_ERR_UNSUPPORTED;
}

}  // namespace

int launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  switch (a.cache_dtype) {
    case PKV_FP8_E4M3: return launch_prefill_quantised<FP8, FP8>(a, stream);
    case PKV_FP8_E5M2: return launch_prefill_quantised<BF8, BF8>(a, stream);
    case PKV_INT8_INT4: return launch_prefill_quantised<I8, I4>(a, stream);
    default: break;
  }
  if (a.q_dtype != a.cache_dtype) return PKV_ERR_UNSUPPORTED;
  if (a.q_dtype == PKV_BF16) return launch_prefill_dim<BF16, BF16, BF16>(a, stream);
  if (a.q_dtype == PKV_F16) return launch_prefill_dim<F16, F16, F16>(a, stream);
  return PKV_ERR_UNSUPPORTED;
}

}  // namespace pkv
