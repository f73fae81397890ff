// Paged decode attention for gfx950: one query token per sequence attends
// over its cached K/V, read through the block table.
//
// Pages: softmax(Q K^T / sqrt(d_k)) V ("企业官网建设流程全解析" §1.2); the query
// attends to every cached token, its own included (§3.2-3.3 of the same
// page); several query heads share one KV head (§2.2 of the same page); the
// block table translates logical blocks to physical blocks and only the
// sequence's own blocks are read ("KV Cache 和 vLLM" §3.2); decode time goes
// to moving the cached K/V out of device memory, so bandwidth sets the speed
// ("KV Cache 和 vLLM" §2.3).
//
// Design (MI355X / CDNA4):
//  * Workgroup = 4 waves for one (sequence, KV head, partition).  A partition
//    is a run of logical positions; wave w takes the partition's 16-token
//    tiles w, w+4, w+8, ... (a tile is 16 rows of one (block, KV head): a
//    16-token block is one tile, a 32-token block two).  Each wave streams
//    its tiles straight from HBM into registers with 16-byte loads, several
//    tiles in flight, and keeps its own online-softmax state; the 4 states
//    merge through LDS at the end.
//  * The whole GQA group is served from one read of each K/V tile: the
//    group's query heads are the 16 columns of an MFMA tile (columns >= G
//    repeat the first head and are discarded), so one 16x16 MFMA output
//    holds 16 tokens x 16 heads.
//      S^T = K_tile (16 tok x D) * Q^T (D x 16 heads)    [16x16x32 MFMA]
//      O  += P (16 heads x 16 tok) * V_tile (16 tok x D) [16x16x16 MFMA]
//    The S^T accumulator layout (lane = head + 16*(token/4), reg = token%4)
//    is exactly the A-operand layout P needs, so no transpose is done.  The
//    contraction index of each MFMA may be permuted freely as long as both
//    operands use the same permutation: each lane loads a contiguous 1/4 of
//    a K row, and 4 V rows x D/16 contiguous columns.
//  * Quantised codes: e4m3 and e5m2 convert exactly to bf16/f16 in
//    hardware, int8 through float; int4 enters the MFMA as MAGIC + x + 8 and
//    a second accumulator removes the offset.  The per-token scales multiply
//    the scores (k) and the probabilities (v), never each element.
//  * The running maximum of a head moves only when a tile's maximum exceeds
//    it by more than 2^8, so the output is rescaled about once per wave.
//  * Probabilities enter the P*V MFMA as a hi + lo pair of 16-bit values, so
//    P carries ~16 significant bits while the MFMA still accumulates in fp32.
//    With a quantised V pool every code converts exactly to f16, and P
//    rounded once to f16 (11 significant bits) takes one MFMA per column
//    tile instead of two.
//  * Long sequences split into partitions, each with its state (max, sum,
//    unnormalised output), merged with the log-sum-exp formula.  Up to two
//    partitions per sequence (four in launches of at most 512 workgroups)
//    the merge happens in this launch: the last workgroup of a (sequence,
//    KV head) to finish, told so by an arrival counter, reads the others'
//    states (stored and loaded at device scope, past the XCD caches - no
//    fences) and writes the output.  With more partitions, or in the split
//    form, every state goes to the workspace
//    (an empty partition writes max -inf) and a second launch merges them;
//    the two places share one merge routine and give the same bits.

#include <limits.h>
#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace pkv {

#ifndef PKV_DECODE_NATK
#define PKV_DECODE_NATK 1     // 16-bit K in the MFMA's contraction order (0: permuted)
#endif
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 4     // waves per workgroup
#endif
#ifndef PKV_DECODE_PIPE
#define PKV_DECODE_PIPE 2      // blocks in flight per wave, 16-bit caches
#endif
#ifndef PKV_DECODE_PIPE_Q
#define PKV_DECODE_PIPE_Q 2    // blocks in flight per wave, quantised caches
#endif
#ifndef PKV_DECODE_NT
#define PKV_DECODE_NT 0        // non-temporal K/V loads (measured slower: off)
#endif
#ifndef PKV_DECODE_LDS
#define PKV_DECODE_LDS 0       // K/V tiles staged in LDS by direct loads (measured against registers: off)
#endif
#ifndef PKV_DECODE_LDS_BUFS
#define PKV_DECODE_LDS_BUFS 3  // tiles in flight per wave when staged in LDS
#endif
#ifndef PKV_DECODE_PV_X32
#define PKV_DECODE_PV_X32 0    // hi and lo probabilities in one 16x16x32 MFMA (measured no faster: off)
#endif
#ifndef PKV_DECODE_PV_F16Q
#define PKV_DECODE_PV_F16Q 1   // quantised V: P rounded once to f16, one MFMA per column tile
#endif
#ifndef PKV_DECODE_I8_MFMA
#define PKV_DECODE_I8_MFMA 1   // int8 K: Q.K^T on int8 MFMA against two digit planes of the query
#endif
#ifndef PKV_DECODE_QK_VALU
#define PKV_DECODE_QK_VALU 0   // Q.K^T on vector ALU dot products (measured against MFMA: off)
#endif
constexpr int kWaves = PKV_DECODE_WAVES;
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxGroup = 16;
constexpr int kMaxOrderSeqs = PKV_MAX_ORDER_SEQS;   // longest-first order: batches of at most this many
constexpr int kOrderThreads = 1024;
static_assert(kMaxRankSeqs <= kThreads, "one ranking thread per sequence");
constexpr int kMaxPartitionBlocks = PKV_MAX_PARTITION_TOKENS / kTileTokens;
constexpr float kLog2e = 1.4426950408889634f;

// ---- raw register loads -------------------------------------------------------

template <int N>
struct Words {
  uint32_t w[N];
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <typename T, bool NT>
__device__ __forceinline__ T load_vec(const uint8_t* p) {
  const T* src = reinterpret_cast<const T*>(p);
  if constexpr (NT) return __builtin_nontemporal_load(src);
  else return *src;
}

template <int N, bool NT>
__device__ __forceinline__ void load_words(Words<N>& dst, const uint8_t* p) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      u32x4_t v = load_vec<u32x4_t, NT>(p + 16 * i);
      dst.w[4 * i + 0] = v[0];
      dst.w[4 * i + 1] = v[1];
      dst.w[4 * i + 2] = v[2];
      dst.w[4 * i + 3] = v[3];
    }
  } else if constexpr (N == 2) {
    u32x2_t v = load_vec<u32x2_t, NT>(p);
    dst.w[0] = v[0];
    dst.w[1] = v[1];
  } else {
    static_assert(N == 1, "unsupported load width");
    dst.w[0] = load_vec<uint32_t, NT>(p);
  }
}

// ---- cross-row reductions (a "row" is 16 lanes) ------------------------------------
// Max / sum over the 4 lanes c, c+16, c+32, c+48 of each column c, with the
// gfx950 row-swap permutes (VALU, no LDS round trip).
__device__ __forceinline__ float col_max4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Pack two fp32 values into a word of two 16-bit values of type QT (RNE).
template <typename QT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (std::is_same<QT, BF16>::value) {
    bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    half2_t v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, v);
  }
}
template <typename QT>
__device__ __forceinline__ float lo16_to_f32(uint32_t w) {
  if constexpr (std::is_same<QT, BF16>::value) return __uint_as_float(w << 16);
  else return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
template <typename QT>
__device__ __forceinline__ float hi16_to_f32(uint32_t w) {
  if constexpr (std::is_same<QT, BF16>::value) return __uint_as_float(w & 0xffff0000u);
  else return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// ---- per-flavour geometry -------------------------------------------------------
//   QT: query/output type (F32, F16, BF16).  KT, VT: element types of the K
//   and V pools - the query type itself, or a quantised format (FP8 e4m3,
//   BF8 e5m2, I8, I4) with a float32 scale per (token, head).
template <typename QT, typename KT, typename VT, int D>
struct Geo {
  static constexpr int qes = QT::bytes;
  static constexpr int kRowBytes = D * KT::bits / 8;
  static constexpr int vRowBytes = D * VT::bits / 8;
  static constexpr int kLaneBytes = kRowBytes / 4;      // 1/4 of a K row per lane
  static constexpr int kWords = kLaneBytes / 4;
  static constexpr int qWords = D / 4 * qes / 4;        // Q words per lane
  static constexpr int DC = D / 16;                     // V columns per lane = P*V tiles
  static constexpr int vLaneBytes = DC * VT::bits / 8;  // one V row's share per lane (2..32 bytes)
  static constexpr int vWords = vLaneBytes < 4 ? 1 : vLaneBytes / 4;
  static constexpr int kTileBytes = kTileTokens * kRowBytes;
  static constexpr int vTileBytes = kTileTokens * vRowBytes;
};

template <typename QT, typename KT, typename VT, int D>
struct BlockRegs {
  using G = Geo<QT, KT, VT, D>;
  Words<G::kWords> k;
  Words<G::vWords> v[4];      // rows 4j..4j+3
  float4 ks, vs;              // scales of tokens 4j..4j+3 (quantised pools)
};

// One V row's share: vLaneBytes bytes (a 16-bit load for 2 bytes).
template <int NB>
__device__ __forceinline__ void load_vrow(Words<(NB < 4 ? 1 : NB / 4)>& dst, const uint8_t* p) {
  if constexpr (NB == 2) dst.w[0] = *reinterpret_cast<const uint16_t*>(p);
  else load_words<NB / 4, PKV_DECODE_NT != 0>(dst, p);
}

// ---- element conversions to the 16-bit MFMA operand type of QT ----------------
// Four 8-bit codes (one word) -> two words of four 16-bit values, in element
// order; every conversion is exact (e4m3, e5m2 and int8 values all fit).
template <typename QT, typename ET>
__device__ __forceinline__ uint2 conv8(uint32_t src) {
  uint2 r;
  if constexpr (std::is_same<ET, FP8>::value) {
    if constexpr (std::is_same<QT, BF16>::value) {
      r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 1.0f, false));
      r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 1.0f, true));
    } else {
      r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, 1.0f, false));
      r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, 1.0f, true));
    }
  } else if constexpr (std::is_same<ET, BF8>::value) {
    if constexpr (std::is_same<QT, BF16>::value) {
      r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(src, 1.0f, false));
      r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(src, 1.0f, true));
    } else {
      r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(src, 1.0f, false));
      r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(src, 1.0f, true));
    }
  } else {
    static_assert(std::is_same<ET, I8>::value, "8-bit format");
    const float f0 = static_cast<float>(static_cast<int8_t>(src & 0xffu));
    const float f1 = static_cast<float>(static_cast<int8_t>((src >> 8) & 0xffu));
    const float f2 = static_cast<float>(static_cast<int8_t>((src >> 16) & 0xffu));
    const float f3 = static_cast<float>(static_cast<int8_t>(src >> 24));
    r.x = pack2<QT>(f0, f1);
    r.y = pack2<QT>(f2, f3);
  }
  return r;
}

// K operand words of MFMA i (8 contraction elements) from the lane's K words.
template <typename QT, typename KT, int D>
__device__ __forceinline__ uint4 k_operand(const Words<Geo<QT, KT, KT, D>::kWords>& k, int i) {
  if constexpr (KT::bits == 16) {
    return make_uint4(k.w[4 * i], k.w[4 * i + 1], k.w[4 * i + 2], k.w[4 * i + 3]);
  } else {
    const uint2 lo = conv8<QT, KT>(k.w[2 * i]);
    const uint2 hi = conv8<QT, KT>(k.w[2 * i + 1]);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// ---- QK^T on MFMA -----------------------------------------------------------------
template <typename QT, typename KT, int D>
__device__ __forceinline__ float4_t qk_tile(const Words<Geo<QT, KT, KT, D>::kWords>& k,
                                            const Words<Geo<QT, KT, KT, D>::qWords>& q) {
  float4_t s = {0.f, 0.f, 0.f, 0.f};
  if constexpr (std::is_same<KT, F32>::value) {
#pragma unroll
    for (int i = 0; i < D / 4; ++i)
      s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.w[i]), __uint_as_float(q.w[i]), s, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const uint4 av = k_operand<QT, KT, D>(k, i);
      const uint4 bv = make_uint4(q.w[4 * i], q.w[4 * i + 1], q.w[4 * i + 2], q.w[4 * i + 3]);
      if constexpr (std::is_same<QT, BF16>::value)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                    __builtin_bit_cast(bf16x8_t, bv), s, 0, 0, 0);
      else
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av),
                                                   __builtin_bit_cast(half8_t, bv), s, 0, 0, 0);
    }
  }
  return s;
}

// ---- Q.K^T on int8 MFMA (int8 K pools) ----------------------------------------------
// The query of each head is taken as a 15-bit fixed-point integer v = q times
// 2^(14 - e), where |q| < 2^e over the head's D values, written in two signed
// base-256 digits, v = 256 d1 + d0.  A 16-bit query value is exact there when
// it is at least 2^-6 (bf16) or 2^-3 (f16) of the head's largest; smaller ones
// are rounded, by at most 2^-14 of the largest.  Each digit plane meets the
// int8 codes of the K tile in exact int32 MFMAs, so the codes need no
// conversion, and the two dot products combine exactly in int32.
typedef int i32x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct QDigits {
  static constexpr int kWords = D / 16;    // a lane's quarter of a head: D/4 bytes
  uint32_t w[2][kWords];                   // planes d0, d1
};

// Digits of this lane's D/4 query values (16-bit words of QT, two per word);
// returns the factor 2^(e - 14) that takes the integer dot product back to
// q.K, or NaN when the head's query is not finite.
template <typename QT, int D, int QW>
__device__ __forceinline__ float q_digits(const Words<QW>& q, QDigits<D>& qd) {
  static_assert(QW * 2 == D / 4, "two query values per word");
  float qf[D / 4];
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    qf[2 * i] = lo16_to_f32<QT>(q.w[i]);
    qf[2 * i + 1] = hi16_to_f32<QT>(q.w[i]);
    mx = fmaxf(mx, fmaxf(fabsf(qf[2 * i]), fabsf(qf[2 * i + 1])));
  }
  mx = col_max4(mx);                       // the head's largest |q| (4 lanes hold it)
  const bool finite = mx <= 3.0e38f;
  int e = 0;
  if (mx > 0.f && finite) frexpf(mx, &e);  // mx = f 2^e, f in [0.5, 1)
  const float up = ldexpf(1.f, 14 - e);
#pragma unroll
  for (int w = 0; w < D / 16; ++w) {
    uint32_t p0 = 0u, p1 = 0u;
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
      const int v = finite ? static_cast<int>(rintf(qf[4 * w + bt] * up)) : 0;   // |v| <= 2^14
      const int d0 = ((v + 128) & 255) - 128;
      const int d1 = (v - d0) >> 8;                                              // |d1| <= 64
      p0 |= static_cast<uint32_t>(d0 & 255) << (8 * bt);
      p1 |= static_cast<uint32_t>(d1 & 255) << (8 * bt);
    }
    qd.w[0][w] = p0;
    qd.w[1][w] = p1;
  }
  return finite ? ldexpf(1.f, e - 14) : __builtin_nanf("");
}

template <int D, int KW>
__device__ __forceinline__ float4_t qk_tile_i8(const Words<KW>& k, const QDigits<D>& qd) {
  static_assert(KW == D / 16, "a lane's quarter of an int8 K row");
  i32x4_t acc[2];
#pragma unroll
  for (int pl = 0; pl < 2; ++pl) {
    acc[pl] = i32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < KW / 4; ++m) {
      const i32x4_t kv = {static_cast<int>(k.w[4 * m]), static_cast<int>(k.w[4 * m + 1]),
                          static_cast<int>(k.w[4 * m + 2]), static_cast<int>(k.w[4 * m + 3])};
      const i32x4_t qv = {static_cast<int>(qd.w[pl][4 * m]), static_cast<int>(qd.w[pl][4 * m + 1]),
                          static_cast<int>(qd.w[pl][4 * m + 2]), static_cast<int>(qd.w[pl][4 * m + 3])};
      acc[pl] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kv, qv, acc[pl], 0, 0, 0);
    }
  }
  float4_t s;
#pragma unroll
  for (int r = 0; r < 4; ++r) s[r] = static_cast<float>(acc[1][r] * 256 + acc[0][r]);   // |.| < 2^29
  return s;
}

// ---- Q.K^T on the vector ALU (build option PKV_DECODE_QK_VALU) -------------
// For groups of up to 4 heads: lane (c, j) holds row c, quarter j of the K
// tile and the same quarter of each head's query; it forms the 4 partial dot
// products with packed 16-bit dot instructions, the 4 lanes of a row sum them
// with row-swap permutes, and the wave's LDS scratch turns "token c, all
// heads" into the MFMA output layout (lane = head + 16 * (token / 4), value r
// = token 4j + r) that the softmax and P.V steps take.
template <typename QT>
__device__ __forceinline__ float dot2acc(uint32_t a, uint32_t b, float c) {
  if constexpr (std::is_same<QT, BF16>::value)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

template <typename QT, typename KT, int D>
__device__ __forceinline__ float4_t qk_tile_valu(const Words<Geo<QT, KT, KT, D>::kWords>& k,
                                                 const uint32_t (&qv)[4][D / 8], float* sm_st, int c, int j) {
  uint32_t kw[D / 8];                       // this lane's 32 K elements as 16-bit pairs, in order
  if constexpr (KT::bits == 16) {
#pragma unroll
    for (int i = 0; i < D / 8; ++i) kw[i] = k.w[i];
  } else {
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
      const uint2 c2 = conv8<QT, KT>(k.w[m]);
      kw[2 * m] = c2.x;
      kw[2 * m + 1] = c2.y;
    }
  }
  float acc[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    acc[h] = 0.f;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) acc[h] = dot2acc<QT>(kw[i], qv[h][i], acc[h]);
    acc[h] = col_sum4(acc[h]);
  }
  if (j == 0) {
#pragma unroll
    for (int h = 0; h < 4; ++h) sm_st[h * 16 + c] = acc[h];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float4_t s = {0.f, 0.f, 0.f, 0.f};
  if (c < 4) {
    const float4 v = *reinterpret_cast<const float4*>(sm_st + c * 16 + 4 * j);
    s[0] = v.x;
    s[1] = v.y;
    s[2] = v.z;
    s[3] = v.w;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();           // the next tile's writes follow these reads
  return s;
}

template <typename QT>
__device__ __forceinline__ float4_t mfma16(uint2 a, uint2 b, float4_t c) {
  if constexpr (std::is_same<QT, BF16>::value)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a),
                                                      __builtin_bit_cast(short4_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a),
                                                 __builtin_bit_cast(half4_t, b), c, 0, 0, 0);
}

// Build option PKV_DECODE_PV_X32: the hi and lo halves of the probabilities
// in one 16x16x32 MFMA (A = hi and lo of tokens 4j..4j+3, B = the same 4 V
// values twice) instead of two 16x16x16 ones; on gfx950 the one takes as long
// as each of the two, but the repeated B operand costs two register copies.
template <typename QT>
__device__ __forceinline__ float4_t mfma_hilo(uint4 p_hilo, uint2 b, float4_t c) {
  const uint4 bb = make_uint4(b.x, b.y, b.x, b.y);
  if constexpr (std::is_same<QT, BF16>::value)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, p_hilo),
                                                   __builtin_bit_cast(bf16x8_t, bb), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, p_hilo),
                                                  __builtin_bit_cast(half8_t, bb), c, 0, 0, 0);
}

// ---- P*V on MFMA -----------------------------------------------------------------
// p[r]: probability (times the V scale of a quantised pool) of token 4j+r for
// head column c.
// INT4 values enter the MFMA with an offset: the code x (two's complement,
// |x| <= 8) becomes the 16-bit value MAGIC + (x + 8) by one AND-OR of its
// nibble into the mantissa of MAGIC (128 in bf16, 1024 in f16, where the
// 16-bit format steps by 1), so a word of 8 codes takes 8 instructions
// instead of an integer-to-float conversion per code.  The offset is taken
// back by a second accumulator fed the same probabilities against the
// constant MAGIC + 8: O = P (V + off) - P off.
template <typename QT>
struct I4Magic {
  static constexpr uint32_t pair = std::is_same<QT, BF16>::value ? 0x43004300u : 0x64006400u;   // MAGIC, MAGIC
  static constexpr uint32_t off = std::is_same<QT, BF16>::value ? 0x43084308u : 0x64086408u;    // MAGIC + 8
};

template <typename QT, typename VT, int D>
__device__ __forceinline__ void pv_tile(const float (&p)[4], const Words<Geo<QT, VT, VT, D>::vWords> (&v)[4],
                                        float4_t (&o)[D / 16], float4_t& ocorr) {
  using G = Geo<QT, VT, VT, D>;
  if constexpr (std::is_same<VT, F32>::value) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int nt = 0; nt < G::DC; ++nt)
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[r], __uint_as_float(v[r].w[nt]), o[nt], 0, 0, 0);
  } else {
    // PT: the 16-bit type of the P*V operands.  Probabilities are split in a
    // hi and a lo half (P keeps ~16 significant bits), except for quantised
    // V (build option PKV_DECODE_PV_F16Q, on): every code converts exactly
    // to f16, and P rounded once to f16 keeps 11 bits in one MFMA per column
    // tile.
    constexpr bool kOne = PKV_DECODE_PV_F16Q && VT::quantised;
    using PT = typename std::conditional<kOne, F16, QT>::type;
    const uint32_t h01 = pack2<PT>(p[0], p[1]);
    const uint32_t h23 = pack2<PT>(p[2], p[3]);
    const uint32_t l01 = kOne ? 0u : pack2<PT>(p[0] - lo16_to_f32<PT>(h01), p[1] - hi16_to_f32<PT>(h01));
    const uint32_t l23 = kOne ? 0u : pack2<PT>(p[2] - lo16_to_f32<PT>(h23), p[3] - hi16_to_f32<PT>(h23));
    const uint2 phi = make_uint2(h01, h23);
    const uint2 plo = make_uint2(l01, l23);
    const uint4 phl = make_uint4(h01, h23, l01, l23);
    auto acc = [&](float4_t& o_, uint2 b_) {
      if constexpr (kOne) {
        o_ = mfma16<PT>(phi, b_, o_);
      } else if constexpr (PKV_DECODE_PV_X32) {
        o_ = mfma_hilo<PT>(phl, b_, o_);
      } else {
        o_ = mfma16<PT>(phi, b_, o_);
        o_ = mfma16<PT>(plo, b_, o_);
      }
    };
    static_assert(VT::bits == 16 || VT::bits == 8 || std::is_same<VT, I4>::value, "V format");
    if constexpr (std::is_same<VT, I4>::value) {
      // word k of row e: columns k (low half) and k + DC/2 (high half),
      // offset by MAGIC + 8; x ^ 8 is x + 8 for a 4-bit two's complement code
      uint32_t w16[4][G::DC / 2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = v[e].w[0] ^ (G::DC == 8 ? 0x88888888u : 0x00008888u);   // DC = 4: one 16-bit row
        const uint32_t s = G::DC == 8 ? u : (u | (u << 8));   // DC = 4: codes 2, 3 move to bits 16..23
#pragma unroll
        for (int k = 0; k < G::DC / 2; ++k) w16[e][k] = ((s >> (4 * k)) & 0x000F000Fu) | I4Magic<PT>::pair;
      }
#pragma unroll
      for (int nt = 0; nt < G::DC; ++nt) {
        const uint32_t sel = (nt >= G::DC / 2) ? 0x07060302u : 0x05040100u;
        const int wi = nt % (G::DC / 2);
        uint2 b;
        b.x = __builtin_amdgcn_perm(w16[1][wi], w16[0][wi], sel);
        b.y = __builtin_amdgcn_perm(w16[3][wi], w16[2][wi], sel);
        acc(o[nt], b);
      }
      acc(ocorr, make_uint2(I4Magic<PT>::off, I4Magic<PT>::off));
    } else if constexpr (VT::bits == 8 && !std::is_same<VT, I8>::value) {
      // fp8 codes: the bytes of rows (0, 1) and (2, 3) are interleaved first
      // - one byte permute per two columns - so that each pair conversion
      // gives an operand word (row 2r, row 2r + 1 of one column) directly
#pragma unroll
      for (int i = 0; i < G::vWords; ++i) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint32_t sel = half ? 0x07030602u : 0x05010400u;
          const uint2 c01 = conv8<PT, VT>(__builtin_amdgcn_perm(v[1].w[i], v[0].w[i], sel));
          const uint2 c23 = conv8<PT, VT>(__builtin_amdgcn_perm(v[3].w[i], v[2].w[i], sel));
          const int nt = 4 * i + 2 * half;
          acc(o[nt], make_uint2(c01.x, c23.x));
          acc(o[nt + 1], make_uint2(c01.y, c23.y));
        }
      }
    } else {
      // 16-bit words of the 4 V rows (int8 codes converted): element nt of
      // row e sits in word nt/2
      uint32_t w16[4][G::DC / 2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int i = 0; i < G::vWords; ++i) {
          if constexpr (VT::bits == 16) {
            w16[e][i] = v[e].w[i];
          } else {
            const uint2 c2 = conv8<PT, VT>(v[e].w[i]);
            w16[e][2 * i] = c2.x;
            w16[e][2 * i + 1] = c2.y;
          }
        }
      }
#pragma unroll
      for (int nt = 0; nt < G::DC; ++nt) {
        const uint32_t sel = (nt & 1) ? 0x07060302u : 0x05040100u;
        const int wi = nt >> 1;
        uint2 b;
        b.x = __builtin_amdgcn_perm(w16[1][wi], w16[0][wi], sel);
        b.y = __builtin_amdgcn_perm(w16[3][wi], w16[2][wi], sel);
        acc(o[nt], b);
      }
    }
  }
}

// ---- log-sum-exp merge of partition states ------------------------------------
// A partition's state is (m, l, acc): its maximum score (log2 units), the
// sum of 2^(s - m) over its tokens and the unnormalised output
// sum 2^(s - m) V.  The merged output is sum_p 2^(m_p - M) acc_p /
// sum_p 2^(m_p - M) l_p with M = max_p m_p ("企业官网建设流程全解析" §1.2:
// the softmax over the whole context, regrouped by partition).  States are
// taken in partition order, up to 8 at a time, with a running maximum.  Both
// places that merge - the merge kernel of the split form and the last
// partition of a sequence to finish in the one-call form - go through this
// function, so the two forms give the same bits.
template <int N>
struct MergeState {
  float M;
  float den;
  float num[N];
};

template <int N>
__device__ __forceinline__ MergeState<N> merge_begin() {
  MergeState<N> s;
  s.M = -INFINITY;
  s.den = 0.f;
#pragma unroll
  for (int e = 0; e < N; ++e) s.num[e] = 0.f;
  return s;
}

// n (<= 8) states of consecutive partitions; empty ones have m = -inf.
template <int N>
__device__ __forceinline__ void merge_chunk(MergeState<N>& s, const float (&mp)[8], const float (&lp)[8],
                                            const float (&ap)[8][N], int n) {
  float cm = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < n) cm = fmaxf(cm, mp[i]);
  const float M_new = fmaxf(s.M, cm);
  if (M_new == -INFINITY) return;
  const float r = __builtin_amdgcn_exp2f(s.M - M_new);   // 0 while s.M is still -inf
  s.den *= r;
#pragma unroll
  for (int e = 0; e < N; ++e) s.num[e] *= r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < n && mp[i] != -INFINITY) {
      const float f = __builtin_amdgcn_exp2f(mp[i] - M_new);
#pragma unroll
      for (int e = 0; e < N; ++e) s.num[e] = __builtin_fmaf(f, ap[i][e], s.num[e]);
      s.den = __builtin_fmaf(f, lp[i], s.den);
    }
  }
  s.M = M_new;
}

template <int N>
__device__ __forceinline__ float merge_result(const MergeState<N>& s, int e) {
  return s.den > 0.f ? s.num[e] / s.den : 0.f;
}

// Partition states written for another workgroup to read go straight to
// memory (agent-scope stores write through the XCD's L2) and are read back
// past the reader's caches (agent-scope loads), so the workgroups of one
// sequence may run on any XCDs.
__device__ __forceinline__ void store_agent2(float* p, float v0, float v1) {
  const uint64_t u = static_cast<uint64_t>(__float_as_uint(v0)) | (static_cast<uint64_t>(__float_as_uint(v1)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_agent2(const float* p) {
  const uint64_t u = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(u)), __uint_as_float(static_cast<uint32_t>(u >> 32)));
}

// ---- the main kernel ------------------------------------------------------------


// ---- longest-first order of a batch (once per call) ----------------------------
// order[r] = the sequence at position r when the batch is sorted by context
// length, longest first, ties by lower index: a permutation of
// 0..num_seqs-1 for any length values.  One workgroup sorts 64-bit keys
// (length above, complement of the index below) in LDS with a bitonic
// network; num_seqs <= kMaxOrderSeqs.
__global__ void __launch_bounds__(kOrderThreads) order_kernel(const int32_t* context_lens, int num_seqs,
                                                              int32_t* order) {
  __shared__ uint64_t key[kMaxOrderSeqs];
  int n = 1;
  while (n < num_seqs) n <<= 1;
  for (int t = threadIdx.x; t < n; t += kOrderThreads) {
    // padding sorts last: every real key is at least 2^32 - kMaxOrderSeqs
    key[t] = t < num_seqs ? (static_cast<uint64_t>(static_cast<uint32_t>(max(context_lens[t], 0))) << 32) |
                                (0xffffffffu - static_cast<uint32_t>(t))
                          : 0ull;
  }
  __syncthreads();
  for (int k = 2; k <= n; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int t = threadIdx.x; t < n; t += kOrderThreads) {
        const int u = t ^ jj;
        if (u > t) {
          const uint64_t x = key[t], y = key[u];
          // descending within blocks whose bit k is clear, ascending otherwise
          const bool desc = (t & k) == 0;
          if (desc ? x < y : x > y) {
            key[t] = y;
            key[u] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = threadIdx.x; r < num_seqs; r += kOrderThreads)
    order[r] = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(key[r]));
}

// Index of the sequence at position r of the longest-first order of the
// batch (ties: lower index first), which is a permutation of 0..num_seqs-1
// for any length values.  Every thread of the workgroup calls it;
// num_seqs <= kMaxRankSeqs.
__device__ __forceinline__ int seq_of_rank(const int32_t* context_lens, int num_seqs, int r, int tid,
                                           int* sm_len, int* sm_part, int* sm_pick) {
  // slots past num_seqs (to a multiple of 4) hold INT_MIN at index >= num_seqs:
  // never longer than a real entry, and never tied with a lower index
  const int padded = (num_seqs + 3) & ~3;
  for (int t = tid; t < padded; t += kThreads) sm_len[t] = t < num_seqs ? context_lens[t] : INT_MIN;
  __syncthreads();
  // a batch already longest first (equal lengths included) is its own order
  int unsorted = 0;
  for (int t = tid; t + 1 < num_seqs; t += kThreads) unsorted |= sm_len[t] < sm_len[t + 1] ? 1 : 0;
  if (!__syncthreads_or(unsorted)) return r;
  // rank of sequence t = entries before it in the order; thread (k, t)
  // counts over the k-th of nk slices of the batch
  const int nk = num_seqs <= kThreads / 4 ? 4 : (num_seqs <= kThreads / 2 ? 2 : 1);
  const int slice = ((padded / nk) + 3) & ~3;
  if (tid < nk * num_seqs) {
    const int t = tid % num_seqs;
    const int k = tid / num_seqs;
    const int lt = sm_len[t];
    int rank = 0;
    for (int u = k * slice; u < min(padded, (k + 1) * slice); u += 4) {
      const int4 lu = *reinterpret_cast<const int4*>(sm_len + u);
      rank += (lu.x > lt || (lu.x == lt && u < t)) ? 1 : 0;
      rank += (lu.y > lt || (lu.y == lt && u + 1 < t)) ? 1 : 0;
      rank += (lu.z > lt || (lu.z == lt && u + 2 < t)) ? 1 : 0;
      rank += (lu.w > lt || (lu.w == lt && u + 3 < t)) ? 1 : 0;
    }
    sm_part[tid] = rank;
  }
  __syncthreads();
  if (tid < num_seqs) {
    int rank = 0;
    for (int k = 0; k < nk; ++k) rank += sm_part[k * num_seqs + tid];
    if (rank == r) *sm_pick = tid;
  }
  __syncthreads();
  return *sm_pick;
}

// Quantised pools keep three waves per SIMD (their tiles are half as large,
// so the registers fit); 16-bit and fp32 pools take two.
template <typename KT>
constexpr int decode_min_blocks() { return KT::quantised && !PKV_DECODE_QK_VALU ? 3 : 2; }

// ORDER: workgroups take sequences longest first (a separate instance, so
// launches without the order carry none of its code or registers).
// MERGE: the instance of one-call launches that merge split sequences in the
// launch (counters given, more than one partition); the others - single
// partitions, the split form - are built without that code, which measured
// 3% faster on long split launches (the register allocation of the whole
// kernel changes with it).
template <typename QT, typename KT, typename VT, int D, int PIPE, bool ORDER, bool MERGE>
__global__ void __launch_bounds__(kThreads, decode_min_blocks<KT>()) paged_decode_kernel(DecodeArgs a) {
  using G = Geo<QT, KT, VT, D>;
  constexpr bool kQK = KT::quantised;
  constexpr bool kQV = VT::quantised;
  constexpr float kNegInf = -INFINITY;
  constexpr float kRebase = 8.0f;          // lazy-rescale threshold (log2 units)

  __shared__ float sm_m[kWaves][kMaxGroup];
  __shared__ float sm_l[kWaves][kMaxGroup];
  __shared__ float sm_o[kWaves][kMaxGroup][D];
  __shared__ int sm_ids[kMaxPartitionBlocks];
  __shared__ __attribute__((aligned(16))) float sm_st[kWaves][PKV_DECODE_QK_VALU ? 64 : 1];   // vector-ALU Q.K^T
  constexpr bool kLdsStage = PKV_DECODE_LDS && KT::bits == 16 && VT::bits == 16 && D == 128;
  __shared__ __attribute__((aligned(16))) uint8_t
      sm_ring[kLdsStage ? kWaves * PKV_DECODE_LDS_BUFS * 2 * Geo<QT, KT, VT, D>::kTileBytes : 16];

  const int P = a.num_partitions;
  const int part = blockIdx.x % P;
  const int g = (blockIdx.x / P) % a.num_kv_heads;
  const int tid = threadIdx.x;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int c = lane & 15;
  const int j = lane >> 4;

  const int PS = a.partition_size;
  const int tok0 = part * PS;
  const int blk0 = tok0 / kTileTokens;       // first 16-token unit of the partition
  const int pblk = PS / kTileTokens;         // units of a full partition
  const int rs = block_shift(a.block_size);
  const int max_units = a.max_blocks_per_seq << rs;
  constexpr int kLoads = (kMaxPartitionBlocks + kThreads - 1) / kThreads;

  // The workgroup's first loads do not depend on each other and are issued
  // together: the context length, the query, the block-table entries of a
  // full partition (read before the length is known; entries past the
  // sequence's end lie inside its table row and are never used) and the
  // fused write's slot.
  // Q^T operand: lane (head column c, k-group j) holds q[head c][j*D/4 ...).
  Words<G::qWords> qop;
  constexpr bool kValuQK = PKV_DECODE_QK_VALU && !std::is_same<KT, F32>::value;
  // 16-bit K meets the query in the MFMA's own contraction order: lane (c, j)
  // takes bytes 64i + 16j .. +15 of K row c for MFMA i (and the same elements
  // of its query), so each load instruction reads 64 contiguous bytes of each
  // of the tile's 16 rows.  The other formats take a contiguous quarter row
  // per lane, the contraction index permuted alike on both operands.
  constexpr bool kNatK = KT::bits == 16 && !kValuQK && !kLdsStage && PKV_DECODE_NATK;
  // vector-ALU form: quarter j of each of the group's (up to 4) queries
  uint32_t qv[4][D / 8];
  int phys[kLoads];
  int64_t new_slot = -1;   // fused cache write: the slot of this step's row
  auto first_loads = [&](int bb) {
    // Columns c >= group of the MFMA tile take a copy of the group's first
    // query: their scores, probabilities and output rows repeat column 0's
    // and are never stored.  (Zeroing them instead would make the wave wait
    // for the query loads before it issues the table loads.)
    const bool valid = c < group;
    const int64_t row0 = static_cast<int64_t>(bb) * a.num_q_heads + static_cast<int64_t>(g) * group;
    if constexpr (kNatK) {
      static_assert(G::qes == 2 && G::qWords == 4 * (D / 32), "16-bit query words, four per MFMA");
      const uint8_t* qr = static_cast<const uint8_t*>(a.q) + (row0 + (valid ? c : 0)) * D * G::qes + 16 * j;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) {
        const u32x4_t v = load_vec<u32x4_t, false>(qr + 64 * i);
        qop.w[4 * i + 0] = v[0];
        qop.w[4 * i + 1] = v[1];
        qop.w[4 * i + 2] = v[2];
        qop.w[4 * i + 3] = v[3];
      }
    } else {
      const uint8_t* qp =
          static_cast<const uint8_t*>(a.q) + ((row0 + (valid ? c : 0)) * D + j * (D / 4)) * G::qes;
      load_words<G::qWords, false>(qop, qp);
    }
    if constexpr (kValuQK) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        Words<D / 8> w;
        const uint8_t* qh = static_cast<const uint8_t*>(a.q) + ((row0 + min(h, group - 1)) * D + j * (D / 4)) * 2;
        load_words<D / 8, false>(w, qh);
#pragma unroll
        for (int i = 0; i < D / 8; ++i) qv[h][i] = h < group ? w.w[i] : 0u;
      }
    }
    const int32_t* table = a.block_tables + static_cast<int64_t>(bb) * a.max_blocks_per_seq;
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int u = blk0 + tid + k * kThreads;
      phys[k] = (tid + k * kThreads < pblk && u < max_units) ? table[u >> rs] : -1;
    }
    // (a scalar load, issued with the others: the workgroup that writes the
    // row then waits for one round trip fewer)
    if (a.slot_mapping != nullptr) new_slot = a.slot_mapping[bb];
  };

  // Workgroups are dispatched in index order.  When many of them share the
  // chip in turns (one partition per sequence), index r takes the r-th
  // longest sequence (the order kernel launched before this one wrote the
  // permutation), so long sequences start first and none starts last.  The
  // loads for sequence r go out together with the read of the order; they
  // are repeated for the sequence the order names only when it is another.
  int b = blockIdx.x / (P * a.num_kv_heads);
  int L = a.context_lens[b];
  first_loads(b);
  if constexpr (ORDER) {
    __shared__ __attribute__((aligned(16))) int sm_len[kMaxRankSeqs];
    __shared__ int sm_part[kThreads];
    __shared__ int sm_pick;
    int pick;
    if (a.num_seqs <= kMaxRankSeqs) {
      pick = seq_of_rank(a.context_lens, a.num_seqs, b, tid, sm_len, sm_part, &sm_pick);
    } else {
      pick = a.seq_order[b];
      if (pick < 0 || pick >= a.num_seqs) pick = b;   // (never: the order is a permutation)
    }
    if (pick != b) {
      b = pick;
      L = a.context_lens[b];
      first_loads(b);
    }
  }
  const int64_t out_row0 = static_cast<int64_t>(b) * a.num_q_heads + static_cast<int64_t>(g) * group;

  // The partition's tiles, staged in LDS once: a per-block table read from
  // global memory in front of the K/V loads would make the wave wait for
  // every load already in flight (vmcnt is in order), while LDS reads are
  // counted separately.  Unit u's entry is its tile index at KV head 0,
  // ((phys * Hkv) << rs) + (u & (2^rs - 1)), or -1 when the table names a
  // block outside the pool.
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const int i = tid + k * kThreads;
    const int u = blk0 + i;
    if (i < pblk)
      sm_ids[i] = (phys[k] >= 0 && phys[k] < a.num_blocks)
                      ? ((phys[k] * a.num_kv_heads) << rs) + (u & ((1 << rs) - 1))
                      : -1;
  }

  L = max(0, min(L, min(a.max_context_len, a.max_blocks_per_seq * a.block_size)));
  const int np_b = (L + PS - 1) / PS;         // non-empty partitions of this sequence
  if (part >= np_b) {
    if (P > 1 && a.counters == nullptr) {
      // split form: the merge kernel reads every partition slot, so mark
      // this one empty
      for (int h = tid; h < group; h += kThreads) {
        const int64_t prow = (out_row0 + h) * P + part;
        a.part_ml[2 * prow] = kNegInf;
        a.part_ml[2 * prow + 1] = 0.0f;
      }
    } else if (part == 0) {
      // an empty context gives a zero output row (merged in this launch, a
      // sequence's states come from its non-empty partitions only)
      for (int i = tid; i < group * D; i += kThreads) store_from_f32<QT>(a.out, out_row0 * D + i, 0.0f);
    }
    return;
  }
  const int tok1 = min(L, tok0 + PS);
  const int nblk = (tok1 - tok0 + kTileTokens - 1) / kTileTokens;
  float qk_scale = a.scale * kLog2e;   // scores in log2 units
  constexpr bool kIntQK = PKV_DECODE_I8_MFMA && std::is_same<KT, I8>::value && D % 64 == 0;
  QDigits<kIntQK ? D : 64> qd;
  if constexpr (kIntQK) qk_scale *= q_digits<QT, D>(qop, qd);

  const uint8_t* kbase = static_cast<const uint8_t*>(a.k_pool);
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v_pool);
  const int64_t k_lane = static_cast<int64_t>(c) * G::kRowBytes + j * (kNatK ? 16 : G::kLaneBytes);
  const int64_t v_lane = static_cast<int64_t>(4 * j) * G::vRowBytes + c * G::vLaneBytes;

  // Fused cache write: the workgroup whose partition holds the sequence's
  // last position writes this step's K and V rows for its KV head (wave 0:
  // K, wave 1: V) before anything is read; the barrier below makes the rows
  // visible to every wave of the workgroup.
  if (a.slot_mapping != nullptr && part == (L - 1) / PS && wave < 2) {
    const int64_t slot = new_slot;
    if (slot >= 0 && slot < static_cast<int64_t>(a.num_blocks) * a.block_size) {
      const int64_t dst_row = slot_row(slot, a.block_size, a.num_kv_heads, g);
      const int64_t src_row = static_cast<int64_t>(b) * a.num_kv_heads + g;
      auto write = [&](auto tag, const void* src, const void* pool_c, const float* scales_c) {
        using T = decltype(tag);
        void* pool = const_cast<void*>(pool_c);
        if constexpr (T::quantised) {
          float* scales = const_cast<float*>(scales_c);
          auto* p8 = static_cast<uint8_t*>(pool);
          if (a.src_dtype == PKV_F32) write_row_quant<F32, D, T>(src, src_row, p8, scales, dst_row, lane);
          else if (a.src_dtype == PKV_F16) write_row_quant<F16, D, T>(src, src_row, p8, scales, dst_row, lane);
          else write_row_quant<BF16, D, T>(src, src_row, p8, scales, dst_row, lane);
        } else {
          write_row_copy(src, src_row, pool, dst_row, D * T::bytes, lane);
        }
      };
      if (wave == 0) write(KT{}, a.k_new, a.k_pool, a.k_scale);
      else write(VT{}, a.v_new, a.v_pool, a.v_scale);
    }
  }
  const int g_tile = g << rs;
  __syncthreads();

  // Load one tile's K/V (and scales) for this lane.  Tiles of blocks outside
  // the pool are read from tile 0 and fully masked.
  auto load_block = [&](BlockRegs<QT, KT, VT, D>& r, int i, bool& ok) {
    int t0 = __builtin_amdgcn_readfirstlane(sm_ids[i]);
    ok = t0 >= 0;
    if (!ok) t0 = -g_tile;
    const int64_t tile = static_cast<int64_t>(t0) + g_tile;
    const uint8_t* kt = kbase + tile * G::kTileBytes;
    const uint8_t* vt = vbase + tile * G::vTileBytes;
    if constexpr (kNatK) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) {
        const u32x4_t v = load_vec<u32x4_t, PKV_DECODE_NT != 0>(kt + k_lane + 64 * i);
        r.k.w[4 * i + 0] = v[0];
        r.k.w[4 * i + 1] = v[1];
        r.k.w[4 * i + 2] = v[2];
        r.k.w[4 * i + 3] = v[3];
      }
    } else {
      load_words<G::kWords, PKV_DECODE_NT>(r.k, kt + k_lane);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) load_vrow<G::vLaneBytes>(r.v[e], vt + v_lane + e * G::vRowBytes);
    if constexpr (kQK) r.ks = *reinterpret_cast<const float4*>(a.k_scale + tile * kTileTokens + 4 * j);
    if constexpr (kQV) r.vs = *reinterpret_cast<const float4*>(a.v_scale + tile * kTileTokens + 4 * j);
  };

  float m = kNegInf;          // running max of head column c (log2 units)
  float l = 0.0f;             // this lane's share of the running sum
  float4_t o[G::DC];
#pragma unroll
  for (int nt = 0; nt < G::DC; ++nt) o[nt] = {0.f, 0.f, 0.f, 0.f};
  float4_t ocorr = {0.f, 0.f, 0.f, 0.f};     // INT4 V: P times the operand offset

  auto compute_block = [&](BlockRegs<QT, KT, VT, D>& r, int i, bool ok) {
    const int base = tok0 + i * kTileTokens;   // logical position of the block's token 0
    float4_t s;
    if constexpr (kValuQK) {
      if (group <= 4) s = qk_tile_valu<QT, KT, D>(r.k, qv, &sm_st[wave][0], c, j);
      else s = qk_tile<QT, KT, D>(r.k, qop);
    } else if constexpr (kIntQK) {
      s = qk_tile_i8<D>(r.k, qd);
    } else {
      s = qk_tile<QT, KT, D>(r.k, qop);
    }
    float sc[4] = {s[0], s[1], s[2], s[3]};
    float ksc[4] = {1.f, 1.f, 1.f, 1.f};
    float vsc[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (kQK) {
      ksc[0] = r.ks.x; ksc[1] = r.ks.y; ksc[2] = r.ks.z; ksc[3] = r.ks.w;
    }
    if constexpr (kQV) {
      vsc[0] = r.vs.x; vsc[1] = r.vs.y; vsc[2] = r.vs.z; vsc[3] = r.vs.w;
    }
    bool valid[4];
    const bool partial = !ok || base + kTileTokens > tok1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      valid[t] = ok && (base + 4 * j + t < tok1);
      float x = sc[t] * ksc[t] * qk_scale;
      sc[t] = valid[t] ? x : kNegInf;
    }
    if (partial) {
      // zero V rows of masked tokens (their slots may hold any bits)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!valid[e]) {
#pragma unroll
          for (int w = 0; w < G::vWords; ++w) r.v[e].w[w] = 0u;
          vsc[e] = 0.f;
        }
      }
    }
    // Lazy rescale: the running max m of a head only moves when the tile's
    // max exceeds it by more than kRebase (log2 units), so p = 2^(s - m)
    // stays below 2^kRebase and O and l are rescaled only then - for random
    // scores about once per wave.  O and l always share one m, so the final
    // O / l is the same function of the scores.
    const float bm = col_max4(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    const bool grow = bm > m + kRebase;       // also true for the first valid tile (m = -inf)
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? bm : m;
      const float alpha = (m_new == kNegInf || !grow) ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
      m = m_new;
      // rescale O: lane (c, j) reg r holds head row 4j+r; alpha of head h
      // sits in lane h (all lanes of column h agree).  With at most 4 heads
      // per group only rows 0..3 (lanes j == 0) matter, and the four factors
      // are wave-uniform: read them into scalar registers.
      float ar[4];
      if (group <= 4) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) ar[rr] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(alpha), rr));
      } else {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) ar[rr] = __shfl(alpha, 4 * j + rr, kWave);
      }
#pragma unroll
      for (int nt = 0; nt < G::DC; ++nt) {
        o[nt][0] *= ar[0];
        o[nt][1] *= ar[1];
        o[nt][2] *= ar[2];
        o[nt][3] *= ar[3];
      }
      if constexpr (std::is_same<VT, I4>::value) {
        ocorr[0] *= ar[0];
        ocorr[1] *= ar[1];
        ocorr[2] *= ar[2];
        ocorr[3] *= ar[3];
      }
    }
    float p[4];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float e = valid[t] ? __builtin_amdgcn_exp2f(sc[t] - m) : 0.0f;
      psum += e;
      p[t] = e * vsc[t];
    }
    l += psum;
    pv_tile<QT, VT, D>(p, r.v, o, ocorr);
  };

  // PIPE blocks in flight per wave: block i is computed while blocks
  // i+4, ..., i+4*(PIPE-1) are being loaded.
  if constexpr (kLdsStage) {
    // Build option PKV_DECODE_LDS (16-bit caches, head_dim 128): each wave
    // streams its tiles into a ring of kBufs LDS slots with direct loads
    // (global_load_lds, no registers held for the tiles in flight), then reads
    // its MFMA operands from LDS.  Within a tile row the 16-byte chunks are
    // XOR-swizzled by the row so that the operand reads (16 rows at one
    // column, or one row's 4 columns) touch distinct banks.
    constexpr int kBufs = PKV_DECODE_LDS_BUFS;
    constexpr int kCh = 16;                                   // 16-byte chunks per 256-byte row
    constexpr int kInsts = kTileTokens * kCh / kWave;         // direct loads per tile (K or V): 4
    uint8_t* ring = sm_ring + wave * kBufs * 2 * G::kTileBytes;
    int lane_off[kInsts];
#pragma unroll
    for (int t = 0; t < kInsts; ++t) {
      const int pos = t * kWave + lane;                       // chunk position in the LDS tile
      const int row = pos / kCh;
      lane_off[t] = row * G::kRowBytes + 16 * ((pos % kCh) ^ (row & 15));
    }
    auto dma = [&](int slot, int i) {
      int t0 = __builtin_amdgcn_readfirstlane(sm_ids[i]);
      if (t0 < 0) t0 = -g_tile;
      const int64_t tile = static_cast<int64_t>(t0) + g_tile;
      uint8_t* kd = ring + slot * 2 * G::kTileBytes;
      uint8_t* vd = kd + G::kTileBytes;
#pragma unroll
      for (int t = 0; t < kInsts; ++t) {
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(kbase + tile * G::kTileBytes + lane_off[t]),
            (__attribute__((address_space(3))) void*)(kd + t * kWave * 16), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(vbase + tile * G::vTileBytes + lane_off[t]),
            (__attribute__((address_space(3))) void*)(vd + t * kWave * 16), 16, 0, 0);
      }
    };
    auto chunk = [&](const uint8_t* base, int row, int col) {
      return *reinterpret_cast<const u32x4_t*>(base + row * G::kRowBytes + 16 * (col ^ (row & 15)));
    };
    if (wave < nblk) {
      const int last = wave + kWaves * ((nblk - 1 - wave) / kWaves);
#pragma unroll
      for (int st = 0; st < kBufs - 1; ++st) dma(st, min(wave + st * kWaves, last));
      int slot = 0;
      for (int i = wave; i < nblk; i += kWaves) {
        dma((slot + kBufs - 1) % kBufs, min(i + (kBufs - 1) * kWaves, last));
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kBufs - 1) * 2 * kInsts) : "memory");
        const uint8_t* kd = ring + slot * 2 * G::kTileBytes;
        const uint8_t* vd = kd + G::kTileBytes;
        BlockRegs<QT, KT, VT, D> r;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4_t x = chunk(kd, c, 4 * j + q);          // K row c, quarter j
          r.k.w[4 * q] = x[0];
          r.k.w[4 * q + 1] = x[1];
          r.k.w[4 * q + 2] = x[2];
          r.k.w[4 * q + 3] = x[3];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const u32x4_t x = chunk(vd, 4 * j + e, c);          // V row 4j+e, columns 8c..8c+7
          r.v[e].w[0] = x[0];
          r.v[e].w[1] = x[1];
          r.v[e].w[2] = x[2];
          r.v[e].w[3] = x[3];
        }
        compute_block(r, i, __builtin_amdgcn_readfirstlane(sm_ids[i]) >= 0);
        slot = slot + 1 == kBufs ? 0 : slot + 1;
      }
    }
  } else if (wave < nblk) {
    // The wave's tiles are wave + k * kWaves, k < n; tile k lives in slot
    // k % PIPE.  Full rounds load only real tiles; the last 1 .. 2*PIPE-1
    // tiles run as straight-line code for their count, so no load goes past
    // the wave's last tile (a re-read there would hold the wave's end for a
    // memory round trip) and every wait still covers just the tile in use.
    const int n = (nblk - 1 - wave) / kWaves + 1;
    auto tile = [&](int k) { return wave + k * kWaves; };
    BlockRegs<QT, KT, VT, D> r[PIPE];
    bool ok[PIPE];
#pragma unroll
    for (int st = 0; st < PIPE; ++st) load_block(r[st], tile(min(st, n - 1)), ok[st]);
    int k = 0;
    for (; k + 2 * PIPE <= n; k += PIPE) {
#pragma unroll
      for (int st = 0; st < PIPE; ++st) {
        compute_block(r[st], tile(k + st), ok[st]);
        load_block(r[st], tile(k + st + PIPE), ok[st]);
      }
    }
    auto finish = [&](auto rem_c) {
      constexpr int R = decltype(rem_c)::value;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        compute_block(r[q % PIPE], tile(k + q), ok[q % PIPE]);
        if (q + PIPE < R) load_block(r[q % PIPE], tile(k + q + PIPE), ok[q % PIPE]);
      }
    };
    static_assert(PIPE >= 1 && PIPE <= 3, "tail cases below cover 2 * PIPE - 1 tiles");
    switch (n - k) {   // 1 .. 2 * PIPE - 1
      case 1: finish(std::integral_constant<int, 1>{}); break;
      case 2: if constexpr (PIPE >= 2) finish(std::integral_constant<int, 2>{}); break;
      case 3: if constexpr (PIPE >= 2) finish(std::integral_constant<int, 3>{}); break;
      case 4: if constexpr (PIPE >= 3) finish(std::integral_constant<int, 4>{}); break;
      case 5: if constexpr (PIPE >= 3) finish(std::integral_constant<int, 5>{}); break;
      default: break;
    }
  }

  if constexpr (std::is_same<VT, I4>::value) {
    // every column of a head row carries the same offset term
#pragma unroll
    for (int nt = 0; nt < G::DC; ++nt) {
      o[nt][0] -= ocorr[0];
      o[nt][1] -= ocorr[1];
      o[nt][2] -= ocorr[2];
      o[nt][3] -= ocorr[3];
    }
  }

  // ---- merge the waves' states ----
  // A sequence split over several partitions and merged in this launch: its
  // workgroups count their arrival on the sequence's (KV head's) counter;
  // the request goes out now and its reply is read after the wave merge.
  // Loads still in flight (the LDS-staged build's, or a short partition's
  // repeated first loads) are drained first: the wait counter is in order,
  // and a wait for them would also wait for whatever was issued after them,
  // the arrival reply among it.
  const bool merge_here = MERGE && np_b > 1;
  if (merge_here) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int* const cnt = merge_here ? a.counters + 2 * (static_cast<int64_t>(b) * a.num_kv_heads + g) : nullptr;
  // (an increment the compiler leaves as one atomic: an add would go
  // through its wave-level combining, whose result it waits for at once)
  int arrival = 0;
  if (merge_here && tid == 0)
    arrival = static_cast<int>(__builtin_amdgcn_atomic_inc32(reinterpret_cast<unsigned*>(cnt), 0xffffffffu,
                                                             __ATOMIC_RELAXED, "agent"));

  l = col_sum4(l);
  if (j == 0 && c < group) {
    sm_m[wave][c] = m;
    sm_l[wave][c] = l;
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int h = 4 * j + rr;
    if (h < group) {
#pragma unroll
      for (int nt = 0; nt < G::DC; ++nt) sm_o[wave][h][G::DC * c + nt] = o[nt][rr];
    }
  }
  __syncthreads();

  if constexpr (!MERGE) {
    // One element (h, d) per thread and step: the output when the workgroup
    // holds the whole sequence, else the partition's state for the merge
    // kernel.
    const bool single = P == 1;
    for (int idx = tid; idx < group * D; idx += kThreads) {
      const int h = idx / D;
      const int d = idx % D;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
      float acc = 0.f, lsum = 0.f;
      if (M != kNegInf) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float mw = sm_m[w][h];
          if (mw != kNegInf) {
            const float f = __builtin_amdgcn_exp2f(mw - M);
            acc += f * sm_o[w][h][d];
            lsum += f * sm_l[w][h];
          }
        }
      }
      const int64_t row = out_row0 + h;
      if (single) {
        store_from_f32<QT>(a.out, row * D + d, lsum > 0.f ? acc / lsum : 0.f);
      } else {
        const int64_t prow = row * P + part;
        a.part_acc[prow * D + d] = acc;
        if (d == 0) {
          a.part_ml[2 * prow] = M;
          a.part_ml[2 * prow + 1] = lsum;
        }
      }
    }
    return;
  }

  // Merging instance.  This workgroup's state, two adjacent output columns
  // (h, d..d+1) per step (the same sums as above, so the split form's states
  // carry the same bits): kPairs steps cover the largest group.
  constexpr int kPairs = (kMaxGroup * D / 2 + kThreads - 1) / kThreads;
  const int n_pairs = group * D / 2;
  float st_m[kPairs], st_l[kPairs], st_a[kPairs][2];
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const int pi = tid + k * kThreads;
    st_m[k] = kNegInf;
    st_l[k] = 0.f;
    st_a[k][0] = st_a[k][1] = 0.f;
    if (pi < n_pairs) {
      const int h = pi / (D / 2);
      const int d = 2 * (pi % (D / 2));
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
      float acc0 = 0.f, acc1 = 0.f, lsum = 0.f;
      if (M != kNegInf) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float mw = sm_m[w][h];
          if (mw != kNegInf) {
            const float f = __builtin_amdgcn_exp2f(mw - M);
            acc0 += f * sm_o[w][h][d];
            acc1 += f * sm_o[w][h][d + 1];
            lsum += f * sm_l[w][h];
          }
        }
      }
      st_m[k] = M;
      st_l[k] = lsum;
      st_a[k][0] = acc0;
      st_a[k][1] = acc1;
    }
  }

  if (np_b == 1) {
    // the workgroup holds the whole sequence: its state is the output (the
    // merge of one state gives the same bits)
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      const int pi = tid + k * kThreads;
      if (pi < n_pairs) {
        const int64_t i = (out_row0 + pi / (D / 2)) * D + 2 * (pi % (D / 2));
        store2_from_f32<QT>(a.out, i, st_l[k] > 0.f ? st_a[k][0] / st_l[k] : 0.f,
                            st_l[k] > 0.f ? st_a[k][1] / st_l[k] : 0.f);
      }
    }
    return;
  }


  // One-call form.  The counter holds arrivals in its low 16 bits and
  // publications above them.  Every workgroup but the last to arrive
  // publishes its state (stored through to memory, then counted as
  // published once the stores are acknowledged); the reply to the last
  // one's arrival usually shows every other state published already, and
  // otherwise it waits until they are - they have all arrived, so only their
  // stores are outstanding.  It merges every state in partition order,
  // writes the output and zeroes the counter for the next call.  The wait
  // is bounded; if it ever ran out the output row would be NaN rather than
  // the kernel hanging.
  constexpr int kPub = 1 << 16;
  __shared__ int sm_arrival;
  if (tid == 0) sm_arrival = arrival;
  __syncthreads();
  const bool last = (sm_arrival & (kPub - 1)) == np_b - 1;
  if (!last) {
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      const int pi = tid + k * kThreads;
      if (pi < n_pairs) {
        const int d = 2 * (pi % (D / 2));
        const int64_t prow = (out_row0 + pi / (D / 2)) * P + part;
        store_agent2(a.part_acc + prow * D + d, st_a[k][0], st_a[k][1]);
        if (d == 0) store_agent2(a.part_ml + 2 * prow, st_m[k], st_l[k]);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // every store of this thread acknowledged
    __syncthreads();
    if (tid == 0) atomicAdd(cnt, kPub);
    return;
  }
  if (tid == 0) {
    constexpr int kMaxSpins = 1 << 20;
    int spins = 0;
    int seen = sm_arrival;
    while ((seen >> 16) < np_b - 1 && spins < kMaxSpins) {
      __builtin_amdgcn_s_sleep(1);
      ++spins;
      seen = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    sm_arrival = (seen >> 16) >= np_b - 1 ? 1 : 0;
  }
  __syncthreads();
  const bool published = sm_arrival != 0;
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const int pi = tid + k * kThreads;
    if (pi >= n_pairs) continue;
    const int d = 2 * (pi % (D / 2));
    const int64_t row = out_row0 + pi / (D / 2);
    MergeState<2> ms = merge_begin<2>();
    for (int p0 = 0; p0 < np_b; p0 += 8) {
      // only existing partitions are read (each agent-scope load goes past
      // the caches: a repeated one would cost another trip to memory)
      float mp[8], lp[8], ap[8][2];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int p = p0 + i;
        const int64_t prow = row * P + p;
        mp[i] = kNegInf;
        lp[i] = 0.f;
        ap[i][0] = ap[i][1] = 0.f;
        if (p >= np_b) {
        } else if (p == part) {
          mp[i] = st_m[k];
          lp[i] = st_l[k];
          ap[i][0] = st_a[k][0];
          ap[i][1] = st_a[k][1];
        } else {
          const float2 ml = load_agent2(a.part_ml + 2 * prow);
          const float2 av = load_agent2(a.part_acc + prow * D + d);
          mp[i] = ml.x;
          lp[i] = ml.y;
          ap[i][0] = av.x;
          ap[i][1] = av.y;
        }
      }
      merge_chunk<2>(ms, mp, lp, ap, min(8, np_b - p0));
    }
    const float nan = __builtin_nanf("");
    store2_from_f32<QT>(a.out, row * D + d, published ? merge_result<2>(ms, 0) : nan,
                        published ? merge_result<2>(ms, 1) : nan);
  }
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- log-sum-exp merge of partitions (second launch) --------------------------------
// One workgroup of D threads per (sequence, query head).  The main kernel
// wrote a state into every partition slot (an empty partition has max -inf),
// so the merge needs no context length and issues all of its loads at once.
template <typename QT, int D>
__global__ void __launch_bounds__(D) partition_merge_kernel(DecodeArgs a) {
  const int row = blockIdx.x;                 // b * Hq + h
  const int d = threadIdx.x;
  const int P = a.num_partitions;
  const float* ml = a.part_ml + static_cast<int64_t>(row) * P * 2;
  const float* acc = a.part_acc + static_cast<int64_t>(row) * P * D;
  // Within a chunk every load is issued before any is used.  The output
  // slot of an empty partition holds stale values and is never used.
  MergeState<1> ms = merge_begin<1>();
  for (int p0 = 0; p0 < P; p0 += 8) {
    float mp[8], lp[8], ap[8][1];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = min(p0 + i, P - 1);
      mp[i] = ml[2 * p];
      lp[i] = ml[2 * p + 1];
      ap[i][0] = acc[static_cast<int64_t>(p) * D + d];
    }
    merge_chunk<1>(ms, mp, lp, ap, min(8, P - p0));
  }
  store_from_f32<QT>(a.out, static_cast<int64_t>(row) * D + d, merge_result<1>(ms, 0));
}

// ---- host side -------------------------------------------------------------------------

int choose_partition_size(int num_seqs, int num_kv_heads, int max_context_len, pkv_dtype cache_dtype) {
  // Pick the number of partitions per sequence, np, as the smallest value
  // for which the launch fills the chip evenly and no wave streams more than
  // kMaxWaveTiles blocks: units * np workgroups should be at least min_wgs and either a
  // whole number of 256-CU rounds or at least four rounds (then the
  // dispatcher balances the remainder).  min_wgs is one workgroup per CU,
  // except for int8 K + int4 V caches, whose decoding takes the most vector
  // instructions per byte: two resident workgroups per CU hide it (16 x 4096
  // at 8 KV heads: 31.0 us against 37.3 us with one).  Each partition keeps
  // >= 4 blocks per wave.  Partitions of one sequence are made as even as a
  // 16-token granule allows.  kMaxWaveTiles = 72 lets 32 x 32768 tokens at
  // 8 KV heads run in 8 partitions (65 blocks per wave, 2048 workgroups):
  // fp8 386.5-387.2 us and int8 K + int4 V 300.2-301.0 us per whole call
  // against 390.2-391.0 and 302.4-303.5 us with the 9 that a cap of 64
  // gave; 6 and 7 partitions measured within 1% of 8.
  constexpr int64_t kCUs = 256;
  constexpr int64_t kMaxWaveTiles = 72;
  const int64_t min_wgs = cache_dtype == PKV_INT8_INT4 ? 2 * kCUs : kCUs;
  const int64_t units = static_cast<int64_t>(num_seqs) * num_kv_heads;
  const int64_t seq_blocks = (static_cast<int64_t>(max_context_len) + kTileTokens - 1) / kTileTokens;
  if (seq_blocks <= 0 || units <= 0) return kTileTokens;
  const int64_t np_min = (seq_blocks + kMaxPartitionBlocks - 1) / kMaxPartitionBlocks;
  int64_t np_max = seq_blocks / (4 * kWaves);
  if (np_max < np_min) np_max = np_min;
  int64_t np = np_max;
  for (int64_t cand = np_min; cand <= np_max; ++cand) {
    const int64_t wgs = units * cand;
    const int64_t per_wave = (seq_blocks + cand * kWaves - 1) / (cand * kWaves);
    if (per_wave <= kMaxWaveTiles && wgs >= min_wgs && (wgs % kCUs == 0 || wgs >= 4 * kCUs)) {
      np = cand;
      break;
    }
  }
  if (np < 1) np = 1;
  const int64_t blocks = (seq_blocks + np - 1) / np;
  return static_cast<int>(blocks * kTileTokens);
}

template <typename QT, typename KT, typename VT, int D>
static int launch_typed(const DecodeArgs& a, hipStream_t stream, int stages) {
  const int64_t grid = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * a.num_partitions;
  if (grid > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  int rc = PKV_OK;
  if (stages & kStageAttend) {
    // Two tiles in flight per wave for every format.  16-bit caches:
    // interleaved A/B 1.3% faster than three on the Llama-3-8B layer shape,
    // 5% on the shared-prefix batch.  Quantised caches (tiles half as large)
    // took three while each wave ended with re-reads of its last tile; with
    // the straight-line tail two are faster (fp8 on the Llama-3-8B shape
    // 30.2-30.4 against 34.2-34.4 us, 32 x 32768 fp8 377.5 against 386.7 us)
    // and three would spill.
    constexpr int pipe = std::is_same<KT, F32>::value ? 2 : (KT::quantised ? PKV_DECODE_PIPE_Q : PKV_DECODE_PIPE);
    // longest first where the dispatcher hands out workgroups in turns and
    // each holds a whole sequence (split sequences already have workgroups of
    // at most one partition each: the order measured no faster there)
    if (a.seq_order != nullptr ||
        (decode_uses_order(a.num_seqs, a.num_kv_heads, a.num_partitions) && a.num_seqs <= kMaxRankSeqs)) {
      // small batches: every workgroup ranks in its prologue (measured faster
      // than a sort launch ahead of the kernel); larger ones: sorted once
      if (a.num_seqs > kMaxRankSeqs) {
        hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, a.context_lens, a.num_seqs,
                           const_cast<int32_t*>(a.seq_order));
        rc = check_launch();
        if (rc != PKV_OK) return rc;
      }
      hipLaunchKernelGGL((paged_decode_kernel<QT, KT, VT, D, pipe, true, false>), dim3(static_cast<unsigned>(grid)),
                         dim3(kThreads), 0, stream, a);
    } else if (a.counters != nullptr && a.num_partitions > 1) {
      hipLaunchKernelGGL((paged_decode_kernel<QT, KT, VT, D, pipe, false, true>),
                         dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream, a);
    } else {
      hipLaunchKernelGGL((paged_decode_kernel<QT, KT, VT, D, pipe, false, false>),
                         dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream, a);
    }
    rc = check_launch();
  }
  // one-call launches with counters merge inside the attention kernel
  if (rc != PKV_OK || !(stages & kStageMerge) || a.num_partitions == 1 || a.counters != nullptr) return rc;
  hipLaunchKernelGGL((partition_merge_kernel<QT, D>), dim3(a.num_seqs * a.num_q_heads), dim3(D), 0, stream, a);
  return check_launch();
}

template <typename QT, typename KT, typename VT>
static int launch_dim(const DecodeArgs& a, hipStream_t stream, int stages) {
  if (a.head_dim == 128) return launch_typed<QT, KT, VT, 128>(a, stream, stages);
  return launch_typed<QT, KT, VT, 64>(a, stream, stages);
}

template <typename KT, typename VT>
static int launch_quantised(const DecodeArgs& a, hipStream_t stream, int stages) {
  if (a.q_dtype == PKV_BF16) return launch_dim<BF16, KT, VT>(a, stream, stages);
  return launch_dim<F16, KT, VT>(a, stream, stages);
}

int launch_decode(const DecodeArgs& a, hipStream_t stream, int stages) {
  switch (a.cache_dtype) {
    case PKV_F32: return launch_dim<F32, F32, F32>(a, stream, stages);
    case PKV_F16: return launch_dim<F16, F16, F16>(a, stream, stages);
    case PKV_BF16: return launch_dim<BF16, BF16, BF16>(a, stream, stages);
    case PKV_FP8_E4M3: return launch_quantised<FP8, FP8>(a, stream, stages);
    case PKV_FP8_E5M2: return launch_quantised<BF8, BF8>(a, stream, stages);
    case PKV_INT8_INT4: return launch_quantised<I8, I4>(a, stream, stages);
  }
  return PKV_ERR_UNSUPPORTED;
}

}  // namespace pkv
