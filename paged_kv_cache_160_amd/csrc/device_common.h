// Device-side helpers shared by the cache-write and decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pagedkv.h"

namespace pkv {

// Kernels walk the pool in tiles of 16 token rows of one (block, KV head): a
// 16-token block is one tile per head, a 32-token block two consecutive ones.
// Tile index of a sequence's 16-token unit u (tokens 16u .. 16u+15) at KV head
// g, with rs = log2(block_size / 16) and phys the block holding the unit:
//   ((phys * num_kv_heads + g) << rs) + (u & ((1 << rs) - 1)),
// and the tile's rows start at row tile * 16 of the pool (scales likewise).
constexpr int kTileTokens = 16;
constexpr int kWave = 64;

// log2(block_size / 16): 0 for 16-token blocks, 1 for 32-token blocks.
__host__ __device__ inline int block_shift(int block_size) { return block_size == 32 ? 1 : 0; }

// Pool row of slot = phys * block_size + offset at KV head g.
__host__ __device__ inline int64_t slot_row(int64_t slot, int block_size, int num_kv_heads, int g) {
  return ((slot / block_size) * num_kv_heads + g) * block_size + slot % block_size;
}

// Storage tags.  Each names the element type a pool or a query holds.
// Quantised tags (codes plus one float32 scale per (token, head) row) carry
// qmax, the largest code magnitude the row's scale maps max|x| to.
struct F32 {
  using storage = float;
  static constexpr int bytes = 4;
  static constexpr int bits = 32;
  static constexpr bool quantised = false;
};
struct F16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
  static constexpr int bits = 16;
  static constexpr bool quantised = false;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
  static constexpr int bits = 16;
  static constexpr bool quantised = false;
};
struct FP8 {            // OCP e4m3 ("FN")
  using storage = uint8_t;
  static constexpr int bytes = 1;
  static constexpr int bits = 8;
  static constexpr bool quantised = true;
  static constexpr float qmax = 448.0f;
};
struct BF8 {            // OCP e5m2
  using storage = uint8_t;
  static constexpr int bytes = 1;
  static constexpr int bits = 8;
  static constexpr bool quantised = true;
  static constexpr float qmax = 57344.0f;
};
struct I8 {             // symmetric two's-complement int8
  using storage = uint8_t;
  static constexpr int bytes = 1;
  static constexpr int bits = 8;
  static constexpr bool quantised = true;
  static constexpr float qmax = 127.0f;
};
struct I4 {             // symmetric two's-complement int4, two per byte (even element low)
  using storage = uint8_t;
  static constexpr int bytes = 1;   // per pair of elements
  static constexpr int bits = 4;
  static constexpr bool quantised = true;
  static constexpr float qmax = 7.0f;
};

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// ---- scalar conversions ------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, bits16));
}
// fp32 -> bf16 / f16 with round-to-nearest-even (hardware conversions).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

template <typename T> __device__ __forceinline__ float load_as_f32(const void* p, int64_t i);
template <> __device__ __forceinline__ float load_as_f32<F32>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <> __device__ __forceinline__ float load_as_f32<F16>(const void* p, int64_t i) {
  return f16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float load_as_f32<BF16>(const void* p, int64_t i) {
  return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <typename T> __device__ __forceinline__ void store_from_f32(void* p, int64_t i, float v);
template <> __device__ __forceinline__ void store_from_f32<F32>(void* p, int64_t i, float v) {
  static_cast<float*>(p)[i] = v;
}
template <> __device__ __forceinline__ void store_from_f32<F16>(void* p, int64_t i, float v) {
  static_cast<uint16_t*>(p)[i] = f32_to_f16_bits(v);
}
template <> __device__ __forceinline__ void store_from_f32<BF16>(void* p, int64_t i, float v) {
  static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(v);
}
// Elements i and i + 1 (i even) in one store.
template <typename T> __device__ __forceinline__ void store2_from_f32(void* p, int64_t i, float v0, float v1);
template <> __device__ __forceinline__ void store2_from_f32<F32>(void* p, int64_t i, float v0, float v1) {
  *reinterpret_cast<float2*>(static_cast<float*>(p) + i) = make_float2(v0, v1);
}
template <> __device__ __forceinline__ void store2_from_f32<F16>(void* p, int64_t i, float v0, float v1) {
  *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p) + i) =
      static_cast<uint32_t>(f32_to_f16_bits(v0)) | (static_cast<uint32_t>(f32_to_f16_bits(v1)) << 16);
}
template <> __device__ __forceinline__ void store2_from_f32<BF16>(void* p, int64_t i, float v0, float v1) {
  *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p) + i) =
      static_cast<uint32_t>(f32_to_bf16_bits(v0)) | (static_cast<uint32_t>(f32_to_bf16_bits(v1)) << 16);
}

// ---- OCP e4m3 encoding ---------------------------------------------------------
// Round-to-nearest-even of a finite y with |y| <= 448 to the E4M3FN code
// (1 sign, 4 exponent bits with bias 7, 3 mantissa bits).  Normal range
// (|y| >= 2^-6): keep the fp32 exponent, round the 23-bit mantissa to 3 bits
// with ties to even; a carry out of the mantissa bumps the exponent, which
// the integer add does by itself.  Subnormal range: the code magnitude is
// |y| * 2^9 rounded to an integer with ties to even (0..8; 8 is the smallest
// normal code).  The sign bit copies y's sign (-0 gives 0x80).
__device__ __forceinline__ uint32_t e4m3_encode_rne(float y) {
  uint32_t bits = __float_as_uint(y);
  uint32_t sign = (bits >> 24) & 0x80u;
  float a = fabsf(y);
  uint32_t mag;
  if (a < 0.015625f) {                       // 2^-6
    mag = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {
    uint32_t abits = bits & 0x7fffffffu;
    int32_t e = static_cast<int32_t>(abits >> 23) - 127;   // -6 .. 8
    uint32_t m = abits & 0x7fffffu;
    uint32_t rounded = (m + 0x7ffffu + ((m >> 20) & 1u)) >> 20;   // 0 .. 8
    mag = (static_cast<uint32_t>(e + 7) << 3) + rounded;
  }
  return sign | mag;
}

// ---- OCP e5m2 encoding ---------------------------------------------------------
// Round-to-nearest-even of a finite y with |y| <= 57344 to the E5M2 code
// (1 sign, 5 exponent bits with bias 15, 2 mantissa bits).  Normal range
// (|y| >= 2^-14): keep the fp32 exponent and round the mantissa to 2 bits
// with ties to even (a carry bumps the exponent through the integer add).
// Subnormal range: |y| * 2^16 rounded to an integer with ties to even (0..4;
// 4 is the smallest normal code).  The sign bit copies y's sign.
__device__ __forceinline__ uint32_t e5m2_encode_rne(float y) {
  uint32_t bits = __float_as_uint(y);
  uint32_t sign = (bits >> 24) & 0x80u;
  float a = fabsf(y);
  uint32_t mag;
  if (a < 6.103515625e-05f) {                 // 2^-14
    mag = static_cast<uint32_t>(__builtin_rintf(a * 65536.0f));
  } else {
    uint32_t abits = bits & 0x7fffffffu;
    int32_t e = static_cast<int32_t>(abits >> 23) - 127;   // -14 .. 15
    uint32_t m = abits & 0x7fffffu;
    uint32_t rounded = (m + 0xfffffu + ((m >> 21) & 1u)) >> 21;   // 0 .. 4
    mag = (static_cast<uint32_t>(e + 15) << 2) + rounded;
  }
  return sign | mag;
}

// Code of y (already divided by the row scale and clamped to +-qmax) in the
// quantised format Q: an 8-bit pattern, or for I4 a nibble in the low bits.
template <typename Q>
__device__ __forceinline__ uint32_t quant_code(float y) {
  if constexpr (std::is_same<Q, FP8>::value) return e4m3_encode_rne(y);
  else if constexpr (std::is_same<Q, BF8>::value) return e5m2_encode_rne(y);
  else if constexpr (std::is_same<Q, I8>::value) return static_cast<uint32_t>(static_cast<int32_t>(__builtin_rintf(y))) & 0xffu;
  else return static_cast<uint32_t>(static_cast<int32_t>(__builtin_rintf(y))) & 0xfu;
}

// ---- wave reductions -----------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// ---- cache-row writes ------------------------------------------------------------
// One wave writes one (token, head) row of D elements to its pool row
// (`dst_row` counts pool rows).  Same dtype: a bit copy in 16-byte chunks.
// Quantised format Q: a = max|x| over the row, s = a / qmax (s = 1 if
// a == 0), codes = quant_code(clamp(x / s, -qmax, qmax)), both divisions
// correctly rounded in fp32; the scale goes to scales[dst_row].  Lane l holds
// elements l*D/64 ..; I4 rows pack two codes per byte, the even element in
// the low nibble (for D = 64 neighbouring lanes pair up).
template <typename Src, int D, typename Q>
__device__ __forceinline__ void write_row_quant(const void* src, int64_t src_row, uint8_t* pool,
                                                float* scales, int64_t dst_row, int lane) {
  constexpr int kPer = D / kWave;   // 1 or 2 elements per lane
  float x[kPer];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    x[i] = load_as_f32<Src>(src, src_row * D + lane * kPer + i);
    amax = fmaxf(amax, fabsf(x[i]));
  }
  amax = wave_max(amax);
  float s = __fdiv_rn(amax, Q::qmax);
  if (amax == 0.0f) s = 1.0f;
  uint32_t code[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    float y = __fdiv_rn(x[i], s);
    y = fminf(fmaxf(y, -Q::qmax), Q::qmax);
    code[i] = quant_code<Q>(y);
  }
  if constexpr (std::is_same<Q, I4>::value) {
    constexpr int row_bytes = D / 2;
    if constexpr (kPer == 2) {
      pool[dst_row * row_bytes + lane] = static_cast<uint8_t>(code[0] | (code[1] << 4));
    } else {
      const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(code[0]), 1, kWave));
      if ((lane & 1) == 0) pool[dst_row * row_bytes + lane / 2] = static_cast<uint8_t>(code[0] | (other << 4));
    }
  } else {
    uint8_t* dst = pool + dst_row * D + lane * kPer;
    if constexpr (kPer == 2) {
      *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(code[0] | (code[1] << 8));
    } else {
      *dst = static_cast<uint8_t>(code[0]);
    }
  }
  if (lane == 0) scales[dst_row] = s;
}

template <typename Src, int D>
__device__ __forceinline__ void write_row_fp8(const void* src, int64_t src_row, uint8_t* pool,
                                              float* scales, int64_t dst_row, int lane) {
  write_row_quant<Src, D, FP8>(src, src_row, pool, scales, dst_row, lane);
}

__device__ __forceinline__ void write_row_copy(const void* src, int64_t src_row, void* pool, int64_t dst_row,
                                               int row_bytes, int lane) {
  const int chunks = row_bytes / 16;
  if (lane < chunks) {
    const uint4* s = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(src) + src_row * row_bytes);
    uint4* d = reinterpret_cast<uint4*>(static_cast<uint8_t*>(pool) + dst_row * row_bytes);
    d[lane] = s[lane];
  }
}

}  // namespace pkv
