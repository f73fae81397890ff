// Device-side helpers shared by the cache-write and decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

constexpr int kBlockTokens = PKV_BLOCK_SIZE;
constexpr int kWave = 64;

// Storage tags.  Each names the element type a pool or a query holds.
struct F32 {
  using storage = float;
  static constexpr int bytes = 4;
};
struct F16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};
struct FP8 {
  using storage = uint8_t;
  static constexpr int bytes = 1;
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

// ---- wave reductions -----------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// ---- cache-row writes ------------------------------------------------------------
// One wave writes one (token, head) row of D elements to its pool row
// (`dst_row` counts rows of D elements).  Same dtype: a bit copy in 16-byte
// chunks.  fp8: a = max|x| over the row, s = a / 448 (s = 1 if a == 0),
// codes = e4m3 RNE of clamp(x / s, -448, 448), with both divisions correctly
// rounded in fp32; the scale goes to scales[dst_row].
template <typename Src, int D>
__device__ __forceinline__ void write_row_fp8(const void* src, int64_t src_row, uint8_t* pool,
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
  float s = __fdiv_rn(amax, 448.0f);
  if (amax == 0.0f) s = 1.0f;
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    float y = __fdiv_rn(x[i], s);
    y = fminf(fmaxf(y, -448.0f), 448.0f);
    packed |= e4m3_encode_rne(y) << (8 * i);
  }
  uint8_t* dst = pool + dst_row * D + lane * kPer;
  if constexpr (kPer == 2) {
    *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(packed);
  } else {
    *dst = static_cast<uint8_t>(packed);
  }
  if (lane == 0) scales[dst_row] = s;
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
