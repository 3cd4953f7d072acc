// Device-side helpers shared by the CSA2 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CSA2_DEV __device__ __forceinline__

typedef int v8i __attribute__((ext_vector_type(8)));          // 32 bytes of FP8
typedef float v16f __attribute__((ext_vector_type(16)));      // 32x32 MFMA accumulator
typedef float v4f __attribute__((ext_vector_type(4)));        // 16x16 MFMA accumulator
typedef _Float16 v8h __attribute__((ext_vector_type(8)));     // 8 fp16 MFMA operand
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));      // 8 bf16 MFMA operand
typedef short v8s __attribute__((ext_vector_type(8)));

namespace csa2 {

constexpr int kIdxHeads = 32;
constexpr int kIdxDim = 128;
constexpr int kHeads = 64;
constexpr int kDim = 512;
constexpr int kRowBytes = 288;
constexpr int kCodeBytes = 256;
constexpr int kTopK = 512;
constexpr int kPoolBlocks = 2048;
constexpr int kBlock = 8;
constexpr int kPoolCand = 16384;
constexpr int kWindow = 128;

CSA2_DEV float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// OCP E4M3FN byte -> float, from the bit fields (bias 7, subnormals m * 2^-9).
// Codes 0x7F/0xFF (NaN) decode to NaN.
CSA2_DEV float e4m3_to_f32(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 0x7u;
  float v;
  if (e == 0) {
    v = (float)m * 0.001953125f;                       // m * 2^-9, exact
  } else if (e == 0xF && m == 0x7) {
    v = __uint_as_float(0x7FC00000u);
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) 2^(e-7)
  }
  return __uint_as_float(__float_as_uint(v) | s);
}

// E2M1 magnitude code (0..7) -> value {0, .5, 1, 1.5, 2, 3, 4, 6}.
CSA2_DEV float e2m1_mag(uint32_t m) {
  // exponent field e = m >> 1 (bias 1), mantissa bit = m & 1
  const uint32_t e = m >> 1, f = m & 1u;
  return e == 0 ? 0.5f * (float)f : __uint_as_float(((e + 126u) << 23) | (f << 22));
}

// Order-preserving map of a float to uint32 (larger key = larger float); -0 and
// +0 share a key. NaN is not supported.
CSA2_DEV uint32_t float_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <typename T>
CSA2_DEV T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace csa2
