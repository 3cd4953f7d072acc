// The rest of the write path around the FP4 main-KV packer: the m-token
// compressor and the E4M3 append of window rows and FP8 indexer keys.
//
// Pages: every m tokens become one compressed entry, m = 2 in the encoder
// groups and m = 1 in the decoder groups ("DeepSeek V4.1-Flash 为什么这么强？
// CED 与 CSA2 架构全拆解", §二 layer layout; "DeepSeek V4.1 Flash vs V4 Pro",
// 黑科技之二); the sliding-window KV stays FP8 (same page §三; "DeepSeek-V4.1-
// Flash：全局 KV 仅 890 B/token", 第三刀) and every layer keeps its own window
// ("DeepSeek V4.1 Flash vs V4 Pro", 黑科技之二).
//
// Compressor: entry j is the mean of token rows jm .. jm+m-1 (fewer for a
// trailing partial group), summed in float32 in token order, divided by the row
// count with a correctly rounded division, rounded to bf16 nearest-even. One
// thread per (entry, 8 channels).
//
// E4M3 append: nearest E4M3 value, ties to the even code, saturating at 448,
// sign bit kept (OCP E4M3FN). Every decision is exact: below 2^-6 the code is
// rint(|x| * 2^9) (the subnormal step; 8 lands on the smallest normal code);
// above, the mantissa is rint((|x| / 2^e - 1) * 8) with the carry into the
// exponent falling out of the code arithmetic; beyond 448 the largest finite
// code. One thread per (row, 8 channels).
#include "device_common.hpp"
#include "launchers.hpp"

namespace csa2 {
namespace {

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;   // finite values
}

__global__ __launch_bounds__(256) void k_compress_rows(const uint16_t* __restrict__ tok,
                                                       int64_t n_tok, int width, int m,
                                                       uint16_t* __restrict__ out, int64_t n_out) {
  const int per = width / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t j = idx / per;
  const int c8 = (int)(idx % per);
  if (j >= n_out) return;
  const int64_t r0 = j * m;
  const int64_t r1 = r0 + m < n_tok ? r0 + m : n_tok;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  for (int64_t r = r0; r < r1; ++r) {
    const uint4 v = *reinterpret_cast<const uint4*>(tok + r * width + 8 * c8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = __fadd_rn(acc[2 * i], bf16_bits_to_f32(w[i] & 0xFFFFu));
      acc[2 * i + 1] = __fadd_rn(acc[2 * i + 1], bf16_bits_to_f32(w[i] >> 16));
    }
  }
  const float cnt = (float)(r1 - r0);
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32_to_bf16_rne(__fdiv_rn(acc[2 * i], cnt)) |
           (f32_to_bf16_rne(__fdiv_rn(acc[2 * i + 1], cnt)) << 16);
  *reinterpret_cast<uint4*>(out + j * width + 8 * c8) = make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ uint32_t e4m3_rne_sat(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t mag;
  if (a > 448.0f) {
    mag = 0x7Eu;
  } else if (a < 0.015625f) {                          // below 2^-6: steps of 2^-9
    mag = (uint32_t)__builtin_rintf(__fmul_rn(a, 512.0f));
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // -6 .. 8
    const float f = __fmul_rn(a, __uint_as_float((uint32_t)(127 - e) << 23));   // [1, 2)
    const uint32_t mm = (uint32_t)__builtin_rintf(__fmul_rn(__fsub_rn(f, 1.0f), 8.0f));
    mag = ((uint32_t)(e + 7) << 3) + mm;               // mm = 8 carries into the exponent
  }
  return mag | sign;
}

__global__ __launch_bounds__(256) void k_quantize_e4m3(const uint16_t* __restrict__ x, int64_t n,
                                                       int width, const int64_t* __restrict__ slot,
                                                       uint8_t* __restrict__ out, int64_t rows) {
  const int per = width / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = idx / per;
  const int c8 = (int)(idx % per);
  if (r >= n) return;
  const int64_t dst = slot ? slot[r] : r;
  if (dst < 0 || dst >= rows) return;
  const uint4 v = *reinterpret_cast<const uint4*>(x + r * width + 8 * c8);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    lo |= e4m3_rne_sat(bf16_bits_to_f32(w[i] & 0xFFFFu)) << (16 * i);
    lo |= e4m3_rne_sat(bf16_bits_to_f32(w[i] >> 16)) << (16 * i + 8);
    hi |= e4m3_rne_sat(bf16_bits_to_f32(w[2 + i] & 0xFFFFu)) << (16 * i);
    hi |= e4m3_rne_sat(bf16_bits_to_f32(w[2 + i] >> 16)) << (16 * i + 8);
  }
  *reinterpret_cast<uint2*>(out + dst * width + 8 * c8) = make_uint2(lo, hi);
}

}  // namespace

hipError_t launch_compress_rows(const uint16_t* tok, int64_t n_tok, int width, int m,
                                uint16_t* out, hipStream_t st) {
  const int64_t n_out = (n_tok + m - 1) / m;
  if (n_out == 0) return hipSuccess;
  const int64_t threads = n_out * (width / 8);
  hipLaunchKernelGGL(k_compress_rows, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     tok, n_tok, width, m, out, n_out);
  return hipGetLastError();
}

hipError_t launch_quantize_e4m3(const uint16_t* x, int64_t n, int width, const int64_t* slot,
                                uint8_t* out, int64_t rows, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t threads = n * (width / 8);
  hipLaunchKernelGGL(k_quantize_e4m3, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     x, n, width, slot, out, rows);
  return hipGetLastError();
}

}  // namespace csa2
