// Write path of the main KV: RoPE on channels 448..511, then FP4 E2M1 codes
// with one E4M3 scale per 16 channels, stored as a 288-byte row.
//
// Pages: the main KV is E2M1 with an E4M3 scale per 16 channels and no
// second-level scale ("DeepSeek V4.1-Flash 为什么这么强？CED 与 CSA2 架构全拆解",
// §三; "DeepSeek V4.1 Flash vs V4 Pro", 黑科技之三), quantised after RoPE
// (same §三; "DeepSeek-V4.1-Flash：全局 KV 仅 890 B/token", 第三刀).
//
// Layout: one wave per row, lane l owns channels 8l..8l+7 (one 16-byte load of
// bf16, one 4-byte store of codes); a 16-channel group is a lane pair. Every
// rounding decision is taken by exact float32 comparisons, so the result is
// bit-exact regardless of instruction order:
//   * scale: the E4M3 code c with 3(v_{c-1}+v_c) < amax <= 3(v_c+v_{c+1}) (the
//     midpoints of amax/6 times 6, all exact in float32), ties to the even code;
//   * element: |y| against t*s for the seven E2M1 midpoints t (exact products),
//     ties to the even code.
#include "device_common.hpp"
#include "launchers.hpp"

namespace csa2 {
namespace {

// Non-negative finite E4M3 value of code c (0..126), exact.
__device__ __forceinline__ float e4m3_pos(int c) {
  const int e = c >> 3, m = c & 7;
  return e == 0 ? (float)m * 0.001953125f : __uint_as_float(((uint32_t)(e + 120) << 23) | ((uint32_t)m << 20));
}

// 6 x (midpoint between codes k and k+1) = 3 (v_k + v_{k+1}); exact in float32.
__device__ __forceinline__ float scale_threshold(int k) {
  return __fmul_rn(3.0f, __fadd_rn(e4m3_pos(k), e4m3_pos(k + 1)));
}

__device__ __forceinline__ int scale_code(float amax) {
  int lo = 0, hi = 126;                       // smallest c with amax <= T(c), else 126
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (amax <= scale_threshold(mid)) hi = mid; else lo = mid + 1;
  }
  if (lo < 126 && (lo & 1) && amax == scale_threshold(lo)) ++lo;   // tie -> even
  return lo;
}

__device__ __forceinline__ uint32_t e2m1_code(float y, float s) {
  const float a = fabsf(y);
  uint32_t m = 0;
  if (s > 0.0f) {
    m = (a > __fmul_rn(0.25f, s)) + (a >= __fmul_rn(0.75f, s)) + (a > __fmul_rn(1.25f, s)) +
        (a >= __fmul_rn(1.75f, s)) + (a > __fmul_rn(2.5f, s)) + (a >= __fmul_rn(3.5f, s)) +
        (a > __fmul_rn(5.0f, s));
  }
  return m | ((__float_as_uint(y) >> 28) & 0x8u);
}

__global__ __launch_bounds__(256) void k_quantize_kv(const uint16_t* __restrict__ kv,
                                                     const float* __restrict__ cs,
                                                     const int64_t* __restrict__ slot, int64_t n,
                                                     uint8_t* __restrict__ cache,
                                                     int64_t cache_rows) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const int64_t dst = slot ? slot[row] : row;
  if (dst < 0 || dst >= cache_rows) return;

  const uint4 raw = *reinterpret_cast<const uint4*>(kv + row * kDim + lane * 8);
  float x[8];
  const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(w4[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_bits_to_f32(w4[i] >> 16);
  }
  if (lane >= 56) {  // channels 448..511: pairs 4(lane-56) .. 4(lane-56)+3
    const float4* c4 = reinterpret_cast<const float4*>(cs + row * 64 + (lane - 56) * 8);
    const float4 p01 = c4[0], p23 = c4[1];
    const float cc[4] = {p01.x, p01.z, p23.x, p23.z};
    const float ss[4] = {p01.y, p01.w, p23.y, p23.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = x[2 * i], x1 = x[2 * i + 1];
      x[2 * i] = __fsub_rn(__fmul_rn(x0, cc[i]), __fmul_rn(x1, ss[i]));
      x[2 * i + 1] = __fadd_rn(__fmul_rn(x0, ss[i]), __fmul_rn(x1, cc[i]));
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = fmaxf(amax, wave_shfl_xor(amax, 1));
  const int sc = scale_code(amax);
  const float s = e4m3_pos(sc);
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) packed |= e2m1_code(x[i], s) << (4 * i);
  uint8_t* dstp = cache + dst * kRowBytes;
  *reinterpret_cast<uint32_t*>(dstp + lane * 4) = packed;
  if ((lane & 1) == 0) dstp[kCodeBytes + (lane >> 1)] = (uint8_t)sc;
}

// ---------------------------------------------------------------------------
// FP4 indexer keys: E2M1 codes with one E8M0 (power-of-two) scale per 32
// channels. The earlier model generation trained its indexer keys in FP4
// ("DeepSeek V4.1 Flash vs V4 Pro", 黑科技之三); the pages' FP4 is of the MXFP4
// family ("DeepSeek V4.1-Flash 为什么这么强？CED 与 CSA2 架构全拆解", §三), and
// the block scale follows the OCP Microscaling (MX) v1.0 conversion rule:
// exponent floor(log2(amax)) - 2, stored with bias 127, clamped to 0..254.
//
// One wave per key, lane l owns channels 2l and 2l+1 (one 4-byte bf16 load,
// one byte of codes); a 32-channel block is a row of 16 lanes. For a normal
// amax with biased exponent E, floor(log2(amax)) - 2 + 127 = E - 2, so the
// scale code is max(E - 2, 0) (zero and subnormal maxima give 0). Dividing by
// the scale is a multiplication by 2^(127 - code), exact for every value whose
// code can be nonzero; the element code then comes from exact comparisons with
// the E2M1 midpoints, ties to the even code, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_code_of_scaled(float x, float inv_scale) {
  const float y = __fmul_rn(fabsf(x), inv_scale);
  uint32_t m = (y > 0.25f) + (y >= 0.75f) + (y > 1.25f) + (y >= 1.75f) + (y > 2.5f) +
               (y >= 3.5f) + (y > 5.0f);
  return m | ((__float_as_uint(x) >> 28) & 8u);
}

__global__ __launch_bounds__(256) void k_quantize_index_k(const uint16_t* __restrict__ k,
                                                          const int64_t* __restrict__ slot,
                                                          int64_t n, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales,
                                                          int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= n) return;
  const int64_t dst = slot ? slot[r] : r;
  if (dst < 0 || dst >= rows) return;
  const uint32_t pair = *reinterpret_cast<const uint32_t*>(k + r * kIdxDim + 2 * lane);
  const float x0 = bf16_bits_to_f32(pair & 0xFFFFu), x1 = bf16_bits_to_f32(pair >> 16);
  uint32_t amax = max(__float_as_uint(x0) & 0x7FFFFFFFu, __float_as_uint(x1) & 0x7FFFFFFFu);
  amax = max(amax, (uint32_t)wave_shfl_xor((int)amax, 1));
  amax = max(amax, (uint32_t)wave_shfl_xor((int)amax, 2));
  amax = max(amax, (uint32_t)wave_shfl_xor((int)amax, 4));
  amax = max(amax, (uint32_t)wave_shfl_xor((int)amax, 8));   // max over the 16-lane row
  const uint32_t E = amax >> 23;
  const uint32_t code = E >= 2u ? E - 2u : 0u;
  const float inv = __uint_as_float((254u - code) << 23);       // 2^(127 - code)
  codes[dst * (kIdxDim / 2) + lane] =
      (uint8_t)(e2m1_code_of_scaled(x0, inv) | (e2m1_code_of_scaled(x1, inv) << 4));
  if ((lane & 15) == 0) scales[dst * 4 + (lane >> 4)] = (uint8_t)code;
}

}  // namespace

hipError_t launch_quantize_index_k(const uint16_t* k, const int64_t* slot, int64_t n,
                                   uint8_t* codes, uint8_t* scales, int64_t rows, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 3) / 4;
  hipLaunchKernelGGL(k_quantize_index_k, dim3((unsigned)blocks), dim3(256), 0, st, k, slot, n,
                     codes, scales, rows);
  return hipGetLastError();
}

hipError_t launch_quantize_kv(const uint16_t* kv, const float* cos_sin, const int64_t* slot,
                              int64_t n, uint8_t* cache, int64_t cache_rows, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 3) / 4;
  hipLaunchKernelGGL(k_quantize_kv, dim3((unsigned)blocks), dim3(256), 0, st, kv, cos_sin, slot,
                     n, cache, cache_rows);
  return hipGetLastError();
}

}  // namespace csa2
