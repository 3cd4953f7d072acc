// Sparse MQA attention over the selected FP4 main-KV rows plus the FP8 window.
//
// Pages: 64 heads of width 512 over the Top-512 selected entries
// ("DeepSeek V4.1-Flash 为什么这么强？CED 与 CSA2 架构全拆解", §二 layer layout)
// plus a 128-token sliding window (same page §一; "DeepSeek V4.1 Flash vs V4
// Pro", 黑科技之一); the FP4 main KV is dequantised before attention and the
// window KV stays FP8 ("DeepSeek-V4.1-Flash：全局 KV 仅 890 B/token", 第三刀);
// every layer has its own query and window ("DeepSeek V4.1 Flash vs V4 Pro",
// 黑科技之二). Key = value = the dequantised 512-wide row (reading in csa2.h).
// The window buffer is linear (row s = token swa_pos0 + s) or a ring (token t
// in row t mod S), the latter for a decode loop that keeps the last n_win
// tokens of window KV per layer ("DeepSeek V4.1 Flash vs V4 Pro", 黑科技之三).
//
// Common to all work shapes: rows are dequantised to fp16 exactly with the
// gfx950 converts (v_cvt_scalef32_pk_f16_fp4 with the power-of-two part of the
// E4M3 scale, then one v_pk_mul_f16 by its mantissa part; window rows with
// v_cvt_scalef32_pk_f16_fp8). Q.K: v_mfma_f32_16x16x32_f16 with 16 keys as A and
// 16 query heads as B (each head scaled by a power of two into fp16 range; the
// logits are scaled back). P.V: v_mfma_f32_16x16x32_f16 with V^T as A, read
// from a row-major fp16 LDS copy by the transposing LDS read
// ds_read_b64_tr_b16, and P as B; P = hi + lo in fp16 (two MFMAs per tile),
// which keeps the product accurate to about 2^-22 of P even for rows with large
// outlier channels. Work-groups that gather the same rows get ids equal mod 8,
// so the dispatcher's round-robin over the 8 XCDs puts them on one XCD (one L2).
//
// Three work shapes, by the number of queries Q in the call:
//   Q <= 12 (decode): one 8-wave work-group per (query, 16 heads, slice of 128
//          key slots); each lane dequantises 128 channels of one key straight
//          into its Q.K operand registers and the slice's LDS copy; the waves
//          agree on the slice maximum through LDS; slices are merged by
//          log-sum-exp in a second kernel (k_attn_merge). Spreads a few
//          queries over 20 work-groups each; with 151 KB of LDS each takes a
//          whole CU, so up to 12 queries (240 work-groups) run in one round
//          over the 256 CUs, and from 13 on the head-group shape below (one
//          round up to 64 queries, no merge) is faster.
//   13 <= Q < 512: one 8-wave work-group per (query, 16 heads), no workspace.
//          The query's 640 key slots form 20 steps of 32; wave pair p takes
//          steps p, p+4, p+8, p+12 (selected rows) and 16+p (window):
//          * wave p + 4h dequantises keys 16h..16h+15 of the step (lane (g, c):
//            key c, channels 128g..128g+127) straight into its Q.K operand
//            registers and into the pair's 32-row fp16 LDS tile, and forms
//            their logits for the 16 heads;
//          * the pair swaps logits through LDS; the logit of key 16t + 4g + r
//            for head c sits in lane (g, c), the lane and order P.V's B operand
//            needs; both waves run the same online softmax over the 32 keys,
//            raising the running maximum only when a step's maximum exceeds it
//            by more than 8 (p stays below e^8, inside fp16);
//          * wave p + 4h accumulates P.V for output channels 256h..256h+255.
//          At the end the four pairs' (max, sum, output) are merged by
//          log-sum-exp through LDS and the work-group writes its 16 heads'
//          output directly.
//   Q >= 512 (prefill): one 8-wave work-group per query over its 640 key slots
//          in chunks of 64 with an online softmax; wave w serves 16 heads
//          (w % 4), and the 4 head groups share each dequantised chunk through
//          LDS (each row is dequantised once for all 64 heads).
#include "device_common.hpp"
#include "launchers.hpp"

namespace csa2 {
namespace {

constexpr int kSlots = kTopK + kWindow;           // 640 key slots per query
constexpr int kHG = 16;                           // heads per work-group
constexpr int kHeadGroups = kHeads / kHG;         // 4
constexpr int kPairs = 4;                         // wave pairs of the head-group shape
constexpr int kWaves = 2 * kPairs;                // 8: two waves per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kStepKeys = 32;                     // keys per softmax step (one P.V MFMA)
constexpr int kSteps = kSlots / kStepKeys / kPairs;      // 5 per pair
constexpr int kMainSteps = kTopK / kStepKeys / kPairs;   // 4 per pair, then 1 window step
constexpr int kHalfTiles = kDim / 16 / 2;         // P.V channel tiles per wave (16)
constexpr int kPvGroup = 4;                       // channel tiles per P.V issue group
constexpr int kVRow = kDim + 8;                   // fp16 per LDS key row
constexpr int kDecodeMaxQueries = 13;             // below: the split decode shape
constexpr int kPrefillMinQueries = 512;           // from here: one work-group per query
constexpr int kOutRow = kDim / 2 + 4;             // floats per LDS row of the final merge
constexpr float kLazyMax = 8.0f;                  // headroom before the running max moves
constexpr int kXcds = 8;
static_assert(kSlots == kSteps * kStepKeys * kPairs, "whole steps per pair");
static_assert(kTopK % (kStepKeys * kPairs) == 0 && kWindow == kStepKeys * kPairs,
              "each pair: whole steps of selected rows, then one window step");
static_assert(kWaves * kHG * kOutRow * 4 <= kPairs * kStepKeys * kVRow * 2,
              "the final merge fits in the key tiles");
static_assert(kHG * kVRow <= kPairs * kStepKeys * kVRow, "the query staging fits in the key tiles");
static_assert(kThreads >= 256, "one thread per E4M3 scale code fills the table");

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

struct AttnArgs {
  const uint16_t* q;
  const uint8_t* cache;
  const int32_t* idx;
  const uint8_t* swa;
  const int64_t* q_pos;
  const int64_t* swa_pos0;
  int T;
  int Q;
  int64_t n_cap;
  int S;
  int ring;
  float scale;
  float* out;
  float* part;     // decode shape: [Q][slices][64][512] unnormalised outputs
  float* part_ml;  // decode shape: [Q][slices][64][2] running max and sum
};

// Exponent shift that brings a per-head maximum |q| into [2^14, 2^15): q * 2^s
// then fits fp16 without overflow, and every element within 2^28 of the maximum
// keeps its full bf16 precision (smaller ones contribute below 2^-28 of it).
__device__ __forceinline__ int q_shift(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127;
  return 14 - e;
}

__device__ __forceinline__ v8h q_to_f16(const uint4& raw, int shift) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  v8h o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = (_Float16)ldexpf(bf16_bits_to_f32(w[i] & 0xFFFFu), shift);
    o[2 * i + 1] = (_Float16)ldexpf(bf16_bits_to_f32(w[i] >> 16), shift);
  }
  return o;
}

__device__ __forceinline__ float bf16x8_absmax(const uint4& raw) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] & 0xFFFFu)));
    m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] >> 16)));
  }
  return m;
}

typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

// Work-group barrier that orders LDS accesses only: it waits for this wave's
// LDS operations, not for its global loads in flight (__syncthreads waits for
// those too, which would expose the latency of rows loaded ahead of use).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Reductions over the four 16-lane rows of a wave (lanes with the same lane %
// 16), in VALU: v_permlane16_swap pairs rows 0/1 and 2/3, v_permlane32_swap
// pairs the halves; every lane ends with (r0 op r1) op (r2 op r3).
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 16 FP4 codes (two 32-bit words, channels 2b, 2b+1 in byte b) with the E4M3
// scale byte c -> 8 fp16 pairs: the power-of-two part of the scale in the
// convert, its mantissa part (1 + M/8, or M for a subnormal scale) in one
// v_pk_mul_f16; exact, as the products have at most 6 significant bits and lie
// in [2^-10, 2688].
__device__ __forceinline__ void fp4x16_to_f16(uint32_t w0, uint32_t w1, uint32_t c, uint32_t* pr) {
  const uint32_t E = (c >> 3) & 15u, M = c & 7u;
  const float hw = __uint_as_float(E ? (E + 120u) << 23 : 118u << 23);
  const _Float16 mf = E ? __builtin_bit_cast(_Float16, (uint16_t)(0x3C00u | (M << 7)))
                        : (_Float16)(float)M;
  const v2h m2 = {mf, mf};
  pr[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, hw, 0) * m2);
  pr[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, hw, 1) * m2);
  pr[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, hw, 2) * m2);
  pr[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, hw, 3) * m2);
  pr[4] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, hw, 0) * m2);
  pr[5] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, hw, 1) * m2);
  pr[6] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, hw, 2) * m2);
  pr[7] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, hw, 3) * m2);
}
// The two factors of an E4M3 scale code c for the FP4 dequantisation above,
// as one table entry: .x = the float power of two 2^(E-7) (2^-6 for a
// subnormal scale, E = 0), .y = its mantissa part twice as an fp16 pair
// (1 + M/8, or M/8 for E = 0). Filled once per work-group into LDS.
__device__ __forceinline__ uint2 scale_entry(uint32_t c) {
  const uint32_t E = (c >> 3) & 15u, M = c & 7u;
  const uint32_t hw = E ? (E + 120u) << 23 : 118u << 23;
  const _Float16 mf = E ? __builtin_bit_cast(_Float16, (uint16_t)(0x3C00u | (M << 7)))
                        : (_Float16)(float)M;
  const uint32_t mb = __builtin_bit_cast(uint16_t, mf);
  return make_uint2(hw, mb | (mb << 16));
}
// 16 FP4 codes with their scale's table entry -> 8 fp16 pairs (exact).
__device__ __forceinline__ void fp4x16_to_f16_t(uint32_t w0, uint32_t w1, uint2 e, uint32_t* pr) {
  const float hw = __uint_as_float(e.x);
  const v2h m2 = __builtin_bit_cast(v2h, e.y);
  pr[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, hw, 0) * m2);
  pr[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, hw, 1) * m2);
  pr[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, hw, 2) * m2);
  pr[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, hw, 3) * m2);
  pr[4] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, hw, 0) * m2);
  pr[5] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, hw, 1) * m2);
  pr[6] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, hw, 2) * m2);
  pr[7] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, hw, 3) * m2);
}
// 4 E4M3 bytes -> 2 fp16 pairs (exact).
__device__ __forceinline__ void fp8x4_to_f16(uint32_t w, uint32_t* pr) {
  pr[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  pr[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// Maximum over each 32-lane half of a wave (DPP within 16-lane rows, then
// v_permlane16_swap across the two rows of the half).
__device__ __forceinline__ float half_max(float m) {
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x141, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x140, 0xF, 0xF, false)));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}


// ------------------------------------------------------- decode kernel --

// Decode shape: 5 slices of 128 key slots (slices 0-3 hold the selected rows,
// slice 4 the window), one work-group of 8 waves per (query, 16-head group,
// slice). Lane (grp, col) of wave w dequantises channels 128grp..128grp+127 of
// key 16w + col into its Q.K operand registers and the slice's row-major LDS
// copy; wave w forms the logits of its 16 keys for the 16 heads and publishes
// its per-head maximum; with the slice maximum (after a barrier) it writes
// p = exp(z - max) of its keys (fp16 hi + lo) and their sum; after a second
// barrier wave w accumulates P.V for output channels 64w..64w+63 over the 128
// keys, reading V through the transposing LDS read (ds_read_b64_tr_b16). The
// slices are merged by log-sum-exp in a second kernel.
constexpr int kDecSplits = 5;
constexpr int kDecKeys = kSlots / kDecSplits;     // 128 key slots per work-group
constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kPRow = kDecKeys + 8;               // fp16 elements per LDS row of P
static_assert(kDecKeys == 16 * kDecWaves, "one 16-key tile per wave");
static_assert(kTopK % kDecKeys == 0, "a slice holds only selected rows or only window rows");

__global__ __launch_bounds__(kDecThreads) void k_sparse_attn_decode(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t krow[kDecKeys * kVRow];
  // fp16 query [16 heads][kVRow] until the logits are formed, then P
  // (hi, lo) [16 heads][kPRow] each
  constexpr int kQP = kHG * kVRow > 2 * kHG * kPRow ? kHG * kVRow : 2 * kHG * kPRow;
  __shared__ __attribute__((aligned(16))) uint16_t qp_buf[kQP];
  __shared__ float wmax[kDecWaves][kHG];
  __shared__ float wsum[kDecWaves][kHG];
  __shared__ int qsh[kHG];
  uint16_t* const qf = qp_buf;
  uint16_t* const pbuf = qp_buf;   // P hi at [0, kHG*kPRow), lo after it

  // ids 32j + 8g + x: unit 8j + x = (query, slice), head group g (the four
  // head-group work-groups of a unit gather the same rows: one XCD, one L2)
  const int id = blockIdx.x;
  const int unit = (id / (kXcds * kHeadGroups)) * kXcds + id % kXcds;
  const int hg = (id % (kXcds * kHeadGroups)) / kXcds;
  if (unit >= a.Q * kDecSplits) return;            // the whole work-group, before any barrier
  const int qi = unit / kDecSplits;
  const int split = unit % kDecSplits;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int b = qi / a.T;
  const int slot0 = split * kDecKeys;
  const bool is_main = slot0 < kTopK;

  // ---- loads. Lane (grp, col) of wave w loads key 16w + col of the slice:
  // channels 128grp .. 128grp+127 of its row. Q.K runs over a permuted channel
  // order that both operands share: MFMA step kb takes channels
  // 128grp + 8kb .. +7 in lane group grp, so each lane's key operand is its own
  // dequantised row slice and needs no LDS round trip.
  const int kk = wave * 16 + col;           // this lane's key in the slice
  int32_t pj = 0;
  if (is_main) pj = a.idx[(size_t)qi * kTopK + slot0 + kk];
  // query staging: wave w converts heads 2w, 2w+1 (lane: head 2w + lane/32,
  // channels 16*(lane%32) .. +15)
  const int qh = 2 * wave + (lane >> 5), qc = 16 * (lane & 31);
  const uint4* qsrc = reinterpret_cast<const uint4*>(
      a.q + ((size_t)qi * kHeads + hg * kHG + qh) * kDim + qc);
  const uint4 qr0 = qsrc[0], qr1 = qsrc[1];
  uint4 raw[8];          // FP4: raw[0..3] codes, raw[4].xy scales; FP8: raw[0..7]
  bool ok;
  if (is_main) {
    ok = pj >= 0 && (int64_t)pj < a.n_cap;
    const uint8_t* row = a.cache + ((size_t)b * (size_t)a.n_cap + (size_t)(ok ? pj : 0)) * kRowBytes;
    const uint4* c4 = reinterpret_cast<const uint4*>(row + 64 * grp);
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = c4[i];
    const uint2 sc = *reinterpret_cast<const uint2*>(row + kCodeBytes + 8 * grp);
    raw[4] = make_uint4(sc.x, sc.y, 0u, 0u);
  } else {
    const int64_t tq = a.q_pos[qi], pos0 = a.swa_pos0[b];
    const int64_t tok = tq - (kWindow - 1) + (slot0 + kk - kTopK);
    ok = tok >= 0 && tok >= pos0 && tok < pos0 + a.S;
    const int64_t rr = !ok ? 0 : (a.ring ? tok % a.S : tok - pos0);
    const uint4* r4 = reinterpret_cast<const uint4*>(
        a.swa + ((size_t)b * (size_t)a.S + (size_t)rr) * kDim + 128 * grp);
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = r4[i];
  }

  // ---- the query in fp16, each head shifted by a power of two (q_shift)
  {
    const float amax = half_max(fmaxf(bf16x8_absmax(qr0), bf16x8_absmax(qr1)));
    const int sh = q_shift(amax);
    const v8h h0 = q_to_f16(qr0, sh), h1 = q_to_f16(qr1, sh);
    *reinterpret_cast<v8h*>(&qf[qh * kVRow + qc]) = h0;
    *reinterpret_cast<v8h*>(&qf[qh * kVRow + qc + 8]) = h1;
    if ((lane & 31) == 0) qsh[qh] = sh;
  }
  lds_barrier();
  v8h qreg[16];
#pragma unroll
  for (int kb = 0; kb < 16; ++kb)
    qreg[kb] = *reinterpret_cast<const v8h*>(&qf[col * kVRow + 128 * grp + 8 * kb]);
  const float zscale = ldexpf(a.scale, -qsh[col]);

  // ---- dequantise this lane's 128 channels: the Q.K operand in registers and
  // the row-major copy in LDS for P.V
  v8h kreg[16];
  {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(raw);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      uint32_t pr[8];
      if (is_main) {
        fp4x16_to_f16(w[2 * m], w[2 * m + 1], (w[16 + m / 4] >> (8 * (m % 4))) & 0xFFu, pr);
      } else {
        fp8x4_to_f16(w[4 * m + 0], pr + 0);
        fp8x4_to_f16(w[4 * m + 1], pr + 2);
        fp8x4_to_f16(w[4 * m + 2], pr + 4);
        fp8x4_to_f16(w[4 * m + 3], pr + 6);
      }
      const uint4 lo = ok ? make_uint4(pr[0], pr[1], pr[2], pr[3]) : make_uint4(0u, 0u, 0u, 0u);
      const uint4 hi = ok ? make_uint4(pr[4], pr[5], pr[6], pr[7]) : make_uint4(0u, 0u, 0u, 0u);
      kreg[2 * m] = __builtin_bit_cast(v8h, lo);
      kreg[2 * m + 1] = __builtin_bit_cast(v8h, hi);
      uint4* dst = reinterpret_cast<uint4*>(&krow[kk * kVRow + 128 * grp + 16 * m]);
      dst[0] = lo;
      dst[1] = hi;
    }
  }
  // presence of keys 16w .. 16w+15 (lanes 0..15 hold them), wave-uniform
  const uint32_t kmask = (uint32_t)__ballot(ok) & 0xFFFFu;

  // ---- phase 2: logits of keys 16w..16w+15 (lane: keys 4grp+r, head col),
  // four independent accumulation chains
  v4f s;
  {
    v4f sc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) sc[c] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 16; ++kb)
      sc[kb & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kreg[kb], qreg[kb], sc[kb & 3], 0, 0, 0);
    s = (sc[0] + sc[1]) + (sc[2] + sc[3]);
  }
  float z[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) z[r] = ((kmask >> (4 * grp + r)) & 1u) ? s[r] * zscale : -INFINITY;
  const float mloc = rows_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
  if (grp == 0) wmax[wave][col] = mloc;
  lds_barrier();
  float M = wmax[0][col];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) M = fmaxf(M, wmax[w][col]);
  {
    float p[4], psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = M == -INFINITY ? 0.0f : __expf(z[r] - M);
      psum += p[r];
    }
    psum = rows_sum(psum);
    if (grp == 0) wsum[wave][col] = psum;
    v4h ph, pl;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const _Float16 h = (_Float16)p[r];
      ph[r] = h;
      pl[r] = (_Float16)(p[r] - (float)h);
    }
    // (every wave has read the query from this buffer before the barrier above)
    *reinterpret_cast<v4h*>(&pbuf[col * kPRow + wave * 16 + 4 * grp]) = ph;
    *reinterpret_cast<v4h*>(&pbuf[kHG * kPRow + col * kPRow + wave * 16 + 4 * grp]) = pl;
  }
  lds_barrier();
  float l = 0.0f;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) l += wsum[w][col];

  // ---- phase 3: P.V for channels 64w..64w+63 (lane: channels 4grp+r of each
  // 16-channel tile, head col). The transposing read hands lane (grp, i) the
  // values of channel c0 + i for keys k0 + 4grp .. +3 when lane (grp, m)
  // points at key k0 + 4grp + m/4, channels c0 + 4(m%4) .. +3.
  // 32 keys per MFMA (v_mfma_f32_16x16x32_f16): lane (grp, i) takes keys
  // 32ks + 8grp .. +7 of channel i, as two transposing reads of 4 keys each.
  // Operands are requested two key steps ahead of their MFMAs.
  constexpr int kKs = kDecKeys / 32;
  v8h ph[kKs], pl[kKs], vv[kKs][4];
  auto fetch = [&](int ks) __attribute__((always_inline)) {
    ph[ks] = *reinterpret_cast<const v8h*>(&pbuf[col * kPRow + ks * 32 + 8 * grp]);
    pl[ks] = *reinterpret_cast<const v8h*>(&pbuf[kHG * kPRow + col * kPRow + ks * 32 + 8 * grp]);
    const uint16_t* vsrc =
        &krow[(ks * 32 + 8 * grp + (col >> 2)) * kVRow + wave * 64 + 4 * (col & 3)];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(vsrc + dt * 16));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(vsrc + 4 * kVRow + dt * 16));
      vv[ks][dt] = __builtin_bit_cast(v8h, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  v4f acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  fetch(0);
  fetch(1);
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks) {
    if (ks + 2 < kKs) fetch(ks + 2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vv[ks][dt], ph[ks], acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vv[ks][dt], pl[ks], acc[dt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // lane holds head 16hg + col, channels 64w + 16dt + 4grp .. +3
  const int head = hg * kHG + col;
  const size_t ps = (size_t)qi * kDecSplits + split;
  float* o = a.part + (ps * kHeads + head) * kDim + wave * 64 + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    *reinterpret_cast<float4*>(o + dt * 16) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
  if (wave == 0 && grp == 0) {
    a.part_ml[(ps * kHeads + head) * 2 + 0] = M;
    a.part_ml[(ps * kHeads + head) * 2 + 1] = l;
  }
}

// Raw bytes of one lane's share of a 16-key tile: FP4 rows v[0..3] codes and
// v[4].xy the 8 scale bytes; window rows v[0..7].
struct Raw {
  uint4 v[8];
};

// 13 <= Q < 512: one 8-wave work-group per (query, 16 heads). Wave pair p
// (waves p and p + 4) takes the 32-key steps p, p+4, p+8, p+12 (selected
// rows) and 16+p (window); in each step wave p + 4h dequantises the step's 16
// keys 16h..16h+15 and forms their logits for the 16 heads, the pair swaps
// logits through LDS, both waves run the same online softmax over the 32 keys
// and wave p + 4h accumulates P.V for output channels 256h..256h+255.
__global__ __launch_bounds__(kThreads) void k_sparse_attn_hg(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[kPairs * kStepKeys * kVRow];
  __shared__ __attribute__((aligned(16))) float4 zx[kPairs][2][64];   // logits swapped in a pair
  __shared__ int qsh[kHG];
  __shared__ float2 mlbuf[kPairs][kHG];
  __shared__ uint2 stab[256];                      // E4M3 scale code -> dequantisation factors

  // ids 32j + 8g + x: query 8j + x, head group g (a query's four work-groups
  // are equal mod 8: one XCD)
  const int id = blockIdx.x;
  const int qi = (id / (kXcds * kHeadGroups)) * kXcds + id % kXcds;
  const int hg = (id % (kXcds * kHeadGroups)) / kXcds;
  if (qi >= a.Q) return;                           // the whole work-group, before any barrier
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int pair = wave % kPairs, half = wave / kPairs;
  const int col = lane & 15, grp = lane >> 4;
  const int b = qi / a.T;
  const int64_t tq = a.q_pos[qi], pos0 = a.swa_pos0[b];

  // first slot of this wave's 16 keys in step s (lane: key col)
  auto tile_slot = [&](int s) __attribute__((always_inline)) -> int {
    return (s < kMainSteps ? kStepKeys * (pair + kPairs * s) : kTopK + kStepKeys * pair) + 16 * half;
  };
  int32_t pj[kMainSteps];
#pragma unroll
  for (int s = 0; s < kMainSteps; ++s) pj[s] = a.idx[(size_t)qi * kTopK + tile_slot(s) + col];
  const uint8_t* cache_b = a.cache + (size_t)b * (size_t)a.n_cap * kRowBytes;
  const uint8_t* swa_b = a.swa + (size_t)b * (size_t)a.S * kDim;
  // this lane's share of its tile of step s: key col, channels 128grp .. 128grp+127
  auto load = [&](int s, Raw& r) __attribute__((always_inline)) -> bool {
    bool ok;
    if (s < kMainSteps) {
      const int32_t p = pj[s];
      ok = p >= 0 && (int64_t)p < a.n_cap;
      const uint8_t* row = cache_b + (size_t)(ok ? p : 0) * kRowBytes;
      const uint4* c4 = reinterpret_cast<const uint4*>(row + 64 * grp);
#pragma unroll
      for (int i = 0; i < 4; ++i) r.v[i] = c4[i];
      const uint2 sc = *reinterpret_cast<const uint2*>(row + kCodeBytes + 8 * grp);
      r.v[4] = make_uint4(sc.x, sc.y, 0u, 0u);
    } else {
      const int64_t tok = tq - (kWindow - 1) + (tile_slot(s) + col - kTopK);
      ok = tok >= 0 && tok >= pos0 && tok < pos0 + a.S;
      const int64_t rr = !ok ? 0 : (a.ring ? tok % a.S : tok - pos0);
      const uint4* r4 = reinterpret_cast<const uint4*>(swa_b + (size_t)rr * kDim + 128 * grp);
#pragma unroll
      for (int i = 0; i < 8; ++i) r.v[i] = r4[i];
    }
    return ok;
  };

  // the first step's rows are requested before the query is set up
  Raw raw;
  bool okr = load(0, raw);

  if (threadIdx.x < 256) stab[threadIdx.x] = scale_entry(threadIdx.x);

  // ---- the query in fp16, staged in the key tiles: wave w converts heads 2w,
  // 2w+1 (lane: head 2w + lane/32, channels 16(lane%32) .. +15), each head
  // shifted by a power of two
  uint16_t* const qf = vbuf;
  {
    const int qh = 2 * wave + (lane >> 5), qc = 16 * (lane & 31);
    const uint4* qsrc = reinterpret_cast<const uint4*>(
        a.q + ((size_t)qi * kHeads + hg * kHG + qh) * kDim + qc);
    const uint4 q0 = qsrc[0], q1 = qsrc[1];
    const int sh = q_shift(half_max(fmaxf(bf16x8_absmax(q0), bf16x8_absmax(q1))));
    *reinterpret_cast<v8h*>(&qf[qh * kVRow + qc]) = q_to_f16(q0, sh);
    *reinterpret_cast<v8h*>(&qf[qh * kVRow + qc + 8]) = q_to_f16(q1, sh);
    if ((lane & 31) == 0) qsh[qh] = sh;
  }
  lds_barrier();
  v8h qreg[16];
#pragma unroll
  for (int kb = 0; kb < 16; ++kb)
    qreg[kb] = *reinterpret_cast<const v8h*>(&qf[col * kVRow + 128 * grp + 8 * kb]);
  const float zscale = ldexpf(a.scale, -qsh[col]);
  lds_barrier();                                   // every wave holds the query: the tiles are free

  uint16_t* const vw = vbuf + pair * kStepKeys * kVRow;   // this pair's 32 key rows
  v4f acc[kHalfTiles];
#pragma unroll
  for (int j = 0; j < kHalfTiles; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const bool main_rows = s < kMainSteps;         // a compile-time constant per step
    // ---- dequantise this wave's 16 keys: the Q.K operand in registers and
    // rows 16half + col of the pair's tile
    float4 z;
    {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(raw.v);
      const bool ok = okr;
      v4f sc[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) sc[c] = v4f{0.f, 0.f, 0.f, 0.f};
      // a skipped key dequantises to zeros: an FP4 row through a zero scale
      // (any code times 0), a window row through zeroed bytes (its bytes could
      // hold NaN codes)
      const uint32_t sc0 = ok ? w[16] : 0u, sc1 = ok ? w[17] : 0u;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        uint32_t pr[8];
        if (main_rows) {
          const uint32_t c = ((m < 4 ? sc0 : sc1) >> (8 * (m % 4))) & 0xFFu;
          fp4x16_to_f16_t(w[2 * m], w[2 * m + 1], stab[c], pr);
        } else {
          fp8x4_to_f16(ok ? w[4 * m + 0] : 0u, pr + 0);
          fp8x4_to_f16(ok ? w[4 * m + 1] : 0u, pr + 2);
          fp8x4_to_f16(ok ? w[4 * m + 2] : 0u, pr + 4);
          fp8x4_to_f16(ok ? w[4 * m + 3] : 0u, pr + 6);
        }
        const uint4 lo = make_uint4(pr[0], pr[1], pr[2], pr[3]);
        const uint4 hi = make_uint4(pr[4], pr[5], pr[6], pr[7]);
        sc[(2 * m) & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, lo),
                                                                 qreg[2 * m], sc[(2 * m) & 3], 0, 0, 0);
        sc[(2 * m + 1) & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            __builtin_bit_cast(v8h, hi), qreg[2 * m + 1], sc[(2 * m + 1) & 3], 0, 0, 0);
        uint4* dst = reinterpret_cast<uint4*>(&vw[(16 * half + col) * kVRow + 128 * grp + 16 * m]);
        dst[0] = lo;
        dst[1] = hi;
      }
      // presence of the 16 keys (lanes 0..15 hold them), wave-uniform
      const uint32_t kmask = (uint32_t)__ballot(ok) & 0xFFFFu;
      // the next step's rows are requested now
      if (s + 1 < kSteps) okr = load(s + 1, raw);
      const v4f sv = (sc[0] + sc[1]) + (sc[2] + sc[3]);
      // lane (grp, col): logits of keys 4grp + r for head col
      z.x = ((kmask >> (4 * grp + 0)) & 1u) ? sv[0] * zscale : -INFINITY;
      z.y = ((kmask >> (4 * grp + 1)) & 1u) ? sv[1] * zscale : -INFINITY;
      z.z = ((kmask >> (4 * grp + 2)) & 1u) ? sv[2] * zscale : -INFINITY;
      z.w = ((kmask >> (4 * grp + 3)) & 1u) ? sv[3] * zscale : -INFINITY;
    }
    zx[pair][half][lane] = z;
    lds_barrier();                                   // both halves' rows and logits are in LDS
    const float4 zo = zx[pair][half ^ 1][lane];
    // P's k index 8grp + 4t + r is key 16t + 4grp + r of the step (t: the half)
    const float4 zt0 = half == 0 ? z : zo, zt1 = half == 0 ? zo : z;
    const float zz[8] = {zt0.x, zt0.y, zt0.z, zt0.w, zt1.x, zt1.y, zt1.z, zt1.w};

    // ---- online softmax for head col over this step's 32 keys (the same in
    // both waves of the pair)
    float zmax = zz[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) zmax = fmaxf(zmax, zz[i]);
    zmax = rows_max(zmax);
    const bool raise = zmax > m_run + kLazyMax || (m_run == -INFINITY && zmax > -INFINITY);
    const float m_new = raise ? zmax : m_run;
    const float alpha = (raise && m_run != -INFINITY) ? __expf(m_run - m_new) : 1.0f;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int j = 0; j < kHalfTiles; ++j) acc[j] *= alpha;
    }
    float psum = 0.0f;
    v8h ph, pl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pv = m_new == -INFINITY ? 0.0f : __expf(zz[i] - m_new);
      psum += pv;
      const _Float16 h = (_Float16)pv;
      ph[i] = h;
      pl[i] = (_Float16)(pv - (float)h);
    }
    l_run = l_run * alpha + rows_sum(psum);
    m_run = m_new;

    // ---- P.V over output channels 256half..: lane (grp, i) reads channel
    // 16ct + i of keys 4grp..+3 of each half (lane (grp, m) points at key
    // 4grp + m/4, channels 16ct + 4(m%4)..+3); four channel tiles at a time,
    // their hi MFMAs before their lo MFMAs
    const uint16_t* vsrc = &vw[(4 * grp + (col >> 2)) * kVRow + 4 * (col & 3) + 256 * half];
#pragma unroll
    for (int cg = 0; cg < kHalfTiles; cg += kPvGroup) {
      v8h v[kPvGroup];
#pragma unroll
      for (int j = 0; j < kPvGroup; ++j) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(vsrc + 16 * (cg + j)));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(vsrc + 16 * kVRow + 16 * (cg + j)));
        v[j] = __builtin_bit_cast(v8h, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int j = 0; j < kPvGroup; ++j)
        acc[cg + j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v[j], ph, acc[cg + j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < kPvGroup; ++j)
        acc[cg + j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v[j], pl, acc[cg + j], 0, 0, 0);
    }
    lds_barrier();                                   // tile reads done before the next step writes
  }

  // ---- merge the four pairs by log-sum-exp and write the 16 heads' output
  if (half == 0 && grp == 0) mlbuf[pair][col] = make_float2(m_run, l_run);
  __syncthreads();
  float M = mlbuf[0][col].x;
#pragma unroll
  for (int w = 1; w < kPairs; ++w) M = fmaxf(M, mlbuf[w][col].x);
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < kPairs; ++w)
    L += mlbuf[w][col].x == -INFINITY ? 0.0f : __expf(mlbuf[w][col].x - M) * mlbuf[w][col].y;
  const float f = (m_run == -INFINITY || !(L > 0.0f)) ? 0.0f : __expf(m_run - M) / L;
  // lane (grp, col) holds channels 256half + 16j + 4grp .. +3 of head col
  float* stage = reinterpret_cast<float*>(vbuf);
#pragma unroll
  for (int j = 0; j < kHalfTiles; ++j)
    *reinterpret_cast<float4*>(&stage[(wave * kHG + col) * kOutRow + 16 * j + 4 * grp]) =
        make_float4(acc[j][0] * f, acc[j][1] * f, acc[j][2] * f, acc[j][3] * f);
  __syncthreads();
  float* out = a.out + ((size_t)qi * kHeads + hg * kHG) * kDim;
#pragma unroll
  for (int i = 0; i < kHG * kDim / 4 / kThreads; ++i) {
    const int e = (int)threadIdx.x + kThreads * i;   // float4 index over 16 heads x 128
    const int h = e / (kDim / 4), c4 = e % (kDim / 4);
    const int hw = c4 / (kDim / 8), cl = 4 * (c4 % (kDim / 8));   // channel half, channel in it
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kPairs; ++w) {
      const float4 x = *reinterpret_cast<const float4*>(
          &stage[((w + kPairs * hw) * kHG + h) * kOutRow + cl]);
      o.x += x.x;
      o.y += x.y;
      o.z += x.z;
      o.w += x.w;
    }
    *reinterpret_cast<float4*>(&out[(size_t)h * kDim + 4 * c4]) = o;
  }
}

// ------------------------------------------------------ prefill kernel --

// 512 queries or more: one 8-wave work-group per query over its 640 key slots
// in 10 chunks of 64 (chunks 0-7 selected rows, 8-9 the window), online
// softmax across chunks. Wave w serves heads 16(w%4)..+15: for Q.K it takes
// 32 of the chunk's keys (w/4 picks the half), for P.V output channels
// 256(w/4)..+255 over all 64 keys. Per chunk: the next chunk's rows are
// requested; barrier (this chunk is in one of two row-major fp16 LDS buffers);
// Q.K with the keys read from LDS and the query in registers; the two waves of
// a head group exchange their maxima; barrier; p (fp16 hi + lo) into LDS;
// barrier; the 512 threads dequantise the next chunk (8 threads per key, 64
// channels each) into the other buffer while P.V runs with V read by
// ds_read_b64_tr_b16.
constexpr int kPfKeys = 64;                       // keys per chunk
constexpr int kPfChunks = kSlots / kPfKeys;       // 10
constexpr int kPfWavesA = 8;
constexpr int kPfThreadsA = kPfWavesA * 64;
constexpr int kPRowPf = kPfKeys + 8;              // fp16 per LDS row of P
static_assert(kTopK % kPfKeys == 0, "a chunk holds only selected rows or only window rows");
static_assert(kPfThreadsA == kPfKeys * 8, "8 threads per key in the dequantisation");

__global__ __launch_bounds__(kPfThreadsA) void k_sparse_attn_prefill(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t krow[2][kPfKeys * kVRow];
  __shared__ __attribute__((aligned(16))) uint16_t pbuf[2][kHeads * kPRowPf];   // hi, lo
  __shared__ float cmax[kPfWavesA][kHG];
  __shared__ float csum[kPfWavesA][kHG];
  __shared__ int kvalid[2][kPfKeys];

  const int qi = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int hg = wave & 3, half = wave >> 2;
  const int col = lane & 15, grp = lane >> 4;
  const int b = qi / a.T;
  const int64_t tq = a.q_pos[qi], pos0 = a.swa_pos0[b];

  // ---- dequantisation role: key dk of each chunk, channels 64*dc .. +63
  const int dk = (int)threadIdx.x >> 3, dc = (int)threadIdx.x & 7;
  int32_t pj[kTopK / kPfKeys];
#pragma unroll
  for (int c = 0; c < kTopK / kPfKeys; ++c) pj[c] = a.idx[(size_t)qi * kTopK + c * kPfKeys + dk];
  const uint8_t* cache_b = a.cache + (size_t)b * (size_t)a.n_cap * kRowBytes;
  const uint8_t* swa_b = a.swa + (size_t)b * (size_t)a.S * kDim;
  // raw bytes of this thread's piece of chunk c: FP4 r[0..1] codes, r[2].x
  // scales; FP8 r[0..3]
  auto load = [&](int c, uint4 (&r)[4]) __attribute__((always_inline)) -> bool {
    bool v;
    if (c * kPfKeys < kTopK) {
      int32_t p = pj[0];
#pragma unroll
      for (int i = 1; i < kTopK / kPfKeys; ++i) p = c == i ? pj[i] : p;
      v = p >= 0 && (int64_t)p < a.n_cap;
      const uint8_t* row = cache_b + (size_t)(v ? p : 0) * kRowBytes;
      const uint4* c4 = reinterpret_cast<const uint4*>(row + 32 * dc);
      r[0] = c4[0];
      r[1] = c4[1];
      r[2].x = *reinterpret_cast<const uint32_t*>(row + kCodeBytes + 4 * dc);
    } else {
      const int64_t tok = tq - (kWindow - 1) + (c * kPfKeys + dk - kTopK);
      v = tok >= 0 && tok >= pos0 && tok < pos0 + a.S;
      const int64_t rr = !v ? 0 : (a.ring ? tok % a.S : tok - pos0);
      const uint4* r4 = reinterpret_cast<const uint4*>(swa_b + (size_t)rr * kDim + 64 * dc);
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = r4[i];
    }
    return v;
  };
  auto store = [&](int c, const uint4 (&r)[4], bool v) __attribute__((always_inline)) {
    uint32_t pr[32];
    if (c * kPfKeys < kTopK) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(r);
#pragma unroll
      for (int m = 0; m < 4; ++m) fp4x16_to_f16(w[2 * m], w[2 * m + 1], (r[2].x >> (8 * m)) & 0xFFu, pr + 8 * m);
    } else {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(r);
#pragma unroll
      for (int m = 0; m < 16; ++m) fp8x4_to_f16(w[m], pr + 2 * m);
    }
    uint4* dst = reinterpret_cast<uint4*>(&krow[c & 1][dk * kVRow + 64 * dc]);
#pragma unroll
    for (int m = 0; m < 8; ++m)
      dst[m] = v ? make_uint4(pr[4 * m], pr[4 * m + 1], pr[4 * m + 2], pr[4 * m + 3])
                 : make_uint4(0u, 0u, 0u, 0u);
    if (dc == 0) kvalid[c & 1][dk] = v;
  };

  uint4 raw[4];
  bool rv = load(0, raw);

  // ---- the query of heads 16hg..+15 (lane: head col, channels kb*32+8grp..+7)
  v8h qreg[16];
  float zscale;
  {
    const uint16_t* qp = a.q + ((size_t)qi * kHeads + hg * kHG + col) * kDim + grp * 8;
    uint4 qr[16];
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) qr[kb] = *reinterpret_cast<const uint4*>(qp + kb * 32);
    float amax = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) amax = fmaxf(amax, bf16x8_absmax(qr[kb]));
    const int sh = q_shift(rows_max(amax));
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) qreg[kb] = q_to_f16(qr[kb], sh);
    zscale = ldexpf(a.scale, -sh);
  }

  v4f acc[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) acc[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  store(0, raw, rv);
  for (int c = 0; c < kPfChunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < kPfChunks) rv = load(c + 1, raw);
    lds_barrier();   // chunk c is in krow[buf]

    // Q.K: keys 32*half + 16kt + 4grp + r, head col
    float z[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      v4f sc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
      const uint16_t* kr = &krow[buf][(32 * half + 16 * kt + col) * kVRow + grp * 8];
#pragma unroll
      for (int kb = 0; kb < 16; ++kb) {
        const v8h kv = *reinterpret_cast<const v8h*>(kr + kb * 32);
        sc[kb & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, qreg[kb], sc[kb & 1], 0, 0, 0);
      }
      const v4f s = sc[0] + sc[1];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        z[kt][r] = kvalid[buf][32 * half + 16 * kt + 4 * grp + r] ? s[r] * zscale : -INFINITY;
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, z[kt][r]);
    mloc = rows_max(mloc);
    if (grp == 0) cmax[wave][col] = mloc;
    lds_barrier();
    const float mc = fmaxf(cmax[hg][col], cmax[hg + 4][col]);
    const float m_new = fmaxf(m_run, mc);
    const float alpha = m_new == -INFINITY ? 1.0f : __expf(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      v4h ph, pl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = m_new == -INFINITY ? 0.0f : __expf(z[kt][r] - m_new);
        psum += p;
        const _Float16 h = (_Float16)p;
        ph[r] = h;
        pl[r] = (_Float16)(p - (float)h);
      }
      const int off = (hg * kHG + col) * kPRowPf + 32 * half + 16 * kt + 4 * grp;
      *reinterpret_cast<v4h*>(&pbuf[0][off]) = ph;
      *reinterpret_cast<v4h*>(&pbuf[1][off]) = pl;
    }
    psum = rows_sum(psum);
    if (grp == 0) csum[wave][col] = psum;
    m_run = m_new;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) acc[dt] *= alpha;
    }
    lds_barrier();   // P of chunk c is complete
    l_run = l_run * alpha + (csum[hg][col] + csum[hg + 4][col]);
    // the next chunk is dequantised into the other buffer here, so its vector
    // work overlaps this chunk's P.V
    if (c + 1 < kPfChunks) store(c + 1, raw, rv);

    // P.V: channels 256*half + 16dt + 4grp + r, head col
#pragma unroll
    for (int ks = 0; ks < kPfKeys / 32; ++ks) {
      const int poff = (hg * kHG + col) * kPRowPf + ks * 32 + 8 * grp;
      const v8h ph = *reinterpret_cast<const v8h*>(&pbuf[0][poff]);
      const v8h pl = *reinterpret_cast<const v8h*>(&pbuf[1][poff]);
      const uint16_t* vsrc =
          &krow[buf][(ks * 32 + 8 * grp + (col >> 2)) * kVRow + 256 * half + 4 * (col & 3)];
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(vsrc + dt * 16));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(vsrc + 4 * kVRow + dt * 16));
        const v8h v = __builtin_bit_cast(v8h, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v, ph, acc[dt], 0, 0, 0);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v, pl, acc[dt], 0, 0, 0);
      }
    }
  }

  // lane holds head 16hg + col, channels 256*half + 16dt + 4grp .. +3
  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  float* o = a.out + ((size_t)qi * kHeads + hg * kHG + col) * kDim + 256 * half + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < 16; ++dt)
    *reinterpret_cast<float4*>(o + dt * 16) =
        make_float4(acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv, acc[dt][3] * inv);
}

// One work-group per (query, head); 128 threads x 4 channels. Every load is
// independent of the others (one round trip), then the slices are combined.
constexpr int kMaxSplits = 8;
__global__ __launch_bounds__(128) void k_attn_merge(const float* __restrict__ part,
                                                    const float* __restrict__ part_ml, int splits,
                                                    float* __restrict__ out) {
  const int qi = blockIdx.y, head = blockIdx.x;
  float m[kMaxSplits], l[kMaxSplits];
  float4 v[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    if (s < splits) {
      const size_t ps = (size_t)qi * splits + s;
      m[s] = part_ml[(ps * kHeads + head) * 2];
      l[s] = part_ml[(ps * kHeads + head) * 2 + 1];
      v[s] = *reinterpret_cast<const float4*>(part + (ps * kHeads + head) * kDim + threadIdx.x * 4);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < splits) M = fmaxf(M, m[s]);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.0f;
  if (M != -INFINITY) {
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
      if (s < splits) {
        const float wgt = m[s] == -INFINITY ? 0.0f : __expf(m[s] - M);
        L += wgt * l[s];
        o.x += wgt * v[s].x;
        o.y += wgt * v[s].y;
        o.z += wgt * v[s].z;
        o.w += wgt * v[s].w;
      }
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  *reinterpret_cast<float4*>(out + ((size_t)qi * kHeads + head) * kDim + threadIdx.x * 4) =
      make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
}

}  // namespace

size_t attn_workspace_bytes(int Q) {
  if (Q >= kDecodeMaxQueries) return 0;
  return (size_t)Q * kDecSplits * kHeads * (kDim + 2) * sizeof(float);
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* cache, const int32_t* idx,
                              const uint8_t* swa, const int64_t* q_pos, const int64_t* swa_pos0,
                              int B, int T, int64_t n_cap, int S, int ring, float scale, float* out,
                              void* ws, hipStream_t st) {
  AttnArgs a;
  a.q = q;
  a.cache = cache;
  a.idx = idx;
  a.swa = swa;
  a.q_pos = q_pos;
  a.swa_pos0 = swa_pos0;
  a.T = T;
  a.Q = B * T;
  a.n_cap = n_cap;
  a.S = S;
  a.ring = ring;
  a.scale = scale;
  a.out = out;
  a.part = nullptr;
  a.part_ml = nullptr;
  if (a.Q >= kPrefillMinQueries) {
    hipLaunchKernelGGL(k_sparse_attn_prefill, dim3((unsigned)a.Q), dim3(kPfThreadsA), 0, st, a);
  } else if (a.Q >= kDecodeMaxQueries) {
    const int groups = (a.Q + kXcds - 1) / kXcds;
    hipLaunchKernelGGL(k_sparse_attn_hg, dim3((unsigned)(groups * kXcds * kHeadGroups)),
                       dim3(kThreads), 0, st, a);
  } else {
    if (!ws) return hipErrorInvalidValue;
    a.part = reinterpret_cast<float*>(ws);
    a.part_ml = a.part + (size_t)a.Q * kDecSplits * kHeads * kDim;
    const int units = a.Q * kDecSplits;
    const int groups = (units + kXcds - 1) / kXcds;
    hipLaunchKernelGGL(k_sparse_attn_decode, dim3((unsigned)(groups * kXcds * kHeadGroups)),
                       dim3(kDecThreads), 0, st, a);
    hipLaunchKernelGGL(k_attn_merge, dim3(kHeads, a.Q), dim3(128), 0, st, a.part, a.part_ml,
                       kDecSplits, out);
  }
  return hipGetLastError();
}

}  // namespace csa2
