// Sparse MQA attention over the selected FP4 main-KV rows plus the FP8 window.
//
// Pages: 64 heads of width 512 over the Top-512 selected entries
// ("DeepSeek V4.1-Flash 为什么这么强？CED 与 CSA2 架构全拆解", §二 layer layout)
// plus a 128-token sliding window (same page §一; "DeepSeek V4.1 Flash vs V4
// Pro", 黑科技之一); the FP4 main KV is dequantised before attention and the
// window KV stays FP8 ("DeepSeek-V4.1-Flash：全局 KV 仅 890 B/token", 第三刀);
// every layer has its own query and window ("DeepSeek V4.1 Flash vs V4 Pro",
// 黑科技之二). Key = value = the dequantised 512-wide row (reading in csa2.h).
//
// Keys are processed 32 at a time. Gather: thread t of the 256 owns channels
// 8p..8p+7 with p = 16*(t/64) + (t%16) -- so wave w owns channels
// 128w..128w+127 -- and keys 8g..8g+7 of the chunk with g = (t%64)/16. It loads
// the FP4 codes (4 bytes) and E4M3 scale of each of its keys, or 8 E4M3 bytes of
// a window row, dequantises them to fp16 (exact) with the gfx950 FP4/FP8
// converts and stores them in LDS twice:
//   krow -- row-major fp16 [key][channel], the A operand of Q.K;
//   vt   -- transposed fp16 [channel][key], the A operand of P.V. Its rows are
//           80 bytes (5 slots of 16 bytes for 4 chunks of 8 keys) and chunk c of
//           row d sits in slot (c + d/8) % 5, which spreads the 16-byte stores
//           of a wave over the LDS banks.
// Q.K: v_mfma_f32_16x16x32_f16 with keys as A and 16 query heads as B (kept in
// registers, each head scaled by a power of two into fp16 range; the logits are
// scaled back). Online softmax per head (one lane column of the 16x16 result).
// P.V: v_mfma_f32_16x16x32_f16 with the transposed keys as A and P as B. P is
// split as P = hi + lo with both parts in fp16 (two MFMAs per tile), which keeps
// the product accurate to about 2^-22 of P even when rows carry large outlier
// channels.
//
// Two work shapes:
//   wide   (512 queries or more): one work-group of 4 waves per query over all
//          640 key slots; wave w owns heads 16w..16w+15 and all 512 output
//          channels, so every gathered row serves all 64 heads;
//   decode (fewer than 512 queries): one work-group of 8 waves per (query, 16-head
//          group, slice of 128 key slots). Each lane dequantises 128 channels
//          of one key straight into its Q.K operand registers (both operands
//          use the same permuted channel order) and into a row-major fp16 copy
//          in LDS; wave w forms the logits of its 16 keys, the work-group
//          agrees on the slice maximum, and wave w accumulates P.V for output
//          channels 64w..64w+63, reading V through the gfx950 transposing LDS
//          read (ds_read_b64_tr_b16) so no transposed copy is stored. The query
//          is converted once per work-group (two heads per wave) and shared
//          through LDS.
//   Slices are merged by log-sum-exp in a second kernel.
#include "device_common.hpp"
#include "launchers.hpp"

#include <utility>

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkKeys = 32;
constexpr int kSlots = kTopK + kWindow;           // 640 key slots per query
constexpr int kChunks = kSlots / kChunkKeys;      // 20
constexpr int kKrowStride = kDim + 8;             // fp16 elements per LDS key row
constexpr int kVtRowHalves = 40;                  // fp16 elements per LDS channel row (80 B)
constexpr int kHG = 16;                           // heads per decode work-group
constexpr int kHeadGroups = kHeads / kHG;
constexpr int kWideMinQueries = 512;

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// Calls f(integral_constant<int, i>) for i = 0..N-1, fully unrolled.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// fp16 element offset of (channel row d, 16-byte key chunk c) in vt.
__device__ __forceinline__ int vt_off(int d, int c) {
  return d * kVtRowHalves + ((c + (d >> 3)) % 5) * 8;
}

struct AttnArgs {
  const uint16_t* q;
  const uint8_t* cache;
  const int32_t* idx;
  const uint8_t* swa;
  const int64_t* q_pos;
  const int64_t* swa_pos0;
  int T;
  int64_t n_cap;
  int S;
  float scale;
  float* out;
  float* part;     // [Q][splits][64][512] unnormalised outputs
  float* part_ml;  // [Q][splits][64][2] running max and sum
  int splits;
};

struct Gather {
  const uint8_t* cache_b;
  const uint8_t* swa_b;
  const int32_t* idx_q;
  int64_t n_cap, tq, pos0;
  int S, piece, kgrp;

  __device__ void init(const AttnArgs& a, int qi) {
    const int b = qi / a.T;
    cache_b = a.cache + (size_t)b * (size_t)a.n_cap * kRowBytes;
    swa_b = a.swa + (size_t)b * (size_t)a.S * kDim;
    idx_q = a.idx + (size_t)qi * kTopK;
    n_cap = a.n_cap;
    tq = a.q_pos[qi];
    pos0 = a.swa_pos0[b];
    S = a.S;
    const int t = threadIdx.x;
    piece = 16 * (t >> 6) + (t & 15);
    kgrp = (t & 63) >> 4;
  }

  // Raw bytes of this thread's 8 keys (8 channels each) of chunk `chunk`; bit j
  // of the result marks key j present. The selected positions come from `sidx`
  // (this work-group's slice of the index list, staged in LDS by stage_idx), so
  // no global load waits on another; every row load is issued unconditionally
  // (an absent key reads row 0, which exists, and is masked afterwards).
  __device__ __forceinline__ uint32_t load(int chunk, int chunk0, const int32_t* sidx,
                                           uint2 (&r)[8]) const {
    const int slot0 = chunk * kChunkKeys + kgrp * 8;
    uint32_t ok = 0;
    if (slot0 < kTopK) {
      const int4 i0 = *reinterpret_cast<const int4*>(sidx + (slot0 - chunk0 * kChunkKeys));
      const int4 i1 = *reinterpret_cast<const int4*>(sidx + (slot0 - chunk0 * kChunkKeys) + 4);
      const int32_t pj[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool v = pj[j] >= 0 && (int64_t)pj[j] < n_cap;
        ok |= (v ? 1u : 0u) << j;
        const uint8_t* row = cache_b + (size_t)(v ? pj[j] : 0) * kRowBytes;
        r[j].x = *reinterpret_cast<const uint32_t*>(row + piece * 4);
        r[j].y = row[kCodeBytes + (piece >> 1)];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t tok = tq - (kWindow - 1) + (slot0 + j - kTopK);
        const int64_t rr = tok - pos0;
        const bool v = tok >= 0 && rr >= 0 && rr < S;
        ok |= (v ? 1u : 0u) << j;
        r[j] = *reinterpret_cast<const uint2*>(swa_b + (size_t)(v ? rr : 0) * kDim + piece * 8);
      }
    }
    return ok;
  }

  // Copies the selected positions of chunks [chunk0, chunk0 + n) into LDS.
  __device__ __forceinline__ void stage_idx(int chunk0, int n, int32_t* sidx) const {
    const int s0 = chunk0 * kChunkKeys;
    const int cnt = min(n * kChunkKeys, kTopK - s0);
    for (int i = threadIdx.x; i < cnt; i += kThreads) sidx[i] = idx_q[s0 + i];
  }

  // Dequantise and store into krow / vt; flags the keys' presence in kvalid.
  // FP4: v_cvt_scalef32_pk_f16_fp4 applies the power-of-two part of the E4M3
  // scale (2^(E-7), or 2^-9 for a subnormal scale), then one v_pk_mul_f16
  // multiplies by its mantissa part (1 + M/8, or M): every step is exact
  // because the products have at most 6 significant bits and lie in
  // [2^-10, 2688]. FP8 window rows: v_cvt_scalef32_pk_f16_fp8 with scale 1.
  __device__ __forceinline__ void store(bool is_main, const uint2 (&r)[8], uint32_t ok,
                                        uint16_t* krow, uint16_t* vt, int* kvalid) const {
    uint32_t pr[8][4];   // [key][channel pair]: fp16 pairs of channels 8p+2b, 8p+2b+1
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (is_main) {
        const uint32_t c = r[j].y;
        const uint32_t E = (c >> 3) & 15u, M = c & 7u;
        const float hw = __uint_as_float(E ? (E + 120u) << 23 : 118u << 23);
        const _Float16 mf = E ? __builtin_bit_cast(_Float16, (uint16_t)(0x3C00u | (M << 7)))
                              : (_Float16)(float)M;
        const v2h m2 = {mf, mf};
        v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r[j].x, hw, 0) * m2;
        v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r[j].x, hw, 1) * m2;
        v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r[j].x, hw, 2) * m2;
        v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r[j].x, hw, 3) * m2;
        pr[j][0] = __builtin_bit_cast(uint32_t, h0);
        pr[j][1] = __builtin_bit_cast(uint32_t, h1);
        pr[j][2] = __builtin_bit_cast(uint32_t, h2);
        pr[j][3] = __builtin_bit_cast(uint32_t, h3);
      } else {
        pr[j][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r[j].x, 1.0f, false));
        pr[j][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r[j].x, 1.0f, true));
        pr[j][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r[j].y, 1.0f, false));
        pr[j][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r[j].y, 1.0f, true));
      }
      if (!((ok >> j) & 1u)) pr[j][0] = pr[j][1] = pr[j][2] = pr[j][3] = 0u;
      const int key = kgrp * 8 + j;
      if ((threadIdx.x & 15) == 0 && (threadIdx.x >> 6) == 0) kvalid[key] = (ok >> j) & 1u;
      *reinterpret_cast<uint4*>(&krow[key * kKrowStride + piece * 8]) =
          make_uint4(pr[j][0], pr[j][1], pr[j][2], pr[j][3]);
    }
    // transpose 8 keys x 8 channels: row 8p + 2b takes the low halves of the
    // pairs, row 8p + 2b + 1 the high halves
    const int slot = ((kgrp + piece) % 5) * 8;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint4 lo = make_uint4(__builtin_amdgcn_perm(pr[1][b], pr[0][b], 0x05040100u),
                                  __builtin_amdgcn_perm(pr[3][b], pr[2][b], 0x05040100u),
                                  __builtin_amdgcn_perm(pr[5][b], pr[4][b], 0x05040100u),
                                  __builtin_amdgcn_perm(pr[7][b], pr[6][b], 0x05040100u));
      const uint4 hi = make_uint4(__builtin_amdgcn_perm(pr[1][b], pr[0][b], 0x07060302u),
                                  __builtin_amdgcn_perm(pr[3][b], pr[2][b], 0x07060302u),
                                  __builtin_amdgcn_perm(pr[5][b], pr[4][b], 0x07060302u),
                                  __builtin_amdgcn_perm(pr[7][b], pr[6][b], 0x07060302u));
      *reinterpret_cast<uint4*>(&vt[(piece * 8 + 2 * b) * kVtRowHalves + slot]) = lo;
      *reinterpret_cast<uint4*>(&vt[(piece * 8 + 2 * b + 1) * kVtRowHalves + slot]) = hi;
    }
  }
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

// P.V operand for one 16-channel tile: channel row `row`, keys
// {4*grp..+3, 16+4*grp..+3}, matching the Q.K result layout of P.
__device__ __forceinline__ v8h vt_operand(const uint16_t* vt, int row, int grp) {
  const uint2 lo = *reinterpret_cast<const uint2*>(&vt[vt_off(row, grp >> 1) + (grp & 1) * 4]);
  const uint2 hi = *reinterpret_cast<const uint2*>(&vt[vt_off(row, 2 + (grp >> 1)) + (grp & 1) * 4]);
  const uint4 v = make_uint4(lo.x, lo.y, hi.x, hi.y);
  return *reinterpret_cast<const v8h*>(&v);
}

// Online softmax step for one chunk. z: this lane's 8 logits (head = column,
// -inf for absent keys). Returns alpha and writes P as hi/lo fp16 operands.
__device__ __forceinline__ float softmax_step(const float (&z)[8], float& m_run, float& l_run,
                                              v8h& p_hi, v8h& p_lo) {
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) mx = fmaxf(mx, z[i]);
  mx = fmaxf(mx, wave_shfl_xor(mx, 16));
  mx = fmaxf(mx, wave_shfl_xor(mx, 32));
  const float m_new = fmaxf(m_run, mx);
  float alpha = 1.0f, psum = 0.0f;
  float p[8];
  if (m_new == -INFINITY) {
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = 0.0f;
  } else {
    alpha = __expf(m_run - m_new);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __expf(z[i] - m_new);
      psum += p[i];
    }
  }
  psum += wave_shfl_xor(psum, 16);
  psum += wave_shfl_xor(psum, 32);
  l_run = l_run * alpha + psum;
  m_run = m_new;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const _Float16 h = (_Float16)p[i];
    p_hi[i] = h;
    p_lo[i] = (_Float16)(p[i] - (float)h);
  }
  return alpha;
}

// Runs chunk(c, raw, ok) for c = 0..CPS-1 of the slice with row loads issued PF
// chunks ahead (register slots are indexed statically).
template <int CPS, int PF, typename Load, typename Chunk>
__device__ __forceinline__ void pipeline(Load&& load, Chunk&& chunk) {
  uint2 raw[PF][8];
  uint32_t ok[PF];
  static_for<PF>([&](auto ii) __attribute__((always_inline)) {
    constexpr int i = decltype(ii)::value;
    if (i < CPS) ok[i] = load(i, raw[i]);
  });
  for (int c0 = 0; c0 < CPS; c0 += PF) {
    static_for<PF>([&](auto ii) __attribute__((always_inline)) {
      constexpr int i = decltype(ii)::value;
      const int c = c0 + i;
      if (c < CPS) {
        uint2 cur[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) cur[j] = raw[i][j];
        const uint32_t cok = ok[i];
        if (c + PF < CPS) ok[i] = load(c + PF, raw[i]);
        chunk(c, cur, cok);
      }
    });
  }
}

// ------------------------------------------------------------ wide kernel --

// One work-group per query (CPS = all chunks of its key slots); wave w owns
// heads 16w..16w+15 and all 512 output channels, so every gathered row serves
// the 64 heads. The output is written directly.
template <int CPS>
__global__ __launch_bounds__(kThreads) void k_sparse_attn_wide(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t krow[kChunkKeys * kKrowStride];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kDim * kVtRowHalves];
  __shared__ int kvalid[kChunkKeys];
  __shared__ __attribute__((aligned(16))) int32_t sidx[CPS * kChunkKeys];

  const int qi = blockIdx.y;
  const int split = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  Gather g;
  g.init(a, qi);
  const int chunk0 = split * CPS;

  v4f acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  v8h qreg[16];
  float zscale;

  // This wave's 16 heads as the B operand of Q.K: head 16*wave + col,
  // channels kb*32 + grp*8 .. +7 for kb = 0..15, in fp16 after the head's shift.
  auto load_q = [&]() __attribute__((always_inline)) {
    const uint16_t* qp = a.q + ((size_t)qi * kHeads + wave * 16 + col) * kDim + grp * 8;
    uint4 raw[16];
    float amax = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) {
      raw[kb] = *reinterpret_cast<const uint4*>(qp + kb * 32);
      amax = fmaxf(amax, bf16x8_absmax(raw[kb]));
    }
    amax = fmaxf(amax, wave_shfl_xor(amax, 16));
    amax = fmaxf(amax, wave_shfl_xor(amax, 32));
    const int sh = q_shift(amax);
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) qreg[kb] = q_to_f16(raw[kb], sh);
    zscale = ldexpf(a.scale, -sh);
  };

  auto chunk = [&](int c, const uint2 (&r)[8], uint32_t ok) __attribute__((always_inline)) {
    g.store((chunk0 + c) * kChunkKeys < kTopK, r, ok, krow, vt, kvalid);
    __syncthreads();
    float z[8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      v4f s = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* kr = &krow[(mt * 16 + col) * kKrowStride + grp * 8];
#pragma unroll
      for (int kb = 0; kb < 16; ++kb) {
        const uint4 v = *reinterpret_cast<const uint4*>(kr + kb * 32);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const v8h*>(&v), qreg[kb], s,
                                                   0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = mt * 16 + 4 * grp + i;
        z[mt * 4 + i] = kvalid[key] ? s[i] * zscale : -INFINITY;
      }
    }
    v8h p_hi, p_lo;
    const float alpha = softmax_step(z, m_run, l_run, p_hi, p_lo);
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) acc[dt] *= alpha;
    }
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const v8h v = vt_operand(vt, dt * 16 + col, grp);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v, p_hi, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v, p_lo, acc[dt], 0, 0, 0);
    }
    __syncthreads();
  };

  g.stage_idx(chunk0, CPS, sidx);
  load_q();
  __syncthreads();
  constexpr int PF = CPS < 2 ? CPS : 2;
  pipeline<CPS, PF>(
      [&](int c, uint2 (&r)[8]) __attribute__((always_inline)) {
        return g.load(chunk0 + c, chunk0, sidx, r);
      },
      chunk);

  // lane holds head 16*wave + col, channels 16*dt + 4*grp .. +3
  const int head = wave * 16 + col;
  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  float* o = a.out + ((size_t)qi * kHeads + head) * kDim + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < 32; ++dt)
    *reinterpret_cast<float4*>(o + dt * 16) =
        make_float4(acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv, acc[dt][3] * inv);
}

// ------------------------------------------------------- decode kernel --

// Decode shape: 5 slices of 128 key slots (slices 0-3 hold the selected rows,
// slice 4 the window), one work-group of 8 waves per (query, 16-head group,
// slice). Three phases separated by two barriers:
//   1. every thread dequantises 4 keys x 32 channels into a row-major fp16
//      buffer of all 128 keys;
//   2. wave w forms the logits of keys 16w..16w+15 for the 16 heads over all
//      512 channels and publishes its per-head maximum; with the slice maximum
//      it writes p = exp(z - max) of its keys (fp16 hi + lo) and their sum;
//   3. wave w accumulates P.V for output channels 64w..64w+63 over the 128 keys,
//      reading V through the transposing LDS read (ds_read_b64_tr_b16).
// The slices are merged by log-sum-exp in a second kernel.
constexpr int kDecSplits = 5;
constexpr int kDecKeys = kSlots / kDecSplits;     // 128 key slots per work-group
constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kPRow = kDecKeys + 8;               // fp16 elements per LDS row of P
static_assert(kDecKeys == 16 * kDecWaves, "one 16-key tile per wave");
static_assert(kTopK % kDecKeys == 0, "a slice holds only selected rows or only window rows");
static_assert(kDecThreads / 16 * 4 == kDecKeys, "4 keys x 32 channels per thread");

typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

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
// scale byte c -> 8 fp16 pairs, exactly as Gather::store dequantises them.
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

__global__ __launch_bounds__(kDecThreads) void k_sparse_attn_decode(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t krow[kDecKeys * kKrowStride];
  // fp16 query [16 heads][kKrowStride] until the logits are formed, then P
  // (hi, lo) [16 heads][kPRow] each
  constexpr int kQP = kHG * kKrowStride > 2 * kHG * kPRow ? kHG * kKrowStride : 2 * kHG * kPRow;
  __shared__ __attribute__((aligned(16))) uint16_t qp_buf[kQP];
  __shared__ float wmax[kDecWaves][kHG];
  __shared__ float wsum[kDecWaves][kHG];
  __shared__ int qsh[kHG];
  uint16_t* const qf = qp_buf;
  uint16_t* const pbuf = qp_buf;   // P hi at [0, kHG*kPRow), lo after it

  const int qi = blockIdx.y;
  const int hg = blockIdx.x % kHeadGroups;
  const int split = blockIdx.x / kHeadGroups;
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
    const int64_t rr = tok - pos0;
    ok = tok >= 0 && rr >= 0 && rr < a.S;
    const uint4* r4 = reinterpret_cast<const uint4*>(
        a.swa + ((size_t)b * (size_t)a.S + (size_t)(ok ? rr : 0)) * kDim + 128 * grp);
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = r4[i];
  }

  // ---- the query in fp16, each head shifted by a power of two (q_shift)
  {
    const float amax = half_max(fmaxf(bf16x8_absmax(qr0), bf16x8_absmax(qr1)));
    const int sh = q_shift(amax);
    const v8h h0 = q_to_f16(qr0, sh), h1 = q_to_f16(qr1, sh);
    *reinterpret_cast<v8h*>(&qf[qh * kKrowStride + qc]) = h0;
    *reinterpret_cast<v8h*>(&qf[qh * kKrowStride + qc + 8]) = h1;
    if ((lane & 31) == 0) qsh[qh] = sh;
  }
  __syncthreads();
  v8h qreg[16];
#pragma unroll
  for (int kb = 0; kb < 16; ++kb)
    qreg[kb] = *reinterpret_cast<const v8h*>(&qf[col * kKrowStride + 128 * grp + 8 * kb]);
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
      uint4* dst = reinterpret_cast<uint4*>(&krow[kk * kKrowStride + 128 * grp + 16 * m]);
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
  __syncthreads();
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
  __syncthreads();
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
        &krow[(ks * 32 + 8 * grp + (col >> 2)) * kKrowStride + wave * 64 + 4 * (col & 3)];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(vsrc + dt * 16));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(vsrc + 4 * kKrowStride + dt * 16));
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

// Work shape per query count: (kernel, slices). Slices divide the 20 chunks.
struct Shape {
  bool wide;
  int splits;
};

Shape attn_shape(int Q) {
  // Measured on MI355X (graph-replayed, 256K-entry caches, random selections):
  // below 512 queries the 16-head work-groups over 5 slices are fastest
  // (32 queries: 28 us vs 46 us for the 64-head work-groups over 4 slices;
  // 128 queries: 84 us vs 91 us); from 512 queries on, one 64-head work-group
  // per query, which writes its output directly.
  Shape sh;
  if (Q < kWideMinQueries) {
    sh.wide = false;
    sh.splits = kDecSplits;
  } else {
    sh.wide = true;
    sh.splits = 1;
  }
  return sh;
}

}  // namespace

size_t attn_workspace_bytes(int Q) {
  const Shape sh = attn_shape(Q);
  if (sh.splits == 1) return 0;
  return (size_t)Q * sh.splits * kHeads * (kDim + 2) * sizeof(float);
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* cache, const int32_t* idx,
                              const uint8_t* swa, const int64_t* q_pos, const int64_t* swa_pos0,
                              int B, int T, int64_t n_cap, int S, float scale, float* out,
                              void* ws, hipStream_t st) {
  const int Q = B * T;
  AttnArgs a;
  a.q = q;
  a.cache = cache;
  a.idx = idx;
  a.swa = swa;
  a.q_pos = q_pos;
  a.swa_pos0 = swa_pos0;
  a.T = T;
  a.n_cap = n_cap;
  a.S = S;
  a.scale = scale;
  a.out = out;
  a.part = nullptr;
  a.part_ml = nullptr;
  const Shape sh = attn_shape(Q);
  if (sh.wide ? sh.splits != 1 : sh.splits != kDecSplits) return hipErrorInvalidValue;
  a.splits = sh.splits;
  if (a.splits > 1) {
    a.part = reinterpret_cast<float*>(ws);
    a.part_ml = a.part + (size_t)Q * a.splits * kHeads * kDim;
  }
  if (sh.wide) {
    const dim3 grid(a.splits, Q);
    hipLaunchKernelGGL(k_sparse_attn_wide<kChunks>, grid, dim3(kThreads), 0, st, a);
  } else {
    const dim3 grid(kDecSplits * kHeadGroups, Q);
    hipLaunchKernelGGL(k_sparse_attn_decode, grid, dim3(kDecThreads), 0, st, a);
  }
  if (a.splits > 1)
    hipLaunchKernelGGL(k_attn_merge, dim3(kHeads, Q), dim3(128), 0, st, a.part, a.part_ml,
                       a.splits, out);
  return hipGetLastError();
}

}  // namespace csa2
