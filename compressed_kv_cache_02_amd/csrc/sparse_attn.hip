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
//   wide   (more than 16 queries): one work-group of 4 waves per (query, slice
//          of the key slots); wave w owns heads 16w..16w+15 and all 512 output
//          channels, so every gathered row serves all 64 heads;
//   decode (up to 16 queries): one work-group of 8 waves per (query, 16-head
//          group, slice). Wave w takes key half w/4 of each 32-key chunk and
//          channel quarter w%4: it dequantises only that quarter of its keys
//          into the row-major buffer, forms partial Q.K sums that the four
//          waves of its half add up through LDS in a fixed order, and
//          accumulates P.V for its 128 channels. Its P.V operand comes straight
//          from the row-major buffer through the gfx950 transposing LDS read
//          (ds_read_b64_tr_b16), so no transposed copy is stored. The two key
//          halves are combined at the end; two waves per SIMD hide each other's
//          LDS and MFMA latencies.
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

// One work-group per (query, slice of CPS chunks); wave w owns heads
// 16w..16w+15 and all 512 output channels, so every gathered row serves the 64
// heads. With one slice per query the output is written directly, otherwise
// the partial state goes to the workspace for the merge kernel.
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
  if (a.splits == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float* o = a.out + ((size_t)qi * kHeads + head) * kDim + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
      *reinterpret_cast<float4*>(o + dt * 16) =
          make_float4(acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv, acc[dt][3] * inv);
  } else {
    const size_t ps = (size_t)qi * a.splits + split;
    float* o = a.part + (ps * kHeads + head) * kDim + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
      *reinterpret_cast<float4*>(o + dt * 16) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    if (grp == 0) {
      a.part_ml[(ps * kHeads + head) * 2 + 0] = m_run;
      a.part_ml[(ps * kHeads + head) * 2 + 1] = l_run;
    }
  }
}

// ------------------------------------------------ decode kernel, 8 waves --

typedef _Float16 v4h __attribute__((ext_vector_type(4)));

// Gather for the 8-wave decode work-group: thread t of wave w owns channels
// 8p..8p+7 with p = 16*(w%4) + t%16, and keys 4g..4g+3 of the chunk with
// g = 4*(w/4) + (t%64)/16 (wave w serves key half w/4 and channel quarter w%4).
struct Gather8 {
  const uint8_t* cache_b;
  const uint8_t* swa_b;
  const int32_t* idx_q;
  int64_t n_cap, tq, pos0;
  int S, piece, g4;

  __device__ void init(const AttnArgs& a, int qi) {
    const int b = qi / a.T;
    cache_b = a.cache + (size_t)b * (size_t)a.n_cap * kRowBytes;
    swa_b = a.swa + (size_t)b * (size_t)a.S * kDim;
    idx_q = a.idx + (size_t)qi * kTopK;
    n_cap = a.n_cap;
    tq = a.q_pos[qi];
    pos0 = a.swa_pos0[b];
    S = a.S;
    const int t = threadIdx.x, w = t >> 6;
    piece = 16 * (w & 3) + (t & 15);
    g4 = 4 * (w >> 2) + ((t & 63) >> 4);
  }

  // This thread's 4 selected positions of `chunk` (unused for window chunks).
  __device__ __forceinline__ int4 load_idx(int chunk) const {
    const int slot0 = chunk * kChunkKeys + g4 * 4;
    return slot0 < kTopK ? *reinterpret_cast<const int4*>(idx_q + slot0) : make_int4(-1, -1, -1, -1);
  }

  // Raw bytes of this thread's 4 keys; bit j marks key j present. Row loads are
  // unconditional (an absent key reads row 0) so none waits on another.
  __device__ __forceinline__ uint32_t load(int chunk, const int4& i4, uint2 (&r)[4]) const {
    const int slot0 = chunk * kChunkKeys + g4 * 4;
    uint32_t ok = 0;
    if (slot0 < kTopK) {
      const int32_t pj[4] = {i4.x, i4.y, i4.z, i4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool v = pj[j] >= 0 && (int64_t)pj[j] < n_cap;
        ok |= (v ? 1u : 0u) << j;
        const uint8_t* row = cache_b + (size_t)(v ? pj[j] : 0) * kRowBytes;
        r[j].x = *reinterpret_cast<const uint32_t*>(row + piece * 4);
        r[j].y = row[kCodeBytes + (piece >> 1)];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t tok = tq - (kWindow - 1) + (slot0 + j - kTopK);
        const int64_t rr = tok - pos0;
        const bool v = tok >= 0 && rr >= 0 && rr < S;
        ok |= (v ? 1u : 0u) << j;
        r[j] = *reinterpret_cast<const uint2*>(swa_b + (size_t)(v ? rr : 0) * kDim + piece * 8);
      }
    }
    return ok;
  }

  // Dequantise (as Gather::store) into krow; flags presence.
  __device__ __forceinline__ void store(bool is_main, const uint2 (&r)[4], uint32_t ok,
                                        uint16_t* krow, int* kvalid) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t pr[4];   // fp16 pairs of channels 8p+2b, 8p+2b+1
      if (is_main) {
        const uint32_t c = r[j].y;
        const uint32_t E = (c >> 3) & 15u, M = c & 7u;
        const float hw = __uint_as_float(E ? (E + 120u) << 23 : 118u << 23);
        const _Float16 mf = E ? __builtin_bit_cast(_Float16, (uint16_t)(0x3C00u | (M << 7)))
                              : (_Float16)(float)M;
        const v2h m2 = {mf, mf};
        pr[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r[j].x, hw, 0) * m2);
        pr[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r[j].x, hw, 1) * m2);
        pr[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r[j].x, hw, 2) * m2);
        pr[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r[j].x, hw, 3) * m2);
      } else {
        pr[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r[j].x, 1.0f, false));
        pr[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r[j].x, 1.0f, true));
        pr[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r[j].y, 1.0f, false));
        pr[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r[j].y, 1.0f, true));
      }
      if (!((ok >> j) & 1u)) pr[0] = pr[1] = pr[2] = pr[3] = 0u;
      const int key = g4 * 4 + j;
      if ((threadIdx.x & 15) == 0 && ((threadIdx.x >> 6) & 3) == 0) kvalid[key] = (ok >> j) & 1u;
      *reinterpret_cast<uint4*>(&krow[key * kKrowStride + piece * 8]) =
          make_uint4(pr[0], pr[1], pr[2], pr[3]);
    }
  }
};

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

// Online softmax step over 16 keys: z = this lane's 4 logits (head = column).
__device__ __forceinline__ float softmax_step16(const float (&z)[4], float& m_run, float& l_run,
                                                v4h& p_hi, v4h& p_lo) {
  const float mx = rows_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
  const float m_new = fmaxf(m_run, mx);
  float alpha = 1.0f, psum = 0.0f;
  float p[4];
  if (m_new == -INFINITY) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = 0.0f;
  } else {
    alpha = __expf(m_run - m_new);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __expf(z[i] - m_new);
      psum += p[i];
    }
  }
  psum = rows_sum(psum);
  l_run = l_run * alpha + psum;
  m_run = m_new;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 h = (_Float16)p[i];
    p_hi[i] = h;
    p_lo[i] = (_Float16)(p[i] - (float)h);
  }
  return alpha;
}

// One work-group of 8 waves per (query, 16-head group, slice of CPS chunks).
// Wave w takes key half w/4 of every chunk and channel quarter w%4: the four
// waves of a half exchange partial Q.K sums through LDS (one barrier per
// chunk), keep their own online-softmax state and P.V accumulators, and the two
// halves are combined at the end. Two waves per SIMD hide each other's LDS and
// MFMA latencies.
template <int CPS>
__global__ __launch_bounds__(512) void k_sparse_attn_decode8(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t krow[kChunkKeys * kKrowStride];
  __shared__ float spart[2][2][4][16][kHG];
  __shared__ int kvalid[2][kChunkKeys];
  __shared__ float qmax[4][kHG];

  const int qi = blockIdx.y;
  const int hg = blockIdx.x % kHeadGroups;
  const int split = blockIdx.x / kHeadGroups;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cq = wave & 3, kh = wave >> 2;
  const int col = lane & 15, grp = lane >> 4;
  Gather8 g;
  g.init(a, qi);
  const int chunk0 = split * CPS;

  v4f acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  v8h qreg[4];
  float zscale = 1.0f;

  auto chunk = [&](int c, const uint2 (&r)[4], uint32_t ok) __attribute__((always_inline)) {
    const int buf = c & 1;
    g.store((chunk0 + c) * kChunkKeys < kTopK, r, ok, krow, kvalid[buf]);
    {
      v4f s = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* kr = &krow[(kh * 16 + col) * kKrowStride + cq * 128 + grp * 8];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint4 v = *reinterpret_cast<const uint4*>(kr + kb * 32);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const v8h*>(&v), qreg[kb], s,
                                                   0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) spart[buf][kh][cq][4 * grp + i][col] = s[i];
    }
    __syncthreads();
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 4 * grp + i;
      const float sv = ((spart[buf][kh][0][k][col] + spart[buf][kh][1][k][col]) +
                        spart[buf][kh][2][k][col]) + spart[buf][kh][3][k][col];
      z[i] = kvalid[buf][kh * 16 + k] ? sv * zscale : -INFINITY;
    }
    v4h p_hi, p_lo;
    const float alpha = softmax_step16(z, m_run, l_run, p_hi, p_lo);
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[dt] *= alpha;
    }
    // P.V operand: the transposing LDS read hands lane (grp, i) the values of
    // channel ch0 + i for keys 16*kh + 4*grp .. +3, when lane (grp, m) points
    // at key 16*kh + 4*grp + m/4, channels ch0 + 4*(m%4) .. +3.
    const uint16_t* vsrc = &krow[(kh * 16 + 4 * grp + (col >> 2)) * kKrowStride + cq * 128 +
                                 4 * (col & 3)];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      typedef short v4s __attribute__((ext_vector_type(4)));
      const v4s raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(vsrc + dt * 16));
      const v4h v = __builtin_bit_cast(v4h, raw);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(v, p_hi, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(v, p_lo, acc[dt], 0, 0, 0);
    }
  };
  // The quarter cq of the 16 heads' query in fp16 after the head's shift.
  auto load_q = [&]() __attribute__((always_inline)) {
    const uint16_t* qp = a.q + ((size_t)qi * kHeads + hg * kHG + col) * kDim + cq * 128 + grp * 8;
    uint4 raw[4];
    float amax = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      raw[kb] = *reinterpret_cast<const uint4*>(qp + kb * 32);
      amax = fmaxf(amax, bf16x8_absmax(raw[kb]));
    }
    amax = rows_max(amax);
    if (grp == 0 && kh == 0) qmax[cq][col] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(qmax[0][col], qmax[1][col]), fmaxf(qmax[2][col], qmax[3][col]));
    const int sh = q_shift(amax);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qreg[kb] = q_to_f16(raw[kb], sh);
    zscale = ldexpf(a.scale, -sh);
  };

  // Every index this thread needs is requested first, then the first rows,
  // so the index -> row chain overlaps the query set-up.
  int4 ix[CPS];
  static_for<CPS>([&](auto ii) __attribute__((always_inline)) {
    constexpr int i = decltype(ii)::value;
    ix[i] = g.load_idx(chunk0 + i);
  });
  constexpr int PF = CPS < 4 ? CPS : 4;
  uint2 raw[PF][4];
  uint32_t okm[PF];
  static_for<PF>([&](auto ii) __attribute__((always_inline)) {
    constexpr int i = decltype(ii)::value;
    if (i < CPS) okm[i] = g.load(chunk0 + i, ix[i], raw[i]);
  });
  load_q();   // ends with a barrier
  for (int c0 = 0; c0 < CPS; c0 += PF) {
    static_for<PF>([&](auto ii) __attribute__((always_inline)) {
      constexpr int i = decltype(ii)::value;
      const int c = c0 + i;
      if (c < CPS) {
        uint2 cur[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) cur[j] = raw[i][j];
        const uint32_t cok = okm[i];
        if (c + PF < CPS) {
          static_for<CPS>([&](auto jj) __attribute__((always_inline)) {
            constexpr int cc = decltype(jj)::value;
            if (cc == c + PF) okm[i] = g.load(chunk0 + cc, ix[cc], raw[i]);
          });
        }
        chunk(c, cur, cok);
      }
    });
  }

  // Combine the two key halves: half 1 hands its state to half 0 through LDS
  // (reusing the key buffer and the partial sums once every wave is done).
  __syncthreads();
  float* xs = reinterpret_cast<float*>(krow);        // [4 quarters][8 tiles][64 lanes][4]
  float* xml = &spart[0][0][0][0][0];                // [4][64 lanes][2]
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(xs + (((size_t)cq * 8 + dt) * 64 + lane) * 4) =
          make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    xml[(cq * 64 + lane) * 2 + 0] = m_run;
    xml[(cq * 64 + lane) * 2 + 1] = l_run;
  }
  __syncthreads();
  if (kh == 1) return;
  {
    const float m1 = xml[(cq * 64 + lane) * 2 + 0], l1 = xml[(cq * 64 + lane) * 2 + 1];
    const float M = fmaxf(m_run, m1);
    const float w0 = m_run == -INFINITY ? 0.0f : __expf(m_run - M);
    const float w1 = m1 == -INFINITY ? 0.0f : __expf(m1 - M);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const float4 o = *reinterpret_cast<const float4*>(xs + (((size_t)cq * 8 + dt) * 64 + lane) * 4);
      acc[dt][0] = acc[dt][0] * w0 + o.x * w1;
      acc[dt][1] = acc[dt][1] * w0 + o.y * w1;
      acc[dt][2] = acc[dt][2] * w0 + o.z * w1;
      acc[dt][3] = acc[dt][3] * w0 + o.w * w1;
    }
    l_run = l_run * w0 + l1 * w1;
    m_run = M;
  }

  // lane holds head 16*hg + col, channels 128*cq + 16*dt + 4*grp .. +3
  const int head = hg * kHG + col;
  const int splits = gridDim.x / kHeadGroups;
  if (splits == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float* o = a.out + ((size_t)qi * kHeads + head) * kDim + cq * 128 + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(o + dt * 16) =
          make_float4(acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv, acc[dt][3] * inv);
  } else {
    const size_t ps = (size_t)qi * splits + split;
    float* o = a.part + (ps * kHeads + head) * kDim + cq * 128 + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(o + dt * 16) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    if (grp == 0 && cq == 0) {
      a.part_ml[(ps * kHeads + head) * 2 + 0] = m_run;
      a.part_ml[(ps * kHeads + head) * 2 + 1] = l_run;
    }
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
  // Measured on MI355X (graph-replayed, 1M-entry caches): up to 16 queries the
  // 16-head work-groups over 5 slices are fastest (8 queries: 22 us vs 25 us
  // for the best 64-head shape); up to 512 queries the 64-head work-groups over
  // 4 slices (64 queries: 49 us vs 67 us); beyond that one slice per query.
  Shape sh;
  if (Q <= 16) {
    sh.wide = false;
    sh.splits = 5;
  } else if (Q < kWideMinQueries) {
    sh.wide = true;
    sh.splits = 4;
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
  if (sh.splits > kMaxSplits || (!sh.wide && sh.splits != 5)) return hipErrorInvalidValue;
  a.splits = sh.splits;
  if (a.splits > 1) {
    a.part = reinterpret_cast<float*>(ws);
    a.part_ml = a.part + (size_t)Q * a.splits * kHeads * kDim;
  }
  if (sh.wide) {
    const dim3 grid(a.splits, Q);
    switch (kChunks / a.splits) {
      case 1: hipLaunchKernelGGL(k_sparse_attn_wide<1>, grid, dim3(kThreads), 0, st, a); break;
      case 2: hipLaunchKernelGGL(k_sparse_attn_wide<2>, grid, dim3(kThreads), 0, st, a); break;
      case 4: hipLaunchKernelGGL(k_sparse_attn_wide<4>, grid, dim3(kThreads), 0, st, a); break;
      case 5: hipLaunchKernelGGL(k_sparse_attn_wide<5>, grid, dim3(kThreads), 0, st, a); break;
      case 10: hipLaunchKernelGGL(k_sparse_attn_wide<10>, grid, dim3(kThreads), 0, st, a); break;
      default: hipLaunchKernelGGL(k_sparse_attn_wide<20>, grid, dim3(kThreads), 0, st, a); break;
    }
  } else {
    // the decode shape always runs 5 slices of 4 chunks
    const dim3 grid(a.splits * kHeadGroups, Q);
    hipLaunchKernelGGL(k_sparse_attn_decode8<kChunks / 5>, grid, dim3(512), 0, st, a);
  }
  if (a.splits > 1)
    hipLaunchKernelGGL(k_attn_merge, dim3(kHeads, Q), dim3(128), 0, st, a.part, a.part_ml,
                       a.splits, out);
  return hipGetLastError();
}

}  // namespace csa2
