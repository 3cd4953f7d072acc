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
// Work split: one work-group per (query, slice of the 640 key slots); 4 waves,
// wave w owns heads 16w..16w+15 and all 512 output channels. Keys are
// processed 32 at a time:
//   gather  -- the work-group loads the 32 rows (FP4 codes + E4M3 scales, or
//              E4M3 window rows), dequantises them (exact in bf16 and fp16) and
//              writes them to LDS twice: row-major bf16 for Q.K and transposed
//              fp16 for P.V;
//   Q.K     -- v_mfma_f32_16x16x32_bf16 with the keys as A (rows) and the
//              wave's 16 query heads as B (kept in registers);
//   softmax -- online (running max and sum per head, which is one lane column
//              of the 16x16 result);
//   P.V     -- v_mfma_f32_16x16x32_f16 with the transposed keys as A and the
//              probabilities (fp16, converted in registers from the Q.K result
//              layout) as B; 32 accumulator tiles hold 512 channels x 16 heads.
// With more than one slice per query the partial (max, sum, unnormalised
// output) go to the workspace and a merge kernel combines them by
// log-sum-exp; with one slice the kernel writes the output directly.
#include "device_common.hpp"
#include "launchers.hpp"

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkKeys = 32;
constexpr int kSlots = kTopK + kWindow;           // 640 key slots per query
constexpr int kChunks = kSlots / kChunkKeys;      // 20
constexpr int kKrowStride = kDim + 8;             // bf16 elements per LDS key row
constexpr int kVtStride = kChunkKeys + 8;         // fp16 elements per LDS channel row

__device__ __forceinline__ uint16_t f32_to_bf16_exact(float v) {
  return (uint16_t)(__float_as_uint(v) >> 16);   // exact for dequantised values
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  const _Float16 h = (_Float16)v;
  return *reinterpret_cast<const uint16_t*>(&h);
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

__global__ __launch_bounds__(kThreads) void k_sparse_attn(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t krow[kChunkKeys * kKrowStride];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kDim * kVtStride];
  __shared__ int kvalid[kChunkKeys];

  const int qi = blockIdx.y;
  const int split = blockIdx.x;
  const int b = qi / a.T;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t tq = a.q_pos[qi];
  const int64_t pos0 = a.swa_pos0[b];

  // This wave's 16 heads as the B operand of Q.K: head 16*wave + col,
  // channels kb*32 + grp*8 .. +7 for kb = 0..15.
  v8bf qreg[16];
  {
    const uint16_t* qp = a.q + ((size_t)qi * kHeads + wave * 16 + col) * kDim + grp * 8;
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) {
      const uint4 v = *reinterpret_cast<const uint4*>(qp + kb * 32);
      qreg[kb] = *reinterpret_cast<const v8bf*>(&v);
    }
  }
  v4f acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  const int chunks_per_split = kChunks / a.splits;
  const int piece = tid & 63;          // channels 8*piece .. +7 in the gather
  const int kgrp = tid >> 6;           // keys 8*kgrp .. +7 of the chunk in the gather
  const uint8_t* cache_b = a.cache + (size_t)b * (size_t)a.n_cap * kRowBytes;
  const uint8_t* swa_b = a.swa + (size_t)b * (size_t)a.S * kDim;
  const int32_t* idx_q = a.idx + (size_t)qi * kTopK;

  for (int c = 0; c < chunks_per_split; ++c) {
    const int slot0 = (split * chunks_per_split + c) * kChunkKeys;
    // ---------------------------------------------------------------- gather
    float vals[8][8];   // [key][channel]
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = kgrp * 8 + j;
      const int slot = slot0 + key;
      bool ok;
      if (slot < kTopK) {
        const int64_t p = idx_q[slot];
        ok = p >= 0 && p < a.n_cap;
        if (ok) {
          const uint8_t* row = cache_b + (size_t)p * kRowBytes;
          const uint32_t codes = *reinterpret_cast<const uint32_t*>(row + piece * 4);
          const float s = e4m3_to_f32(row[kCodeBytes + (piece >> 1)]);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t cd = (codes >> (4 * i)) & 0xFu;
            const float m = e2m1_mag(cd & 7u) * s;
            vals[j][i] = (cd & 8u) ? -m : m;
          }
        }
      } else {
        const int64_t tok = tq - (kWindow - 1) + (slot - kTopK);
        const int64_t r = tok - pos0;
        ok = tok >= 0 && r >= 0 && r < a.S;
        if (ok) {
          const uint2 raw = *reinterpret_cast<const uint2*>(swa_b + (size_t)r * kDim + piece * 8);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            vals[j][i] = e4m3_to_f32((raw.x >> (8 * i)) & 0xFFu);
            vals[j][4 + i] = e4m3_to_f32((raw.y >> (8 * i)) & 0xFFu);
          }
        }
      }
      if (!ok) {
#pragma unroll
        for (int i = 0; i < 8; ++i) vals[j][i] = 0.0f;
      }
      if (piece == 0) kvalid[key] = ok ? 1 : 0;
      // row-major bf16 copy: key row, channels 8*piece .. +7
      uint4 w;
      w.x = f32_to_bf16_exact(vals[j][0]) | ((uint32_t)f32_to_bf16_exact(vals[j][1]) << 16);
      w.y = f32_to_bf16_exact(vals[j][2]) | ((uint32_t)f32_to_bf16_exact(vals[j][3]) << 16);
      w.z = f32_to_bf16_exact(vals[j][4]) | ((uint32_t)f32_to_bf16_exact(vals[j][5]) << 16);
      w.w = f32_to_bf16_exact(vals[j][6]) | ((uint32_t)f32_to_bf16_exact(vals[j][7]) << 16);
      *reinterpret_cast<uint4*>(&krow[key * kKrowStride + piece * 8]) = w;
    }
    // transposed fp16 copy: channel row, keys 8*kgrp .. +7
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 w;
      w.x = f32_to_f16_bits(vals[0][i]) | ((uint32_t)f32_to_f16_bits(vals[1][i]) << 16);
      w.y = f32_to_f16_bits(vals[2][i]) | ((uint32_t)f32_to_f16_bits(vals[3][i]) << 16);
      w.z = f32_to_f16_bits(vals[4][i]) | ((uint32_t)f32_to_f16_bits(vals[5][i]) << 16);
      w.w = f32_to_f16_bits(vals[6][i]) | ((uint32_t)f32_to_f16_bits(vals[7][i]) << 16);
      *reinterpret_cast<uint4*>(&vt[(piece * 8 + i) * kVtStride + kgrp * 8]) = w;
    }
    __syncthreads();

    // ------------------------------------------------------------------- Q.K
    v4f sc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      v4f s = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* kr = &krow[(mt * 16 + col) * kKrowStride + grp * 8];
#pragma unroll
      for (int kb = 0; kb < 16; ++kb) {
        const uint4 v = *reinterpret_cast<const uint4*>(kr + kb * 32);
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const v8bf*>(&v), qreg[kb], s,
                                                    0, 0, 0);
      }
      sc[mt] = s;
    }
    // --------------------------------------------------------------- softmax
    // lane holds head `col`, keys mt*16 + 4*grp + i
    float z[8];
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = mt * 16 + 4 * grp + i;
        const float v = kvalid[key] ? sc[mt][i] * a.scale : -INFINITY;
        z[mt * 4 + i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    float alpha = 1.0f;
    float psum = 0.0f;
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
    for (int i = 0; i < 32; ++i) acc[i] *= alpha;
    v8h pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[i] = (_Float16)p[i];
    // ------------------------------------------------------------------- P.V
    // A operand: channel row 16*dt + col, keys {4*grp .. +3} and {16 + 4*grp .. +3}
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const uint16_t* vr = &vt[(dt * 16 + col) * kVtStride + 4 * grp];
      const uint2 lo = *reinterpret_cast<const uint2*>(vr);
      const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
      const uint4 v = make_uint4(lo.x, lo.y, hi.x, hi.y);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const v8h*>(&v), pb,
                                                       acc[dt], 0, 0, 0);
    }
    __syncthreads();
  }

  // lane holds head 16*wave + col, channels 16*dt + 4*grp .. +3
  const int head = wave * 16 + col;
  if (a.splits == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float* o = a.out + ((size_t)qi * kHeads + head) * kDim + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const float4 v = make_float4(acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv,
                                   acc[dt][3] * inv);
      *reinterpret_cast<float4*>(o + dt * 16) = v;
    }
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

// One work-group per (query, head); 128 threads x 4 channels.
__global__ __launch_bounds__(128) void k_attn_merge(const float* __restrict__ part,
                                                    const float* __restrict__ part_ml, int splits,
                                                    float* __restrict__ out) {
  const int qi = blockIdx.y, head = blockIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s)
    M = fmaxf(M, part_ml[(((size_t)qi * splits + s) * kHeads + head) * 2]);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const size_t ps = (size_t)qi * splits + s;
      const float m = part_ml[(ps * kHeads + head) * 2];
      const float l = part_ml[(ps * kHeads + head) * 2 + 1];
      const float wgt = m == -INFINITY ? 0.0f : __expf(m - M);
      L += wgt * l;
      const float4 v = *reinterpret_cast<const float4*>(part + (ps * kHeads + head) * kDim + threadIdx.x * 4);
      o.x += wgt * v.x;
      o.y += wgt * v.y;
      o.z += wgt * v.z;
      o.w += wgt * v.w;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  *reinterpret_cast<float4*>(out + ((size_t)qi * kHeads + head) * kDim + threadIdx.x * 4) =
      make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
}

int choose_splits(int Q) {
  // enough work-groups to cover the chip; splits divide the 20 chunks
  static const int opts[] = {1, 2, 4, 5, 10, 20};
  int best = 1;
  for (int s : opts)
    if ((int64_t)Q * best < 512) best = s;
  return best;
}

}  // namespace

size_t attn_workspace_bytes(int Q) {
  const int s = choose_splits(Q);
  if (s == 1) return 0;
  return (size_t)Q * s * kHeads * (kDim + 2) * sizeof(float);
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
  a.splits = choose_splits(Q);
  a.part = reinterpret_cast<float*>(ws);
  a.part_ml = a.part + (size_t)Q * a.splits * kHeads * kDim;
  hipLaunchKernelGGL(k_sparse_attn, dim3(a.splits, Q), dim3(kThreads), 0, st, a);
  if (a.splits > 1)
    hipLaunchKernelGGL(k_attn_merge, dim3(kHeads, Q), dim3(128), 0, st, a.part, a.part_ml,
                       a.splits, out);
  return hipGetLastError();
}

}  // namespace csa2
