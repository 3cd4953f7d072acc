// Sparse-indexer scan, decode shape: score(n) = sum_h w_h * relu(q_h . k_n).
//
// Pages: 32 index query heads of width 128 and Top-512 per query ("DeepSeek
// V4.1-Flash 为什么这么强？CED 与 CSA2 架构全拆解", §二 layer layout); the first
// Full layer scores every visible position and Reindex layers score only inside
// the pool (same §二, hierarchical sparse indexer; "DeepSeek-V4.1-Flash：全局 KV
// 仅 890 B/token", 第二刀 and Fig. 5). The weighted ReLU sum is the reading
// stated in the header csa2.h.
//
// Mapping: per query the 32 x 128 indexer query is the A operand of
// v_mfma_f32_32x32x64_f8f6f4 (rows = heads) and 32 keys are the B operand
// (columns = positions), two MFMAs per 32 positions (K = 128). Lane l holds
// head/position l%32 and bytes (l/32)*64 .. +63 of the 128-byte row, so a wave
// streams 32 whole rows (4 KiB) per tile with 16-byte loads. The channel order
// inside a lane is irrelevant to the dot product as long as A and B agree.
// The accumulator holds, per lane, 16 of the 32 head dot products of one
// position; the epilogue applies ReLU and the head weights and adds the other
// half with one cross-half shuffle. The scan is HBM-bound (64 FLOP per byte);
// the MFMA only keeps the 4096 MACs per key off the vector ALU.
#include "device_common.hpp"
#include "launchers.hpp"

namespace csa2 {
namespace {

constexpr int kTilePos = 32;       // positions per MFMA tile
constexpr int kTilesPerWave = 8;
constexpr int kWaves = 4;
constexpr int kItemsPerWG = kTilePos * kTilesPerWave * kWaves;   // 1024

// Row (head) of accumulator register r in lane `lane` of a 32x32 MFMA result.
__device__ __forceinline__ int acc32_row(int lane, int r) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

struct KTile {
  uint4 v[4];
};

__device__ __forceinline__ void load_tile(KTile& t, const uint8_t* p, bool ok) {
  if (ok) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    t.v[0] = q[0];
    t.v[1] = q[1];
    t.v[2] = q[2];
    t.v[3] = q[3];
  } else {
    t.v[0] = t.v[1] = t.v[2] = t.v[3] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ v8i as_v8i(const uint4& a, const uint4& b) {
  v8i r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
  return r;
}

template <int MODE>
__global__ __launch_bounds__(256) void k_index_score_decode(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ n_vis,
    const int32_t* __restrict__ pool, int T, int64_t n_cap, int64_t n_items,
    float* __restrict__ scores, float* __restrict__ bmax) {
  const int qi = blockIdx.y;
  const int b = qi / T;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  int64_t nv = n_vis[qi];
  nv = nv < 0 ? 0 : (nv > n_cap ? n_cap : nv);
  const int64_t n_blk = (n_cap + kBlock - 1) / kBlock;

  const uint8_t* qp = q_idx + (size_t)qi * (kIdxHeads * kIdxDim) + col * kIdxDim + half * 64;
  const uint4* q4 = reinterpret_cast<const uint4*>(qp);
  const v8i a0 = as_v8i(q4[0], q4[1]);
  const v8i a1 = as_v8i(q4[2], q4[3]);
  float wr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wr[r] = w[(size_t)qi * kIdxHeads + acc32_row(lane, r)];

  const uint8_t* kbase = k_idx + (size_t)b * (size_t)n_cap * kIdxDim + half * 64;
  const int32_t* pl = MODE == 1 ? pool + (size_t)qi * kPoolBlocks : nullptr;
  float* srow = scores + (size_t)qi * (size_t)n_items;
  float* brow = bmax ? bmax + (size_t)qi * (size_t)n_blk : nullptr;

  const int64_t wave_base = (int64_t)blockIdx.x * kItemsPerWG + (int64_t)wave * kTilePos * kTilesPerWave;

  // Reindex: the pool entries of all of this wave's tiles are fetched first, so
  // a tile's key loads never wait on a pool lookup.
  int32_t blk[kTilesPerWave];
#pragma unroll
  for (int it = 0; it < kTilesPerWave; ++it) {
    const int64_t item = wave_base + (int64_t)it * kTilePos + col;
    blk[it] = (MODE == 1 && item < n_items) ? pl[item >> 3] : -1;
  }
  auto position_of = [&](int it, bool& ok) __attribute__((always_inline)) -> int64_t {
    const int64_t item = wave_base + (int64_t)it * kTilePos + col;
    if (MODE == 0) {
      ok = item < nv;
      return ok ? item : 0;
    }
    const int64_t b8 = blk[it];
    const int64_t pos = b8 * kBlock + (item & 7);
    ok = b8 >= 0 && b8 < n_blk && pos < nv;
    return ok ? pos : 0;
  };

  KTile cur, nxt;
  bool cur_ok;
  {
    const int64_t pos = position_of(0, cur_ok);
    load_tile(cur, kbase + pos * kIdxDim, cur_ok);
  }
#pragma unroll
  for (int it = 0; it < kTilesPerWave; ++it) {
    const int64_t tile0 = wave_base + (int64_t)it * kTilePos;
    if (tile0 >= n_items) break;
    bool nxt_ok = false;
    if (it + 1 < kTilesPerWave) {
      const int64_t pos = position_of(it + 1, nxt_ok);
      load_tile(nxt, kbase + pos * kIdxDim, nxt_ok);
    }
    float s = -INFINITY;
    // Skip the MFMA when no lane of the wave holds a visible position.
    if (__any(cur_ok)) {
      v16f acc = {};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, as_v8i(cur.v[0], cur.v[1]), acc,
                                                            0, 0, 0, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, as_v8i(cur.v[2], cur.v[3]), acc,
                                                            0, 0, 0, 0, 0, 0);
      float part = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) part = fmaf(wr[r], fmaxf(acc[r], 0.0f), part);
      part += wave_shfl_xor(part, 32);
      if (cur_ok) s = part;
    }
    const int64_t item = tile0 + col;
    if (half == 0 && item < n_items) srow[item] = s;
    if (brow) {
      float m = s;
      m = fmaxf(m, wave_shfl_xor(m, 1));
      m = fmaxf(m, wave_shfl_xor(m, 2));
      m = fmaxf(m, wave_shfl_xor(m, 4));
      if (half == 0 && (col & 7) == 0 && item < n_items) brow[item >> 3] = m;
    }
    cur = nxt;
    cur_ok = nxt_ok;
  }
}

}  // namespace

hipError_t launch_index_score_decode(int mode, const uint8_t* q_idx, const float* w,
                                     const uint8_t* k_idx, const int32_t* n_vis,
                                     const int32_t* pool, int B, int T, int64_t n_cap,
                                     float* scores, float* bmax, hipStream_t st) {
  const int Q = B * T;
  const int64_t n_items = mode == 0 ? n_cap : (int64_t)kPoolCand;
  const int64_t gx = (n_items + kItemsPerWG - 1) / kItemsPerWG;
  const dim3 grid((unsigned)gx, (unsigned)Q);
  if (mode == 0) {
    hipLaunchKernelGGL(k_index_score_decode<0>, grid, dim3(256), 0, st, q_idx, w, k_idx, n_vis,
                       pool, T, n_cap, n_items, scores, bmax);
  } else {
    hipLaunchKernelGGL(k_index_score_decode<1>, grid, dim3(256), 0, st, q_idx, w, k_idx, n_vis,
                       pool, T, n_cap, n_items, scores, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_index_score_prefill(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                                      const int32_t* n_vis, int B, int T, int64_t n_cap,
                                      float* scores, float* bmax, hipStream_t st) {
  return launch_index_score_decode(0, q_idx, w, k_idx, n_vis, nullptr, B, T, n_cap, scores, bmax,
                                   st);
}

}  // namespace csa2
