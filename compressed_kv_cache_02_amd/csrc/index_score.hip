// Sparse-indexer scan, decode shape: score(n) = sum_h w_h * relu(q_h . k_n).
//
// Pages: 32 index query heads of width 128 and Top-512 per query ("DeepSeek
// V4.1-Flash 为什么这么强？CED 与 CSA2 架构全拆解", §二 layer layout); the first
// Full layer scores every visible position and Reindex layers score only inside
// the pool (same §二, hierarchical sparse indexer; "DeepSeek-V4.1-Flash：全局 KV
// 仅 890 B/token", 第二刀 and Fig. 5). The weighted ReLU sum is the reading
// stated in the header csa2.h.
//
// Mapping (decode shape): per query the 32 x 128 indexer query is the A
// operand of v_mfma_f32_32x32x16_f16 (rows = heads) and 32 keys are the B
// operand (columns = positions), eight MFMAs per 32 positions (K = 128). Lane
// l holds head/position l%32 and bytes (l/32)*64 .. +63 of the 128-byte row,
// so a wave streams 32 whole rows (4 KiB) per tile with 16-byte loads; the
// E4M3 bytes are converted to fp16 in registers (exact) just before their
// MFMA. The channel order inside a lane is irrelevant to the dot product as
// long as A and B agree. The accumulator holds, per lane, 16 of the 32 head
// dot products of one position; the epilogue applies ReLU and the head
// weights and adds the other half with one cross-half shuffle. The scan is
// HBM-bound (64 FLOP per byte); the MFMA keeps the 4096 MACs per key off the
// vector ALU.
//
// Why fp16 and not the FP8 MFMA here: on gfx950 v_mfma_f32_32x32x64_f8f6f4
// truncates each product to 13 fractional bits below the largest product of
// the instruction (measured with in-bounds probes: beside a product 2^8 a
// product below 2^-5 is dropped, 3 * 2^-6 becomes 2^-5), so its scores carry
// errors of 2e-5 .. 2e-4 of the 512-th score on the workloads' values, more
// than the 1e-5 near-tie band of the Top-K. The fp16 MFMA keeps products to
// 24 bits with round-to-nearest-even (beside 2^16 a product 2^-7 survives,
// 3 * 2^-8 rounds to 2^-6), i.e. FP32 accumulation; E4M3 and E2M1 values are
// exact in fp16. Every Top-K and pool decision is therefore taken on scores
// of this kernel.
//
// Variants of the same kernel (one instruction sequence per score, so every
// variant produces the same bits for a position): FP4 indexer keys (E2M1 codes
// with one E8M0 scale per 32 channels: codes converted to fp16 with the block
// scale relative to the key's largest block scale, that largest scale applied
// to the finished score as an exact power of two); NQ query tokens of one
// sequence per wave sharing each key tile; and scores of per-query block lists
// (the Reindex pool, or the blocks that a fused Top-K re-scores). The prefill
// shape further down shares key chunks among 16 or 32 queries through LDS and
// keeps the FP8 contraction (its roofline): its scores only narrow the
// candidates of a fused Top-K, which re-scores them here.
#include <type_traits>

#include "device_common.hpp"
#include "launchers.hpp"

namespace csa2 {
namespace {

constexpr int kTilePos = 32;       // positions per MFMA tile
constexpr int kWaves = 4;          // waves per work-group of the decode scan
// MODE 0: the Full scan; MODE 1: scores of listed blocks (Reindex inside the
// pool, or the re-scoring of a fused Top-K); MODE 2: as MODE 1, shaped for
// many queries (8 tiles per wave instead of 2).
// Tiles per wave (default): 8 for the Full scan (long rows, many work-groups
// anyway); 2 for a block list of a few queries, where more, shorter
// work-groups spread the work over more of the chip; 8 again once the queries
// alone fill it. A Full scan over few sequences takes 4 (kSmallFullGrid).
template <int MODE>
constexpr int tiles_per_wave() { return MODE == 1 ? 2 : 8; }
template <int MODE>
constexpr int items_per_wg(int tiles = tiles_per_wave<MODE>()) {
  return kTilePos * tiles * kWaves;
}
// Tiles in registers per wave (one scored, the rest in flight), as deep as
// three waves per SIMD allow the Full scan (at most 168 registers with the 16
// accumulators): 4 for FP8 keys (16 registers a tile; 1% faster than 3), 5 for
// FP4 keys (9 registers a tile; 3% faster decoder steps than 3, 6 is slower).
// The many-query block-list shape (MODE 2, FP8) then runs two waves per SIMD,
// as fast as with 3 tiles and three.
template <int KF>
constexpr int prefetch_tiles() { return KF ? 5 : 4; }

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

// max(x, 0) as one integer max on the bit pattern: every negative float
// (including -0) is a negative int32 and maps to +0; non-negative floats keep
// their bits. (fmaxf costs an extra canonicalising instruction per value.)
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Maximum over each aligned group of 8 lanes (a pool block of 8 positions),
// with DPP lane moves: swap neighbours, swap pairs, then mirror within 8 lanes.
__device__ __forceinline__ float max_over_8_lanes(float m) {
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x141, 0xF, 0xF, false)));
  return m;
}

// One 16-byte global -> LDS copy per lane, with no registers on the way: the
// wave's 64 pieces land in 64 consecutive 16-byte slots starting at `dst`
// (wave-uniform). Written as assembly so that the compiler does not make
// every later LDS read wait for the copy: the reads of the other buffer may
// proceed while it is in flight. wait_lds_dma() waits for all of them.
__device__ __forceinline__ void lds_dma16(const uint4* src, uint4* dst) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4*)dst;
  // m0 is saved and restored around the copy (the compiler reserves it)
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
               "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(lds_addr) : "memory");
}
// The same for one 4-byte word per lane (64 consecutive words at `dst`).
__device__ __forceinline__ void lds_dma4(const uint32_t* src, uint32_t* dst) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)dst;
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
               "global_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(lds_addr) : "memory");
}
// The same copies with the address split into a wave-uniform base (SGPRs)
// and a 32-bit per-lane byte offset: no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void lds_dma16_sv(uint32_t voff, const void* sbase, uint4* dst) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4*)dst;
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
               "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(lds_addr) : "memory");
}
__device__ __forceinline__ void lds_dma4_sv(uint32_t voff, const void* sbase, uint32_t* dst) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)dst;
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
               "global_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(lds_addr) : "memory");
}
__device__ __forceinline__ void wait_lds_dma() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// sum over the lane's 16 accumulator rows of w_r * relu(acc_r), in row order
__device__ __forceinline__ float weighted_relu_sum(const v16f& acc, const float* wr) {
  float part = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) part = fmaf(wr[r], relu_bits(acc[r]), part);
  return part;
}

// FP4 indexer keys (KF = 1): one key is 64 bytes of E2M1 codes plus 4 E8M0
// scales, one per 32 channels. The scaled FP8 x FP4 MFMA applies them itself:
// in v_mfma_scale_f32_32x32x64_f8f6f4 an FP4 B lane (column, half h) holds K
// values 32h..32h+31 in nibble order and its scale byte covers exactly those
// 32, while an FP8 A lane of half h holds K values 16h..16h+15 (bytes 0..15)
// and 32+16h..32+16h+15 (bytes 16..31) (measured with in-bounds impulse
// probes on gfx950). So MFMA j (channels 64j..64j+63) takes from a key lane
// code bytes 32j+16h..+15 with scale byte 2j+h, and from a query lane the
// 16-byte pieces 4j+h and 4j+2+h. The prefill shape feeds these bytes to that
// instruction; the decode shape loads the same bytes per lane (KTile4) and
// converts them to fp16 for the fp16 MFMA, its query operands staged in the
// matching channel order.
struct KTile4 {
  uint4 c[2];      // code bytes 16h..16h+15 and 32+16h..32+16h+15 of the key
  uint32_t sc;     // the key's four scale bytes (byte b: channels 32b..32b+31)
};

__device__ __forceinline__ void load_tile4(KTile4& t, const uint8_t* codes, const uint8_t* scales,
                                           bool ok) {
  if (ok) {
    t.c[0] = *reinterpret_cast<const uint4*>(codes);
    t.c[1] = *reinterpret_cast<const uint4*>(codes + 32);
    t.sc = *reinterpret_cast<const uint32_t*>(scales);
  } else {
    t.c[0] = t.c[1] = make_uint4(0, 0, 0, 0);
    t.sc = 0;
  }
}

__device__ __forceinline__ v8i fp4_operand(const uint4& a) {
  v8i r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = r[5] = r[6] = r[7] = 0;   // an FP4 operand uses the first four registers
  return r;
}

// 8 E4M3 bytes (two words) -> 8 fp16 values, exact.
__device__ __forceinline__ v8h e4m3x8_to_f16(uint32_t d0, uint32_t d1) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true);
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}
// 8 E2M1 codes (one word, channel 2k in the low nibble of byte k) times the
// power of two `scale` -> 8 fp16 values (exact while the product stays in the
// fp16 range).
__device__ __forceinline__ v8h e2m1x8_to_f16(uint32_t d, float scale) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 0);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 1);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 2);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 3);
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// The query operands of the eight fp16 MFMAs of a tile (lane: head l%32,
// half h = l/32). FP8 keys: MFMA j takes channels 64h + 8j .. +7. FP4 keys:
// MFMA j < 4 takes channels 32h + 8j .. +7 (scale block h), j >= 4 channels
// 64 + 32h + 8(j-4) .. +7 (block 2 + h), the order of the key lane's codes.
template <int KF>
__device__ __forceinline__ void query_f16(const uint4* q4, int half, v8h (&a)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int byte = KF ? (j < 4 ? 32 * half + 8 * j : 64 + 32 * half + 8 * (j - 4))
                        : 64 * half + 8 * j;
    const uint4 u = q4[byte >> 4];
    const bool hi = (byte & 8) != 0;
    a[j] = e4m3x8_to_f16(hi ? u.z : u.x, hi ? u.w : u.y);
  }
}

// 2^e as a float for any integer e >= -149 (exact).
__device__ __forceinline__ float pow2f(int e) { return ldexpf(1.0f, e); }

// The 32x32 head-by-position dot products of one tile, FP32-accurate; for FP4
// keys also the power of two that the finished score must be multiplied by.
__device__ __forceinline__ v16f dots_tile(const v8h (&a)[8], const KTile& t, float& post) {
  v16f acc = {};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint4& u = t.v[j >> 1];
    const v8h b = e4m3x8_to_f16((j & 1) ? u.z : u.x, (j & 1) ? u.w : u.y);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b, acc, 0, 0, 0);
  }
  post = 1.0f;
  return acc;
}
__device__ __forceinline__ v16f dots_tile(const v8h (&a)[8], const KTile4& t, float& post,
                                          int half) {
  // block scales relative to the key's largest, so every code fits fp16
  const uint32_t s0 = (t.sc >> (8 * half)) & 0xFFu, s1 = (t.sc >> (16 + 8 * half)) & 0xFFu;
  const uint32_t m01 = max(t.sc & 0xFFu, (t.sc >> 8) & 0xFFu);
  const uint32_t m23 = max((t.sc >> 16) & 0xFFu, t.sc >> 24);
  const int smax = (int)max(m01, m23);
  const float f0 = pow2f(max((int)s0 - smax, -126)), f1 = pow2f(max((int)s1 - smax, -126));
  v16f acc = {};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint4& u = t.c[j >> 2];
    const uint32_t d = (j & 3) == 0 ? u.x : (j & 3) == 1 ? u.y : (j & 3) == 2 ? u.z : u.w;
    const v8h b = e2m1x8_to_f16(d, j < 4 ? f0 : f1);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b, acc, 0, 0, 0);
  }
  post = pow2f(smax - 127);
  return acc;
}

// NQ > 1 (Full mode, several query tokens of one sequence, e.g. speculative
// decode): a wave scores NQ consecutive queries of the sequence against each key
// tile it loads, so a sequence's keys are read once per NQ queries. Every query
// runs the same instruction sequence as with NQ = 1 (same bits); each keeps its
// own visibility limit.
template <int MODE, int KF, int NQ, int TPW = tiles_per_wave<MODE>()>
__global__ __launch_bounds__(256) void k_index_score_decode(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, const uint8_t* __restrict__ k_scales,
    const int32_t* __restrict__ n_vis,
    const int32_t* __restrict__ pool, int T, int64_t n_cap, int64_t n_items,
    float* __restrict__ scores, float* __restrict__ bmax) {
  static_assert(MODE == 0 || NQ == 1, "query groups share keys only in the Full scan");
  const int groups = (T + NQ - 1) / NQ;           // query groups per sequence
  const int b = blockIdx.y / groups;
  const int t0 = (blockIdx.y % groups) * NQ;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int64_t n_blk = (n_cap + kBlock - 1) / kBlock;

  // per query of the group: index, visibility (0 past T), A operands (fp16,
  // in the channel order of the key lane's bytes; see query_f16), weights.
  int qi[NQ];
  bool real[NQ];
  int64_t nv[NQ];
  v8h a16[NQ][8];
  float wr[NQ][16];     // weights of the lane's 16 accumulator rows: 4 runs of 4 heads
  int64_t nv_max = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    real[q] = t0 + q < T;
    qi[q] = b * T + (real[q] ? t0 + q : T - 1);
    int64_t v = n_vis[qi[q]];
    v = v < 0 ? 0 : (v > n_cap ? n_cap : v);
    nv[q] = real[q] ? v : 0;
    nv_max = nv[q] > nv_max ? nv[q] : nv_max;
    const uint4* q4 = reinterpret_cast<const uint4*>(q_idx + (size_t)qi[q] * (kIdxHeads * kIdxDim) +
                                                     col * kIdxDim);
    query_f16<KF>(q4, half, a16[q]);
    const float4* w4 = reinterpret_cast<const float4*>(w + (size_t)qi[q] * kIdxHeads);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 x = w4[2 * j + half];   // heads 8j + 4*half .. +3
      wr[q][4 * j + 0] = x.x;
      wr[q][4 * j + 1] = x.y;
      wr[q][4 * j + 2] = x.z;
      wr[q][4 * j + 3] = x.w;
    }
  }

  constexpr int kKeyBytes = KF ? kIdxDim / 2 : kIdxDim;
  const uint8_t* kbase = k_idx + (size_t)b * (size_t)n_cap * kKeyBytes + half * (KF ? 16 : 64);
  const uint8_t* sbase = KF ? k_scales + (size_t)b * (size_t)n_cap * 4 : nullptr;
  // a Reindex query's block list: n_items / 8 entries (the pool's 2,048, or the
  // 512 best blocks of a fused Top-K)
  const int32_t* pl = MODE != 0 ? pool + (size_t)qi[0] * (size_t)(n_items >> 3) : nullptr;

  constexpr int kTilesPerWave = TPW;
  constexpr int kPrefetch = prefetch_tiles<KF>();
  const int64_t wave_base = (int64_t)blockIdx.x * items_per_wg<MODE>(TPW) +
                            (int64_t)wave * kTilePos * kTilesPerWave;

  // Reindex: the pool entries of all of this wave's tiles are fetched first, so
  // a tile's key loads never wait on a pool lookup.
  int32_t blk[kTilesPerWave];
#pragma unroll
  for (int it = 0; it < kTilesPerWave; ++it) {
    const int64_t item = wave_base + (int64_t)it * kTilePos + col;
    blk[it] = (MODE != 0 && item < n_items) ? pl[item >> 3] : -1;
  }
  // A tile is loaded where some query of the group sees the position.
  auto position_of = [&](int it, bool& ok) __attribute__((always_inline)) -> int64_t {
    const int64_t item = wave_base + (int64_t)it * kTilePos + col;
    if (MODE == 0) {
      ok = item < nv_max;
      return ok ? item : 0;
    }
    const int64_t b8 = blk[it];
    const int64_t pos = b8 * kBlock + (item & 7);
    ok = b8 >= 0 && b8 < n_blk && pos < nv[0];
    return ok ? pos : 0;
  };

  // Tiles are loaded kPrefetch - 1 ahead of the one being scored.
  using Tile = typename std::conditional<KF == 1, KTile4, KTile>::type;
  Tile buf[kPrefetch];
  bool okb[kPrefetch];
  auto load = [&](Tile& t, int64_t pos, bool ok) __attribute__((always_inline)) {
    if constexpr (KF == 1)
      load_tile4(t, kbase + pos * kKeyBytes, sbase + pos * 4, ok);
    else
      load_tile(t, kbase + pos * kKeyBytes, ok);
  };
  // (never beyond this wave's own tiles: blk[] holds kTilesPerWave entries)
#pragma unroll
  for (int i = 0; i < kPrefetch - 1 && i < kTilesPerWave; ++i) {
    const int64_t pos = position_of(i, okb[i]);
    load(buf[i], pos, okb[i]);
  }
#pragma unroll
  for (int it = 0; it < kTilesPerWave; ++it) {
    const int64_t tile0 = wave_base + (int64_t)it * kTilePos;
    if (tile0 >= n_items) break;
    constexpr int kAhead = kPrefetch - 1;
    if (it + kAhead < kTilesPerWave) {
      const int nb = (it + kAhead) % kPrefetch;
      const int64_t pos = position_of(it + kAhead, okb[nb]);
      load(buf[nb], pos, okb[nb]);
    }
    const Tile& cur = buf[it % kPrefetch];
    const bool cur_ok = okb[it % kPrefetch];
    const int64_t item = tile0 + col;
    const bool any_ok = __any(cur_ok);   // skip the MFMAs when no lane holds a visible key
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float s = -INFINITY;
      if (any_ok) {
        float post;
        v16f acc;
        if constexpr (KF == 1)
          acc = dots_tile(a16[q], cur, post, half);
        else
          acc = dots_tile(a16[q], cur, post);
        const float part = weighted_relu_sum(acc, wr[q]);
        // lo-half + hi-half row sums, in every lane
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                         __float_as_uint(part), false, false);
        const float tot = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * post;
        const bool vis = MODE == 0 ? item < nv[q] : cur_ok;
        if (cur_ok && vis) s = tot;
      }
      if (!real[q]) continue;
      if (scores && half == 0 && item < n_items) scores[(size_t)qi[q] * (size_t)n_items + item] = s;
      if (bmax) {
        const float m = max_over_8_lanes(s);
        if (half == 0 && (col & 7) == 0 && item < n_items)
          bmax[(size_t)qi[q] * (size_t)n_blk + (item >> 3)] = m;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill shape: many queries share each sequence's keys, so the scan is a
// dense FP8 contraction of (queries x 32 heads) x 128 against positions x 128,
// followed by the ReLU-weighted head sum. A work-group of 8 waves takes 32
// consecutive queries of one sequence (4 per wave, their A operands and head
// weights held in registers; 16 queries, 2 per wave, when a sequence has at
// most 16, so that more waves hold real queries) and 4,096 positions, streamed
// through LDS in double-buffered chunks of 256 keys (32 KiB each) so every key
// byte read from L2 feeds all of the tile's queries. Waves whose queries are
// all padding skip their MFMAs. The 16-byte pieces of a key row are stored at piece
// index (p ^ (row & 7)), which makes the B-operand reads (8 consecutive rows
// per lane group) and the chunk writes conflict-free. Per 32-position tile and
// query: two MFMAs, then 16 max + 16 fma per lane; the two half-sums of a
// query pair are combined with one v_permlane32_swap (lanes 0..31 end up with
// the first query's 32 scores, lanes 32..63 with the second's), so each store
// writes 2 x 128 contiguous bytes. The head sum runs in the same order as in
// the decode kernel, but the dot products come from the FP8 MFMA (which drops
// product bits below 2^-13 of each instruction's largest product) instead of
// the fp16 MFMA on exactly converted keys (float32-accurate), so the scores
// agree with the decode kernel's within that truncation bound, not bit for bit.
constexpr int kPfQPerWave = 4;
constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kPfSmallTile = 16;                     // 2 queries per wave up to this T
constexpr int kPfChunk = 256;                        // keys per LDS chunk
constexpr int kPfChunksPerWG = 16;
constexpr int kPfKeysPerWG = kPfChunk * kPfChunksPerWG;   // 4096
constexpr int kPfPieces = kPfChunk * (kIdxDim / 16);      // 2048 16-byte pieces
constexpr int kPfLoads = kPfPieces / kPfThreads;            // 4 per thread
static_assert(kPfPieces % kPfThreads == 0, "a chunk is a whole number of loads per thread");

// FP4 keys (KF = 1): a chunk holds 256 x 64 bytes of codes (4 pieces per key,
// piece j of row r at slot 4r + (j ^ ((r/8) & 3))) and the keys' 4-byte scale
// words; the B operand of MFMA j is code piece 2j + h with scale byte 2j + h
// (the operand order measured for the scaled FP8 x FP4 instruction, see
// above). The scale word rides in the FP4 operand's four unused registers.
constexpr int kPfPieces4 = kPfChunk * (kIdxDim / 2 / 16);   // 1024 code pieces
constexpr int kPfLoads4 = kPfPieces4 / kPfThreads;           // 2 per thread
static_assert(kPfChunk % 64 == 0 && kPfChunk / 64 <= kPfWaves, "one scale word per lane");

template <bool BMAX, int KF, int QPW, bool SC>
__global__ __launch_bounds__(kPfThreads) void k_index_score_prefill(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, const uint8_t* __restrict__ k_scales,
    const int32_t* __restrict__ n_vis, int T, int64_t n_cap,
    int n_kb, int n_qb, float* __restrict__ scores, float* __restrict__ bmax) {
  __shared__ uint4 lds[2][KF ? kPfPieces4 : kPfPieces];
  __shared__ uint32_t lsc[2][KF ? kPfChunk : 1];
  // Key blocks vary slowest over the grid: the work-groups that run together
  // share a key block through L2, and the last (ragged, shorter) key block's
  // work-groups come last, where they fill the tail instead of leaving whole
  // work-groups to start late (c3: 2.05 -> 1.97 ms).
  const int per_kb = (int)(gridDim.x / (unsigned)n_kb);   // work-groups per key block
  const int kb = (int)blockIdx.x / per_kb;
  const int rest = (int)blockIdx.x % per_kb;
  const int qb = rest % n_qb;
  const int b = rest / n_qb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int half = lane >> 5;
  const int col = lane & 31;
  const int64_t n_blk = (n_cap + kBlock - 1) / kBlock;

  // this wave's queries (clamped for loads; stores check t < T)
  int tq[QPW];
  int64_t nv[QPW];
  v8i a0[QPW], a1[QPW];
  float wr[QPW][16];
  int64_t nv_max = 0, nv_min = n_cap;
#pragma unroll
  for (int q = 0; q < QPW; ++q) {
    tq[q] = qb * (QPW * kPfWaves) + wave * QPW + q;
    const int tc = tq[q] < T ? tq[q] : T - 1;
    const size_t qi = (size_t)b * T + tc;
    int64_t v = n_vis[qi];
    v = v < 0 ? 0 : (v > n_cap ? n_cap : v);
    nv[q] = tq[q] < T ? v : 0;
    nv_max = nv[q] > nv_max ? nv[q] : nv_max;
    nv_min = nv[q] < nv_min ? nv[q] : nv_min;
    const uint4* q4 = reinterpret_cast<const uint4*>(q_idx + qi * (kIdxHeads * kIdxDim) +
                                                     col * kIdxDim);
    a0[q] = KF ? as_v8i(q4[half], q4[2 + half]) : as_v8i(q4[4 * half], q4[4 * half + 1]);
    a1[q] = KF ? as_v8i(q4[4 + half], q4[6 + half]) : as_v8i(q4[4 * half + 2], q4[4 * half + 3]);
#pragma unroll
    for (int r = 0; r < 16; ++r) wr[q][r] = w[qi * kIdxHeads + acc32_row(lane, r)];
  }

  const int64_t key0 = (int64_t)kb * kPfKeysPerWG;
  int64_t span = n_cap - key0;
  span = span < kPfKeysPerWG ? span : kPfKeysPerWG;
  const int n_chunks = (int)((span + kPfChunk - 1) / kPfChunk);
  constexpr int kKeyBytes = KF ? kIdxDim / 2 : kIdxDim;
  const uint8_t* kseq = k_idx + (size_t)b * (size_t)n_cap * kKeyBytes;
  const uint32_t* sseq = KF ? reinterpret_cast<const uint32_t*>(k_scales) + (size_t)b * (size_t)n_cap
                            : nullptr;

  // K rows of chunk c go straight from global memory into LDS buffer `buf`
  // (no registers on the way): LDS slot s = row*8 + j holds piece
  // j ^ ((row/8) & 7) of the chunk's row `row` (FP4: slot row*4 + j holds
  // piece j ^ ((row/8) & 3), and waves 0..3 copy the scale words). Each wave's
  // load fills 64 consecutive slots. Rows past n_cap repeat the last row; their
  // scores are masked to -inf.
  // Byte offsets of this thread's pieces inside a whole chunk (the same for
  // every chunk): with them a chunk that lies below n_cap is copied from a
  // wave-uniform base.
  constexpr int kLoads = KF ? kPfLoads4 : kPfLoads;
  uint32_t poff[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int slot = tid + i * kPfThreads;
    const int row = KF ? slot >> 2 : slot >> 3;
    const int piece = KF ? (slot & 3) ^ ((row >> 3) & 3) : (slot & 7) ^ ((row >> 3) & 7);
    poff[i] = (uint32_t)(row * kKeyBytes + piece * 16);
  }
  auto load_chunk = [&](int c, int buf) __attribute__((always_inline)) {
    const int64_t first = key0 + (int64_t)c * kPfChunk;
    if (first + kPfChunk <= n_cap) {
      const uint8_t* base = kseq + first * kKeyBytes;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) lds_dma16_sv(poff[i], base, &lds[buf][i * kPfThreads + wave * 64]);
      if constexpr (KF == 1) {
        if (wave < kPfChunk / 64) lds_dma4_sv((uint32_t)tid * 4u, sseq + first, &lsc[buf][wave * 64]);
      }
      return;
    }
    if constexpr (KF == 1) {
#pragma unroll
      for (int i = 0; i < kPfLoads4; ++i) {
        const int slot = tid + i * kPfThreads;
        const int row = slot >> 2;
        int64_t krow = key0 + (int64_t)c * kPfChunk + row;
        krow = krow < n_cap ? krow : n_cap - 1;
        const int piece = (slot & 3) ^ ((row >> 3) & 3);
        lds_dma16(reinterpret_cast<const uint4*>(kseq + krow * kKeyBytes) + piece,
                  &lds[buf][i * kPfThreads + wave * 64]);
      }
      if (wave < kPfChunk / 64) {
        int64_t krow = key0 + (int64_t)c * kPfChunk + tid;
        krow = krow < n_cap ? krow : n_cap - 1;
        lds_dma4(sseq + krow, &lsc[buf][wave * 64]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kPfLoads; ++i) {
        const int slot = tid + i * kPfThreads;
        const int row = slot >> 3;
        int64_t krow = key0 + (int64_t)c * kPfChunk + row;
        krow = krow < n_cap ? krow : n_cap - 1;
        const int piece = (slot & 7) ^ ((row >> 3) & 7);
        lds_dma16(reinterpret_cast<const uint4*>(kseq + krow * kIdxDim) + piece,
                  &lds[buf][i * kPfThreads + wave * 64]);
      }
    }
  };

  // B operand of tile tt of an LDS chunk: column `col` of tile tt is key
  // 8*col + tt of the chunk, so over the chunk's 8 tiles a lane sees one whole
  // block of 8 positions (its block maximum stays in a register). Pieces are
  // swizzled by row/8, which differs across 8 consecutive lanes.
  int cur_buf = 0;     // the buffer load_b reads (FP4 scale words)
  auto load_b = [&](const uint4* L, int tt, v8i& b0, v8i& b1) __attribute__((always_inline)) {
    const int row = kBlock * col + tt;
    if constexpr (KF == 1) {
      const int sw = col & 3;
      const uint4 c0 = L[row * 4 + (half ^ sw)], c1 = L[row * 4 + ((2 + half) ^ sw)];
      const uint32_t scw = lsc[cur_buf][row] >> (8 * half);
      b0 = fp4_operand(c0);
      b1 = fp4_operand(c1);
      b0[4] = (int)scw;            // scale bytes 0 and 2: MFMA 0 and MFMA 1
      b1[4] = (int)(scw >> 16);
    } else {
      const int sw = col & 7;
      b0 = as_v8i(L[row * 8 + ((half * 4 + 0) ^ sw)], L[row * 8 + ((half * 4 + 1) ^ sw)]);
      b1 = as_v8i(L[row * 8 + ((half * 4 + 2) ^ sw)], L[row * 8 + ((half * 4 + 3) ^ sw)]);
    }
  };
  auto mfma2 = [&](int q, const v8i& b0, const v8i& b1) __attribute__((always_inline)) -> v16f {
    v16f acc = {};
    if constexpr (KF == 1) {
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0[q], b0, acc, 0, 4, 0, 127, 0, b0[4]);
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1[q], b1, acc, 0, 4, 0, 127, 0, b1[4]);
    } else {
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0[q], b0, acc, 0, 0, 0, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1[q], b1, acc, 0, 0, 0, 0, 0, 0);
    }
    return acc;
  };
  constexpr int kPairs = QPW / 2;
  // Lanes 0..31 take query 2qp, lanes 32..63 query 2qp+1 of each pair after
  // the swap; bm[qp] is the running maximum of this lane's block.
  float bm[kPairs];
  // Slow path (ragged chunk or partial wave): every check per key.
  auto emit = [&](int64_t chunk0, int tt, const float* p) __attribute__((always_inline)) {
    const int64_t key = chunk0 + kBlock * col + tt;
#pragma unroll
    for (int qp = 0; qp < kPairs; ++qp) {
      const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[2 * qp]),
                                                        __float_as_uint(p[2 * qp + 1]), false, false);
      float s = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
      const int64_t nvq = half ? nv[2 * qp + 1] : nv[2 * qp];
      const int tqq = half ? tq[2 * qp + 1] : tq[2 * qp];
      if (key >= nvq) s = -INFINITY;
      const bool store = tqq < T && key < n_cap;
      const size_t qi = (size_t)b * T + (size_t)tqq;
      if (SC && store) scores[qi * (size_t)n_cap + key] = s;
      bm[qp] = fmaxf(bm[qp], s);
    }
  };
  // Block maxima of the chunk: lane col holds block chunk0/8 + col.
  auto emit_bmax = [&](int64_t chunk0) __attribute__((always_inline)) {
    if (!BMAX) return;
    const int64_t blk = (chunk0 >> 3) + col;
#pragma unroll
    for (int qp = 0; qp < kPairs; ++qp) {
      const int tqq = half ? tq[2 * qp + 1] : tq[2 * qp];
      const size_t qi = (size_t)b * T + (size_t)tqq;
      if (tqq < T && blk < n_blk) bmax[qi * (size_t)n_blk + blk] = bm[qp];
    }
  };

  // Stores of a fast-path tile: every query of the wave is real and every key
  // below n_cap, so the chunk's code is one basic block (no exec branches).
  // Per chunk each lane keeps one score pointer (its block's first position)
  // and one visibility limit per query pair.
  float* sp[kPairs];
  int lim[kPairs];
  auto chunk_setup = [&](int64_t chunk0) __attribute__((always_inline)) {
#pragma unroll
    for (int qp = 0; qp < kPairs; ++qp) {
      const int64_t nvq = half ? nv[2 * qp + 1] : nv[2 * qp];
      const int tqq = half ? tq[2 * qp + 1] : tq[2 * qp];
      const size_t qi = (size_t)b * T + (size_t)tqq;
      if constexpr (SC) sp[qp] = scores + qi * (size_t)n_cap + chunk0 + kBlock * col;
      int64_t l = nvq - chunk0 - kBlock * col;
      lim[qp] = (int)(l < -1 ? -1 : (l > kBlock ? kBlock : l));
      bm[qp] = -INFINITY;
    }
  };
  auto emit_fast = [&](int t, const float* p, auto masked) __attribute__((always_inline)) {
#pragma unroll
    for (int qp = 0; qp < kPairs; ++qp) {
      const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[2 * qp]),
                                                        __float_as_uint(p[2 * qp + 1]), false, false);
      float s = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
      if constexpr (decltype(masked)::value) s = t < lim[qp] ? s : -INFINITY;
      if constexpr (SC) sp[qp][t] = s;
      if (BMAX) bm[qp] = fmaxf(bm[qp], s);
    }
  };
  const bool wave_full = tq[QPW - 1] < T;

  constexpr int kTiles = kPfChunk / kTilePos;     // 8
  load_chunk(0, 0);
  wait_lds_dma();
  __syncthreads();
  for (int c = 0; c < n_chunks; ++c) {
    if (c + 1 < n_chunks) load_chunk(c + 1, (c + 1) & 1);
    const uint4* L = lds[c & 1];
    cur_buf = c & 1;
    const int64_t chunk0 = key0 + (int64_t)c * kPfChunk;
    if (wave_full && chunk0 + kPfChunk <= n_cap && chunk0 < nv_max) {
      // Whole chunk in range: a flat software pipeline over the 32 (tile,
      // query) steps; step j+1's MFMAs are issued before step j's epilogue, and
      // the next tile's B operand is read from LDS as soon as the last MFMA on
      // the current one has been issued. Chunks that every query of the wave
      // sees whole skip the per-key visibility test (masked = false).
      auto run_fast = [&](auto masked) __attribute__((always_inline)) {
        v8i bb0, bb1;
        v16f acc[2];
        float p[QPW];
        chunk_setup(chunk0);
        load_b(L, 0, bb0, bb1);
        acc[0] = mfma2(0, bb0, bb1);
#pragma unroll
        for (int j = 0; j < kTiles * QPW; ++j) {
          const int t = j / QPW, q = j % QPW;
          if (j + 1 < kTiles * QPW) {
            const int t1 = (j + 1) / QPW, q1 = (j + 1) % QPW;
            // raised wave priority while issuing: the matrix core is kept fed
            // when the other wave on this SIMD is also ready to issue
            __builtin_amdgcn_s_setprio(1);
            acc[(j + 1) & 1] = mfma2(q1, bb0, bb1);
            __builtin_amdgcn_s_setprio(0);
            // the last MFMA on tile t1 is issued: fetch the next tile's operand
            if (q1 == QPW - 1 && t1 + 1 < kTiles) load_b(L, t1 + 1, bb0, bb1);
          }
          // Keep this order: the epilogue below reads results issued one step
          // earlier, so it runs on the vector ALU while the matrix core works
          // on the MFMAs just issued.
          __builtin_amdgcn_sched_barrier(0);
          p[q] = weighted_relu_sum(acc[j & 1], wr[q]);
          // The empty asm makes p[q] exist here: otherwise the compiler sinks
          // each epilogue to its use in emit_fast and runs the four queries'
          // epilogues back to back after their MFMAs, the last one waiting for
          // results just issued (and 15 more registers live).
          asm volatile("" : "+v"(p[q]));
          if (q == QPW - 1) emit_fast(t, p, masked);
          __builtin_amdgcn_sched_barrier(0);
        }
        emit_bmax(chunk0);
      };
      if (chunk0 + kPfChunk <= nv_min)
        run_fast(std::false_type{});
      else
        run_fast(std::true_type{});
    } else {
      // Ragged last chunk, a partial wave, or nothing visible to this wave's
      // queries (rows past n_cap repeat the last row; keys checked one by one).
#pragma unroll
      for (int qp = 0; qp < kPairs; ++qp) bm[qp] = -INFINITY;
      const bool any_vis = chunk0 < nv_max;
#pragma unroll 1
      for (int tt = 0; tt < kTiles; ++tt) {
        float p[QPW];
        if (any_vis) {
          v8i b0, b1;
          load_b(L, tt, b0, b1);
#pragma unroll
          for (int q = 0; q < QPW; ++q) p[q] = weighted_relu_sum(mfma2(q, b0, b1), wr[q]);
        } else {
#pragma unroll
          for (int q = 0; q < QPW; ++q) p[q] = 0.0f;
        }
        emit(chunk0, tt, p);
      }
      emit_bmax(chunk0);
    }
    wait_lds_dma();   // the next chunk has landed in LDS
    __syncthreads();
  }
}

}  // namespace

// Queries per wave of the Full scan when several query tokens of one sequence
// share each key tile: 2 (each query's fp16 operands take 32 registers).
template <int KF>
constexpr int decode_group() { return 2; }

// From this many queries on, the Reindex scan over the pool uses 8 tiles per
// wave (2 below it, where more work-groups per query pay off): 1-2% faster
// steps at 64-256 queries of 1M-entry contexts.
constexpr int kPoolManyQueries = 64;

// A single-token Full scan whose default grid has fewer work-groups than this
// (a few sequences, e.g. 8 x 1M positions: 8,192) runs 4 tiles per wave: the
// shorter work-groups leave a shorter tail before the dependent selection
// (2% faster decoder steps at 8 x 1M); 64 x 512K (32,768) keeps 8.
constexpr int64_t kSmallFullGrid = 16384;

template <int KF>
hipError_t launch_decode(int mode, const uint8_t* q_idx, const float* w, const uint8_t* keys,
                         const uint8_t* scales, const int32_t* n_vis, const int32_t* pool, int B,
                         int T, int64_t n_cap, float* scores, float* bmax, hipStream_t st) {
  const int64_t n_items = mode == 0 ? n_cap : (int64_t)kPoolCand;
  const int64_t per_wg = mode == 0 ? items_per_wg<0>() : items_per_wg<1>();
  const unsigned gx = (unsigned)((n_items + per_wg - 1) / per_wg);
  if (mode == 1 && B * T >= kPoolManyQueries) {
    constexpr int64_t per2 = items_per_wg<2>();
    hipLaunchKernelGGL((k_index_score_decode<2, KF, 1>), dim3((unsigned)((n_items + per2 - 1) / per2),
                       (unsigned)(B * T)), dim3(256), 0, st, q_idx, w, keys, scales, n_vis, pool, T,
                       n_cap, n_items, scores, nullptr);
  } else if (mode == 1) {
    hipLaunchKernelGGL((k_index_score_decode<1, KF, 1>), dim3(gx, (unsigned)(B * T)), dim3(256), 0,
                       st, q_idx, w, keys, scales, n_vis, pool, T, n_cap, n_items, scores, nullptr);
  } else if (T == 1 && (int64_t)gx * B < kSmallFullGrid) {
    constexpr int64_t per4 = items_per_wg<0>(4);
    hipLaunchKernelGGL((k_index_score_decode<0, KF, 1, 4>),
                       dim3((unsigned)((n_items + per4 - 1) / per4), (unsigned)B), dim3(256), 0,
                       st, q_idx, w, keys, scales, n_vis, pool, T, n_cap, n_items, scores, bmax);
  } else if (T == 1) {
    hipLaunchKernelGGL((k_index_score_decode<0, KF, 1>), dim3(gx, (unsigned)B), dim3(256), 0, st,
                       q_idx, w, keys, scales, n_vis, pool, T, n_cap, n_items, scores, bmax);
  } else {
    constexpr int G = decode_group<KF>();
    const unsigned gy = (unsigned)(B * ((T + G - 1) / G));
    hipLaunchKernelGGL((k_index_score_decode<0, KF, G>), dim3(gx, gy), dim3(256), 0, st,
                       q_idx, w, keys, scales, n_vis, pool, T, n_cap, n_items, scores, bmax);
  }
  return hipGetLastError();
}

// From this many queries on, a block-list re-scoring uses 8 tiles per wave.
constexpr int kManyQueries = 512;

hipError_t launch_rescore_blocks(const uint8_t* q_idx, const float* w, const uint8_t* keys,
                                 const uint8_t* scales, const int32_t* n_vis, const int32_t* blocks,
                                 int n_blocks, int B, int T, int64_t n_cap, float* vals,
                                 hipStream_t st) {
  const int64_t n_items = (int64_t)n_blocks * kBlock;
  const int Q = B * T;
  auto go = [&](auto mode_c, auto kf_c) {
    constexpr int M = decltype(mode_c)::value, K = decltype(kf_c)::value;
    const int64_t per_wg = items_per_wg<M>();
    hipLaunchKernelGGL((k_index_score_decode<M, K, 1>),
                       dim3((unsigned)((n_items + per_wg - 1) / per_wg), (unsigned)Q), dim3(256),
                       0, st, q_idx, w, keys, scales, n_vis, blocks, T, n_cap, n_items, vals,
                       nullptr);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if (Q >= kManyQueries) {
    if (scales) go(I2{}, I1{}); else go(I2{}, I0{});
  } else {
    if (scales) go(I1{}, I1{}); else go(I1{}, I0{});
  }
  return hipGetLastError();
}

hipError_t launch_index_score_decode(int mode, const uint8_t* q_idx, const float* w,
                                     const uint8_t* k_idx, const int32_t* n_vis,
                                     const int32_t* pool, int B, int T, int64_t n_cap,
                                     float* scores, float* bmax, hipStream_t st) {
  return launch_decode<0>(mode, q_idx, w, k_idx, nullptr, n_vis, pool, B, T, n_cap, scores, bmax,
                          st);
}

hipError_t launch_index_score_decode_fp4k(int mode, const uint8_t* q_idx, const float* w,
                                          const uint8_t* k_codes, const uint8_t* k_scales,
                                          const int32_t* n_vis, const int32_t* pool, int B, int T,
                                          int64_t n_cap, float* scores, float* bmax,
                                          hipStream_t st) {
  return launch_decode<1>(mode, q_idx, w, k_codes, k_scales, n_vis, pool, B, T, n_cap, scores,
                          bmax, st);
}

template <int KF>
hipError_t launch_prefill(const uint8_t* q_idx, const float* w, const uint8_t* keys,
                          const uint8_t* scales, const int32_t* n_vis, int B, int T, int64_t n_cap,
                          float* scores, float* bmax, hipStream_t st) {
  const int n_kb = (int)((n_cap + kPfKeysPerWG - 1) / kPfKeysPerWG);
  auto go = [&](auto qpw_c) {
    constexpr int QPW = decltype(qpw_c)::value;
    constexpr int kQ = QPW * kPfWaves;
    const int n_qb = (T + kQ - 1) / kQ;
    const int64_t grid = (int64_t)n_kb * n_qb * B;
    if (bmax && scores)
      hipLaunchKernelGGL((k_index_score_prefill<true, KF, QPW, true>), dim3((unsigned)grid),
                         dim3(kPfThreads), 0, st, q_idx, w, keys, scales, n_vis, T, n_cap, n_kb,
                         n_qb, scores, bmax);
    else if (bmax)
      hipLaunchKernelGGL((k_index_score_prefill<true, KF, QPW, false>), dim3((unsigned)grid),
                         dim3(kPfThreads), 0, st, q_idx, w, keys, scales, n_vis, T, n_cap, n_kb,
                         n_qb, scores, bmax);
    else
      hipLaunchKernelGGL((k_index_score_prefill<false, KF, QPW, true>), dim3((unsigned)grid),
                         dim3(kPfThreads), 0, st, q_idx, w, keys, scales, n_vis, T, n_cap, n_kb,
                         n_qb, scores, bmax);
  };
  // up to 16 query tokens per sequence: 16-query tiles (2 per wave) keep twice
  // as many waves busy as half-empty 32-query tiles
  if (T <= kPfSmallTile)
    go(std::integral_constant<int, 2>{});
  else
    go(std::integral_constant<int, kPfQPerWave>{});
  return hipGetLastError();
}

hipError_t launch_index_score_prefill(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                                      const int32_t* n_vis, int B, int T, int64_t n_cap,
                                      float* scores, float* bmax, hipStream_t st) {
  return launch_prefill<0>(q_idx, w, k_idx, nullptr, n_vis, B, T, n_cap, scores, bmax, st);
}

hipError_t launch_index_score_prefill_fp4k(const uint8_t* q_idx, const float* w,
                                           const uint8_t* k_codes, const uint8_t* k_scales,
                                           const int32_t* n_vis, int B, int T, int64_t n_cap,
                                           float* scores, float* bmax, hipStream_t st) {
  return launch_prefill<1>(q_idx, w, k_codes, k_scales, n_vis, B, T, n_cap, scores, bmax, st);
}

}  // namespace csa2
