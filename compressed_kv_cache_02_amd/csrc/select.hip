// Exact Top-K selection (Top-512 per query; 2,048 blocks for the pool) by radix
// select on order-preserving 32-bit keys of the float scores.
//
// Pages: Top-512 per query ("DeepSeek V4.1-Flash 为什么这么强？CED 与 CSA2
// 架构全拆解", §二 layer layout); Full picks its own Top-K over every visible
// position, Reindex its own inside the pool, Reuse copies (same §二, mode
// table); the pool keeps the 2,048 blocks of 8 with the highest in-block maximum
// (same §二, hierarchical sparse indexer; "DeepSeek-V4.1-Flash：全局 KV 仅
// 890 B/token", 第二刀 and Fig. 5). Ties go to the lower position and the result
// is emitted in ascending order (the reading stated in csa2.h).
//
// Items are visited in position order (Full: item = position; Reindex: the
// pool is ascending, so item order is position order; pool: item = block id).
//
// Small inputs (<= 16,384 items per query, e.g. every Reindex layer): one
// work-group of 1,024 threads per query holds 16 consecutive items per thread
// in registers, runs three histogram levels (bits 31..21, 20..10, 9..0) in LDS
// to find the exact K-th key, takes the ties lowest-position first with a block
// prefix sum, and writes the selection ascending with a second prefix sum (the
// items are already in position order, so no sort is needed).
//
// Large inputs: a grid over (chunk, query) per pass --
//   zero   -- clear the per-query histograms and counters (a fill kernel, safe
//             to capture in a HIP graph);
//   hist1  -- 2,048-bin histogram of key bits 31..21, then one work-group per
//             query derives the bin holding the K-th key;
//   hist2  -- 2,048-bin histogram of bits 20..10 inside that bin, then one
//             work-group per query derives the 22-bit prefix of the K-th key;
//   filter -- items above that prefix are certain (fewer than K) and appended
//             to one list, items sharing it to a candidate list;
//   final  -- one work-group per query ranks the candidates by (key desc,
//             position asc), sorts the K positions and writes them. If the
//             candidates overflow their buffer (tie-heavy input) it falls back
//             to a third histogram level and an in-order scan of the input:
//             exact but slow.
#include "device_common.hpp"
#include "launchers.hpp"

namespace csa2 {
namespace {

constexpr int kBins = 2048;
constexpr int kCandCap = 4096;
constexpr int kThreads = 256;
constexpr int kItemsPerThread = 16;
constexpr int kChunk = kThreads * kItemsPerThread;   // 4096 items per work-group
constexpr int kSmallThreads = 1024;
constexpr int kSmallMax = kSmallThreads * kItemsPerThread;   // 16,384
constexpr int kFinalThreads = 1024;

// Per-query thresholds derived after each histogram pass.
struct Thresh {
  uint32_t all;      // 1: every valid item is selected
  uint32_t b1;       // bin of bits 31..21 holding the K-th key
  uint32_t above1;   // items in higher bins
  uint32_t b2;       // bin of bits 20..10 (inside b1) holding the K-th key
  uint32_t above;    // items with a higher 22-bit prefix
  uint32_t kk;       // number selected = min(K, valid items)
  uint32_t pad[2];
};

// Per-query workspace record.
struct SelWs {
  uint32_t hist1[kBins];
  uint32_t hist2[kBins];
  uint32_t cnt[8];           // [0] sure, [1] candidates
  Thresh th;
  uint32_t pad[48];
};

__host__ __device__ inline size_t sel_stride(int K) {
  return sizeof(SelWs) + (size_t)K * 8 + (size_t)kCandCap * 8;
}

struct Items {
  int kind;
  const float* values;
  const int32_t* n_vis;
  const int32_t* pool;
  int64_t n_items;   // values per query row
  int64_t n_cap;

  // Validity, key and position of item i of query q. The score load does not
  // depend on the pool lookup (it is indexed by the item, clamped into the row),
  // so both are in flight together.
  __device__ __forceinline__ bool get(int q, int64_t i, int64_t nv, const int32_t* pl,
                                      uint32_t& key, uint32_t& pos) const {
    const bool in = i < n_items;
    const int64_t ic = in ? i : 0;
    const float val = values[(size_t)q * (size_t)n_items + ic];
    int64_t p = ic;
    bool v;
    if (kind == kSelFull) {
      v = in && i < nv;
    } else if (kind == kSelPool) {
      v = in && i < (nv + kBlock - 1) / kBlock;
    } else {
      const int64_t blk = pl[ic >> 3];
      const int64_t n_blk = (n_cap + kBlock - 1) / kBlock;
      p = blk * kBlock + (ic & 7);
      v = in && blk >= 0 && blk < n_blk && p < nv;
    }
    key = float_key(val);
    pos = (uint32_t)p;
    return v;
  }

  __device__ __forceinline__ int64_t visible(int q) const {
    int64_t nv = n_vis[q];
    return nv < 0 ? 0 : (nv > n_cap ? n_cap : nv);
  }
};

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Exclusive scan over the NT threads of a block; also returns the total.
// `sh` holds NT/64 words.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v, lane);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  uint32_t base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t x = sh[w];
    if (w < wave) base += x;
    total += x;
  }
  __syncthreads();
  return base + inc - v;
}

// Highest bin b of an LDS histogram with sum(hist[b..]) >= k (1 <= k <= total),
// and above = sum(hist[b+1..]). NT threads each own kBins/NT bins from the top.
// `sh` holds NT/64 + 2 words. Every thread gets the result.
template <int NT>
__device__ void find_threshold(const uint32_t* hist, uint32_t k, uint32_t* sh, uint32_t& bin_out,
                               uint32_t& above_out) {
  constexpr int per = kBins / NT;
  const int hi = kBins - per * (int)threadIdx.x;   // owns bins [hi-per, hi)
  uint32_t s = 0;
#pragma unroll
  for (int j = 1; j <= per; ++j) s += hist[hi - j];
  uint32_t total;
  const uint32_t before = block_excl_scan<NT>(s, sh, total);
  if (before < k && before + s >= k) {
    uint32_t run = before;
#pragma unroll
    for (int j = 1; j <= per; ++j) {
      const uint32_t h = hist[hi - j];
      if (run + h >= k) {
        sh[NT / 64] = (uint32_t)(hi - j);
        sh[NT / 64 + 1] = run;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
  bin_out = sh[NT / 64];
  above_out = sh[NT / 64 + 1];
  __syncthreads();
}

__device__ __forceinline__ void hist_add(uint32_t* lh, uint32_t bin, bool pred) {
  if (pred) atomicAdd(&lh[bin], 1u);
}

// ------------------------------------------------------------ small inputs --

__global__ __launch_bounds__(kSmallThreads) void k_sel_small(Items it, int K, int32_t* out) {
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t sh[kSmallThreads / 64 + 2];
  const int q = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t nv = it.visible(q);
  const int32_t* pl = it.kind == kSelReindex ? it.pool + (size_t)q * kPoolBlocks : nullptr;
  uint32_t key[kItemsPerThread], pos[kItemsPerThread];
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < kItemsPerThread; ++j) {
    const int64_t i = (int64_t)t * kItemsPerThread + j;
    key[j] = 0;
    pos[j] = 0;
    if (it.get(q, i, nv, pl, key[j], pos[j])) valid |= 1u << j;
  }
  uint32_t total;
  block_excl_scan<kSmallThreads>(__popc(valid), sh, total);
  const uint32_t kk = total < (uint32_t)K ? total : (uint32_t)K;
  uint32_t kth = 0, ties_needed = 0;   // select key > kth, plus the first ties_needed == kth
  const bool all = total <= (uint32_t)K;
  if (!all) {
    uint32_t prefix = 0, above = 0;
    // three levels: bits 31..21, 20..10, 9..0
#pragma unroll
    for (int level = 0; level < 3; ++level) {
      const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
      const uint32_t mask = level == 2 ? 0x3FFu : 0x7FFu;
      for (int i = t; i < kBins; i += kSmallThreads) lh[i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kItemsPerThread; ++j) {
        const bool in = ((valid >> j) & 1u) &&
                        (level == 0 || (key[j] >> (shift + (level == 1 ? 11 : 10))) == prefix);
        hist_add(lh, (key[j] >> shift) & mask, in);
      }
      __syncthreads();
      uint32_t bin, ab;
      find_threshold<kSmallThreads>(lh, (uint32_t)K - above, sh, bin, ab);
      above += ab;
      // prefix after level 0: bits 31..21; level 1: bits 31..10; level 2: the key
      prefix = level == 0 ? bin : ((prefix << (level == 1 ? 11 : 10)) | bin);
    }
    kth = prefix;
    ties_needed = (uint32_t)K - above;
  }
  // ties: the first `ties_needed` items equal to kth, in item order
  uint32_t nt = 0;
#pragma unroll
  for (int j = 0; j < kItemsPerThread; ++j) nt += (((valid >> j) & 1u) && !all && key[j] == kth);
  uint32_t tie_tot;
  uint32_t tie_rank = block_excl_scan<kSmallThreads>(nt, sh, tie_tot);
  uint32_t sel = 0;
#pragma unroll
  for (int j = 0; j < kItemsPerThread; ++j) {
    if (!((valid >> j) & 1u)) continue;
    bool s = all || key[j] > kth;
    if (!all && key[j] == kth) {
      s = tie_rank < ties_needed;
      ++tie_rank;
    }
    if (s) sel |= 1u << j;
  }
  uint32_t sel_tot;
  uint32_t rank = block_excl_scan<kSmallThreads>(__popc(sel), sh, sel_tot);
  int32_t* o = out + (size_t)q * K;
#pragma unroll
  for (int j = 0; j < kItemsPerThread; ++j)
    if ((sel >> j) & 1u) o[rank++] = (int32_t)pos[j];
  for (int i = (int)kk + t; i < K; i += kSmallThreads) o[i] = -1;
}

// ------------------------------------------------------------ large inputs --

__device__ __forceinline__ SelWs* ws_of(void* ws, int q, int K) {
  return reinterpret_cast<SelWs*>(reinterpret_cast<uint8_t*>(ws) + (size_t)q * sel_stride(K));
}
__device__ __forceinline__ uint2* sure_of(SelWs* w) { return reinterpret_cast<uint2*>(w + 1); }
__device__ __forceinline__ uint2* cand_of(SelWs* w, int K) { return sure_of(w) + K; }

__global__ __launch_bounds__(kThreads) void k_sel_zero(void* ws, int K) {
  SelWs* w = ws_of(ws, blockIdx.x, K);
  for (int i = threadIdx.x; i < kBins; i += kThreads) {
    w->hist1[i] = 0;
    w->hist2[i] = 0;
  }
  if (threadIdx.x < 8) w->cnt[threadIdx.x] = 0;
}

template <int LEVEL>
__global__ __launch_bounds__(kThreads) void k_sel_hist(Items it, void* ws, int K) {
  __shared__ uint32_t lh[kBins];
  const int q = blockIdx.y;
  SelWs* w = ws_of(ws, q, K);
  uint32_t b1 = 0;
  if (LEVEL == 2) {
    if (w->th.all) return;
    b1 = w->th.b1;
  }
  for (int i = threadIdx.x; i < kBins; i += kThreads) lh[i] = 0;
  __syncthreads();
  const int64_t nv = it.visible(q);
  const int32_t* pl = it.kind == kSelReindex ? it.pool + (size_t)q * kPoolBlocks : nullptr;
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  for (int j = 0; j < kItemsPerThread; ++j) {
    const int64_t i = base + j * kThreads + threadIdx.x;
    if (__all(i >= it.n_items)) break;
    uint32_t key = 0, pos = 0;
    const bool ok = it.get(q, i, nv, pl, key, pos);
    if (LEVEL == 1)
      hist_add(lh, key >> 21, ok);
    else
      hist_add(lh, (key >> 10) & 0x7FF, ok && (key >> 21) == b1);
  }
  __syncthreads();
  uint32_t* gh = LEVEL == 1 ? w->hist1 : w->hist2;
  for (int i = threadIdx.x; i < kBins; i += kThreads)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// One work-group per query: the threshold after a histogram pass.
template <int LEVEL>
__global__ __launch_bounds__(kThreads) void k_sel_thresh(void* ws, int K) {
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t sh[kThreads / 64 + 2];
  SelWs* w = ws_of(ws, blockIdx.x, K);
  if (LEVEL == 2 && w->th.all) return;
  const uint32_t* gh = LEVEL == 1 ? w->hist1 : w->hist2;
  for (int i = threadIdx.x; i < kBins; i += kThreads) lh[i] = gh[i];
  __syncthreads();
  if (LEVEL == 1) {
    uint32_t s = 0;
    for (int i = threadIdx.x; i < kBins; i += kThreads) s += lh[i];
    uint32_t total;
    block_excl_scan<kThreads>(s, sh, total);
    uint32_t bin = 0, above = 0;
    const bool all = total <= (uint32_t)K;
    if (!all) find_threshold<kThreads>(lh, (uint32_t)K, sh, bin, above);
    if (threadIdx.x == 0) {
      w->th.all = all ? 1u : 0u;
      w->th.b1 = bin;
      w->th.above1 = above;
      w->th.kk = all ? total : (uint32_t)K;
    }
  } else {
    uint32_t bin, above;
    find_threshold<kThreads>(lh, (uint32_t)K - w->th.above1, sh, bin, above);
    if (threadIdx.x == 0) {
      w->th.b2 = bin;
      w->th.above = w->th.above1 + above;
    }
  }
}

// Wave-aggregated append: returns this lane's slot (valid only where pred).
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
  const uint64_t m = __ballot(pred);
  if (m == 0) return 0;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)m) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
  base = __shfl(base, leader, 64);
  return base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
}

__global__ __launch_bounds__(kThreads) void k_sel_filter(Items it, void* ws, int K) {
  const int q = blockIdx.y;
  SelWs* w = ws_of(ws, q, K);
  const bool all = w->th.all != 0;
  const uint32_t prefix = (w->th.b1 << 11) | w->th.b2;
  const int64_t nv = it.visible(q);
  const int32_t* pl = it.kind == kSelReindex ? it.pool + (size_t)q * kPoolBlocks : nullptr;
  uint2* sure = sure_of(w);
  uint2* cand = cand_of(w, K);
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  for (int j = 0; j < kItemsPerThread; ++j) {
    const int64_t i = base + j * kThreads + threadIdx.x;
    if (__all(i >= it.n_items)) break;
    uint32_t key = 0, pos = 0;
    const bool ok = it.get(q, i, nv, pl, key, pos);
    bool is_sure = false, is_cand = false;
    if (ok) {
      if (all) {
        is_sure = true;
      } else {
        const uint32_t p = key >> 10;
        is_sure = p > prefix;
        is_cand = p == prefix;
      }
    }
    const uint32_t ss = wave_append(is_sure, &w->cnt[0]);
    if (is_sure && ss < (uint32_t)K) sure[ss] = make_uint2(key, pos);
    const uint32_t cs = wave_append(is_cand, &w->cnt[1]);
    if (is_cand && cs < (uint32_t)kCandCap) cand[cs] = make_uint2(key, pos);
  }
}

template <typename T>
__device__ void bitonic_sort(T* a, int n) {   // n a power of two, ascending
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += kFinalThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const bool up = (i & k) == 0;
          const T x = a[i], y = a[ixj];
          if ((x > y) == up) {
            a[i] = y;
            a[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// One work-group per query.
__global__ __launch_bounds__(kFinalThreads) void k_sel_final(Items it, void* ws, int K,
                                                            int32_t* out) {
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t sh[kFinalThreads / 64 + 2];
  __shared__ uint64_t cs[kCandCap];
  __shared__ uint32_t fin[kPoolBlocks];
  __shared__ uint32_t nfin;
  const int q = blockIdx.x;
  SelWs* w = ws_of(ws, q, K);
  const bool all = w->th.all != 0;
  const uint32_t kk = w->th.kk;
  const uint32_t n_sure = w->cnt[0] < (uint32_t)K ? w->cnt[0] : (uint32_t)K;
  const uint32_t n_cand = w->cnt[1];
  const uint2* sure = sure_of(w);
  for (uint32_t i = threadIdx.x; i < n_sure; i += kFinalThreads) fin[i] = sure[i].y;
  if (threadIdx.x == 0) nfin = n_sure;
  __syncthreads();

  if (!all) {
    const uint32_t need = kk - n_sure;   // >= 1
    if (n_cand <= (uint32_t)kCandCap) {
      const uint2* cand = cand_of(w, K);
      if (n_cand <= (uint32_t)kFinalThreads) {
        // rank each candidate by counting the candidates that beat it
        for (uint32_t i = threadIdx.x; i < n_cand; i += kFinalThreads)
          cs[i] = ((uint64_t)(~cand[i].x) << 32) | cand[i].y;
        __syncthreads();
        if (threadIdx.x < n_cand) {
          const uint64_t me = cs[threadIdx.x];
          uint32_t r = 0;
          for (uint32_t j = 0; j < n_cand; ++j) r += cs[j] < me;
          if (r < need && n_sure + r < (uint32_t)K) fin[n_sure + r] = (uint32_t)me;
        }
      } else {
        const int n = next_pow2((int)n_cand);
        for (int i = threadIdx.x; i < n; i += kFinalThreads)
          cs[i] = i < (int)n_cand ? ((uint64_t)(~cand[i].x) << 32) | cand[i].y : ~0ull;
        __syncthreads();
        bitonic_sort(cs, n);
        for (uint32_t i = threadIdx.x; i < need && n_sure + i < (uint32_t)K; i += kFinalThreads)
          fin[n_sure + i] = (uint32_t)cs[i];
      }
      __syncthreads();
    } else {
      // Fallback: third level over bits 9..0 of the keys sharing the prefix,
      // then an in-order scan that keeps ties in position order.
      const uint32_t prefix = (w->th.b1 << 11) | w->th.b2;
      const int64_t nv = it.visible(q);
      const int32_t* pl = it.kind == kSelReindex ? it.pool + (size_t)q * kPoolBlocks : nullptr;
      for (int i = threadIdx.x; i < kBins; i += kFinalThreads) lh[i] = 0;
      __syncthreads();
      for (int64_t i = threadIdx.x; i < it.n_items; i += kFinalThreads) {
        uint32_t key, pos;
        if (it.get(q, i, nv, pl, key, pos) && (key >> 10) == prefix)
          atomicAdd(&lh[1024 + (key & 0x3FF)], 1u);
      }
      __syncthreads();
      uint32_t b3, above3;
      find_threshold<kFinalThreads>(lh, need, sh, b3, above3);
      const uint32_t kth = (prefix << 10) | (b3 - 1024);
      const uint32_t ties_needed = need - above3;
      uint32_t ties_taken = 0;   // uniform across the block
      for (int64_t i0 = 0; i0 < it.n_items; i0 += kFinalThreads) {
        const int64_t i = i0 + threadIdx.x;
        uint32_t key = 0, pos = 0;
        const bool ok = it.get(q, i, nv, pl, key, pos);
        const bool gt = ok && (key >> 10) == prefix && key > kth;
        const bool eq = ok && key == kth;
        uint32_t tot;
        const uint32_t r = block_excl_scan<kFinalThreads>(eq ? 1u : 0u, sh, tot);
        if (gt) {
          const uint32_t slot = atomicAdd(&nfin, 1u);
          if (slot < (uint32_t)K) fin[slot] = pos;
        }
        if (eq && ties_taken + r < ties_needed) {
          const uint32_t slot = atomicAdd(&nfin, 1u);
          if (slot < (uint32_t)K) fin[slot] = pos;
        }
        ties_taken += tot;
      }
    }
  }
  __syncthreads();
  const int n = next_pow2(K);
  for (int i = threadIdx.x + (int)kk; i < n; i += kFinalThreads) fin[i] = 0xFFFFFFFFu;
  __syncthreads();
  bitonic_sort(fin, n);
  int32_t* o = out + (size_t)q * K;
  for (int i = threadIdx.x; i < K; i += kFinalThreads) o[i] = i < (int)kk ? (int32_t)fin[i] : -1;
}

__global__ void k_block_max(const float* __restrict__ scores, const int32_t* __restrict__ n_vis,
                            int64_t n_cap, float* __restrict__ bmax) {
  const int q = blockIdx.y;
  const int64_t n_blk = (n_cap + kBlock - 1) / kBlock;
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n_blk) return;
  int64_t nv = n_vis[q];
  nv = nv < 0 ? 0 : (nv > n_cap ? n_cap : nv);
  const float* s = scores + (size_t)q * (size_t)n_cap;
  float m = -INFINITY;
  for (int r = 0; r < kBlock; ++r) {
    const int64_t p = j * kBlock + r;
    if (p < nv) m = fmaxf(m, s[p]);
  }
  bmax[(size_t)q * (size_t)n_blk + j] = m;
}

__global__ void k_copy_i32(const int32_t* __restrict__ src, int32_t* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

}  // namespace

size_t select_workspace_bytes(int Q, int K) { return (size_t)Q * sel_stride(K); }

hipError_t launch_select(int kind, const float* values, const int32_t* n_vis, const int32_t* pool,
                         int Q, int64_t n_items, int64_t n_cap, int K, int32_t* out, void* ws,
                         hipStream_t st) {
  Items it;
  it.kind = kind;
  it.values = values;
  it.n_vis = n_vis;
  it.pool = pool;
  it.n_items = n_items;
  it.n_cap = n_cap;
  if (n_items <= kSmallMax) {
    hipLaunchKernelGGL(k_sel_small, dim3(Q), dim3(kSmallThreads), 0, st, it, K, out);
    return hipGetLastError();
  }
  const unsigned gx = (unsigned)((n_items + kChunk - 1) / kChunk);
  hipLaunchKernelGGL(k_sel_zero, dim3(Q), dim3(kThreads), 0, st, ws, K);
  hipLaunchKernelGGL(k_sel_hist<1>, dim3(gx, Q), dim3(kThreads), 0, st, it, ws, K);
  hipLaunchKernelGGL(k_sel_thresh<1>, dim3(Q), dim3(kThreads), 0, st, ws, K);
  hipLaunchKernelGGL(k_sel_hist<2>, dim3(gx, Q), dim3(kThreads), 0, st, it, ws, K);
  hipLaunchKernelGGL(k_sel_thresh<2>, dim3(Q), dim3(kThreads), 0, st, ws, K);
  hipLaunchKernelGGL(k_sel_filter, dim3(gx, Q), dim3(kThreads), 0, st, it, ws, K);
  hipLaunchKernelGGL(k_sel_final, dim3(Q), dim3(kFinalThreads), 0, st, it, ws, K, out);
  return hipGetLastError();
}

hipError_t launch_block_max(const float* scores, const int32_t* n_vis, int Q, int64_t n_cap,
                            float* bmax, hipStream_t st) {
  const int64_t n_blk = (n_cap + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(k_block_max, dim3((unsigned)((n_blk + 255) / 256), Q), dim3(256), 0, st,
                     scores, n_vis, n_cap, bmax);
  return hipGetLastError();
}

hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, dst, n);
  return hipGetLastError();
}

}  // namespace csa2
