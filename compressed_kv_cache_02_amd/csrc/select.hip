// Exact Top-K selection (Top-512 per query; 2,048 blocks for the pool) by a
// multi-work-group radix select on order-preserving 32-bit keys of the float
// scores.
//
// Pages: Top-512 per query ("DeepSeek V4.1-Flash 为什么这么强？CED 与 CSA2
// 架构全拆解", §二 layer layout); Full picks its own Top-K over every visible
// position, Reindex its own inside the pool, Reuse copies (same §二, mode
// table); the pool keeps the 2,048 blocks of 8 with the highest in-block maximum
// (same §二, hierarchical sparse indexer; "DeepSeek-V4.1-Flash：全局 KV 仅
// 890 B/token", 第二刀 and Fig. 5). Ties go to the lower position and the result
// is emitted in ascending order (the reading stated in csa2.h).
//
// Passes (each a grid over (chunk, query) except the last):
//   zero   -- clear the per-query histograms and counters (a fill kernel, so the
//             sequence stays safe to capture in a HIP graph);
//   hist1  -- 2,048-bin histogram of key bits 31..21;
//   hist2  -- 2,048-bin histogram of key bits 20..10 among items in the bin
//             that holds the K-th largest key;
//   filter -- items whose 22-bit prefix is above the K-th key's prefix are
//             certain ("sure", fewer than K); items sharing it are candidates;
//   final  -- one work-group per query ranks the candidates by (key desc,
//             position asc), merges them with the sure items and emits the K
//             positions ascending. If the candidates overflow their buffer
//             (tie-heavy input) it falls back to a third histogram level and an
//             in-order scan of the input, which is exact but slow.
#include "device_common.hpp"
#include "launchers.hpp"

namespace csa2 {
namespace {

constexpr int kBins = 2048;
constexpr int kCandCap = 4096;
constexpr int kThreads = 256;
constexpr int kItemsPerThread = 16;
constexpr int kChunk = kThreads * kItemsPerThread;   // 4096 items per work-group

// Per-query workspace record.
struct SelWs {
  uint32_t hist1[kBins];
  uint32_t hist2[kBins];
  uint32_t cnt[64];          // [0] sure count, [1] candidate count
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

  // Returns validity and the position of item i of query q.
  __device__ __forceinline__ bool get(int q, int64_t i, int64_t nv, const int32_t* pl,
                                      uint32_t& key, uint32_t& pos) const {
    int64_t p;
    if (kind == kSelFull) {
      if (i >= nv) return false;
      p = i;
    } else if (kind == kSelPool) {
      if (i >= (nv + kBlock - 1) / kBlock) return false;
      p = i;
    } else {
      const int64_t blk = pl[i >> 3];
      const int64_t n_blk = (n_cap + kBlock - 1) / kBlock;
      if (blk < 0 || blk >= n_blk) return false;
      p = blk * kBlock + (i & 7);
      if (p >= nv) return false;
    }
    key = float_key(values[(size_t)q * (size_t)n_items + i]);
    pos = (uint32_t)p;
    return true;
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

// Exclusive scan over the 256 threads of a block; also returns the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh4, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v, lane);
  if (lane == 63) sh4[wave] = inc;
  __syncthreads();
  uint32_t base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    if (w < wave) base += sh4[w];
    total += sh4[w];
  }
  __syncthreads();
  return base + inc - v;
}

// Given a 2,048-bin histogram in LDS, find the highest bin b with
// sum(hist[b..]) >= k (k >= 1, k <= total), and above = sum(hist[b+1..]).
// Every thread gets the result. `sh` needs 8 words of LDS scratch.
__device__ void find_threshold(const uint32_t* hist, uint32_t k, uint32_t* sh, int& bin_out,
                               uint32_t& above_out) {
  const int t = threadIdx.x;
  const int hi = kBins - 8 * t;   // this thread owns bins [hi-8, hi)
  uint32_t s = 0;
#pragma unroll
  for (int j = 1; j <= 8; ++j) s += hist[hi - j];
  uint32_t total;
  const uint32_t before = block_excl_scan(s, sh, total);
  if (before < k && before + s >= k) {
    uint32_t run = before;
    for (int j = 1; j <= 8; ++j) {
      const uint32_t h = hist[hi - j];
      if (run + h >= k) {
        sh[4] = (uint32_t)(hi - j);
        sh[5] = run;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
  bin_out = (int)sh[4];
  above_out = sh[5];
  __syncthreads();
}

struct Thresh {
  bool all;        // every valid item is selected
  int b1, b2;
  uint32_t above;  // items above prefix (b1, b2)
  uint32_t kk;     // number selected = min(K, total)
};

// Recomputes the selection thresholds from the two histograms (level 2 only
// when `need2`). Uses LDS `lh` (kBins words) and `sh` (8 words).
__device__ Thresh thresholds(const SelWs* ws, int K, bool need2, uint32_t* lh, uint32_t* sh) {
  Thresh th;
  for (int i = threadIdx.x; i < kBins; i += kThreads) lh[i] = ws->hist1[i];
  __syncthreads();
  uint32_t s = 0;
  for (int i = threadIdx.x; i < kBins; i += kThreads) s += lh[i];
  uint32_t total;
  block_excl_scan(s, sh, total);
  th.kk = total < (uint32_t)K ? total : (uint32_t)K;
  th.all = total <= (uint32_t)K;
  th.b1 = -1;
  th.b2 = -1;
  th.above = 0;
  if (th.all) return th;
  uint32_t above1;
  find_threshold(lh, (uint32_t)K, sh, th.b1, above1);
  th.above = above1;
  if (!need2) return th;
  for (int i = threadIdx.x; i < kBins; i += kThreads) lh[i] = ws->hist2[i];
  __syncthreads();
  uint32_t above2;
  find_threshold(lh, (uint32_t)K - above1, sh, th.b2, above2);
  th.above = above1 + above2;
  return th;
}

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
  if (threadIdx.x < 64) w->cnt[threadIdx.x] = 0;
}

template <int LEVEL>
__global__ __launch_bounds__(kThreads) void k_sel_hist(Items it, void* ws, int K) {
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t sh[8];
  const int q = blockIdx.y;
  SelWs* w = ws_of(ws, q, K);
  int b1 = -1;
  if (LEVEL == 2) {
    const Thresh th = thresholds(w, K, false, lh, sh);
    if (th.all) return;
    b1 = th.b1;
  }
  for (int i = threadIdx.x; i < kBins; i += kThreads) lh[i] = 0;
  __syncthreads();
  const int64_t nv = it.visible(q);
  const int32_t* pl = it.kind == kSelReindex ? it.pool + (size_t)q * kPoolBlocks : nullptr;
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  for (int j = 0; j < kItemsPerThread; ++j) {
    const int64_t i = base + j * kThreads + threadIdx.x;
    if (i >= it.n_items) break;
    uint32_t key, pos;
    if (!it.get(q, i, nv, pl, key, pos)) continue;
    if (LEVEL == 1) {
      atomicAdd(&lh[key >> 21], 1u);
    } else if ((int)(key >> 21) == b1) {
      atomicAdd(&lh[(key >> 10) & 0x7FF], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = LEVEL == 1 ? w->hist1 : w->hist2;
  for (int i = threadIdx.x; i < kBins; i += kThreads)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
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
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t sh[8];
  const int q = blockIdx.y;
  SelWs* w = ws_of(ws, q, K);
  const Thresh th = thresholds(w, K, true, lh, sh);
  const int64_t nv = it.visible(q);
  const int32_t* pl = it.kind == kSelReindex ? it.pool + (size_t)q * kPoolBlocks : nullptr;
  uint2* sure = sure_of(w);
  uint2* cand = cand_of(w, K);
  const uint32_t prefix = ((uint32_t)th.b1 << 11) | (uint32_t)th.b2;
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  for (int j = 0; j < kItemsPerThread; ++j) {
    const int64_t i = base + j * kThreads + threadIdx.x;
    if (__all(i >= it.n_items)) break;
    uint32_t key = 0, pos = 0;
    const bool ok = i < it.n_items && it.get(q, i, nv, pl, key, pos);
    bool is_sure = false, is_cand = false;
    if (ok) {
      if (th.all) {
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
      for (int i = threadIdx.x; i < n; i += kThreads) {
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

// One work-group per query. LDS: candidates as 64-bit (~key << 32 | pos) and the
// final position list.
__global__ __launch_bounds__(kThreads) void k_sel_final(Items it, void* ws, int K, int32_t* out) {
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t sh[8];
  __shared__ uint64_t cs[kCandCap];
  __shared__ uint32_t fin[kPoolBlocks];
  __shared__ uint32_t nfin;
  const int q = blockIdx.x;
  SelWs* w = ws_of(ws, q, K);
  const Thresh th = thresholds(w, K, true, lh, sh);
  const uint32_t n_sure = w->cnt[0] < (uint32_t)K ? w->cnt[0] : (uint32_t)K;
  const uint32_t n_cand = w->cnt[1];
  const uint2* sure = sure_of(w);
  for (uint32_t i = threadIdx.x; i < n_sure; i += kThreads) fin[i] = sure[i].y;
  if (threadIdx.x == 0) nfin = n_sure;
  __syncthreads();

  if (!th.all) {
    const uint32_t need = th.kk - n_sure;   // >= 1
    if (n_cand <= (uint32_t)kCandCap) {
      const uint2* cand = cand_of(w, K);
      const int n = next_pow2((int)n_cand);
      for (int i = threadIdx.x; i < n; i += kThreads)
        cs[i] = i < (int)n_cand ? ((uint64_t)(~cand[i].x) << 32) | cand[i].y : ~0ull;
      __syncthreads();
      bitonic_sort(cs, n);
      for (uint32_t i = threadIdx.x; i < need && n_sure + i < (uint32_t)K; i += kThreads)
        fin[n_sure + i] = (uint32_t)cs[i];
      __syncthreads();
    } else {
      // Fallback: third level over bits 9..0 of the keys with the shared prefix,
      // then an in-order scan that keeps ties in position order.
      const uint32_t prefix = ((uint32_t)th.b1 << 11) | (uint32_t)th.b2;
      const int64_t nv = it.visible(q);
      const int32_t* pl = it.kind == kSelReindex ? it.pool + (size_t)q * kPoolBlocks : nullptr;
      for (int i = threadIdx.x; i < kBins; i += kThreads) lh[i] = 0;
      __syncthreads();
      for (int64_t i = threadIdx.x; i < it.n_items; i += kThreads) {
        uint32_t key, pos;
        if (it.get(q, i, nv, pl, key, pos) && (key >> 10) == prefix) atomicAdd(&lh[key & 0x3FF], 1u);
      }
      __syncthreads();
      // the 1,024 low bins live in lh[0..1023]; shift them to the top of a
      // 2,048-bin view so find_threshold can be reused.
      for (int i = threadIdx.x; i < 1024; i += kThreads) lh[1024 + i] = lh[i];
      __syncthreads();
      for (int i = threadIdx.x; i < 1024; i += kThreads) lh[i] = 0;
      __syncthreads();
      int b3;
      uint32_t above3;
      find_threshold(lh, need, sh, b3, above3);
      const uint32_t kth = (prefix << 10) | (uint32_t)(b3 - 1024);
      const uint32_t ties_needed = need - above3;
      uint32_t ties_taken = 0;     // uniform across the block
      for (int64_t i0 = 0; i0 < it.n_items; i0 += kThreads) {
        const int64_t i = i0 + threadIdx.x;
        uint32_t key = 0, pos = 0;
        const bool ok = i < it.n_items && it.get(q, i, nv, pl, key, pos);
        const bool gt = ok && (key >> 10) == prefix && key > kth;
        const bool eq = ok && key == kth;
        uint32_t tot;
        const uint32_t r = block_excl_scan(eq ? 1u : 0u, sh, tot);
        if (gt) {
          const uint32_t slot = atomicAdd(&nfin, 1u);
          if (slot < (uint32_t)K) fin[slot] = pos;
        }
        if (eq && ties_taken + r < ties_needed) {
          const uint32_t slot = atomicAdd(&nfin, 1u);
          if (slot < (uint32_t)K) fin[slot] = pos;
        }
        ties_taken += tot;
        __syncthreads();
      }
    }
  }
  __syncthreads();
  const int n = next_pow2(K);
  for (int i = threadIdx.x + (int)th.kk; i < n; i += kThreads) fin[i] = 0xFFFFFFFFu;
  __syncthreads();
  bitonic_sort(fin, n);
  int32_t* o = out + (size_t)q * K;
  for (int i = threadIdx.x; i < K; i += kThreads) o[i] = i < (int)th.kk ? (int32_t)fin[i] : -1;
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
  const unsigned gx = (unsigned)((n_items + kChunk - 1) / kChunk);
  hipLaunchKernelGGL(k_sel_zero, dim3(Q), dim3(kThreads), 0, st, ws, K);
  hipLaunchKernelGGL(k_sel_hist<1>, dim3(gx, Q), dim3(kThreads), 0, st, it, ws, K);
  hipLaunchKernelGGL(k_sel_hist<2>, dim3(gx, Q), dim3(kThreads), 0, st, it, ws, K);
  hipLaunchKernelGGL(k_sel_filter, dim3(gx, Q), dim3(kThreads), 0, st, it, ws, K);
  hipLaunchKernelGGL(k_sel_final, dim3(Q), dim3(kThreads), 0, st, it, ws, K, out);
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
