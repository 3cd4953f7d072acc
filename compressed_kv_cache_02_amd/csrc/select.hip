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
// Selection is exact at every step and hierarchical where inputs are large. A
// position among the best 512 lies in one of the best 512 blocks of 8 (ranked
// by block maximum, ties to the lower block): every block ranked ahead of its
// block holds, as its maximum, a distinct position ranked ahead of it. The same
// holds one level up for blocks inside super-blocks of 8 blocks. Hence
//   Full Top-512 = the best 512 positions inside the best 512 blocks, found
//                  directly among at most 16,384 blocks and otherwise inside
//                  the best 512 super-blocks (after the first, each selection
//                  sees at most 4,096 candidates); or, when the group has built
//                  the pool from the same scores, the best 512 of the pool's
//                  16,384 positions;
//   pool         = the best 2,048 blocks inside the best 2,048 super-blocks.
// It is the pages' hierarchical indexer applied once more, one level up.
//
// One selection = one work-group per query that holds its items in registers,
// in item order (= id order): 512 threads x 8 items up to 4,096 items, 512 x 16
// up to 8,192, 1,024 x 16 up to 16,384. It finds the exact K-th key by radix
// select on order-preserving 32-bit keys; the digits (12 bits, 4,096 bins) are
// taken from the offset to the smallest valid key, so the first level spreads
// values of any range over its bins. Once the bin holding the K-th key has at
// most NT/8 items, those are gathered into LDS and ranked against each other
// by (key descending, item ascending) instead of further levels. Otherwise ties
// are taken lowest id first with a block prefix sum. The selected ids are
// written ascending with a second prefix sum (no sort).
//
// Inputs beyond 2^20 positions per query use a multi-pass radix path over the
// raw values instead (a grid over chunks x queries):
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

// ------------------------------------------------- one query per work-group --

// Where one selection stage takes its items from.
//   kDirect: item i is id i of a value row (visible while i < the limit);
//   kChild:  item i is child (i % 8) of parent sel[i / 8] (ids ascending,
//            -1 padded): id = 8 * parent + i % 8, visible while below the limit;
//            its value is indexed by the id;
//   kChildItem: as kChild, but the value is indexed by the item (Reindex
//            scores), so value loads do not wait for the parents.
enum SrcKind { kDirect = 0, kChild = 2, kChildItem = 3 };

struct Src {
  const float* vals;     // value rows, vstride floats per query
  int64_t vstride;
  const int32_t* sel;    // kChild: parent ids [Q][sel_stride]
  int sel_stride;
  int by_item;           // kChild: value indexed by item (1) or by child id (0)
  int unit;              // positions per id: 1 (positions), 8 (blocks), 64 (super-blocks)
  const int32_t* n_vis;
  int64_t n_cap;
  int64_t n_items;       // items per query
  int vec;               // value rows start 16-byte aligned (vstride % 4 == 0)

  // ids below this limit are visible
  __device__ __forceinline__ int64_t limit(int q) const {
    int64_t nv = n_vis[q];
    nv = nv < 0 ? 0 : (nv > n_cap ? n_cap : nv);
    return (nv + unit - 1) / unit;
  }
};

// Items t*IPT .. t*IPT+IPT-1 of query q. Every load is issued before any is
// used (indices are clamped into the row instead of branching), so a thread's
// loads are in flight together: parents first (kChild), then values, 16 bytes
// at a time where the row allows it.
template <int KIND, int IPT>
__device__ __forceinline__ uint32_t load_items(const Src& src, int q, int t, int64_t lim,
                                               uint32_t* key, uint32_t* id) {
  static_assert(IPT % kBlock == 0, "whole groups of 8 per thread");
  const float* row = src.vals + (size_t)q * (size_t)src.vstride;
  // ids, item counts and limits stay below 2^31 + 8 (n_cap < 2^31): 32-bit math
  const uint32_t n_items = (uint32_t)src.n_items;
  const uint32_t lim32 = (uint32_t)lim;
  const uint32_t i0 = (uint32_t)t * IPT;
  float v[IPT];
  uint32_t c[IPT];
  bool ok[IPT];
  // 8 consecutive values starting at `base` (clamped element-wise at the row end)
  auto load8 = [&](uint32_t base, float* dst) __attribute__((always_inline)) {
    if (src.vec && (int64_t)base + kBlock <= src.vstride) {
      const float4* r4 = reinterpret_cast<const float4*>(row + base);
      const float4 a = r4[0], b = r4[1];
      dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
      dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
    } else {
#pragma unroll
      for (int r = 0; r < kBlock; ++r) {
        const int64_t k = (int64_t)base + r;
        dst[r] = row[k < src.vstride ? k : src.vstride - 1];
      }
    }
  };
  if (KIND == kDirect) {
#pragma unroll
    for (int g = 0; g < IPT / kBlock; ++g) load8(i0 + g * kBlock, v + g * kBlock);
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      c[j] = i0 + j;
      ok[j] = c[j] < n_items && c[j] < lim32;
    }
  } else {
    int32_t par[IPT / kBlock];
#pragma unroll
    for (int p = 0; p < IPT / kBlock; ++p) {
      const uint32_t i = i0 + p * kBlock;
      par[p] = i < n_items ? src.sel[(size_t)q * src.sel_stride + (i >> 3)] : -1;
    }
    if (KIND == kChildItem) {
#pragma unroll
      for (int p = 0; p < IPT / kBlock; ++p) load8(i0 + p * kBlock, v + p * kBlock);
    }
#pragma unroll
    for (int p = 0; p < IPT / kBlock; ++p) {
      const bool has = par[p] >= 0;
      const uint32_t cb = has ? (uint32_t)par[p] * kBlock : 0u;
      if (KIND == kChild) load8(has && cb < lim32 ? cb : 0u, v + p * kBlock);
#pragma unroll
      for (int r = 0; r < kBlock; ++r) {
        c[p * kBlock + r] = cb + r;
        ok[p * kBlock + r] = has && cb + r < lim32;
      }
    }
  }
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    key[j] = float_key(v[j]);
    id[j] = c[j];
    valid |= (ok[j] ? 1u : 0u) << j;
  }
  return valid;
}

// --- wave / block primitives without LDS round trips where possible --------

// Maximum over each row of 16 lanes with DPP moves, then over the four rows
// with lane reads (scalar).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  return max(max(a, b), max(c, d));
}

// Inclusive prefix sum over the wave with DPP: shifts of 1, 2, 4, 8 inside
// each row of 16 lanes, then the row totals carried across rows (lane 15 to
// rows 1 and 3, lane 31 to rows 2 and 3).
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
  return v;
}

// Exclusive prefix over the block. `sh` holds NT/64 words and must alternate
// between regions on consecutive calls (so no trailing barrier is needed).
template <int NT>
__device__ __forceinline__ uint32_t block_prefix(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan_dpp(v);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t x = sh[w];
    base += w < wave ? x : 0u;
    tot += x;
  }
  total = tot;
  return base + incl - v;
}

constexpr int kSelBins = 4096;       // 12-bit digits: two levels cover 24 bits
constexpr int kSelDigit = 12;

// Largest K-th bin ranked item against item instead of by further radix
// levels: NT/8 candidates, so that each thread compares at most 16 pairs.
template <int NT>
constexpr int sel_cand_max() { return NT / 8; }

// LDS of one selection: the radix histogram, the per-wave exchange words
// (regions: 0-2 count/range, 0/3 levels, 4 ties, 5 output), the result of
// each level's threshold search, and the candidates of the K-th bin with their
// ranks and the per-thread masks of the items taken from them.
template <int NT>
struct SelLds {
  __align__(16) uint32_t lh[kSelBins];
  uint32_t sh[6][NT / 64];
  uint32_t res[3];
  uint32_t n_cand;
  uint2 cand[sel_cand_max<NT>()];    // (key, item) of each item in the K-th bin
  uint32_t ahead[sel_cand_max<NT>()];
  uint32_t take[NT];
};

// The items of the K-th bin -- those whose offset d = key - kmin has the top
// bits d >> nb == prefix, n_c of them -- ranked by (key descending, item
// ascending); the first `need` are selected. Returns this thread's selection:
// its items above that bin and its selected candidates. The candidates are
// appended to LDS one wave-aggregated atomic at a time (their order there is
// arbitrary: the rank compares keys and item numbers, not slots).
template <int NT, int IPT>
__device__ uint32_t select_candidates(const uint32_t* key, uint32_t valid, uint32_t kmin, int nb,
                                      uint32_t prefix, uint32_t need, uint32_t n_c,
                                      SelLds<NT>& L) {
  const int t = threadIdx.x, lane = t & 63;
  uint32_t sel = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const bool v = (valid >> j) & 1u;
    const uint32_t top = (key[j] - kmin) >> nb;      // 0 < nb < 32
    if (v && top > prefix) sel |= 1u << j;
    const bool c = v && top == prefix;
    const uint64_t m = __ballot(c);
    if (m) {
      const int leader = __ffsll((unsigned long long)m) - 1;
      uint32_t base = 0;
      if (lane == leader) base = atomicAdd(&L.n_cand, (uint32_t)__popcll(m));
      base = __shfl(base, leader, 64);
      if (c)
        L.cand[base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull))] =
            make_uint2(key[j], (uint32_t)(t * IPT + j));
    }
  }
  __syncthreads();
  // thread t ranks candidate t % P against slice t / P of the candidates
  // (P a power of two >= n_c, at least a wave, so a wave reads one slice in
  // step: LDS broadcasts)
  int P = 64;
  while (P < (int)n_c) P <<= 1;
  const int S = NT / P;
  const int c = t & (P - 1), s = t / P;
  if (c < (int)n_c) {
    const uint2 me = L.cand[c];
    const int per = ((int)n_c + S - 1) / S;
    const int i0 = s * per, i1 = min((int)n_c, i0 + per);
    uint32_t ahead = 0;
    for (int i = i0; i < i1; ++i) {
      const uint2 o = L.cand[i];
      ahead += (o.x > me.x || (o.x == me.x && o.y < me.y)) ? 1u : 0u;
    }
    if (ahead) atomicAdd(&L.ahead[c], ahead);
  }
  __syncthreads();
  if (t < (int)n_c && L.ahead[t] < need) {
    const uint32_t item = L.cand[t].y;
    atomicOr(&L.take[item / IPT], 1u << (item % IPT));
  }
  __syncthreads();
  return sel | L.take[t];
}

// The selection of query q by one work-group of NT threads: writes the ids of
// the K best items ascending to o[0..K), -1 padded (o may point to LDS).
template <int KIND, int NT, int IPT>
__device__ __forceinline__ void select_wg(const Src& src, int q, int K, int32_t* o,
                                          SelLds<NT>& L) {
  static_assert(IPT <= 32, "item masks are 32-bit");
  static_assert(sel_cand_max<NT>() <= NT, "one thread per candidate");
  constexpr int NW = NT / 64;
  constexpr int PER = kSelBins / NT;                 // bins per thread in the threshold search
  uint32_t* const lh = L.lh;
  uint32_t (*const sh)[NW] = L.sh;
  uint32_t* const res = L.res;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int64_t lim = src.limit(q);
  uint32_t key[IPT], id[IPT];
  const uint32_t valid = load_items<KIND, IPT>(src, q, t, lim, key, id);
  // the first level's histogram and the candidate records are cleared while
  // the loads are in flight (the exchange barrier below orders both)
  {
    uint4* l4 = reinterpret_cast<uint4*>(lh);
    for (int i = t; i < kSelBins / 4; i += NT) l4[i] = make_uint4(0, 0, 0, 0);
    if (t < sel_cand_max<NT>()) L.ahead[t] = 0;
    L.take[t] = 0;
    if (t == 0) L.n_cand = 0;
  }
  // one exchange for the count of valid items and their key range
  uint32_t mx = 0, cmn = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j)
    if ((valid >> j) & 1u) {
      mx = max(mx, key[j]);
      cmn = max(cmn, ~key[j]);   // min as the max of complements
    }
  {
    const uint32_t cnt = wave_incl_scan_dpp(__popc(valid));
    mx = wave_max_u32(mx);
    cmn = wave_max_u32(cmn);
    if (lane == 63) {
      sh[0][wave] = cnt;
      sh[1][wave] = mx;
      sh[2][wave] = cmn;
    }
  }
  __syncthreads();
  uint32_t total = 0, kmax = 0, kcmn = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    total += sh[0][w];
    kmax = max(kmax, sh[1][w]);
    kcmn = max(kcmn, sh[2][w]);
  }
  const uint32_t kmin = ~kcmn;
  const uint32_t kk = total < (uint32_t)K ? total : (uint32_t)K;
  const bool all = total <= (uint32_t)K;
  uint32_t kth = 0, ties_needed = 0;   // select key > kth, plus the first ties_needed == kth
  uint32_t eq_count = total;           // items equal to kth (all of them if the range is 0)
  uint32_t sel = 0;
  bool ranked = false;                 // selection made by ranking the K-th bin's items
  if (!all) {
    // radix select on d = key - kmin, digits of up to 12 bits from the top,
    // until the K-th bin is small enough to rank its items directly
    const uint32_t range = kmax - kmin;
    int nb = range ? 32 - __clz(range) : 0;
    uint32_t prefix = 0, above = 0;
    int reg = 3;
    bool clear = false;                // the first level's histogram is clear already
    while (nb > 0) {                   // uniform across the block
      const int lo = nb > kSelDigit ? nb - kSelDigit : 0;
      const uint32_t mask = (1u << (nb - lo)) - 1u;
      if (clear) {
        uint4* l4 = reinterpret_cast<uint4*>(lh);
        for (int i = t; i < kSelBins / 4; i += NT) l4[i] = make_uint4(0, 0, 0, 0);
        __syncthreads();
      }
      clear = true;
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        const uint32_t d = key[j] - kmin;
        if (((valid >> j) & 1u) && ((uint64_t)d >> nb) == prefix) atomicAdd(&lh[(d >> lo) & mask], 1u);
      }
      __syncthreads();
      // thread t owns bins [hi - PER, hi), counted from the top bin down
      const int hi = kSelBins - PER * t;
      uint32_t c[PER];
      uint32_t s = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        c[j] = lh[hi - 1 - j];
        s += c[j];
      }
      uint32_t tot;
      reg = reg == 3 ? 0 : 3;
      const uint32_t before = block_prefix<NT>(s, sh[reg], tot);
      const uint32_t need = (uint32_t)K - above;
      if (before < need && before + s >= need) {
        uint32_t run = before;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          if (run + c[j] >= need) {
            res[0] = (uint32_t)(hi - 1 - j);
            res[1] = run;
            res[2] = c[j];
            break;
          }
          run += c[j];
        }
      }
      __syncthreads();
      const uint32_t bin = res[0];
      above += res[1];
      eq_count = res[2];   // after the last level: the items equal to the K-th key
      prefix = (prefix << (nb - lo)) | bin;
      nb = lo;
      if (nb > 0 && eq_count <= (uint32_t)sel_cand_max<NT>()) {
        sel = select_candidates<NT, IPT>(key, valid, kmin, nb, prefix, (uint32_t)K - above,
                                         eq_count, L);
        ranked = true;
        break;
      }
    }
    kth = kmin + prefix;
    ties_needed = (uint32_t)K - above;
  }
  if (ranked) {
    // selected above
  } else if (!all && ties_needed < eq_count) {
    // ties: the first `ties_needed` items equal to kth, in item order
    uint32_t nt = 0;
#pragma unroll
    for (int j = 0; j < IPT; ++j) nt += (((valid >> j) & 1u) && key[j] == kth);
    uint32_t tie_tot;
    uint32_t tie_rank = block_prefix<NT>(nt, sh[4], tie_tot);
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      if (!((valid >> j) & 1u)) continue;
      bool s = key[j] > kth;
      if (key[j] == kth) {
        s = tie_rank < ties_needed;
        ++tie_rank;
      }
      if (s) sel |= 1u << j;
    }
  } else {
    // every item equal to the K-th key is taken: no tie ranking needed
#pragma unroll
    for (int j = 0; j < IPT; ++j)
      if (((valid >> j) & 1u) && (all || key[j] >= kth)) sel |= 1u << j;
  }
  uint32_t sel_tot;
  uint32_t rank = block_prefix<NT>(__popc(sel), sh[5], sel_tot);
#pragma unroll
  for (int j = 0; j < IPT; ++j)
    if ((sel >> j) & 1u) o[rank++] = (int32_t)id[j];
  for (int i = (int)kk + t; i < K; i += NT) o[i] = -1;
}

// One work-group per query: exact selection of the K best items (NT threads x
// IPT items). Writes ids ascending to out[q * out_stride + r], -1 padded to K.
template <int KIND, int NT, int IPT>
__global__ __launch_bounds__(NT) void k_select(Src src, int K, int32_t* __restrict__ out,
                                               int out_stride) {
  __shared__ SelLds<NT> L;
  const int q = blockIdx.x;
  select_wg<KIND, NT, IPT>(src, q, K, out + (size_t)q * out_stride, L);
}

// Two chained selections in one work-group per query: the K1 best parents
// (super-blocks) by their values, kept in LDS, then the K2 best of their
// children (blocks, value indexed by the child id). The same result as two
// k_select launches, without the second launch and its load of the parents.
template <int NT, int IPT>
__global__ __launch_bounds__(NT) void k_select_pair(Src parents, int K1, Src children, int K2,
                                                    int32_t* __restrict__ out, int out_stride) {
  __shared__ SelLds<NT> L;
  __shared__ int32_t par[kPoolBlocks];
  const int q = blockIdx.x;
  select_wg<kDirect, NT, IPT>(parents, q, K1, par, L);
  __syncthreads();                 // the parents are in LDS; the exchange words are free
  Src c = children;
  c.sel = par;                     // read through a generic pointer: LDS
  c.sel_stride = 0;
  c.n_items = (int64_t)K1 * kBlock;
  select_wg<kChild, NT, IPT>(c, q, K2, out + (size_t)q * out_stride, L);
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

// Maxima of super-blocks of 8 consecutive blocks (-inf where none is finite).
// VEC: rows start 16-byte aligned, so a super-block's 8 maxima are two float4
// loads.
template <bool VEC>
__global__ void k_super_max(const float* __restrict__ bmax, int64_t n_blk, int64_t n_sb,
                            float* __restrict__ smax) {
  const int q = blockIdx.y;
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n_sb) return;
  const float* b = bmax + (size_t)q * (size_t)n_blk;
  float v[kBlock];
  if (VEC && (j + 1) * kBlock <= n_blk) {
    const float4* b4 = reinterpret_cast<const float4*>(b + j * kBlock);
    const float4 x = b4[0], y = b4[1];
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else {
#pragma unroll
    for (int r = 0; r < kBlock; ++r) {
      const int64_t k = j * kBlock + r;
      v[r] = k < n_blk ? b[k] : -INFINITY;
    }
  }
  float m = v[0];
#pragma unroll
  for (int r = 1; r < kBlock; ++r) m = fmaxf(m, v[r]);
  smax[(size_t)q * (size_t)n_sb + j] = m;
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

// ------------------------------------------------------------ launchers --

namespace {

constexpr int64_t kOneWgMax = 16384;                 // items one work-group selects over
constexpr size_t kWsAlign = 256;
inline size_t up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

inline int64_t n_blocks(int64_t n) { return (n + kBlock - 1) / kBlock; }

// One per-query selection stage over up to 16,384 items.
template <int KIND>
hipError_t run_stage_k(const Src& s, int Q, int K, int32_t* out, int out_stride, hipStream_t st) {
  if (s.n_items <= 4096)
    hipLaunchKernelGGL((k_select<KIND, 512, 8>), dim3(Q), dim3(512), 0, st, s, K, out,
                       out_stride);
  else if (s.n_items <= 8192)
    hipLaunchKernelGGL((k_select<KIND, 512, 16>), dim3(Q), dim3(512), 0, st, s, K, out,
                       out_stride);
  else
    hipLaunchKernelGGL((k_select<KIND, 1024, 16>), dim3(Q), dim3(1024), 0, st, s, K, out,
                       out_stride);
  return hipGetLastError();
}

struct Stage {
  int kind;
  Src src;
};

hipError_t run_stage(const Stage& g, int Q, int K, int32_t* out, int out_stride, hipStream_t st) {
  if (g.kind == kDirect) return run_stage_k<kDirect>(g.src, Q, K, out, out_stride, st);
  if (g.kind == kChildItem) return run_stage_k<kChildItem>(g.src, Q, K, out, out_stride, st);
  return run_stage_k<kChild>(g.src, Q, K, out, out_stride, st);
}

// Parents (a direct stage) and children (a child stage by id) chained in one
// work-group per query; the children's parent list is the first selection's
// result in LDS.
hipError_t run_pair(const Stage& parents, int K1, const Stage& children, int K2, int Q,
                    int32_t* out, int out_stride, hipStream_t st) {
  if (parents.kind != kDirect || children.kind != kChild || K1 > kPoolBlocks)
    return hipErrorInvalidValue;
  const int64_t n = parents.src.n_items > (int64_t)K1 * kBlock ? parents.src.n_items
                                                                : (int64_t)K1 * kBlock;
  if (n <= 4096)
    hipLaunchKernelGGL((k_select_pair<512, 8>), dim3(Q), dim3(512), 0, st, parents.src, K1,
                       children.src, K2, out, out_stride);
  else if (n <= 8192)
    hipLaunchKernelGGL((k_select_pair<512, 16>), dim3(Q), dim3(512), 0, st, parents.src, K1,
                       children.src, K2, out, out_stride);
  else
    hipLaunchKernelGGL((k_select_pair<1024, 16>), dim3(Q), dim3(1024), 0, st, parents.src, K1,
                       children.src, K2, out, out_stride);
  return hipGetLastError();
}

Stage direct(const float* vals, int64_t vstride, int unit, const int32_t* n_vis, int64_t n_cap,
             int64_t n_items) {
  Stage g;
  g.kind = kDirect;
  g.src.vals = vals;
  g.src.vstride = vstride;
  g.src.sel = nullptr;
  g.src.sel_stride = 0;
  g.src.by_item = 0;
  g.src.unit = unit;
  g.src.n_vis = n_vis;
  g.src.n_cap = n_cap;
  g.src.n_items = n_items;
  g.src.vec = vstride % 4 == 0 && (reinterpret_cast<uintptr_t>(vals) & 15u) == 0;
  return g;
}

Stage child(const float* vals, int64_t vstride, int unit, const int32_t* sel, int sel_stride,
            int by_item, const int32_t* n_vis, int64_t n_cap) {
  Stage g = direct(vals, vstride, unit, n_vis, n_cap, (int64_t)sel_stride * kBlock);
  g.kind = by_item ? kChildItem : kChild;
  g.src.sel = sel;
  g.src.sel_stride = sel_stride;
  g.src.by_item = by_item;
  return g;
}

hipError_t launch_super_max(const float* bmax, int Q, int64_t n_blk, float* smax, hipStream_t st) {
  const int64_t n_sb = (n_blk + kBlock - 1) / kBlock;
  const dim3 grid((unsigned)((n_sb + 255) / 256), Q);
  if ((n_blk & 3) == 0 && (reinterpret_cast<uintptr_t>(bmax) & 15) == 0)
    hipLaunchKernelGGL(k_super_max<true>, grid, dim3(256), 0, st, bmax, n_blk, n_sb, smax);
  else
    hipLaunchKernelGGL(k_super_max<false>, grid, dim3(256), 0, st, bmax, n_blk, n_sb, smax);
  return hipGetLastError();
}

Items large_items(int kind, const float* values, const int32_t* n_vis, int64_t n_items,
                  int64_t n_cap) {
  Items it;
  it.kind = kind;
  it.values = values;
  it.n_vis = n_vis;
  it.pool = nullptr;
  it.n_items = n_items;
  it.n_cap = n_cap;
  return it;
}

hipError_t run_large(const Items& it, int Q, int K, int32_t* out, void* ws, hipStream_t st) {
  const unsigned gx = (unsigned)((it.n_items + kChunk - 1) / kChunk);
  hipLaunchKernelGGL(k_sel_zero, dim3(Q), dim3(kThreads), 0, st, ws, K);
  hipLaunchKernelGGL(k_sel_hist<1>, dim3(gx, Q), dim3(kThreads), 0, st, it, ws, K);
  hipLaunchKernelGGL(k_sel_thresh<1>, dim3(Q), dim3(kThreads), 0, st, ws, K);
  hipLaunchKernelGGL(k_sel_hist<2>, dim3(gx, Q), dim3(kThreads), 0, st, it, ws, K);
  hipLaunchKernelGGL(k_sel_thresh<2>, dim3(Q), dim3(kThreads), 0, st, ws, K);
  hipLaunchKernelGGL(k_sel_filter, dim3(gx, Q), dim3(kThreads), 0, st, it, ws, K);
  hipLaunchKernelGGL(k_sel_final, dim3(Q), dim3(kFinalThreads), 0, st, it, ws, K, out);
  return hipGetLastError();
}

// Workspace layout shared by the Full Top-K and the pool:
//   [block maxima, when computed here][super-block maxima][block ids Q x 512]
//   [large path]
struct WsLayout {
  size_t bmax, smax, sel_b, large, total;
};

WsLayout layout(int Q, int64_t n_cap, int K) {
  WsLayout l;
  const int64_t n_blk = n_blocks(n_cap);
  l.bmax = 0;
  l.smax = up((size_t)Q * n_blk * sizeof(float));
  l.sel_b = l.smax + up((size_t)Q * n_blocks(n_blk) * sizeof(float));
  l.large = l.sel_b + up((size_t)Q * kTopK * sizeof(int32_t));
  const bool need_large = n_blocks(n_blk) > kOneWgMax;
  l.total = l.large + (need_large ? up((size_t)Q * sel_stride(K)) : 0);
  return l;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

}  // namespace

size_t topk_workspace_bytes(int Q, int64_t n_cap) {
  if (n_cap <= kOneWgMax) return 0;
  return layout(Q, n_cap, kTopK).total;
}

size_t pool_workspace_bytes(int Q, int64_t n_cap) { return layout(Q, n_cap, kPoolBlocks).total; }

hipError_t launch_topk_full(const float* scores, const float* bmax, const int32_t* pool,
                            const int32_t* n_vis, int Q, int64_t n_cap, int32_t* out, void* ws,
                            hipStream_t st) {
  if (n_cap <= kOneWgMax)
    return run_stage(direct(scores, n_cap, 1, n_vis, n_cap, n_cap), Q, kTopK, out, kTopK, st);
  if (pool)   // the best 512 positions of the pool built from these scores
    return run_stage(child(scores, n_cap, 1, pool, kPoolBlocks, 0, n_vis, n_cap), Q, kTopK, out,
                     kTopK, st);
  const int64_t n_blk = n_blocks(n_cap);
  const int64_t n_sb = n_blocks(n_blk);
  const WsLayout l = layout(Q, n_cap, kTopK);
  if (n_sb > kOneWgMax)
    return run_large(large_items(kSelFull, scores, n_vis, n_cap, n_cap), Q, kTopK, out,
                     at<void>(ws, l.large), st);
  hipError_t e;
  if (!bmax) {
    e = launch_block_max(scores, n_vis, Q, n_cap, at<float>(ws, l.bmax), st);
    if (e != hipSuccess) return e;
    bmax = at<float>(ws, l.bmax);
  }
  float* smax = at<float>(ws, l.smax);
  int32_t* sel_blk = at<int32_t>(ws, l.sel_b);
  if (n_blk <= kOneWgMax) {
    // few enough blocks for one selection: the best 512 directly
    e = run_stage(direct(bmax, n_blk, 8, n_vis, n_cap, n_blk), Q, kTopK, sel_blk, kTopK, st);
  } else {
    // best 512 super-blocks, then the best 512 of their blocks
    if ((e = launch_super_max(bmax, Q, n_blk, smax, st)) != hipSuccess) return e;
    e = run_pair(direct(smax, n_sb, 64, n_vis, n_cap, n_sb), kTopK,
                 child(bmax, n_blk, 8, nullptr, kTopK, 0, n_vis, n_cap), kTopK, Q, sel_blk, kTopK,
                 st);
  }
  if (e != hipSuccess) return e;
  // then the best 512 of their positions
  return run_stage(child(scores, n_cap, 1, sel_blk, kTopK, 0, n_vis, n_cap), Q, kTopK, out, kTopK,
                   st);
}

size_t best_blocks_workspace_bytes(int Q, int64_t n_cap) {
  const int64_t n_sb = n_blocks(n_blocks(n_cap));
  return up((size_t)Q * n_sb * sizeof(float));        // super-block maxima
}

hipError_t launch_best_blocks(const float* bmax, const int32_t* n_vis, int Q, int64_t n_cap,
                              int n_best, int32_t* sel_blk, void* ws, hipStream_t st) {
  const int64_t n_blk = n_blocks(n_cap);
  const int64_t n_sb = n_blocks(n_blk);
  if (n_sb > kOneWgMax || n_best < 1 || n_best > kPoolBlocks) return hipErrorInvalidValue;
  if (n_blk <= kOneWgMax)   // one selection over the block maxima
    return run_stage(direct(bmax, n_blk, 8, n_vis, n_cap, n_blk), Q, n_best, sel_blk, n_best, st);
  float* smax = at<float>(ws, 0);
  hipError_t e;
  if ((e = launch_super_max(bmax, Q, n_blk, smax, st)) != hipSuccess) return e;
  return run_pair(direct(smax, n_sb, 64, n_vis, n_cap, n_sb), n_best,
                  child(bmax, n_blk, 8, nullptr, n_best, 0, n_vis, n_cap), n_best, Q, sel_blk,
                  n_best, st);
}

hipError_t launch_topk_of_blocks(const float* vals, const int32_t* sel_blk, int n_best,
                                 const int32_t* n_vis, int Q, int64_t n_cap, int32_t* out,
                                 hipStream_t st) {
  return run_stage(child(vals, (int64_t)n_best * kBlock, 1, sel_blk, n_best, 1, n_vis, n_cap), Q,
                   kTopK, out, kTopK, st);
}

hipError_t launch_topk_direct(const float* scores, const int32_t* n_vis, int Q, int64_t n_cap,
                              int32_t* out, hipStream_t st) {
  if (n_cap > kOneWgMax) return hipErrorInvalidValue;
  return run_stage(direct(scores, n_cap, 1, n_vis, n_cap, n_cap), Q, kTopK, out, kTopK, st);
}

hipError_t launch_topk_reindex(const float* scores_pool, const int32_t* pool, const int32_t* n_vis,
                               int Q, int64_t n_cap, int32_t* out, hipStream_t st) {
  return run_stage(child(scores_pool, kPoolCand, 1, pool, kPoolBlocks, 1, n_vis, n_cap), Q, kTopK,
                   out, kTopK, st);
}

hipError_t launch_build_pool(const float* src, int is_bmax, const int32_t* n_vis, int Q,
                             int64_t n_cap, int32_t* pool, void* ws, hipStream_t st) {
  const int64_t n_blk = n_blocks(n_cap);
  const int64_t n_sb = n_blocks(n_blk);
  const WsLayout l = layout(Q, n_cap, kPoolBlocks);
  const float* bm = src;
  hipError_t e;
  if (!is_bmax) {
    e = launch_block_max(src, n_vis, Q, n_cap, at<float>(ws, l.bmax), st);
    if (e != hipSuccess) return e;
    bm = at<float>(ws, l.bmax);
  }
  if (n_blk <= kOneWgMax)
    return run_stage(direct(bm, n_blk, 8, n_vis, n_cap, n_blk), Q, kPoolBlocks, pool, kPoolBlocks,
                     st);
  if (n_sb > kOneWgMax)
    return run_large(large_items(kSelPool, bm, n_vis, n_blk, n_cap), Q, kPoolBlocks, pool,
                     at<void>(ws, l.large), st);
  // best 2,048 super-blocks, then the best 2,048 of their 16,384 blocks
  float* smax = at<float>(ws, l.smax);
  if ((e = launch_super_max(bm, Q, n_blk, smax, st)) != hipSuccess) return e;
  return run_pair(direct(smax, n_sb, 64, n_vis, n_cap, n_sb), kPoolBlocks,
                  child(bm, n_blk, 8, nullptr, kPoolBlocks, 0, n_vis, n_cap), kPoolBlocks, Q, pool,
                  kPoolBlocks, st);
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
