// C ABI of libcsa2: argument validation, workspace sizing and dispatch to the
// kernels. Every check happens before anything is enqueued; no exception leaves
// this file. See include/csa2.h for the contract of each call.
#include "csa2.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "launchers.hpp"

namespace {

constexpr size_t kAlign = 256;

inline size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool opt_aligned16(const void* p) { return !p || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool aligned4(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

inline bool sizes_ok(int B, int T, int64_t n_cap) {
  if (B < 1 || T < 1 || n_cap < 1 || n_cap >= (int64_t(1) << 31)) return false;
  if ((int64_t)B * T > 65535) return false;   // one grid row per query
  return true;
}

inline int status_of(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_EHIP; }

// Workspace of csa2_index_topk. Decode-shaped scans (FP32-accurate scores):
// the whole score rows when one selection covers them (n_cap <= 16,384);
// otherwise block maxima, the 512 best blocks, their 4,096 re-scored
// positions and the best-blocks selection's own scratch. Prefill-shaped scans
// (the FP8 contraction, whose scores only narrow the candidates): block
// maxima, the 1,024 best blocks and their 8,192 positions re-scored.
struct FusedWs {
  size_t scores, bmax, sel_blk, vals, blocks_ws, total;
  int n_best;     // 0: one selection over the score rows
};

// Best blocks kept for re-scoring: 512 when the block maxima come from
// FP32-accurate scores (the 512 best positions lie in the 512 best blocks),
// 1,024 when they come from the FP8 contraction. There a block holding one of
// the 512 best positions could only fall out of the list if more than 512
// other blocks' maxima came within twice the contraction's error (below
// 2.5e-4 of the score on the workloads) of its own.
constexpr int kBestExact = CSA2_TOPK;
constexpr int kBestNarrowed = 2 * CSA2_TOPK;

inline bool prefill_shaped(int T, bool fp4) {
  return T >= (fp4 ? CSA2_PREFILL_MIN_T_FP4 : CSA2_PREFILL_MIN_T_FP8);
}

inline FusedWs fused_layout(int Q, int64_t n_cap, bool narrowed) {
  FusedWs l{};
  if (!narrowed && n_cap <= CSA2_POOL_CAND) {
    l.total = round_up((size_t)Q * (size_t)n_cap * sizeof(float));
    return l;
  }
  l.n_best = narrowed ? kBestNarrowed : kBestExact;
  const int64_t n_blk = (n_cap + CSA2_BLOCK - 1) / CSA2_BLOCK;
  l.bmax = 0;
  l.sel_blk = round_up((size_t)Q * (size_t)n_blk * sizeof(float));
  l.vals = l.sel_blk + round_up((size_t)Q * l.n_best * sizeof(int32_t));
  l.blocks_ws = l.vals + round_up((size_t)Q * l.n_best * CSA2_BLOCK * sizeof(float));
  l.total = l.blocks_ws + round_up(csa2::best_blocks_workspace_bytes(Q, n_cap));
  return l;
}

// Scratch of csa2_index_topk_noalloc: a file-scope device array, so the call
// needs no allocation. Every GPU the library runs on holds its own copy until
// the process ends. Its address is resolved once per device, with that device
// current, and kept; host code never passes the array's name itself.
constexpr size_t kScratchBytes = CSA2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

template <typename T>
inline T* ws_at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int csa2_abi_version(void) { return CSA2_ABI_VERSION; }

const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_EINVAL: return "invalid argument";
    case CSA2_EUNSUPPORTED: return "unsupported request";
    case CSA2_EWORKSPACE: return "workspace too small";
    case CSA2_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t csa2_workspace_bytes(int op, int mode, int B, int T, int64_t n_cap) {
  if (!sizes_ok(B, T, n_cap)) return 0;
  const int Q = B * T;
  switch (op) {
    case CSA2_OP_INDEX_SCORE: return 0;
    case CSA2_OP_BUILD_POOL: return round_up(csa2::pool_workspace_bytes(Q, n_cap));
    case CSA2_OP_TOPK:
      if (mode == CSA2_FULL) return round_up(csa2::topk_workspace_bytes(Q, n_cap));
      return 0;
    case CSA2_OP_SPARSE_ATTN: return round_up(csa2::attn_workspace_bytes(Q));
    case CSA2_OP_INDEX_TOPK: {
      // enough for either key format at this T
      const FusedWs a = fused_layout(Q, n_cap, prefill_shaped(T, false));
      const FusedWs b = fused_layout(Q, n_cap, prefill_shaped(T, true));
      return a.total > b.total ? a.total : b.total;
    }
    default: return 0;
  }
}

int csa2_rope_table(const int64_t* pos, int64_t n, float* cos_sin) {
  if (n < 0 || (n > 0 && (!pos || !cos_sin))) return CSA2_EINVAL;
  double theta[CSA2_ROPE_PAIRS];
  for (int i = 0; i < CSA2_ROPE_PAIRS; ++i) theta[i] = std::pow(10000.0, -(double)i / 32.0);
  for (int64_t r = 0; r < n; ++r)
    if (pos[r] < 0) return CSA2_EINVAL;
  for (int64_t r = 0; r < n; ++r) {
    const double p = (double)pos[r];
    for (int i = 0; i < CSA2_ROPE_PAIRS; ++i) {
      const double ang = p * theta[i];
      cos_sin[(r * CSA2_ROPE_PAIRS + i) * 2 + 0] = (float)std::cos(ang);
      cos_sin[(r * CSA2_ROPE_PAIRS + i) * 2 + 1] = (float)std::sin(ang);
    }
  }
  return CSA2_OK;
}

int csa2_quantize_kv(const void* kv_bf16, const float* cos_sin, const int64_t* dst_slot, int64_t n,
                     uint8_t* cache, int64_t cache_rows, void* stream) {
  if (n < 0 || cache_rows < 1) return CSA2_EINVAL;
  if (n == 0) return CSA2_OK;
  if (!aligned16(kv_bf16) || !aligned16(cos_sin) || !aligned16(cache) || !opt_aligned16(dst_slot))
    return CSA2_EINVAL;
  if (!dst_slot && n > cache_rows) return CSA2_EINVAL;
  return status_of(csa2::launch_quantize_kv(static_cast<const uint16_t*>(kv_bf16), cos_sin,
                                            dst_slot, n, cache, cache_rows, as_stream(stream)));
}

int csa2_index_score(int mode, const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                     const int32_t* n_vis, const int32_t* pool, int B, int T, int64_t n_cap,
                     float* scores, float* bmax, void* stream) {
  if (mode != CSA2_FULL && mode != CSA2_REINDEX) return CSA2_EINVAL;
  if (!sizes_ok(B, T, n_cap)) return CSA2_EINVAL;
  if (!aligned16(q_idx) || !aligned16(w) || !aligned16(k_idx) || !aligned16(n_vis) ||
      !opt_aligned16(scores) || !opt_aligned16(bmax))
    return CSA2_EINVAL;
  if (!scores && (mode != CSA2_FULL || !bmax)) return CSA2_EINVAL;   // something to write
  if (mode == CSA2_REINDEX && (!aligned16(pool) || bmax)) return CSA2_EINVAL;
  hipError_t e;
  if (mode == CSA2_FULL && T >= CSA2_PREFILL_MIN_T_FP8)
    e = csa2::launch_index_score_prefill(q_idx, w, k_idx, n_vis, B, T, n_cap, scores, bmax,
                                         as_stream(stream));
  else
    e = csa2::launch_index_score_decode(mode, q_idx, w, k_idx, n_vis, pool, B, T, n_cap, scores,
                                        bmax, as_stream(stream));
  return status_of(e);
}

int csa2_compress_tokens(const void* tokens_bf16, int64_t n_tok, int width, int m,
                         void* out_bf16, void* stream) {
  if (n_tok < 0 || m < 1 || m > CSA2_MAX_M || width < 8 || width > CSA2_MAX_WIDTH || width % 8)
    return CSA2_EINVAL;
  if (n_tok == 0) return CSA2_OK;
  if (!aligned16(tokens_bf16) || !aligned16(out_bf16)) return CSA2_EINVAL;
  return status_of(csa2::launch_compress_rows(static_cast<const uint16_t*>(tokens_bf16), n_tok,
                                              width, m, static_cast<uint16_t*>(out_bf16),
                                              as_stream(stream)));
}

int csa2_quantize_e4m3(const void* rows_bf16, int64_t n, int width, const int64_t* dst_slot,
                       uint8_t* out, int64_t rows, void* stream) {
  if (n < 0 || rows < 1 || width < 8 || width > CSA2_MAX_WIDTH || width % 8) return CSA2_EINVAL;
  if (n == 0) return CSA2_OK;
  if (!aligned16(rows_bf16) || !aligned16(out) || !opt_aligned16(dst_slot)) return CSA2_EINVAL;
  if (!dst_slot && n > rows) return CSA2_EINVAL;
  return status_of(csa2::launch_quantize_e4m3(static_cast<const uint16_t*>(rows_bf16), n, width,
                                              dst_slot, out, rows, as_stream(stream)));
}

int csa2_quantize_index_k(const void* k_bf16, const int64_t* dst_slot, int64_t n,
                          uint8_t* codes, uint8_t* scales, int64_t rows, void* stream) {
  if (n < 0 || rows < 1) return CSA2_EINVAL;
  if (n == 0) return CSA2_OK;
  if (!aligned16(k_bf16) || !aligned16(codes) || !aligned4(scales) || !opt_aligned16(dst_slot))
    return CSA2_EINVAL;
  if (!dst_slot && n > rows) return CSA2_EINVAL;
  return status_of(csa2::launch_quantize_index_k(static_cast<const uint16_t*>(k_bf16), dst_slot, n,
                                                 codes, scales, rows, as_stream(stream)));
}

int csa2_index_score_fp4k(int mode, const uint8_t* q_idx, const float* w, const uint8_t* k_codes,
                          const uint8_t* k_scales, const int32_t* n_vis, const int32_t* pool,
                          int B, int T, int64_t n_cap, float* scores, float* bmax, void* stream) {
  if (mode != CSA2_FULL && mode != CSA2_REINDEX) return CSA2_EINVAL;
  if (!sizes_ok(B, T, n_cap)) return CSA2_EINVAL;
  if (!aligned16(q_idx) || !aligned16(w) || !aligned16(k_codes) || !aligned4(k_scales) ||
      !aligned16(n_vis) || !opt_aligned16(scores) || !opt_aligned16(bmax))
    return CSA2_EINVAL;
  if (!scores && (mode != CSA2_FULL || !bmax)) return CSA2_EINVAL;
  if (mode == CSA2_REINDEX && (!aligned16(pool) || bmax)) return CSA2_EINVAL;
  if (mode == CSA2_FULL && T >= CSA2_PREFILL_MIN_T_FP4)
    return status_of(csa2::launch_index_score_prefill_fp4k(q_idx, w, k_codes, k_scales, n_vis, B, T,
                                                           n_cap, scores, bmax, as_stream(stream)));
  return status_of(csa2::launch_index_score_decode_fp4k(mode, q_idx, w, k_codes, k_scales, n_vis,
                                                        pool, B, T, n_cap, scores, bmax,
                                                        as_stream(stream)));
}

int csa2_index_topk(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                    const uint8_t* k_scales, const int32_t* n_vis, int B, int T, int64_t n_cap,
                    int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  if (!sizes_ok(B, T, n_cap)) return CSA2_EINVAL;
  if (!aligned16(q_idx) || !aligned16(w) || !aligned16(k_idx) || !aligned16(n_vis) ||
      !aligned16(idx) || (k_scales && !aligned4(k_scales)))
    return CSA2_EINVAL;
  if (n_cap > CSA2_INDEX_TOPK_MAX_CAP) return CSA2_EUNSUPPORTED;
  const bool fp4 = k_scales != nullptr;
  const bool narrowed = prefill_shaped(T, fp4);
  const FusedWs l = fused_layout(B * T, n_cap, narrowed);
  if (!aligned16(ws)) return ws ? CSA2_EINVAL : CSA2_EWORKSPACE;
  if (ws_bytes < l.total) return CSA2_EWORKSPACE;
  hipStream_t st = as_stream(stream);
  const int Q = B * T;
  // the Full scan: score rows (short contexts, decode shape) or block maxima only
  float* scores = l.n_best == 0 ? ws_at<float>(ws, l.scores) : nullptr;
  float* bmax = scores ? nullptr : ws_at<float>(ws, l.bmax);
  hipError_t e;
  if (fp4 && narrowed)
    e = csa2::launch_index_score_prefill_fp4k(q_idx, w, k_idx, k_scales, n_vis, B, T, n_cap, scores,
                                              bmax, st);
  else if (fp4)
    e = csa2::launch_index_score_decode_fp4k(CSA2_FULL, q_idx, w, k_idx, k_scales, n_vis, nullptr,
                                             B, T, n_cap, scores, bmax, st);
  else if (narrowed)
    e = csa2::launch_index_score_prefill(q_idx, w, k_idx, n_vis, B, T, n_cap, scores, bmax, st);
  else
    e = csa2::launch_index_score_decode(CSA2_FULL, q_idx, w, k_idx, n_vis, nullptr, B, T, n_cap,
                                        scores, bmax, st);
  if (e != hipSuccess) return CSA2_EHIP;
  if (scores) return status_of(csa2::launch_topk_direct(scores, n_vis, Q, n_cap, idx, st));
  // the best blocks by block maximum, their positions re-scored by the
  // FP32-accurate decode-shaped kernel, the Top-512 of those
  int32_t* sel_blk = ws_at<int32_t>(ws, l.sel_blk);
  float* vals = ws_at<float>(ws, l.vals);
  if ((e = csa2::launch_best_blocks(bmax, n_vis, Q, n_cap, l.n_best, sel_blk,
                                    ws_at<void>(ws, l.blocks_ws), st)) != hipSuccess)
    return CSA2_EHIP;
  if ((e = csa2::launch_rescore_blocks(q_idx, w, k_idx, k_scales, n_vis, sel_blk, l.n_best, B, T,
                                       n_cap, vals, st)) != hipSuccess)
    return CSA2_EHIP;
  return status_of(
      csa2::launch_topk_of_blocks(vals, sel_blk, l.n_best, n_vis, Q, n_cap, idx, st));
}

int csa2_index_topk_noalloc(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                            const uint8_t* k_scales, const int32_t* n_vis, int B, int T,
                            int64_t n_cap, int32_t* idx, void* stream) {
  if (!sizes_ok(B, T, n_cap)) return CSA2_EINVAL;
  if (n_cap > CSA2_INDEX_TOPK_MAX_CAP) return CSA2_EUNSUPPORTED;
  const FusedWs l = fused_layout(B * T, n_cap, prefill_shaped(T, k_scales != nullptr));
  if (l.total > kScratchBytes) return CSA2_EWORKSPACE;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return CSA2_EHIP;
  return csa2_index_topk(q_idx, w, k_idx, k_scales, n_vis, B, T, n_cap, idx, ws, kScratchBytes,
                         stream);
}

int csa2_build_pool(const float* src, int is_bmax, const int32_t* n_vis, int B, int T,
                    int64_t n_cap, int32_t* pool, void* ws, size_t ws_bytes, void* stream) {
  if (!sizes_ok(B, T, n_cap)) return CSA2_EINVAL;
  if (!aligned16(src) || !aligned16(n_vis) || !aligned16(pool)) return CSA2_EINVAL;
  const size_t need = csa2_workspace_bytes(CSA2_OP_BUILD_POOL, 0, B, T, n_cap);
  if (need > 0) {
    if (!aligned16(ws)) return ws ? CSA2_EINVAL : CSA2_EWORKSPACE;
    if (ws_bytes < need) return CSA2_EWORKSPACE;
  }
  return status_of(csa2::launch_build_pool(src, is_bmax, n_vis, B * T, n_cap, pool, ws,
                                           as_stream(stream)));
}

int csa2_topk(int mode, const float* scores, const float* bmax, const int32_t* n_vis,
              const int32_t* pool, const int32_t* src_idx, int B, int T, int64_t n_cap,
              int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  if (!sizes_ok(B, T, n_cap)) return CSA2_EINVAL;
  if (!aligned16(idx)) return CSA2_EINVAL;
  const int Q = B * T;
  hipStream_t st = as_stream(stream);
  if (mode == CSA2_REUSE) {
    if (!aligned16(src_idx)) return CSA2_EINVAL;
    if (src_idx == idx) return CSA2_OK;
    return status_of(csa2::launch_copy_i32(src_idx, idx, (int64_t)Q * CSA2_TOPK, st));
  }
  if (mode != CSA2_FULL && mode != CSA2_REINDEX) return CSA2_EINVAL;
  if (!aligned16(scores) || !aligned16(n_vis)) return CSA2_EINVAL;
  if (mode == CSA2_REINDEX) {
    if (!aligned16(pool) || bmax) return CSA2_EINVAL;
    return status_of(csa2::launch_topk_reindex(scores, pool, n_vis, Q, n_cap, idx, st));
  }
  if (!opt_aligned16(bmax) || !opt_aligned16(pool)) return CSA2_EINVAL;
  const size_t need = csa2_workspace_bytes(CSA2_OP_TOPK, mode, B, T, n_cap);
  if (need > 0) {
    if (!aligned16(ws)) return ws ? CSA2_EINVAL : CSA2_EWORKSPACE;
    if (ws_bytes < need) return CSA2_EWORKSPACE;
  }
  return status_of(csa2::launch_topk_full(scores, bmax, pool, n_vis, Q, n_cap, idx, ws, st));
}

namespace {

int sparse_attn(const void* q_bf16, const uint8_t* cache, const int32_t* idx, const uint8_t* swa,
                const int64_t* q_pos, const int64_t* swa_pos0, int B, int T, int64_t n_cap, int S,
                int ring, float softmax_scale, float* out, void* ws, size_t ws_bytes,
                void* stream) {
  if (!sizes_ok(B, T, n_cap) || S < 1) return CSA2_EINVAL;
  if (!std::isfinite(softmax_scale)) return CSA2_EINVAL;
  if (!aligned16(q_bf16) || !aligned16(cache) || !aligned16(idx) || !aligned16(swa) ||
      !aligned16(q_pos) || !aligned16(swa_pos0) || !aligned16(out))
    return CSA2_EINVAL;
  const size_t need = csa2_workspace_bytes(CSA2_OP_SPARSE_ATTN, 0, B, T, n_cap);
  if (need > 0) {
    if (!aligned16(ws)) return ws ? CSA2_EINVAL : CSA2_EWORKSPACE;
    if (ws_bytes < need) return CSA2_EWORKSPACE;
  }
  return status_of(csa2::launch_sparse_attn(static_cast<const uint16_t*>(q_bf16), cache, idx, swa,
                                            q_pos, swa_pos0, B, T, n_cap, S, ring, softmax_scale,
                                            out, need > 0 ? ws : nullptr, as_stream(stream)));
}

}  // namespace

int csa2_sparse_attn(const void* q_bf16, const uint8_t* cache, const int32_t* idx,
                     const uint8_t* swa, const int64_t* q_pos, const int64_t* swa_pos0, int B,
                     int T, int64_t n_cap, int S, float softmax_scale, float* out, void* ws,
                     size_t ws_bytes, void* stream) {
  return sparse_attn(q_bf16, cache, idx, swa, q_pos, swa_pos0, B, T, n_cap, S, 0, softmax_scale,
                     out, ws, ws_bytes, stream);
}

int csa2_sparse_attn_ring(const void* q_bf16, const uint8_t* cache, const int32_t* idx,
                          const uint8_t* swa, const int64_t* q_pos, const int64_t* swa_pos0, int B,
                          int T, int64_t n_cap, int S, float softmax_scale, float* out, void* ws,
                          size_t ws_bytes, void* stream) {
  return sparse_attn(q_bf16, cache, idx, swa, q_pos, swa_pos0, B, T, n_cap, S, 1, softmax_scale,
                     out, ws, ws_bytes, stream);
}

}  // extern "C"
