// Host-side launchers of the CSA2 kernels; called by the C-ABI layer after it
// has validated every argument. Each returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

hipError_t launch_quantize_kv(const uint16_t* kv, const float* cos_sin, const int64_t* slot,
                              int64_t n, uint8_t* cache, int64_t cache_rows, hipStream_t st);

// Write path around the FP4 packer: m-token mean compressor (bf16 -> bf16) and
// E4M3 append of bf16 rows (window rows, FP8 indexer keys).
hipError_t launch_compress_rows(const uint16_t* tok, int64_t n_tok, int width, int m,
                                uint16_t* out, hipStream_t st);
hipError_t launch_quantize_e4m3(const uint16_t* x, int64_t n, int width, const int64_t* slot,
                                uint8_t* out, int64_t rows, hipStream_t st);

// FP4 indexer keys (E2M1 codes [rows][64] + E8M0 scales [rows][4]) from bf16 keys.
hipError_t launch_quantize_index_k(const uint16_t* k, const int64_t* slot, int64_t n,
                                   uint8_t* codes, uint8_t* scales, int64_t rows, hipStream_t st);

// Decode-shaped scan: one query per grid row, positions split over work-groups.
hipError_t launch_index_score_decode(int mode, const uint8_t* q_idx, const float* w,
                                     const uint8_t* k_idx, const int32_t* n_vis,
                                     const int32_t* pool, int B, int T, int64_t n_cap,
                                     float* scores, float* bmax, hipStream_t st);

// Decode-shaped scan over FP4 indexer keys (codes [B][n_cap][64], scales [B][n_cap][4]).
hipError_t launch_index_score_decode_fp4k(int mode, const uint8_t* q_idx, const float* w,
                                          const uint8_t* k_codes, const uint8_t* k_scales,
                                          const int32_t* n_vis, const int32_t* pool, int B, int T,
                                          int64_t n_cap, float* scores, float* bmax,
                                          hipStream_t st);

// Prefill-shaped scan over FP4 indexer keys (the scaled FP8 x FP4 contraction).
hipError_t launch_index_score_prefill_fp4k(const uint8_t* q_idx, const float* w,
                                           const uint8_t* k_codes, const uint8_t* k_scales,
                                           const int32_t* n_vis, int B, int T, int64_t n_cap,
                                           float* scores, float* bmax, hipStream_t st);

// Prefill-shaped scan: a dense FP8 contraction over (queries x 32 heads) x positions.
hipError_t launch_index_score_prefill(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                                      const int32_t* n_vis, int B, int T, int64_t n_cap,
                                      float* scores, float* bmax, hipStream_t st);

// Exact Top-K selection (hierarchical; see select.hip).
enum SelectKind { kSelFull = 0, kSelReindex = 1, kSelPool = 2 };
size_t topk_workspace_bytes(int Q, int64_t n_cap);
size_t pool_workspace_bytes(int Q, int64_t n_cap);
hipError_t launch_topk_full(const float* scores, const float* bmax, const int32_t* pool,
                            const int32_t* n_vis, int Q, int64_t n_cap, int32_t* out, void* ws,
                            hipStream_t st);
hipError_t launch_topk_reindex(const float* scores_pool, const int32_t* pool, const int32_t* n_vis,
                               int Q, int64_t n_cap, int32_t* out, hipStream_t st);
hipError_t launch_build_pool(const float* src, int is_bmax, const int32_t* n_vis, int Q,
                             int64_t n_cap, int32_t* pool, void* ws, hipStream_t st);
hipError_t launch_block_max(const float* scores, const int32_t* n_vis, int Q, int64_t n_cap,
                            float* bmax, hipStream_t st);
hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int64_t n, hipStream_t st);

// Fused Full Top-K pieces: the n_best (<= 2,048) best blocks from block maxima
// (super-block maxima, then two chained selections in one kernel; workspace
// best_blocks_workspace_bytes), the re-scoring of a per-query block list
// ([Q][n_blocks] block ids, -1 padded; values [Q][8 * n_blocks] by item), the
// Top-512 of the re-scored positions, and the Top-512 of a short score row
// (n_cap <= 16,384).
size_t best_blocks_workspace_bytes(int Q, int64_t n_cap);
hipError_t launch_best_blocks(const float* bmax, const int32_t* n_vis, int Q, int64_t n_cap,
                              int n_best, int32_t* sel_blk, void* ws, hipStream_t st);
hipError_t launch_rescore_blocks(const uint8_t* q_idx, const float* w, const uint8_t* keys,
                                 const uint8_t* scales, const int32_t* n_vis, const int32_t* blocks,
                                 int n_blocks, int B, int T, int64_t n_cap, float* vals,
                                 hipStream_t st);
hipError_t launch_topk_of_blocks(const float* vals, const int32_t* sel_blk, int n_best,
                                 const int32_t* n_vis, int Q, int64_t n_cap, int32_t* out,
                                 hipStream_t st);
hipError_t launch_topk_direct(const float* scores, const int32_t* n_vis, int Q, int64_t n_cap,
                              int32_t* out, hipStream_t st);

// Sparse attention; the workspace holds the key slices' partial results when
// a call has at most 12 queries (attn_workspace_bytes). ring != 0: the
// window buffer is a ring, token t in row t mod S; else row s holds token
// swa_pos0 + s.
size_t attn_workspace_bytes(int Q);
hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* cache, const int32_t* idx,
                              const uint8_t* swa, const int64_t* q_pos, const int64_t* swa_pos0,
                              int B, int T, int64_t n_cap, int S, int ring, float scale, float* out,
                              void* ws, hipStream_t st);

}  // namespace csa2
