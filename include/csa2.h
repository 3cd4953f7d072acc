/*
 * csa2.h -- C ABI of libcsa2, the per-layer hot path of CSA2 (Compressed Sparse
 * Attention 2) on AMD Instinct MI355X (gfx950).
 *
 * Pages the operations come from (cited below by tag):
 *   [P1] "DeepSeek V4.1-Flash 为什么这么强？CED 与 CSA2 架构全拆解" (deepseek.csdn.net)
 *   [P2] "DeepSeek V4.1 Flash vs V4 Pro" (my-blog-5oz.pages.dev)
 *   [P3] "DeepSeek-V4.1-Flash：全局 KV 仅 890 B/token，百万上下文怎么做成的？"
 *        (landx.limxdynamics.com)
 *   [P4] "DeepSeek-V4.1-Flash KV cache compression architecture analysis" (www.ic.work)
 *
 * Conventions shared by every call:
 *   - "device" pointers are HIP device (or managed) memory; "host" pointers are
 *     ordinary host memory. Every device pointer must be 16-byte aligned.
 *     Tensors are contiguous and row-major in the order written.
 *   - The caller owns every buffer, the workspace and the stream. The library
 *     never allocates or frees memory, never synchronises, never copies between
 *     host and device, and keeps no state between calls; every device call only
 *     enqueues kernels on `stream` (a hipStream_t passed as void*; NULL = the
 *     default stream), so it can be captured into a HIP graph.
 *   - Arguments are validated on the host before anything is enqueued; a bad
 *     argument returns CSA2_EINVAL (or CSA2_EUNSUPPORTED / CSA2_EWORKSPACE) and
 *     launches nothing. CSA2_EHIP reports a launch failure. Device-side faults
 *     surface at the caller's next synchronisation. No C++ exception crosses
 *     this boundary.
 *   - Values inside device buffers cannot be checked on the host. Where a
 *     device value is out of range (an index, a slot, a position) the kernels
 *     skip it rather than touch memory outside the buffer, as stated per call.
 *
 * Fixed shapes (from [P1] §二 layer layout and hierarchical indexer):
 *   indexer: 32 query heads x 128 (E4M3), one 128-wide key per position;
 *   main attention: 64 heads x 512 over one shared 512-wide latent per position;
 *   Top-512 per query; pool = 2,048 blocks x 8 positions = 16,384 candidates;
 *   sliding window of 128 tokens ([P1] §一, [P2] 黑科技之一).
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 7

#define CSA2_IDX_HEADS 32
#define CSA2_IDX_DIM 128
#define CSA2_HEADS 64
#define CSA2_DIM 512
#define CSA2_ROW_BYTES 288      /* 256 bytes of E2M1 codes + 32 E4M3 scales */
#define CSA2_TOPK 512
#define CSA2_POOL_BLOCKS 2048
#define CSA2_BLOCK 8
#define CSA2_POOL_CAND 16384
#define CSA2_WINDOW 128
#define CSA2_ROPE_PAIRS 32      /* RoPE on channels 448..511, adjacent pairs */
#define CSA2_INDEX_TOPK_MAX_CAP 1048576   /* longest context csa2_index_topk serves */
#define CSA2_MAX_M 64                /* largest compression ratio csa2_compress_tokens accepts */
#define CSA2_MAX_WIDTH 8192          /* widest row of the write-path helpers */
#define CSA2_IDX_FP4_CODE_BYTES 64   /* FP4 indexer key: 128 E2M1 codes ... */
#define CSA2_IDX_FP4_SCALES 4        /* ... and one E8M0 scale per 32 channels */
#define CSA2_NOALLOC_SCRATCH_BYTES 33554432   /* 32 MiB: scratch of csa2_index_topk_noalloc */
/* Query tokens per sequence from which a FULL scan (csa2_index_score,
 * csa2_index_score_fp4k, csa2_index_topk) takes the prefill-shaped contraction:
 * 16 (up to 16 tokens) or 32 queries x 4,096 keys per work-group, keys staged
 * through LDS, on the FP8 MFMA. Below it the decode shape scores the tokens in
 * pairs per wave that each read the keys again, on the fp16 MFMA.
 *
 * Precision. The decode shape (and every REINDEX scan and re-scoring) converts
 * E4M3 and E2M1 values exactly to fp16 and accumulates with the fp16 MFMA,
 * which keeps products to 24 bits and rounds to nearest: float32 accuracy. The
 * prefill shape's FP8 MFMA truncates each product to 13 fractional bits below
 * the largest product of its 64-term instruction, so a prefill-shaped score may
 * be off by up to 2 * 63 * 2^-13 * sum_h w_h max_c |q_hc k_c| (about 2e-5 of
 * the score on N(0,1) values). csa2_index_topk therefore narrows with those
 * scores and decides on re-scored float32-accurate ones. */
#define CSA2_PREFILL_MIN_T_FP8 4
#define CSA2_PREFILL_MIN_T_FP4 5

/* Layer mode ([P1] §二 mode table; [P2] 黑科技之二; [P3] 第二刀, Fig. 4):
 *   FULL    -- own indexer keys, own scores over every visible position, own Top-K;
 *   REINDEX -- an earlier layer's keys, own indexer query, scores only inside the
 *              candidate pool, own Top-K;
 *   REUSE   -- an earlier layer's Top-K indices, unchanged. */
typedef enum { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2 } csa2_mode;

enum {
  CSA2_OK = 0,
  CSA2_EINVAL = -1,        /* null/misaligned pointer, bad size, bad mode combination */
  CSA2_EUNSUPPORTED = -2,  /* valid request the library does not implement */
  CSA2_EWORKSPACE = -3,    /* workspace smaller than csa2_workspace_bytes() */
  CSA2_EHIP = -4           /* a HIP launch failed */
};

/* Operation ids for csa2_workspace_bytes(). */
enum {
  CSA2_OP_INDEX_SCORE = 0,
  CSA2_OP_BUILD_POOL = 1,
  CSA2_OP_TOPK = 2,
  CSA2_OP_SPARSE_ATTN = 3,
  CSA2_OP_INDEX_TOPK = 4
};

/* Version of this ABI (CSA2_ABI_VERSION). */
int csa2_abi_version(void);

/* Static, human-readable text for a status code. Never NULL. */
const char* csa2_status_string(int status);

/* Workspace (device bytes) an operation needs for the given sizes; 0 if none.
 * `mode` matters for CSA2_OP_TOPK only. Returns 0 for invalid sizes. */
size_t csa2_workspace_bytes(int op, int mode, int B, int T, int64_t n_cap);

/* HOST. RoPE table for the main-KV write path (the main KV is quantised after
 * RoPE: [P1] §三, [P3] 第三刀). For each of `n` positions pos[r] (host) and pair
 * i = 0..31 writes cos_sin[r][i][0] = (float)cos(pos[r] * theta_i) and
 * cos_sin[r][i][1] = (float)sin(pos[r] * theta_i), theta_i = 10000^(-i/32),
 * evaluated in double and rounded once (host buffer of n*64 floats).
 * Errors: CSA2_EINVAL if a pointer is NULL, n < 0 or a position is negative. */
int csa2_rope_table(const int64_t* pos, int64_t n, float* cos_sin);

/* DEVICE. Write path: RoPE, then FP4 packing, then the store ([P1] §三; [P2]
 * 黑科技之三; [P3] 第三刀).
 *   kv_bf16   [n][512] bf16 latent rows (device);
 *   cos_sin   [n][32][2] float table for each row's position (device; see
 *             csa2_rope_table);
 *   dst_slot  [n] int64 destination row in `cache` (device), or NULL to store
 *             row r at row r; slots outside [0, cache_rows) are skipped;
 *   cache     [cache_rows][288] packed rows (device, written).
 * Per row: channels 448 + 2i and 449 + 2i are rotated in float32 with each
 * product and sum rounded separately; then per 16-channel group g the scale is
 * the E4M3 value nearest amax/6 (ties to even, saturating at 448) stored at byte
 * 256 + g, and each element is the E2M1 code nearest |y|/scale (ties to even,
 * saturating at 6; sign bit = sign of y; a zero scale gives magnitude 0), two
 * codes per byte with the even channel in the low nibble. Inputs must be finite.
 * Errors: CSA2_EINVAL for NULL/misaligned pointers, n < 0, cache_rows < 1. */
int csa2_quantize_kv(const void* kv_bf16, const float* cos_sin, const int64_t* dst_slot,
                     int64_t n, uint8_t* cache, int64_t cache_rows, void* stream);

/* DEVICE. Sparse-indexer scores ([P1] §二 layer layout and hierarchical sparse
 * indexer; [P3] 第二刀, Fig. 5). For query (b,t) and position n:
 *   score = sum_{h<32} w[b][t][h] * max(0, sum_{c<128} q_idx[b][t][h][c] * k_idx[b][n][c]).
 *   mode FULL:    scores[b][t][n] for every n < n_cap; n >= n_vis[b][t] gets -inf.
 *                 If `bmax` is not NULL, bmax[b][t][j] = max of scores over
 *                 positions 8j..8j+7 (visible ones; -inf if none), j < ceil(n_cap/8).
 *                 `scores` may be NULL when `bmax` is not: only the block maxima
 *                 are written (below CSA2_PREFILL_MIN_T_FP8 the scores of chosen
 *                 positions can be recomputed bit for bit with REINDEX, which
 *                 evaluates each position the same way).
 *   mode REINDEX: scores[b][t][i] for i < 16384 at position 8*pool[b][t][i/8] + i%8;
 *                 -inf where the pool entry is -1 or the position is >= n_vis.
 *                 `bmax` must be NULL.
 *   q_idx [B][T][32][128] E4M3, w [B][T][32] float, k_idx [B][n_cap][128] E4M3,
 *   n_vis [B][T] int32 (device; values are clamped to [0, n_cap]),
 *   pool  [B][T][2048] int32 (device, REINDEX only; entries >= ceil(n_cap/8) are
 *         treated as -1).
 * Below T = CSA2_PREFILL_MIN_T_FP8 products are exact and sums float32 (MFMA
 * accumulation order), and a query's score is the same bits whatever T is; in
 * FULL mode the query tokens of a sequence (T >= 2, e.g. speculative decode)
 * share each key read, two at a time, and from CSA2_PREFILL_MIN_T_FP8 on in
 * tiles of 16 or 32 through the FP8 contraction (precision: see above).
 * Errors: CSA2_EINVAL for REUSE, NULL/misaligned pointers, REINDEX without a
 * pool, nothing to write, B < 1, T < 1, n_cap < 1 or n_cap >= 2^31. */
int csa2_index_score(int mode, const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                     const int32_t* n_vis, const int32_t* pool, int B, int T, int64_t n_cap,
                     float* scores, float* bmax, void* stream);

/* DEVICE. Sequence compressor of the write path: every m tokens become one
 * compressed entry ([P1] §二 layer layout: m = 2 in encoder groups, 1 in decoder
 * groups; [P2] 黑科技之二). The learned compressor of the real model is not on the
 * pages; this library takes the mean the workloads fix:
 *   out[j][c] = bf16( (sum_{r = jm .. min(jm+m, n_tok)-1} tokens[r][c]) / count ),
 * summed in float32 in token order, divided with a correctly rounded float32
 * division, rounded to bf16 nearest-even. A trailing partial group is the mean of
 * the rows present (a decode step re-compresses the open group when its second
 * token arrives; only complete entries are visible to queries).
 *   tokens_bf16 [n_tok][width] (device), out_bf16 [ceil(n_tok/m)][width] (device,
 *   written), width a multiple of 8 up to CSA2_MAX_WIDTH, 1 <= m <= CSA2_MAX_M.
 * Rows of several sequences compress in one call when each contributes a whole
 * number of groups. Inputs must be finite.
 * Errors: CSA2_EINVAL for NULL/misaligned pointers or bad sizes. */
int csa2_compress_tokens(const void* tokens_bf16, int64_t n_tok, int width, int m,
                         void* out_bf16, void* stream);

/* DEVICE. E4M3 append of the write path: the sliding-window KV stays FP8 ([P1]
 * §三; [P3] 第三刀) and every layer keeps its own window ([P2] 黑科技之二); FP8
 * indexer keys are E4M3 as in every workload.
 *   rows_bf16 [n][width] (device); dst_slot [n] int64 destination row (device) or
 *   NULL for row r -> row r, slots outside [0, rows) skipped; out [rows][width]
 *   E4M3 codes (device, written); width a multiple of 8 up to CSA2_MAX_WIDTH.
 * Each value becomes the nearest E4M3 (OCP E4M3FN) value, ties to the even code,
 * saturating at +-448, sign bit kept. Inputs must be finite.
 * Errors: CSA2_EINVAL for NULL/misaligned pointers, bad sizes, n > rows without
 * slots. */
int csa2_quantize_e4m3(const void* rows_bf16, int64_t n, int width, const int64_t* dst_slot,
                       uint8_t* out, int64_t rows, void* stream);

/* DEVICE. FP4 indexer keys. An earlier model generation already trained the
 * indexer's keys in FP4 ([P2] 黑科技之三) and the pages' FP4 belongs to the MXFP4
 * family ([P1] §三); they give no block size or scale type for the indexer, so
 * this library takes the OCP Microscaling (MX) v1.0 layout and conversion rule:
 *   k_bf16   [n][128] bf16 keys (device, finite values);
 *   dst_slot [n] int64 destination row (device), or NULL for row r -> row r;
 *            slots outside [0, rows) are skipped;
 *   codes    [rows][64] (device, written): byte j = E2M1 code of channel 2j in the
 *            low nibble, channel 2j+1 in the high nibble;
 *   scales   [rows][4] (device, written): byte b = E8M0 scale of channels
 *            32b..32b+31, max(E - 2, 0) for the biased exponent E of the block's
 *            largest |value| (= floor(log2(amax)) - 2 + 127; 0 for a zero block).
 * Each element is the E2M1 code nearest |v| / 2^(scale - 127) (ties to the even
 * code, saturating at 6); its sign bit is the sign bit of v.
 * Errors: CSA2_EINVAL for NULL/misaligned pointers, n < 0, rows < 1. */
/* (`scales` needs only 4-byte alignment, so one sequence's slice of a [B][n_cap][4]
 * buffer can be passed.) */
int csa2_quantize_index_k(const void* k_bf16, const int64_t* dst_slot, int64_t n,
                          uint8_t* codes, uint8_t* scales, int64_t rows, void* stream);

/* DEVICE. csa2_index_score over FP4 indexer keys (csa2_quantize_index_k's
 * layout): k_codes [B][n_cap][64], k_scales [B][n_cap][4] (device) take the
 * place of k_idx; the key value of channel c is E2M1(code) * 2^(scale - 127),
 * multiplied exactly with the E4M3 query by the scaled FP8 x FP4 matrix
 * instruction. Modes, outputs, masking and errors are those of
 * csa2_index_score (FULL from T = CSA2_PREFILL_MIN_T_FP4 on runs the
 * prefill-shaped contraction, below it the decode shape with two query tokens
 * per key read); every decode shape, and REINDEX, gives a position the same
 * bits, and the prefill-shaped scores lie within the FP8 contraction's
 * truncation bound of them. `k_scales` needs only 4-byte alignment. */
int csa2_index_score_fp4k(int mode, const uint8_t* q_idx, const float* w, const uint8_t* k_codes,
                          const uint8_t* k_scales, const int32_t* n_vis, const int32_t* pool,
                          int B, int T, int64_t n_cap, float* scores, float* bmax, void* stream);

/* DEVICE. Fused Full-mode scan and Top-512 ([P1] §二 layer layout, mode table
 * and hierarchical sparse indexer): the exact Top-512 of the float32-accurate
 * (decode-shaped) scores, without writing any score row.
 * Below CSA2_PREFILL_MIN_T_FP8 (E4M3 keys) / _FP4 (FP4 keys) query tokens: up to
 * 16,384 positions the score rows go to the workspace and one selection takes
 * the Top-512; beyond, the scan keeps only block maxima, the 512 best blocks of
 * 8 (by block maximum, ties to the lower block; found through the 512 best
 * super-blocks of 8 blocks) are re-scored position by position to the scan's
 * own bits, and the Top-512 is taken among those 4,096 positions. This is
 * exact: each block ranked ahead of the block holding one of the 512 best
 * positions holds, as its maximum, a distinct position ranked ahead of it, so
 * the 512 best positions lie in the 512 best blocks.
 * From that T on the scan is the prefill-shaped FP8 contraction: its block
 * maxima narrow the candidates to the 1,024 best blocks, whose 8,192 positions
 * are re-scored float32-accurately before the selection. A block holding one
 * of the 512 best positions could drop out of that list only if more than 512
 * other blocks came within twice the contraction's error of its maximum.
 *   q_idx, w, n_vis: as csa2_index_score; k_idx [B][n_cap][128] E4M3 keys when
 *   k_scales is NULL, else [B][n_cap][64] FP4 codes with k_scales [B][n_cap][4]
 *   (csa2_quantize_index_k's layout; 4-byte aligned);
 *   idx [B][T][512] int32 (device, written) as csa2_topk writes it: ascending,
 *   -1 padded; ranking by (score descending, position ascending);
 *   ws   csa2_workspace_bytes(CSA2_OP_INDEX_TOPK, 0, B, T, n_cap) bytes (device).
 * Errors: CSA2_EINVAL (pointers, sizes), CSA2_EWORKSPACE, CSA2_EUNSUPPORTED for
 * n_cap > CSA2_INDEX_TOPK_MAX_CAP. */
int csa2_index_topk(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                    const uint8_t* k_scales, const int32_t* n_vis, int B, int T, int64_t n_cap,
                    int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* DEVICE. csa2_index_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, kernels and result, with the workspace
 * taken from a library-owned device array of CSA2_NOALLOC_SCRATCH_BYTES (32 MiB)
 * instead of a caller buffer. The call allocates nothing; each GPU holds its
 * own copy of the array from the first call on that device until the process
 * ends. Every call on a GPU shares that GPU's array, so calls that overlap in
 * time on one GPU (on different streams, or from several threads) race and
 * must be ordered by the caller; no part of the array needs to start at zero
 * (each call writes every byte it later reads). Arguments as csa2_index_topk,
 * without `ws` and `ws_bytes`.
 * Errors: as csa2_index_topk; CSA2_EWORKSPACE when the request needs more than
 * CSA2_NOALLOC_SCRATCH_BYTES (csa2_workspace_bytes(CSA2_OP_INDEX_TOPK, ...)
 * bytes: e.g. 64 sequences x 524,288 positions need about 18 MB, a
 * 4,096-query prefill chunk over 133,120 positions far more); CSA2_EHIP if the
 * array's device address cannot be resolved. */
int csa2_index_topk_noalloc(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                            const uint8_t* k_scales, const int32_t* n_vis, int B, int T,
                            int64_t n_cap, int32_t* idx, void* stream);

/* DEVICE. Hierarchical candidate pool ([P1] §二 hierarchical sparse indexer;
 * [P3] 第二刀, Fig. 5): per query, among blocks j < ceil(n_vis/8), the 2,048
 * with the largest block max (ties to the lower block id), written as block ids
 * in ascending order and padded with -1.
 *   src    [B][T][ceil(n_cap/8)] block maxima when is_bmax != 0 (as written by
 *          csa2_index_score), else [B][T][n_cap] FULL scores (device);
 *   pool   [B][T][2048] int32 (device, written);
 *   ws     device workspace of at least csa2_workspace_bytes(CSA2_OP_BUILD_POOL, ...)
 *          bytes (may be NULL when that is 0).
 * Errors: CSA2_EINVAL (pointers, sizes), CSA2_EWORKSPACE. */
int csa2_build_pool(const float* src, int is_bmax, const int32_t* n_vis, int B, int T,
                    int64_t n_cap, int32_t* pool, void* ws, size_t ws_bytes, void* stream);

/* DEVICE. Top-512 per query ([P1] §二 mode table and layer layout; [P2] 黑科技之二).
 *   FULL:    the 512 highest of scores[b][t][0 .. n_vis) ([B][T][n_cap]).
 *            Optional helpers, both computed from these same scores and n_vis:
 *            `bmax` [B][T][ceil(n_cap/8)] block maxima as csa2_index_score
 *            writes them (NULL: computed into the workspace), and `pool`
 *            [B][T][2048] as csa2_build_pool writes it (NULL: not used). With a
 *            pool the search runs over its 16,384 positions; this is exact
 *            because the 512 best positions always lie inside the 2,048 best
 *            blocks of 8 ([P1] §二 hierarchical sparse indexer).
 *   REINDEX: the 512 highest of the pool candidates scores[b][t][i], i < 16384
 *            ([B][T][16384], from csa2_index_score REINDEX with the same pool);
 *            `bmax` must be NULL.
 *   REUSE:   idx = src_idx byte for byte (a device copy; nothing when idx == src_idx).
 * Ranking is by (score descending, position ascending); the selected positions
 * are written to idx [B][T][512] int32 in ascending order, padded with -1 when
 * fewer than 512 candidates exist. Scores must not be NaN. FULL needs a
 * workspace of csa2_workspace_bytes(CSA2_OP_TOPK, CSA2_FULL, ...) bytes (0 when
 * n_cap <= 16384; then `ws` may be NULL); REINDEX and REUSE need none.
 * Errors: CSA2_EINVAL (pointers, sizes, REINDEX without pool or with bmax,
 * REUSE without src_idx), CSA2_EWORKSPACE. */
int csa2_topk(int mode, const float* scores, const float* bmax, const int32_t* n_vis,
              const int32_t* pool, const int32_t* src_idx, int B, int T, int64_t n_cap,
              int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* DEVICE. Sparse MQA attention over the selected FP4 main-KV rows plus the
 * 128-token FP8 window ([P1] §二 layer layout, §三; [P3] 第三刀: dequantise
 * before attention, window KV stays FP8; [P2] 黑科技之二: every layer has its
 * own query and window KV).
 *   q        [B][T][64][512] bf16 (device);
 *   cache    [B][n_cap][288] packed rows (device); key = value = the dequantised row;
 *   idx      [B][T][512] int32 selected positions (device); -1 and values outside
 *            [0, n_cap) are skipped;
 *   swa      [B][S][512] E4M3 window rows (device), row s of sequence b holds
 *            token swa_pos0[b] + s;
 *   q_pos    [B][T] int64 token position t of each query (device);
 *   swa_pos0 [B] int64 (device).
 * Keys = the selected rows and the window tokens max(0, t-127) .. t (tokens
 * outside [swa_pos0, swa_pos0 + S) are skipped); one softmax over all of them of
 * scale * q_h . key; out[b][t][h] = sum_j p_hj key_j, float32 [B][T][64][512].
 * Needs csa2_workspace_bytes(CSA2_OP_SPARSE_ATTN, 0, B, T, n_cap) bytes of
 * workspace: the partial results of 5 key slices per query when B*T <= 12 (a
 * few queries spread over more work-groups), none from 13 queries on (then `ws`
 * may be NULL).
 * Errors: CSA2_EINVAL (pointers, sizes, S < 1, a non-finite scale), CSA2_EWORKSPACE. */
int csa2_sparse_attn(const void* q_bf16, const uint8_t* cache, const int32_t* idx,
                     const uint8_t* swa, const int64_t* q_pos, const int64_t* swa_pos0, int B,
                     int T, int64_t n_cap, int S, float softmax_scale, float* out, void* ws,
                     size_t ws_bytes, void* stream);

/* DEVICE. csa2_sparse_attn over a window kept as a ring buffer: the window KV
 * of the last n_win = 128 tokens per layer, replayed as a bounded span ([P2]
 * 黑科技之三, SWA Bounded Replay; [P3] 第三刀). Token tok of sequence b sits in
 * row tok mod S of swa [B][S][512]; the rows hold tokens
 * [swa_pos0[b], swa_pos0[b] + S), and window tokens outside that range are
 * skipped. A decode loop appends token t into row t mod S (csa2_quantize_e4m3
 * with dst_slot = b * S + t mod S) and sets swa_pos0 = max(0, t - S + 1); with
 * S >= 127 + T every query of a T-token step sees its whole window. Arguments,
 * workspace, result and errors otherwise as csa2_sparse_attn. */
int csa2_sparse_attn_ring(const void* q_bf16, const uint8_t* cache, const int32_t* idx,
                          const uint8_t* swa, const int64_t* q_pos, const int64_t* swa_pos0, int B,
                          int T, int64_t n_cap, int S, float softmax_scale, float* out, void* ws,
                          size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
