"""Sparse MQA attention over the selected main-KV rows plus the sliding window
(oracle; test-only).

Pages: main attention has 64 heads of width 512 [P1 §二 layer layout]; it runs
over the Top-512 selected global entries plus a 128-token sliding window
[P1 §一 (n = 128); P2 黑科技之一; P4 架构重构的三级挤压]; the FP4 main KV is
dequantised before attention [P3 第三刀] while the window KV stays FP8
[P1 §三; P3 第三刀]; every layer keeps its own query and window KV
[P1 §二; P2 黑科技之二].
Readings taken:
  * Heads share one 512-wide latent per key (MQA over the shared latent); the
    same dequantised row is both key and value; the output is not un-rotated.
  * Window = tokens max(0, t - 127) .. t, the current token included. Window
    rows are 512-wide E4M3 codes with no scale.
  * One softmax over the union of the (up to) 512 selected rows and the window
    rows; no sink; no de-duplication (they are different tensors).
  * logits z = scale * q_h . key with q taken exactly from bf16; the 1/sqrt(512)
    factor of the configs is folded into q, so scale = 1 there.
  * All arithmetic in float64; the output is rounded to float32.
  * What a caller's buffers may not hold is skipped, not guessed: a selected
    index outside [0, rows of the cache) contributes no key, and a window token
    that the window buffer does not hold (outside [swa_pos0, swa_pos0 + S))
    contributes no key.
  * The window buffer is addressed in one of two ways. Linear: row s holds token
    swa_pos0 + s. Ring: token tok sits in row tok mod S, so a decode loop appends
    token t into row t mod S and advances swa_pos0 to max(0, t - S + 1); the
    pages keep the window KV of the last n_win = 128 tokens per layer and replay
    exactly that span ("DeepSeek V4.1 Flash vs V4 Pro", 黑科技之三;
    "DeepSeek-V4.1-Flash：全局 KV 仅 890 B/token", 第三刀), which a ring of
    S >= 128 rows holds.
"""

import numpy as np

from .formats import dequantize_rows, e4m3_decode

N_WIN = 128
N_HEADS = 64
D_MAIN = 512


def swa_tokens(t, n_win=N_WIN):
    """Tokens of the sliding window of the query at token t."""
    return np.arange(max(0, int(t) - n_win + 1), int(t) + 1, dtype=np.int64)


def softmax_attention(q, keys, scale):
    """Textbook softmax attention of float64 queries q [H, D] over rows keys
    [n, D] used as both key and value. Returns float64 [H, D]."""
    z = scale * (q @ keys.T)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ keys


def window_rows(t, swa_pos0, S, ring=False):
    """(tokens, rows) of the window tokens of the query at token t that a
    window buffer of S rows holds: tokens in [swa_pos0, swa_pos0 + S), each
    at row tok - swa_pos0 (linear) or tok mod S (ring)."""
    toks = swa_tokens(t)
    toks = toks[(toks >= int(swa_pos0)) & (toks < int(swa_pos0) + int(S))]
    rows = toks % int(S) if ring else toks - int(swa_pos0)
    return toks, rows


def gather_keys(cache_rows, idx, swa_codes, t, swa_pos0, ring=False):
    """Dequantised key rows for one query: selected main rows (0 <= idx < rows
    of the cache) in idx order, then the window rows the buffer holds, in token
    order."""
    idx = np.asarray(idx, dtype=np.int64)
    sel = idx[(idx >= 0) & (idx < len(cache_rows))]
    main = dequantize_rows(np.asarray(cache_rows[sel]))
    swa_codes = np.asarray(swa_codes)
    _, rows = window_rows(t, swa_pos0, swa_codes.shape[0], ring)
    swa = e4m3_decode(swa_codes[rows])
    return np.concatenate([main, swa], axis=0)


def sparse_attention(q, cache_rows, idx, swa_codes, t, swa_pos0, scale=1.0, ring=False):
    """One query's output [64, 512] float32.

    q: float array [64, 512] holding the bf16 query values exactly;
    cache_rows: packed 288-byte main-KV rows indexed by position (an array, or
    any object with len() and row indexing by an index array);
    idx: the selected positions (-1 padded); swa_codes: uint8 [S, 512] E4M3
    window rows (linear: row s holds token swa_pos0 + s; ring: token tok sits
    in row tok mod S); t: the query's token."""
    keys = gather_keys(cache_rows, idx, swa_codes, t, swa_pos0, ring)
    q = np.asarray(q, dtype=np.float64).reshape(N_HEADS, D_MAIN)
    return softmax_attention(q, keys, float(scale)).astype(np.float32)
