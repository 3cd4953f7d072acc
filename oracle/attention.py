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


def gather_keys(cache_rows, idx, swa_codes, t, swa_pos0):
    """Dequantised key rows for one query: selected main rows (idx >= 0) in idx
    order, then the window rows in token order."""
    idx = np.asarray(idx, dtype=np.int64)
    sel = idx[idx >= 0]
    main = dequantize_rows(np.asarray(cache_rows[sel]))
    toks = swa_tokens(t)
    swa = e4m3_decode(np.asarray(swa_codes)[toks - int(swa_pos0)])
    return np.concatenate([main, swa], axis=0)


def sparse_attention(q, cache_rows, idx, swa_codes, t, swa_pos0, scale=1.0):
    """One query's output [64, 512] float32.

    q: float array [64, 512] holding the bf16 query values exactly;
    cache_rows: packed 288-byte main-KV rows indexed by position;
    idx: the selected positions (-1 padded); swa_codes: uint8 [S, 512] E4M3
    window rows where row s holds token swa_pos0 + s; t: the query's token."""
    keys = gather_keys(cache_rows, idx, swa_codes, t, swa_pos0)
    q = np.asarray(q, dtype=np.float64).reshape(N_HEADS, D_MAIN)
    return softmax_attention(q, keys, float(scale)).astype(np.float32)
