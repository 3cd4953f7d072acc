"""Sequence compression and causal visibility (oracle; test-only).

The pages say every m tokens become one compressed entry, with m = 2 in the
encoder groups and m = 1 in the decoder groups [P1 §二 layer layout; P2
黑科技之二]. The real compressor is learned and out of scope; the spec of this
path fixes m = 2 as the mean of token pairs. Readings taken:
  * Entry j covers tokens [j m, j m + m). It is the mean of those bf16 token
    rows computed in float32 (rows summed in token order, then divided by the
    row count) and rounded to bf16, nearest-even. A trailing partial group is the
    mean of the rows present. The entry count for N tokens is ceil(N / m).
  * A query at token t sees only complete entries: n_vis(t) = floor((t + 1) / m).
"""

import numpy as np


def n_entries(n_tokens, m):
    """Number of compressed entries for ``n_tokens`` tokens: ceil(N / m)."""
    return -(-int(n_tokens) // int(m))


def n_visible(t, m):
    """Compressed entries visible to the query at token ``t`` (complete ones only)."""
    return (np.asarray(t, dtype=np.int64) + 1) // int(m)


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even) as uint16 bit
    patterns. Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact bf16 -> float32 decode of uint16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def compress_mean(token_bits, m):
    """Mean-pool bf16 token rows (uint16 bits, shape [N, D]) in groups of ``m``.
    Returns bf16 bits of shape [ceil(N/m), D]."""
    tok = bf16_bits_to_f32(token_bits)
    n, d = tok.shape
    k = n_entries(n, m)
    out = np.empty((k, d), dtype=np.float32)
    for j in range(k):
        rows = tok[j * m: min(n, (j + 1) * m)]
        acc = np.zeros(d, dtype=np.float32)
        for r in rows:
            acc = acc + r                      # float32, token order
        out[j] = acc / np.float32(rows.shape[0])
    return f32_to_bf16_bits(out)
