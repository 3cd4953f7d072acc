"""Sparse-indexer scores (oracle; test-only).

The pages give the indexer's shape only: 32 index query heads of width 128,
Top-512 per query [P1 §二 layer layout]. They say the first index layer scores
every causally visible compressed position [P1 §二 hierarchical indexer; P3
第二刀, Fig. 5]. Readings taken (the spec of this path fixes the formula):
  * score(n) = sum over heads h of w_h * max(0, q_h . k_n), one 128-wide key
    k_n per compressed position shared by the 32 heads, one weight w_h per query
    token and head, no further scale.
  * q and k are FP8 E4M3 codes; w is float32.
  * The dot products are exact in float64 (every E4M3 x E4M3 product is a
    multiple of 2^-18 below 2^18, so 128-term sums stay below 2^25 and need at
    most 43 bits). The weighted head sum runs in float64 in ascending h and is
    rounded once to float32.
  * Positions n >= n_vis are not visible and score -inf.
  * With FP4 keys (E2M1 codes plus one power-of-two scale per 32 channels, see
    ``mxfp4``) the dequantised key takes the place of the E4M3 key; nothing
    else changes.
"""

import numpy as np

from .formats import e4m3_decode
from .mxfp4 import dequantize_index_keys

N_IDX_HEADS = 32
D_IDX = 128
BLOCK = 8          # positions per pool block [P1 §二 hierarchical indexer]


def index_scores(q_codes, w, k_codes, n_vis, positions=None, chunk=65536, k_scales=None):
    """Scores of one query.

    q_codes: uint8 [32, 128] E4M3 indexer query; w: float32 [32];
    k_codes: uint8 [n_cap, 128] E4M3 indexer keys, or, with ``k_scales``
    (uint8 [n_cap, 4] E8M0), uint8 [n_cap, 64] packed FP4 keys; n_vis: visible count;
    positions: int array of positions to score (default: all 0..n_cap-1).
    Returns float32 scores for ``positions`` (-inf where position >= n_vis).
    """
    q = e4m3_decode(np.asarray(q_codes).reshape(N_IDX_HEADS, D_IDX))   # f64
    w = np.asarray(w, dtype=np.float32).astype(np.float64).reshape(N_IDX_HEADS)
    k_codes = np.asarray(k_codes)
    n_cap = k_codes.shape[0]
    if positions is None:
        positions = np.arange(n_cap, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    out = np.full(positions.shape[0], -np.inf, dtype=np.float32)
    vis = np.nonzero(positions < int(n_vis))[0]
    for c0 in range(0, vis.shape[0], chunk):
        sel = vis[c0:c0 + chunk]
        if k_scales is None:
            k = e4m3_decode(k_codes[positions[sel]])                    # [c,128]
        else:
            k = dequantize_index_keys(k_codes[positions[sel]], k_scales[positions[sel]])
        d = k @ q.T                                                     # exact
        acc = np.zeros(sel.shape[0], dtype=np.float64)
        for h in range(N_IDX_HEADS):
            acc = acc + w[h] * np.maximum(d[:, h], 0.0)
        out[sel] = acc.astype(np.float32)
    return out


def block_max(scores, n_vis):
    """Per block of 8 consecutive positions: the largest score over its visible
    positions; -inf for blocks with none visible. ``scores`` is one query's
    full-length score vector."""
    scores = np.asarray(scores, dtype=np.float32)
    n_cap = scores.shape[0]
    n_blk = -(-n_cap // BLOCK)
    pad = np.full(n_blk * BLOCK, -np.inf, dtype=np.float32)
    vis = min(int(n_vis), n_cap)
    pad[:vis] = scores[:vis]
    return pad.reshape(n_blk, BLOCK).max(axis=1)
