"""Top-512 selection and the hierarchical candidate pool (oracle; test-only).

Pages:
  * Each layer is statically Full, Reindex or Reuse. Full picks its own Top-K
    over everything it can see; Reindex re-scores with its own indexer query and
    picks its own Top-K; Reuse carries the earlier layer's indices unchanged
    [P1 §二 mode table; P2 黑科技之二; P3 第二刀, Fig. 4].
  * Top-512 per query [P1 §二 layer layout; P4 架构重构的三级挤压].
  * The first Full layer, after its full scan, keeps the blocks with the highest
    in-block maximum score as a shared candidate pool of 2,048 blocks x 8
    positions = 16,384 positions; Reindex layers score only inside it
    [P1 §二 hierarchical indexer; P3 第二刀, Fig. 5].
Readings taken:
  * Ranking is by (score descending, position ascending): a tie goes to the lower
    position. The selected positions are emitted in ascending order; when fewer
    than K candidates exist the list is padded with -1.
  * A pool block is 8 consecutive compressed positions; its key is the maximum
    over its visible positions; ties go to the lower block id; at most 2,048
    blocks among the ceil(n_vis / 8) blocks that hold a visible position; block
    ids are emitted ascending, -1 padded.
  * Reindex candidates are the pool positions 8 b + r (r < 8) below n_vis.
"""

import numpy as np

TOPK = 512
POOL_BLOCKS = 2048
BLOCK = 8


def topk_positions(scores, cand_positions, k=TOPK):
    """Plain definition: stable sort of the candidates by (-score, position),
    keep the first min(k, #candidates), return them ascending, -1 padded.

    scores: float32 per candidate; cand_positions: int per candidate."""
    scores = np.asarray(scores, dtype=np.float32)
    pos = np.asarray(cand_positions, dtype=np.int64)
    assert scores.shape == pos.shape
    order = np.lexsort((pos, -scores.astype(np.float64)))
    keep = np.sort(pos[order[:k]])
    out = np.full(k, -1, dtype=np.int32)
    out[:keep.shape[0]] = keep
    return out


def build_pool(bmax, n_vis, n_blocks=POOL_BLOCKS):
    """Top ``n_blocks`` block ids by (block max descending, block id ascending)
    among blocks 0..ceil(n_vis/8)-1; ascending, -1 padded."""
    bmax = np.asarray(bmax, dtype=np.float32)
    n_blk = min(-(-int(n_vis) // BLOCK), bmax.shape[0])
    ids = np.arange(n_blk, dtype=np.int64)
    return topk_positions(bmax[:n_blk], ids, k=n_blocks)


def reindex_candidates(pool, n_vis):
    """Positions a Reindex layer scores: 8 b + r for pooled blocks b, r < 8,
    below n_vis; ascending (the pool is ascending)."""
    pool = np.asarray(pool, dtype=np.int64)
    b = pool[pool >= 0]
    pos = (b[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
    return pos[pos < int(n_vis)]
