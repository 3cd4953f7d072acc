"""Layer-group schedules and one query's pass through a group (oracle; test-only).

Pages:
  * Mode table: Full generates its own main KV and indexer K and picks its own
    Top-K; Reindex reuses an earlier layer's main KV and indexer K but picks its
    own Top-K with its own indexer query; Reuse reuses main KV and Top-K indices
    and computes no indexer query [P1 §二 mode table; P2 黑科技之二; P3 第二刀].
  * Layout: encoder layers 3-20 in 3 groups of [1 Full + 5 Reuse] at m = 2;
    decoder 20 layers in 5 groups, the first [1 Full + 3 Reuse], the other four
    [1 Reindex + 3 Reuse], at m = 1 [P1 §二 layer layout]. Another page says
    only 4 backbone layers generate KV state, numbered 2, 8, 14 and 20
    [P4 架构重构的三级挤压]; that agrees with the layout if those numbers are
    0-based (1-based 3, 9, 15 and 21).
  * Every layer computes its own main query and window KV [P1 §二; P2 黑科技之二].
  * The pool is built by the first Full layer after its full scan and used by the
    later Reindex layers [P1 §二 hierarchical indexer; P3 第二刀, Fig. 5].
Reading taken for the short decoder group used as a workload (1 Full, 3
Reindex, 3 Reuse layers, order not given): [F, X1, U1, X2, U2, X3, U3], each
Reuse layer reusing the indices of the Reindex layer just before it, and every
layer reading the Full layer's main KV and indexer K.
"""

import numpy as np

from .indexer import index_scores, block_max
from .select import topk_positions, build_pool, reindex_candidates
from .attention import sparse_attention

FULL, REINDEX, REUSE = "F", "X", "U"


def model_layout():
    """The 40-layer backbone's CSA2 modes, 1-based layer number -> (mode, m).

    Layers 1-2 of the encoder are not CSA2 layers in the layout the pages give
    and are reported as None."""
    modes = {1: None, 2: None}
    layer = 3
    for _ in range(3):                       # encoder: 3 x [Full + 5 Reuse]
        for j in range(6):
            modes[layer] = (FULL if j == 0 else REUSE, 2)
            layer += 1
    for g in range(5):                       # decoder: 5 groups
        head = FULL if g == 0 else REINDEX
        for j in range(4):
            modes[layer] = (head if j == 0 else REUSE, 1)
            layer += 1
    assert layer == 41
    return modes


def layer_schedule(kind):
    """(mode, source layer index) per layer of a workload group.

    'decoder': [F, X1, U1, X2, U2, X3, U3]; 'encoder': [F, U1..U5];
    'full': a single Full layer."""
    if kind == "full":
        return [(FULL, None)]
    if kind == "encoder":
        return [(FULL, None)] + [(REUSE, 0)] * 5
    if kind == "decoder":
        sched = [(FULL, None)]
        for _ in range(3):
            sched.append((REINDEX, 0))
            sched.append((REUSE, len(sched) - 1))
        return sched
    raise ValueError(kind)


def run_group(schedule, q_idx, w, q, swa, k_codes, cache_rows, n_vis, t,
              swa_pos0, scale=1.0, with_pool=True, k_scales=None, ring=False):
    """One query through a layer group.

    q_idx / w: dict layer -> indexer query [32,128] E4M3 codes / weights [32]
    (only index-producing layers need them); q / swa: dict layer -> main query
    [64,512] (bf16 values as floats) / window rows [S,512] E4M3 codes;
    k_codes [n_cap,128] and cache_rows [n_cap,288] are the group's shared
    indexer keys and packed main KV (with ``k_scales`` [n_cap,4], k_codes are
    [n_cap,64] packed FP4 keys; see ``mxfp4``). ``ring``: the window buffers
    are rings (token tok in row tok mod S; see ``attention``). Returns (idx per
    layer, out per layer, pool, scores per index-producing layer)."""
    idx_of, out_of, scores_of = {}, {}, {}
    pool = None
    for li, (mode, src) in enumerate(schedule):
        if mode == FULL:
            s = index_scores(q_idx[li], w[li], k_codes, n_vis, k_scales=k_scales)
            nv = min(int(n_vis), s.shape[0])
            idx_of[li] = topk_positions(s[:nv], np.arange(nv))
            if with_pool and pool is None:
                pool = build_pool(block_max(s, n_vis), n_vis)
            scores_of[li] = s
        elif mode == REINDEX:
            cand = reindex_candidates(pool, n_vis)
            s = index_scores(q_idx[li], w[li], k_codes, n_vis, positions=cand,
                             k_scales=k_scales)
            idx_of[li] = topk_positions(s, cand)
            scores_of[li] = (cand, s)
        elif mode == REUSE:
            idx_of[li] = idx_of[src].copy()
        else:
            raise ValueError(mode)
        out_of[li] = sparse_attention(q[li], cache_rows, idx_of[li], swa[li], t,
                                      swa_pos0, scale, ring=ring)
    return idx_of, out_of, pool, scores_of
