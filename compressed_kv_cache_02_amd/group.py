"""Layer-group step: the sequence of libcsa2 calls for one decode (or prefill)
step through a group of CSA2 layers.

Pages: each layer is statically Full, Reindex or Reuse ("DeepSeek V4.1-Flash
为什么这么强？CED 与 CSA2 架构全拆解", §二 mode table); encoder groups are
[Full + 5 Reuse] at m = 2 and decoder groups [Full or Reindex + 3 Reuse] at
m = 1 (same §二, layer layout); the first Full layer builds the candidate pool
that later Reindex layers score inside (same §二, hierarchical sparse indexer);
every layer keeps its own main query and window KV ("DeepSeek V4.1 Flash vs V4
Pro", 黑科技之二).

This module only sequences calls and owns the intermediate device buffers; all
arithmetic runs in the library's kernels.
"""

import torch

from . import (INDEX_TOPK_MAX_CAP, PREFILL_MIN_T_FP8, PREFILL_MIN_T_FP4, CSA2_FULL,
               CSA2_REINDEX, CSA2_REUSE, CSA2_OP_BUILD_POOL, CSA2_OP_INDEX_TOPK,
               CSA2_OP_SPARSE_ATTN, CSA2_OP_TOPK, POOL_BLOCKS, POOL_CAND, TOPK, HEADS, DIM, BLOCK,
               csa2_build_pool, csa2_index_score, csa2_index_score_fp4k, csa2_index_topk,
               csa2_quantize_kv, csa2_sparse_attn, csa2_topk, csa2_workspace_bytes)

FULL, REINDEX, REUSE = "F", "X", "U"


def schedule(kind):
    """(mode, source layer) per layer: 'full' = [F]; 'encoder' = [F, U x5];
    'decoder' = [F, X, U, X, U, X, U] where each U reuses the X just before it
    and every X reads the Full layer's keys, main KV and pool."""
    if kind == "full":
        return [(FULL, None)]
    if kind == "encoder":
        return [(FULL, None)] + [(REUSE, 0)] * 5
    if kind == "decoder":
        s = [(FULL, None)]
        for _ in range(3):
            s.append((REINDEX, 0))
            s.append((REUSE, len(s) - 1))
        return s
    raise ValueError(kind)


def index_score(mode, q_idx, w, keys, n_vis, pool, scores, bmax=None, stream=None):
    """csa2_index_score over FP8 keys (a [B, n_cap, 128] uint8 tensor) or
    csa2_index_score_fp4k over FP4 keys (a (codes [B, n_cap, 64],
    scales [B, n_cap, 4]) pair)."""
    if isinstance(keys, tuple):
        codes, scales = keys
        csa2_index_score_fp4k(mode, q_idx, w, codes, scales, n_vis, pool, scores, bmax,
                              stream=stream)
    else:
        csa2_index_score(mode, q_idx, w, keys, n_vis, pool, scores, bmax, stream=stream)


def fused_topk_auto(T, n_cap):
    """Whether a group without a pool takes the fused scan + Top-K by default:
    whenever the scan is prefill-shaped (from PREFILL_MIN_T_FP8 query tokens
    per sequence: its FP8 contraction's scores only narrow the candidates,
    which the fused call re-scores FP32-accurately before selecting), and for
    decode over at least 262,144 positions, within the context the fused entry
    point serves."""
    return ((T >= min(PREFILL_MIN_T_FP8, PREFILL_MIN_T_FP4) or n_cap >= (1 << 18))
            and n_cap <= INDEX_TOPK_MAX_CAP)


def visible_entries(t, m):
    """Complete compressed entries visible at token t: floor((t + 1) / m)."""
    return (t + 1) // m


class LayerGroup:
    """Intermediate buffers for one group step of B sequences x T queries."""

    def __init__(self, kind, B, T, n_cap, device="cuda", keep_scores=False, fused_topk="auto"):
        """fused_topk: a group without a pool takes its Full layer's Top-K from
        the fused csa2_index_topk (no score rows written) instead of a scan
        followed by csa2_topk. "auto" does so whenever the scan is
        prefill-shaped (its FP8 scores only narrow the candidates; the fused
        call re-scores them FP32-accurately) and for decode steps over at least
        262,144 positions, where the score rows saved outweigh re-scoring 4,096
        positions per query (measured on MI355X: c4 +4%; c1, 65,536 entries, 3%
        slower fused)."""
        self.sched = schedule(kind)
        self.B, self.T, self.n_cap = B, T, n_cap
        dev = torch.device(device)
        L = len(self.sched)
        n_blk = (n_cap + BLOCK - 1) // BLOCK
        need_pool = any(m == REINDEX for m, _ in self.sched)
        if fused_topk == "auto":
            fused_topk = fused_topk_auto(T, n_cap)
        self.fused = bool(fused_topk) and not need_pool and not keep_scores
        # Block maxima come with the scan and drive the hierarchical selections.
        # A group with a pool writes no full score rows: its Full layer
        # re-scores the pool's 16,384 positions (bit-identical to a
        # decode-shaped scan) and takes its Top-K there, exact because the 512
        # best positions always lie inside the 2,048 best blocks.
        self.bmax = torch.empty((B, T, n_blk), dtype=torch.float32, device=dev)
        self.scores = None if (need_pool or self.fused) else torch.empty(
            (B, T, n_cap), dtype=torch.float32, device=dev)
        self.ws_fused = (torch.empty((csa2_workspace_bytes(CSA2_OP_INDEX_TOPK, 0, B, T, n_cap),),
                                     dtype=torch.uint8, device=dev) if self.fused else None)
        self.pool = torch.empty((B, T, POOL_BLOCKS), dtype=torch.int32, device=dev) if need_pool else None
        self.scores_full_pool = (torch.empty((B, T, POOL_CAND), dtype=torch.float32, device=dev)
                                 if need_pool else None)
        self.scores_pool = (torch.empty((B, T, POOL_CAND), dtype=torch.float32, device=dev)
                            if need_pool else None)
        self.idx = [None] * L
        for li, (m, src) in enumerate(self.sched):
            # a Reuse layer aliases its source's index buffer (no copy)
            self.idx[li] = self.idx[src] if m == REUSE else torch.empty(
                (B, T, TOPK), dtype=torch.int32, device=dev)
        self.out = [torch.empty((B, T, HEADS, DIM), dtype=torch.float32, device=dev)
                    for _ in range(L)]
        ws = max(csa2_workspace_bytes(CSA2_OP_TOPK, CSA2_FULL, B, T, n_cap),
                 csa2_workspace_bytes(CSA2_OP_TOPK, CSA2_REINDEX, B, T, n_cap),
                 csa2_workspace_bytes(CSA2_OP_SPARSE_ATTN, 0, B, T, n_cap),
                 csa2_workspace_bytes(CSA2_OP_BUILD_POOL, 0, B, T, n_cap) if need_pool else 0)
        self.ws = torch.empty((max(ws, 256),), dtype=torch.uint8, device=dev)
        self.keep_scores = keep_scores
        self.saved_scores = {}

    def step(self, k_idx, cache, n_vis, q_pos, swa_pos0, q_idx, w, q, swa, scale=1.0,
             write=None, stream=None, hooks=None):
        """One pass of the whole group.

        k_idx [B,n_cap,128] FP8 keys, or a (codes [B,n_cap,64], scales
        [B,n_cap,4]) pair of FP4 keys; cache [B,n_cap,288]: the group's shared
        keys and packed main KV; n_vis [B,T] int32; q_pos [B,T] int64; swa_pos0 [B] int64;
        q_idx / w: per index-producing layer (dict or list indexed by layer);
        q / swa: per layer. write = (kv_bf16 [n,512], cos_sin [n,32,2],
        dst_slot [n]) runs the write path first. hooks: optional dict of
        callables ('scan_begin', 'scan_end') run around the Full-layer scan."""
        hooks = hooks or {}
        self.write(cache, write, stream=stream)
        if "scan_begin" in hooks:
            hooks["scan_begin"]()
        self.scan(k_idx, n_vis, q_idx, w, stream=stream)
        if "scan_end" in hooks:
            hooks["scan_end"]()
        self.rest(k_idx, cache, n_vis, q_pos, swa_pos0, q_idx, w, q, swa, scale, stream=stream)
        return self.out

    def write(self, cache, write, stream=None):
        """The write path: new rows RoPE'd, packed to FP4 and stored."""
        if write is not None:
            kv, cs, slot = write
            csa2_quantize_kv(kv, cs, slot, cache, stream=stream)

    def scan(self, k_idx, n_vis, q_idx, w, stream=None):
        """The Full layer's scan of every visible position, with block maxima
        (nothing here when the fused Top-K runs the scan itself)."""
        if not self.fused:
            self.scan_only(k_idx, n_vis, q_idx, w, stream=stream)

    def scan_only(self, k_idx, n_vis, q_idx, w, stream=None):
        """The Full-layer scan alone (scores only where the group keeps them)."""
        li = [i for i, (m, _) in enumerate(self.sched) if m == FULL][0]
        index_score(CSA2_FULL, q_idx[li], w[li], k_idx, n_vis, None, self.scores, self.bmax,
                    stream=stream)   # scores is None with a pool or a fused Top-K

    def rest(self, k_idx, cache, n_vis, q_pos, swa_pos0, q_idx, w, q, swa, scale=1.0,
             stream=None):
        """Everything after the Full scan: pool, Top-K per mode, attention per layer."""
        for li, (mode, src) in enumerate(self.sched):
            if mode == FULL:
                if self.pool is not None:
                    csa2_build_pool(self.bmax, True, n_vis, self.n_cap, self.pool, self.ws,
                                    stream=stream)
                    index_score(CSA2_REINDEX, q_idx[li], w[li], k_idx, n_vis, self.pool,
                                self.scores_full_pool, None, stream=stream)
                    csa2_topk(CSA2_REINDEX, self.scores_full_pool, n_vis, self.pool, None,
                              self.n_cap, self.idx[li], self.ws, stream=stream)
                elif self.fused:
                    csa2_index_topk(q_idx[li], w[li], k_idx, n_vis, self.idx[li], self.ws_fused,
                                    stream=stream)
                else:
                    csa2_topk(CSA2_FULL, self.scores, n_vis, None, None, self.n_cap,
                              self.idx[li], self.ws, stream=stream, bmax=self.bmax)
                if self.keep_scores:
                    self.saved_scores[li] = (self.scores if self.scores is not None
                                             else self.scores_full_pool).clone()
            elif mode == REINDEX:
                index_score(CSA2_REINDEX, q_idx[li], w[li], k_idx, n_vis, self.pool,
                            self.scores_pool, None, stream=stream)
                csa2_topk(CSA2_REINDEX, self.scores_pool, n_vis, self.pool, None, self.n_cap,
                          self.idx[li], self.ws, stream=stream)
                if self.keep_scores:
                    self.saved_scores[li] = self.scores_pool.clone()
            else:
                csa2_topk(CSA2_REUSE, None, None, None, self.idx[src], self.n_cap, self.idx[li],
                          None, stream=stream)
            csa2_sparse_attn(q[li], cache, self.idx[li], swa[li], q_pos, swa_pos0, scale,
                             self.out[li], self.ws, stream=stream)
