"""End-to-end GPU parity of layer-group steps (the whole hot path) against the
oracle: Full / Reindex / Reuse layers, the pool, the write path, attention.

Top-K sets are compared under the near-tie rule on the oracle's scores;
attention outputs are compared for every query whose index set equals the
oracle's (a near-tie swap changes which row is attended, so such a query is
counted and only its indices are checked)."""

import numpy as np
import pytest
import torch

import compressed_kv_cache_02_amd as C
from compressed_kv_cache_02_amd.group import LayerGroup, visible_entries
from oracle import group as OG
from oracle import indexer as OI
from oracle.compress import n_visible
import synth
from synth.configs import WORKLOADS, make_inputs, scaled
from tests.helpers import (NEAR_TIE, OracleCache, assert_attn_close, assert_topk_near, to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _stage(*a):
    print("[gpu-test]", *a, flush=True)


def build_cache(inp, w, B):
    """Device cache from the bf16 main rows via the write path kernel."""
    n_cap = w.n_cap
    cache = torch.empty((B, n_cap, 288), dtype=torch.uint8, device=DEV)
    cs = torch.from_numpy(C.csa2_rope_table(np.arange(n_cap, dtype=np.int64) * w.m)).to(DEV)
    for b in range(B):
        C.csa2_quantize_kv(inp["main"][b], cs, None, cache[b])
    return cache


def run_gpu(w, inp, B, write=None):
    cache = build_cache(inp, w, B)
    n_vis = visible_entries(inp["q_pos"], w.m).to(torch.int32)
    g = LayerGroup(w.kind, B, w.T, w.n_cap, keep_scores=True)
    g.step(inp["k_idx"], cache, n_vis, inp["q_pos"], inp["swa_pos0"], inp["q_idx"], inp["w"],
           inp["q"], inp["swa"], write=write)
    torch.cuda.synchronize()
    return g, cache


def check_group(w, inp, g, B, main_rows_np_override=None):
    """Compare every layer of every query with the oracle."""
    sched = OG.layer_schedule(w.kind)
    n_attn_checked = n_swaps = 0
    kn = to_np(inp["k_idx"])
    for b in range(B):
        oc = OracleCache(inp["main"][b], w.m)
        if main_rows_np_override is not None:
            oc.cache.update(main_rows_np_override(b))
        for t in range(w.T):
            tq = w.q_positions[t]
            nv = int(n_visible(tq, w.m))
            qi = {li: to_np(inp["q_idx"][li])[b, t] for li in inp["q_idx"]}
            wi = {li: to_np(inp["w"][li])[b, t] for li in inp["w"]}
            q = {li: inp["q"][li][b, t].float().cpu().numpy() for li in range(len(sched))}
            swa = {li: to_np(inp["swa"][li])[b] for li in range(len(sched))}
            o_idx, o_out, o_pool, o_scores = OG.run_group(sched, qi, wi, q, swa, kn[b], oc, nv, tq,
                                                          w.swa_pos0)
            pool_g = to_np(g.pool)[b, t] if g.pool is not None else None
            pool_diff = set()
            if pool_g is not None:
                bm = OI.block_max(o_scores[0], nv)
                a, o = set(pool_g[pool_g >= 0].tolist()), set(o_pool[o_pool >= 0].tolist())
                pool_diff = a ^ o
                if pool_diff:
                    kth = min(float(bm[x]) for x in o)
                    for x in pool_diff:
                        assert abs(float(bm[x]) - kth) <= NEAR_TIE * abs(kth), ("pool", b, t, x)
            for li, (mode, src) in enumerate(sched):
                gi = to_np(g.idx[li])[b, t]
                if mode == OG.FULL:
                    s = o_scores[li]
                    n_swaps += assert_topk_near(gi, o_idx[li], lambda p: s[p],
                                                what="F b%d t%d" % (b, t))
                elif mode == OG.REINDEX:
                    cand, s = o_scores[li]
                    full = OI.index_scores(qi[li], wi[li], kn[b], nv)   # all positions
                    n_swaps += assert_topk_near(
                        gi, o_idx[li], lambda p: full[p],
                        extra_allowed=lambda p: (p // 8) in pool_diff,
                        what="X%d b%d t%d" % (li, b, t))
                else:
                    assert gi.tobytes() == to_np(g.idx[src])[b, t].tobytes()
                if np.array_equal(gi, o_idx[li]):
                    assert_attn_close(to_np(g.out[li])[b, t], o_out[li], "L%d b%d t%d" % (li, b, t))
                    n_attn_checked += 1
    return n_attn_checked, n_swaps


def _inputs(w, B, seed=0):
    inp = make_inputs(w, DEV, seed=seed, keep_main_bf16=True, B=B)
    inp["main"] = [inp["main_bf16"][b].contiguous() for b in range(B)]
    return inp


def test_c0_full_decode_end_to_end():
    """The 8,192-token Full-mode decode workload at its full size."""
    w = WORKLOADS["c0"]
    _stage("c0 group", w)
    inp = _inputs(w, w.B)
    g, _ = run_gpu(w, inp, w.B)
    checked, swaps = check_group(w, inp, g, w.B)
    print("attention checked:", checked, "near-tie swaps:", swaps)
    assert checked >= w.B * w.T - swaps


def test_decoder_group_small_context():
    """[F, X, U, X, U, X, U] at 40,000 positions (5,000 blocks > 2,048 pooled)."""
    w = scaled(WORKLOADS["c2"], 40000, 40000, "c2_40k")
    B = 2
    _stage("decoder group", w)
    inp = _inputs(w, B, seed=3)
    g, _ = run_gpu(w, inp, B)
    checked, swaps = check_group(w, inp, g, B)
    print("attention checked:", checked, "near-tie swaps:", swaps)
    assert checked >= 7 * B - 2 * swaps
    # Reuse layers alias their source buffers; source indices never change
    snap = [to_np(x).copy() for x in g.idx]
    for li, (m, src) in enumerate(g.sched):
        if m == "U":
            assert snap[li].tobytes() == snap[src].tobytes()


def test_encoder_group_write_path_outliers():
    """[F, U x5] at m = 2 with the write path and 1% x8 outlier channels."""
    w = scaled(WORKLOADS["c4"], 24000, 12000, "c4_24k")
    B = 3
    _stage("encoder group", w)
    inp = _inputs(w, B, seed=4)
    n_cap = w.n_cap
    slot = torch.arange(B, dtype=torch.int64, device=DEV) * n_cap + (n_cap - 1)
    cs = torch.from_numpy(C.csa2_rope_table(np.full(B, (n_cap - 1) * w.m, dtype=np.int64))).to(DEV)
    write = (inp["write_bf16"], cs, slot)
    g, cache = run_gpu(w, inp, B, write=write)
    # the oracle sees the new row in the newest slot
    for b in range(B):
        inp["main"][b] = inp["main"][b].clone()
        inp["main"][b][n_cap - 1] = inp["write_bf16"][b]
    checked, swaps = check_group(w, inp, g, B)
    print("attention checked:", checked, "near-tie swaps:", swaps)
    assert checked >= 6 * B - 5 * swaps
    # the written rows are bit-exact
    oc = [OracleCache(inp["main"][b], w.m) for b in range(B)]
    got = to_np(cache)[:, n_cap - 1]
    for b in range(B):
        assert np.array_equal(got[b], oc[b][[n_cap - 1]][0])
