"""Comparison of a device layer-group step with the oracle, query by query.

Top-K sets are compared under the near-tie rule on the oracle's scores (a
position may differ only where its oracle score is within 1e-5 relative of the
oracle's 512-th score; for Reindex layers also where the pool itself differed
by a near-tie); attention outputs are compared for every query whose index set
equals the oracle's. Reuse layers must hold their source's indices byte for
byte."""

import numpy as np

from oracle import group as OG
from oracle import indexer as OI
from oracle import mxfp4 as OM
from oracle.compress import n_visible
from tests.helpers import NEAR_TIE, assert_attn_close, assert_topk_near, to_np


def check_queries(w, inp, g, samples, cache_of, log=print):
    """Check the (b, t) query pairs in `samples`.

    w: the workload; inp: its device inputs; g: the LayerGroup after a step;
    cache_of(b): an object whose [sel] gives the oracle's packed rows of
    sequence b. With FP4 indexer keys (inp["k_bf16"]) the oracle quantises the
    bf16 keys itself. Returns (attention outputs checked, near-tie swaps)."""
    sched = OG.layer_schedule(w.kind)
    n_checked = n_swaps = 0
    idx_host = [to_np(x) for x in g.idx]
    out_host = {}
    pool_host = to_np(g.pool) if g.pool is not None else None
    by_seq = {}
    for b, t in samples:
        by_seq.setdefault(b, []).append(t)
    for b, ts in sorted(by_seq.items()):
        if inp.get("k_bf16") is not None:
            kn, ks = OM.quantize_index_keys(inp["k_bf16"][b].float().cpu().numpy())
        else:
            kn, ks = to_np(inp["k_idx"][b]), None
        oc = cache_of(b)
        for t in ts:
            tq = w.q_positions[t]
            nv = int(n_visible(tq, w.m))
            qi = {li: to_np(inp["q_idx"][li][b, t]) for li in inp["q_idx"]}
            wi = {li: to_np(inp["w"][li][b, t]) for li in inp["w"]}
            q = {li: inp["q"][li][b, t].float().cpu().numpy() for li in range(len(sched))}
            swa = {li: to_np(inp["swa"][li][b]) for li in range(len(sched))}
            o_idx, o_out, o_pool, o_scores = OG.run_group(sched, qi, wi, q, swa, kn, oc, nv, tq,
                                                          w.swa_pos0, k_scales=ks)
            pool_diff = set()
            if pool_host is not None:
                pg = pool_host[b, t]
                bm = OI.block_max(o_scores[0], nv)
                a, o = set(pg[pg >= 0].tolist()), set(o_pool[o_pool >= 0].tolist())
                assert list(pg) == sorted(a) + [-1] * int((pg < 0).sum()), ("pool order", b, t)
                pool_diff = a ^ o
                if pool_diff:
                    kth = min(float(bm[x]) for x in o)
                    for x in pool_diff:
                        assert abs(float(bm[x]) - kth) <= NEAR_TIE * abs(kth), ("pool", b, t, x)
            for li, (mode, src) in enumerate(sched):
                gi = idx_host[li][b, t]
                tag = "%s%d b%d t%d" % (mode, li, b, t)
                if mode == OG.FULL:
                    s = o_scores[li]
                    n_swaps += assert_topk_near(gi, o_idx[li], lambda p: s[p], what=tag)
                elif mode == OG.REINDEX:
                    full = {}

                    def score(p, li=li):
                        # oracle score of any visible position, computed only
                        # when the sets differ
                        if "s" not in full:
                            full["s"] = OI.index_scores(qi[li], wi[li], kn, nv, k_scales=ks)
                        return full["s"][p]

                    n_swaps += assert_topk_near(gi, o_idx[li], score,
                                                extra_allowed=lambda p: (p // 8) in pool_diff,
                                                what=tag)
                else:
                    assert gi.tobytes() == idx_host[src][b, t].tobytes(), tag
                if np.array_equal(gi, o_idx[li]):
                    if li not in out_host:
                        out_host[li] = g.out[li]
                    got = out_host[li][b, t].cpu().numpy()
                    assert_attn_close(got, o_out[li], tag)
                    n_checked += 1
            log("checked b=%d t=%d (n_vis %d)" % (b, t, nv))
    return n_checked, n_swaps
