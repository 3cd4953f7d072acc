"""Comparison of a device layer-group step with the oracle, query by query.

  * Top-K sets are compared under the near-tie rule on the oracle's scores (a
    position may differ only where its oracle score is within 1e-5 relative of
    the oracle's 512-th score). The pool may differ only by near-ties of its
    2,048-th block maximum; where it does, a Reindex layer is compared with the
    oracle's Top-512 over the device pool's candidates. Reuse layers must hold
    their source's indices byte for byte.
  * Attention is compared in every layer of every checked query: against the
    oracle's output when the device picked the oracle's set, otherwise against
    the oracle's attention over the device's own set (the end-to-end rule).
  * Device scores, where the step keeps them, are compared with the oracle's
    exact scores at the positions that decide the selection (the oracle's best
    1,024 and the device's chosen ones) under the score bound, and the largest
    error (in units of 2^-24 * sum_h w_h sum_c |q_hc k_c| and relative to the
    512-th score) and the oracle's relative gap at the cutoff are recorded.
"""

import numpy as np

from compressed_kv_cache_02_amd import PREFILL_MIN_T_FP4, PREFILL_MIN_T_FP8
from oracle import attention as OA
from oracle import formats as OF
from oracle import group as OG
from oracle import indexer as OI
from oracle import mxfp4 as OM
from oracle import select as OS
from oracle.compress import n_visible
from tests.helpers import (NEAR_TIE, SCORE_GAMMA, assert_attn_close, assert_topk_near,
                           fp8_contraction_bound, to_np)

UNIT = 2.0 ** -24


class Stats:
    """Running maxima and minima over the checked queries."""

    def __init__(self):
        self.queries = 0
        self.attn = 0
        self.swaps = 0
        self.attn_own_set = 0
        self.score_pos = 0
        self.max_units = 0.0
        self.max_rel = 0.0
        self.min_gap = float("inf")
        self.attn_max_abs = 0.0
        self.attn_max_rel = 0.0
        self.fp8_pos = 0
        self.fp8_max_units = 0.0
        self.pool_swaps = 0

    def line(self):
        return ("queries %d, attention outputs %d (%d on the device's own set), near-tie swaps %d; "
                "scores at %d deciding positions: max error %.1f units = %.2e of the 512th score, "
                "smallest cutoff gap %.2e; attention max-abs %.2e, rel-L2 %.2e" % (
                    self.queries, self.attn, self.attn_own_set, self.swaps, self.score_pos,
                    self.max_units, self.max_rel, self.min_gap, self.attn_max_abs,
                    self.attn_max_rel) +
                ("; prefill-shaped score rows at %d positions: max error %.1f units" % (
                    self.fp8_pos, self.fp8_max_units) if self.fp8_pos else "") +
                ("; Reindex layers over a pool that differs by near-ties: %d" % self.pool_swaps
                 if self.pool_swaps else ""))


def _abs_keys(kn, ks, pos):
    if ks is None:
        return np.abs(OF.e4m3_decode(kn[pos]))
    return np.abs(OM.dequantize_index_keys(kn[pos], ks[pos]))


def _check_scores(st, qi, wi, kn, ks, o_scores_vis, o_set, gpu_pos, gpu_val, g_set, what,
                  fp8=False):
    """Bound check at the deciding positions (the float32 bound; with fp8, the
    FP8 contraction bound of a prefill-shaped scan's score rows); updates st."""
    nv = o_scores_vis.shape[0]
    if nv <= 512 or gpu_pos.size == 0:
        return
    order = np.argsort(-o_scores_vis.astype(np.float64), kind="stable")
    s512 = float(o_scores_vis[order[511]])
    s513 = float(o_scores_vis[order[512]])
    if s512 != 0.0:
        st.min_gap = min(st.min_gap, (s512 - s513) / abs(s512))
    want = set(order[:1024].tolist()) | set(int(x) for x in g_set)
    have = {int(p): i for i, p in enumerate(gpu_pos)}
    pos = np.array(sorted(p for p in want if p in have), dtype=np.int64)
    if pos.size == 0:
        return
    got = np.array([gpu_val[have[int(p)]] for p in pos], dtype=np.float64)
    ref = o_scores_vis[pos].astype(np.float64)
    q = np.abs(OF.e4m3_decode(qi.reshape(32, 128)))
    unit = UNIT * (_abs_keys(kn, ks, pos) @ q.T) @ np.abs(wi.astype(np.float64).reshape(32))
    err = np.abs(got - ref)
    if fp8:
        kv = (OF.e4m3_decode(kn[pos]) if ks is None
              else OM.dequantize_index_keys(kn[pos], ks[pos]))
        lim = fp8_contraction_bound(OF.e4m3_decode(qi.reshape(32, 128)), wi, kv)
        assert np.all(err <= lim), "%s: prefill-shaped score beyond the FP8 bound" % what
        st.fp8_pos += int(pos.size)
        st.fp8_max_units = max(st.fp8_max_units, float((err / np.maximum(unit, 1e-300)).max()))
        return
    assert np.all(err <= SCORE_GAMMA / UNIT * unit + 1e-30), \
        "%s: score error %.1f units > 160" % (what, float((err / np.maximum(unit, 1e-300)).max()))
    st.score_pos += int(pos.size)
    st.max_units = max(st.max_units, float((err / np.maximum(unit, 1e-300)).max()))
    if s512 != 0.0:
        st.max_rel = max(st.max_rel, float(err.max()) / abs(s512))


def check_queries(w, inp, g, samples, cache_of, log=print, stats=None):
    """Check the (b, t) query pairs in `samples`.

    w: the workload; inp: its device inputs; g: the LayerGroup after a step;
    cache_of(b): an object whose [sel] gives the oracle's packed rows of
    sequence b (and whose len() is the number of rows). With FP4 indexer keys
    (inp["k_bf16"]) the oracle quantises the bf16 keys itself. Returns the
    Stats of the checked queries."""
    st = stats if stats is not None else Stats()
    sched = OG.layer_schedule(w.kind)
    # full score rows written by a prefill-shaped scan (FP8 contraction), unless
    # the caller replaced them with decode-shaped ones (attribute rows_accurate)
    fp4 = inp.get("k_bf16") is not None
    fp8_rows = (w.T >= (PREFILL_MIN_T_FP4 if fp4 else PREFILL_MIN_T_FP8)
                and not getattr(g, "rows_accurate", False))
    idx_host = [to_np(x) for x in g.idx]
    out_host = {}
    pool_host = to_np(g.pool) if g.pool is not None else None
    last_x = max([li for li, (mode, _) in enumerate(sched) if mode == OG.REINDEX], default=-1)
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
            pg = None
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
                    st.swaps += assert_topk_near(gi, o_idx[li], lambda p: s[p], what=tag)
                    gp, gv, rows = _device_scores(g, li, b, t, pg, nv, full=True)
                    _check_scores(st, qi[li], wi[li], kn, ks, s[:nv], o_idx[li], gp, gv,
                                  gi[gi >= 0], tag, fp8=rows and fp8_rows)
                elif mode == OG.REINDEX:
                    full = {}

                    def score(p, li=li):
                        # oracle score of any visible position, computed only
                        # when the sets differ or scores are compared
                        if "s" not in full:
                            full["s"] = OI.index_scores(qi[li], wi[li], kn, nv, k_scales=ks)
                        return full["s"][p]

                    if pool_diff:
                        # the pools differ by near-ties: the reference is the
                        # oracle's Top-512 over the device pool's candidates
                        cand = OS.reindex_candidates(pg, nv)
                        sc = np.asarray(score(cand), dtype=np.float32)
                        ref_set = OS.topk_positions(sc, cand)
                        st.pool_swaps += 1
                    else:
                        ref_set = o_idx[li]
                    st.swaps += assert_topk_near(gi, ref_set, score, what=tag)
                    if li == last_x or li in getattr(g, "saved_scores", {}):
                        gp, gv, _ = _device_scores(g, li, b, t, pg, nv, full=False)
                        if gp.size and not pool_diff:
                            # the oracle's Reindex ranking is over its pool: the
                            # deciding positions are its pool candidates' best
                            cand, cs = o_scores[li]
                            s_pool = np.full(nv, -np.inf, dtype=np.float32)
                            s_pool[cand] = cs
                            _check_scores(st, qi[li], wi[li], kn, ks, s_pool, o_idx[li], gp, gv,
                                          gi[gi >= 0], tag)
                else:
                    assert gi.tobytes() == idx_host[src][b, t].tobytes(), tag
                if li not in out_host:
                    out_host[li] = g.out[li]
                got = out_host[li][b, t].cpu().numpy()
                if np.array_equal(gi, o_idx[li]):
                    ref = o_out[li]
                else:
                    ref = OA.sparse_attention(q[li], oc, gi, swa[li], tq, w.swa_pos0)
                    st.attn_own_set += 1
                mx, rl = assert_attn_close(got, ref, tag)
                st.attn += 1
                st.attn_max_abs = max(st.attn_max_abs, mx)
                st.attn_max_rel = max(st.attn_max_rel, rl)
            st.queries += 1
            log("checked b=%d t=%d (n_vis %d)" % (b, t, nv))
    return st


def _device_scores(g, li, b, t, pool_row, nv, full):
    """(positions, values, from full score rows) of the scores the device step
    kept for layer li."""
    saved = getattr(g, "saved_scores", {}).get(li)
    if full and saved is None and g.scores is not None:
        saved = g.scores
    if saved is None:
        saved = g.scores_full_pool if full else g.scores_pool
    if saved is None:
        return np.zeros(0, np.int64), np.zeros(0, np.float32), False
    row = to_np(saved[b, t])
    if row.shape[0] != 16384 or pool_row is None:
        pos = np.arange(min(nv, row.shape[0]), dtype=np.int64)
        return pos, row[:pos.shape[0]], True
    blocks = np.asarray(pool_row, dtype=np.int64)
    pos = (blocks[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    ok = (np.repeat(blocks, 8) >= 0) & (pos < nv)
    return pos[ok], row[ok], False
