"""Parity at the full workload sizes, in the launch configuration the benchmark
times: the write path, the scan, the pool, Top-K and attention of a whole
layer-group step captured as HIP graphs and replayed (twice: the step is
idempotent, and both replays must give the same bytes: indices, pool and
attention outputs).

  * queries are compared with the oracle one by one (rules of
    tests/group_check.py): every query of the decode workloads, 64 evenly
    spaced queries of the prefill chunk;
  * every query is checked for properties that hold at any size: Top-K and the
    pool are exact selections of the device's own scores and block maxima
    (ties to the lower position / block), ascending with -1 padding and
    min(K, visible) entries; block maxima equal the maxima of the scores; Reuse
    layers hold their source's indices; attention outputs are finite.

Workloads: Full decode, 32 x 65,536 entries; the decoder group at 1,048,576
positions, batch 8 (also with FP4 indexer keys, and with 16 or 5 query tokens
per sequence: the prefill-shaped scan with 16-query tiles and, at 128 queries,
the 8-tile Reindex scan); a Full prefill chunk of 4,096 queries over
131,072-133,120 entries; the encoder group with write path and outliers at
524,288 entries, batch 64."""

import dataclasses

import numpy as np
import pytest
import torch

import compressed_kv_cache_02_amd as C
from compressed_kv_cache_02_amd.group import LayerGroup, index_score, visible_entries
import synth
from synth.configs import WORKLOADS, make_inputs
from tests.group_check import check_queries
from tests.helpers import OracleCache

pytestmark = pytest.mark.gpu
DEV = "cuda"
K = C.TOPK


def _stage(*a):
    print("[gpu-fullsize]", *a, flush=True)


def setup(w, seed=0, write_path=True, index_k="fp8"):
    """Inputs, the packed cache built by the write-path kernel, and the
    per-step write (one new row per sequence into the newest slot). With FP4
    indexer keys, inp["keys"] is the device-quantised (codes, scales) pair."""
    inp = make_inputs(w, DEV, seed=seed, index_k=index_k)
    if index_k == "fp4":
        codes = torch.empty((w.B, w.n_cap, 64), dtype=torch.uint8, device=DEV)
        scales = torch.empty((w.B, w.n_cap, 4), dtype=torch.uint8, device=DEV)
        C.csa2_quantize_index_k(inp["k_bf16"].reshape(w.B * w.n_cap, 128), None, codes, scales)
        inp["keys"] = (codes, scales)
    else:
        inp["keys"] = inp["k_idx"]
    B, n_cap, m = w.B, w.n_cap, w.m
    cache = torch.empty((B, n_cap, 288), dtype=torch.uint8, device=DEV)
    cs_all = torch.from_numpy(C.csa2_rope_table(np.arange(n_cap, dtype=np.int64) * m)).to(DEV)
    for b in range(B):
        C.csa2_quantize_kv(inp["main_rows_per_seq"][b], cs_all, None, cache[b])
    inp["main_rows_per_seq"] = None
    del cs_all
    write = None
    if write_path:
        new_rows = inp.get("write_bf16")
        if new_rows is None:
            new_rows = synth.token_rows_bf16(B, DEV, seed, w.name, "write")
        inp["write_bf16"] = new_rows
        slot = torch.arange(B, dtype=torch.int64, device=DEV) * n_cap + (n_cap - 1)
        cs = torch.from_numpy(C.csa2_rope_table(np.full(B, (n_cap - 1) * m, dtype=np.int64))).to(DEV)
        write = (new_rows, cs, slot)
    torch.cuda.synchronize()
    return inp, cache, write


def run_graph_step(w, inp, cache, write, replays=2):
    n_vis = visible_entries(inp["q_pos"], w.m).to(torch.int32)
    g = LayerGroup(w.kind, w.B, w.T, w.n_cap, device=DEV)

    def step():
        g.step(inp["keys"], cache, n_vis, inp["q_pos"], inp["swa_pos0"], inp["q_idx"], inp["w"],
               inp["q"], inp["swa"], write=write)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    first = None
    for r in range(replays):
        graph.replay()
        torch.cuda.synchronize()
        snap = [t.clone() for t in g.idx + g.out] + ([g.pool.clone()] if g.pool is not None else [])
        if first is None:
            first = snap
        else:
            # determinism: every replay gives the same bytes (indices, pool, outputs)
            for a, b in zip(first, snap):
                assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float32 else a,
                                   b.view(torch.uint8) if b.dtype == torch.float32 else b), \
                    "replay %d differs from the first" % r
    return g, n_vis


def regen_cache(w, inp, seed):
    """cache_of(b) for the oracle: sequence b's bf16 rows regenerated from the
    same seeded streams, with the write-path row in the newest slot."""
    def cache_of(b):
        rows = synth.pooled_main_rows(w.n_cap, w.m, DEV, seed, w.name, "main", b,
                                      outliers=w.outliers)
        if inp.get("write_bf16") is not None:
            rows[w.n_cap - 1] = inp["write_bf16"][b]
        return OracleCache(rows, w.m)
    return cache_of


# ---------------------------------------------------------------- properties

def check_selection(idx, vals, n_items_vis, what, k=K):
    """idx [Q, k] ascending item ids (-1 padded) must be the exact top
    min(k, n_items_vis) of vals [Q, n] by (value desc, id asc).

    n_items_vis [Q]: number of leading valid items per query (or None for all
    finite values)."""
    Q, n = vals.shape
    valid = idx >= 0
    cnt = valid.sum(dim=1)
    want = torch.clamp(n_items_vis, max=k) if n_items_vis is not None else \
        torch.clamp(torch.isfinite(vals).sum(dim=1), max=k)
    assert torch.equal(cnt, want.to(cnt.dtype)), what + ": counts"
    # padding at the end, strictly ascending ids in front
    pos = torch.arange(k, device=idx.device).expand(Q, k)
    assert torch.equal(valid, pos < cnt[:, None]), what + ": padding"
    d = idx[:, 1:] - idx[:, :-1]
    assert bool(((d > 0) | ~valid[:, 1:]).all()), what + ": not ascending"
    assert bool((idx < n).all()), what + ": id out of range"
    safe = torch.where(valid, idx, torch.zeros_like(idx)).long()
    sel = torch.gather(vals, 1, safe)
    sel = torch.where(valid, sel, torch.full_like(sel, float("inf")))
    kth = sel.min(dim=1).values                                  # K-th value
    assert bool(torch.isfinite(kth[cnt > 0]).all()), what + ": selected -inf"
    # the largest selected id among those equal to the K-th value
    last_tie = torch.where(valid & (sel == kth[:, None]), idx, torch.full_like(idx, -1)).max(dim=1).values
    # padding entries go to a spare column n
    mask = torch.zeros((Q, n + 1), dtype=torch.bool, device=vals.device)
    mask.scatter_(1, torch.where(valid, safe, torch.full_like(safe, n)), True)
    rest = torch.where(mask[:, :n], torch.full_like(vals, -float("inf")), vals)
    assert bool((rest.max(dim=1).values <= kth).all()), what + ": a larger value was left out"
    ids = torch.arange(n, device=vals.device).expand(Q, n)
    tie_out = (rest == kth[:, None]) & (ids < last_tie[:, None].long())
    assert not bool(tie_out.any()), what + ": tie not resolved to the lower id"


def check_pool_topk(idx, sp, pool, nv, n_cap, what):
    """idx must be the exact Top-K of the pool candidates' scores sp (slot i is
    position 8 * pool[i // 8] + i % 8), written as ascending positions."""
    Q = idx.shape[0]
    pool = pool.long()
    cand = (pool[:, :, None] * 8 + torch.arange(8, device=DEV)).reshape(Q, -1)
    cand = torch.where((pool[:, :, None] >= 0).expand(-1, -1, 8).reshape(Q, -1), cand,
                       torch.full_like(cand, -1))
    ok = (cand >= 0) & (cand < nv[:, None])
    assert bool(torch.isneginf(sp[~ok]).all()), what + ": non-candidates must be -inf"
    # map selected positions back to candidate slots and check there
    slot_of = torch.full((Q, n_cap), -1, dtype=torch.long, device=DEV)
    q_ids = torch.arange(Q, device=DEV)[:, None].expand_as(cand)
    slot_of[q_ids[ok], cand[ok]] = torch.arange(cand.shape[1], device=DEV).expand_as(cand)[ok]
    v = idx >= 0
    sidx = torch.where(v, slot_of.gather(1, torch.where(v, idx, 0).long()), -1)
    assert bool((sidx[v] >= 0).all()), what + ": a position outside the pool"
    # candidate slots ascend with positions, so the plain check applies
    check_selection(sidx.to(torch.int32), sp, None, what)


def fused_scores(w, g, inp, n_vis):
    """A group with the fused Full Top-K writes neither score rows nor block
    maxima; recompute both with a decode-shaped FULL scan (the FP32-accurate
    scores the fused call selects on; one query token per call when the step
    has enough tokens for the prefill shape) to check its selection against."""
    li = [i for i, (mode, _) in enumerate(g.sched) if mode == "F"][0]
    scores = torch.empty((w.B, w.T, w.n_cap), dtype=torch.float32, device=DEV)
    fp4 = isinstance(inp["keys"], tuple)
    if w.T < (C.PREFILL_MIN_T_FP4 if fp4 else C.PREFILL_MIN_T_FP8):
        index_score(C.CSA2_FULL, inp["q_idx"][li], inp["w"][li], inp["keys"], n_vis, None, scores,
                    g.bmax)
    else:
        one_s = torch.empty((w.B, 1, w.n_cap), dtype=torch.float32, device=DEV)
        one_b = torch.empty((w.B, 1, g.bmax.shape[2]), dtype=torch.float32, device=DEV)
        for t in range(w.T):
            index_score(C.CSA2_FULL, inp["q_idx"][li][:, t:t + 1].contiguous(),
                        inp["w"][li][:, t:t + 1].contiguous(), inp["keys"],
                        n_vis[:, t:t + 1].clone(), None, one_s, one_b)
            scores[:, t] = one_s[:, 0]
            g.bmax[:, t] = one_b[:, 0]
    torch.cuda.synchronize()
    g.rows_accurate = True
    return scores


def check_properties(w, g, n_vis, inp=None):
    Q = w.B * w.T
    nv = n_vis.reshape(Q).long()
    n_blk = (w.n_cap + 7) // 8
    if g.fused:
        g.scores = fused_scores(w, g, inp, n_vis)
    bmax = g.bmax.reshape(Q, n_blk)
    nb = (nv + 7) // 8
    blk_vis = torch.arange(n_blk, device=DEV)[None, :] < nb[:, None]
    assert bool(torch.isneginf(bmax[~blk_vis]).all()), "invisible blocks must have -inf maxima"
    assert bool(torch.isfinite(bmax[blk_vis]).all()), "visible blocks must have finite maxima"
    if g.scores is not None:
        scores = g.scores.reshape(Q, w.n_cap)
        ids = torch.arange(w.n_cap, device=DEV)
        vis = ids[None, :] < nv[:, None]
        assert bool(torch.isneginf(scores[~vis]).all()), "invisible positions must score -inf"
        assert bool(torch.isfinite(scores[vis]).all()), "visible scores must be finite"
        pad = torch.full((Q, n_blk * 8), -float("inf"), device=DEV)
        pad[:, :w.n_cap] = scores
        assert torch.equal(bmax, pad.reshape(Q, n_blk, 8).max(dim=2).values), "block maxima"
    last_x = max([li for li, (mode, _) in enumerate(g.sched) if mode == "X"], default=-1)
    for li, (mode, src) in enumerate(g.sched):
        idx = g.idx[li].reshape(Q, K)
        if mode == "F" and g.scores is not None:
            check_selection(idx, g.scores.reshape(Q, w.n_cap), nv, "Full Top-K")
        elif mode == "F":
            # Full Top-K taken inside the pool from the re-scored candidates
            check_pool_topk(idx, g.scores_full_pool.reshape(Q, -1), g.pool.reshape(Q, -1), nv,
                            w.n_cap, "Full Top-K in the pool")
        elif mode == "X" and li == last_x:
            # (the Reindex layers share one score buffer: the last one's remains)
            check_pool_topk(idx, g.scores_pool.reshape(Q, -1), g.pool.reshape(Q, -1), nv,
                            w.n_cap, "Reindex Top-K")
        elif mode == "U":
            assert torch.equal(idx, g.idx[src].reshape(Q, K)), "Reuse differs from its source"
        assert bool(torch.isfinite(g.out[li]).all()), "attention output not finite (layer %d)" % li
    if g.pool is not None:
        check_selection(g.pool.reshape(Q, -1), bmax, nb, "pool", k=C.POOL_BLOCKS)


# ---------------------------------------------------------------- tests

def _cases(w, spec):
    """Queries compared with the oracle: every query of the decode workloads,
    64 evenly spaced queries (first and last included) of the prefill chunk, and
    for several query tokens per sequence the first and last token of every
    sequence plus one in between."""
    if w.T >= 64:
        ts = sorted(set(np.linspace(0, w.T - 1, 64).round().astype(int).tolist()))
        return [(0, t) for t in ts]
    if spec > 1:
        return sorted({(b, t) for b in range(w.B) for t in (0, w.T - 1)} | {(w.B - 1, w.T // 2)})
    return [(b, t) for b in range(w.B) for t in range(w.T)]


@pytest.mark.parametrize("name,index_k,spec", [("c1", "fp8", 1), ("c2", "fp8", 1), ("c3", "fp8", 1),
                                               ("c4", "fp8", 1), ("c2", "fp4", 1), ("c2", "fp8", 16),
                                               ("c2", "fp4", 5)])
def test_full_size_workload(name, index_k, spec):
    w = WORKLOADS[name]
    if spec > 1:
        # several query tokens per sequence (speculative decode), as bench.py --spec-tokens
        w = dataclasses.replace(w, T=spec, first_q=w.first_q - (spec - 1))
    cases = _cases(w, spec)
    seed = 0
    _stage(name, index_k, "T=%d" % w.T, "inputs")
    inp, cache, write = setup(w, seed, write_path=(w.kind != "full" or w.T == 1), index_k=index_k)
    _stage(name, "graph step")
    g, n_vis = run_graph_step(w, inp, cache, write)
    _stage(name, "properties of every query")
    check_properties(w, g, n_vis, inp)
    _stage(name, "oracle on %d queries" % len(cases))
    st = check_queries(w, inp, g, cases, regen_cache(w, inp, seed),
                       log=lambda s: _stage(name, s))
    _stage(name, index_k, "T=%d" % w.T, st.line())
    # every layer of every compared query had its attention checked
    assert st.queries == len(cases) and st.attn == len(cases) * w.n_layers
