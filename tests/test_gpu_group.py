"""End-to-end GPU parity of layer-group steps (the whole hot path) against the
oracle: Full / Reindex / Reuse layers, the pool, the write path, attention.

The comparison rules are those of tests/group_check.py."""

import numpy as np
import pytest
import torch

import compressed_kv_cache_02_amd as C
from compressed_kv_cache_02_amd.group import LayerGroup, visible_entries
from synth.configs import WORKLOADS, make_inputs, scaled
from tests.group_check import check_queries
from tests.helpers import OracleCache, to_np

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
    # score buffers are kept for the comparison with the oracle where the scan is
    # decode-shaped; a prefill-shaped step (c0's 4 tokens) takes the fused Top-K
    g = LayerGroup(w.kind, B, w.T, w.n_cap, keep_scores=w.T < C.PREFILL_MIN_T_FP8)
    g.step(inp["k_idx"], cache, n_vis, inp["q_pos"], inp["swa_pos0"], inp["q_idx"], inp["w"],
           inp["q"], inp["swa"], write=write)
    torch.cuda.synchronize()
    return g, cache


def check_group(w, inp, g, B):
    """Compare every query of every sequence with the oracle."""
    samples = [(b, t) for b in range(B) for t in range(w.T)]
    return check_queries(w, inp, g, samples, lambda b: OracleCache(inp["main"][b], w.m),
                         log=lambda *a: None)


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
    st = check_group(w, inp, g, w.B)
    print(st.line())
    assert st.attn == st.queries * len(g.sched) and st.queries == w.B * w.T


def test_decoder_group_small_context():
    """[F, X, U, X, U, X, U] at 40,000 positions (5,000 blocks > 2,048 pooled)."""
    w = scaled(WORKLOADS["c2"], 40000, 40000, "c2_40k")
    B = 2
    _stage("decoder group", w)
    inp = _inputs(w, B, seed=3)
    g, _ = run_gpu(w, inp, B)
    st = check_group(w, inp, g, B)
    print(st.line())
    assert st.attn == st.queries * len(g.sched) and st.queries == B * w.T
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
    st = check_group(w, inp, g, B)
    print(st.line())
    assert st.attn == st.queries * len(g.sched) and st.queries == B * w.T
    # the written rows are bit-exact
    oc = [OracleCache(inp["main"][b], w.m) for b in range(B)]
    got = to_np(cache)[:, n_cap - 1]
    for b in range(B):
        assert np.array_equal(got[b], oc[b][[n_cap - 1]][0])


def test_encoder_group_fused_topk():
    """[F, U x5] at m = 2 over 40,000 entries with the Full Top-K from the fused
    scan + Top-K entry point (no score rows), checked against the oracle."""
    w = scaled(WORKLOADS["c4"], 80000, 40000, "c4_80k_fused")
    B = 2
    _stage("encoder group fused", w)
    inp = _inputs(w, B, seed=6)
    cache = build_cache(inp, w, B)
    n_vis = visible_entries(inp["q_pos"], w.m).to(torch.int32)
    g = LayerGroup(w.kind, B, w.T, w.n_cap, fused_topk=True)
    assert g.fused and g.scores is None
    g.step(inp["k_idx"], cache, n_vis, inp["q_pos"], inp["swa_pos0"], inp["q_idx"], inp["w"],
           inp["q"], inp["swa"])
    torch.cuda.synchronize()
    st = check_group(w, inp, g, B)
    print(st.line())
    assert st.attn == st.queries * len(g.sched) and st.queries == B * w.T
