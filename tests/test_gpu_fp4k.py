"""GPU parity of the FP4 indexer-key path (E2M1 codes + one E8M0 scale per 32
channels) against the oracle, through the C ABI: the key quantiser bit for bit,
FULL and REINDEX scores within the score bound, block maxima and re-scoring bit
for bit, and a decoder layer group end to end. The oracle quantises the bf16
keys itself; nothing it is given comes from the HIP path."""

import numpy as np
import pytest
import torch

import compressed_kv_cache_02_amd as C
from compressed_kv_cache_02_amd.group import LayerGroup, visible_entries
from oracle import indexer as OI
from oracle import mxfp4 as OM
from oracle import select as OS
from oracle import formats as OF
import synth
from synth.configs import WORKLOADS, make_inputs, scaled
from tests.group_check import check_queries
from tests.helpers import SCORE_GAMMA, OracleCache, assert_scores_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _stage(*a):
    print("[gpu-test]", *a, flush=True)


def _special_keys():
    """bf16-representable edge rows: zero and -0 blocks, exact E2M1 midpoints and
    saturation relative to each block's scale, subnormal and huge maxima."""
    rows = np.zeros((10, 128), dtype=np.float32)
    rows[1, :] = -0.0
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 7.5, 0.5, 3.0], np.float32)
    rng = np.random.default_rng(9)
    for r in range(2, 6):
        for b in range(4):
            e = int(rng.integers(-20, 20))
            v = rng.choice(mids, 32) * rng.choice([-1, 1], 32)
            v[0] = 4.0                       # amax in [4, 8): scale 2^e exactly
            rows[r, 32 * b:32 * b + 32] = v * np.float32(2.0 ** e)
    rows[6, :32] = np.float32(2.0 ** -127)   # subnormal maxima: scale code 0
    rows[6, 32:64] = np.float32(2.0 ** -133)
    rows[6, 64] = np.float32(2.0 ** -126)    # smallest normal: exponent field 1 -> code 0
    rows[6, 96] = np.float32(2.0 ** -124)    # exponent field 3 -> code 1
    rows[7, :] = np.float32(1.5 * 2.0 ** 127)     # the largest exponent field (254)
    rows[7, ::5] = np.float32(-(2.0 ** 126))
    rows[8, 5] = np.float32(1.0)             # one nonzero channel per block
    rows[8, 40] = np.float32(-448.0)
    rows[8, 70] = np.float32(2.0 ** -10)
    rows[8, 127] = np.float32(6.0)
    rows[9] = torch.from_numpy(rng.standard_normal(128).astype(np.float32) * 8.0).to(
        torch.bfloat16).float().numpy()
    t = torch.from_numpy(rows).to(torch.bfloat16)
    assert torch.equal(t.float(), torch.from_numpy(rows)), "edge rows must be bf16 values"
    return t


@pytest.mark.parametrize("n,outliers", [(5003, False), (2048, True)])
def test_quantize_index_k_bitexact(n, outliers):
    _stage("quantize_index_k", n, outliers)
    k = synth.normal_rows(n, 128, DEV, 21, "kq", outliers=outliers).to(torch.bfloat16)
    k = torch.cat([k, _special_keys().to(DEV)]).contiguous()
    n = k.shape[0]
    codes = torch.empty((n, 64), dtype=torch.uint8, device=DEV)
    scales = torch.empty((n, 4), dtype=torch.uint8, device=DEV)
    C.csa2_quantize_index_k(k, None, codes, scales)
    torch.cuda.synchronize()
    rc, rs = OM.quantize_index_keys(k.float().cpu().numpy())
    assert np.array_equal(to_np(codes), rc)
    assert np.array_equal(to_np(scales), rs)


def test_quantize_index_k_slots():
    """Rows go to their slots; slots outside the buffers are skipped."""
    _stage("quantize_index_k slots")
    n, rows = 40, 64
    k = synth.normal_rows(n, 128, DEV, 22, "ks").to(torch.bfloat16)
    slot = torch.arange(n, dtype=torch.int64, device=DEV).flip(0) * 3 % rows
    slot[5] = -1
    slot[6] = rows
    codes = torch.full((rows, 64), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((rows, 4), 0xCD, dtype=torch.uint8, device=DEV)
    C.csa2_quantize_index_k(k, slot, codes, scales)
    torch.cuda.synchronize()
    rc, rs = OM.quantize_index_keys(k.float().cpu().numpy())
    wc = np.full((rows, 64), 0xAB, np.uint8)
    ws = np.full((rows, 4), 0xCD, np.uint8)
    for i, s in enumerate(to_np(slot)):
        if 0 <= s < rows:
            wc[s], ws[s] = rc[i], rs[i]
    assert np.array_equal(to_np(codes), wc) and np.array_equal(to_np(scales), ws)


def _inputs(B, T, n_cap, seed, outliers=False):
    q = synth.e4m3_rows(B * T * 32, 128, DEV, seed, "q", outliers=outliers).view(B, T, 32, 128)
    w = synth.head_weights(B * T, DEV, seed, "w").view(B, T, 32)
    kb = synth.normal_rows(B * n_cap, 128, DEV, seed, "k4", outliers=outliers).to(torch.bfloat16)
    codes = torch.empty((B, n_cap, 64), dtype=torch.uint8, device=DEV)
    scales = torch.empty((B, n_cap, 4), dtype=torch.uint8, device=DEV)
    C.csa2_quantize_index_k(kb, None, codes, scales)
    oc, os_ = OM.quantize_index_keys(kb.float().cpu().numpy())
    return q, w, codes, scales, oc.reshape(B, n_cap, 64), os_.reshape(B, n_cap, 4)


def _bound(q_codes, w, kc, ks):
    q = np.abs(OF.e4m3_decode(q_codes.reshape(32, 128)))
    k = np.abs(OM.dequantize_index_keys(kc, ks))
    return SCORE_GAMMA * (k @ q.T) @ np.abs(np.asarray(w, dtype=np.float64).reshape(32))


@pytest.mark.parametrize("B,T,n_cap", [(2, 3, 5003), (1, 1, 31), (3, 2, 40000)])
def test_index_score_fp4k_full(B, T, n_cap):
    _stage("index_score_fp4k full", B, T, n_cap)
    q, w, codes, scales, oc, os_ = _inputs(B, T, n_cap, n_cap, outliers=(n_cap == 40000))
    assert np.array_equal(to_np(codes), oc) and np.array_equal(to_np(scales), os_)
    rng = np.random.default_rng(n_cap)
    nv = rng.integers(0, n_cap + 1, (B, T)).astype(np.int32)
    nv.flat[0] = n_cap
    if nv.size > 2:
        nv.flat[1] = 0
        nv.flat[2] = min(n_cap, 33)
    n_vis = torch.from_numpy(nv).to(DEV)
    scores = torch.empty((B, T, n_cap), dtype=torch.float32, device=DEV)
    bmax = torch.empty((B, T, (n_cap + 7) // 8), dtype=torch.float32, device=DEV)
    C.csa2_index_score_fp4k(C.CSA2_FULL, q, w, codes, scales, n_vis, None, scores, bmax)
    torch.cuda.synchronize()
    qn, wn, sn, bn = to_np(q), to_np(w), to_np(scores), to_np(bmax)
    for b in range(B):
        for t in range(T):
            ref = OI.index_scores(qn[b, t], wn[b, t], oc[b], nv[b, t], k_scales=os_[b])
            assert_scores_close(sn[b, t], ref, _bound(qn[b, t], wn[b, t], oc[b], os_[b]),
                                "b%d t%d" % (b, t))
            assert np.array_equal(bn[b, t], OI.block_max(sn[b, t], nv[b, t]))


def test_fp4k_block_maxima_only_and_rescoring():
    """Block maxima alone equal those of the full scan, and REINDEX over a pool
    re-scores each position to the FULL scan's bits."""
    B, T, n_cap = 2, 3, 40003
    _stage("fp4k bmax-only + rescoring", B, T, n_cap)
    q, w, codes, scales, _, _ = _inputs(B, T, n_cap, 13)
    rng = np.random.default_rng(13)
    nv = rng.integers(n_cap // 2, n_cap + 1, (B, T)).astype(np.int32)
    nv.flat[0] = n_cap
    n_vis = torch.from_numpy(nv).to(DEV)
    nb = (n_cap + 7) // 8
    scores = torch.empty((B, T, n_cap), dtype=torch.float32, device=DEV)
    bmax = torch.empty((B, T, nb), dtype=torch.float32, device=DEV)
    bmax2 = torch.full_like(bmax, 7.0)
    C.csa2_index_score_fp4k(C.CSA2_FULL, q, w, codes, scales, n_vis, None, scores, bmax)
    C.csa2_index_score_fp4k(C.CSA2_FULL, q, w, codes, scales, n_vis, None, None, bmax2)
    pool = torch.empty((B, T, 2048), dtype=torch.int32, device=DEV)
    ws = torch.empty(C.csa2_workspace_bytes(C.CSA2_OP_BUILD_POOL, 0, B, T, n_cap),
                     dtype=torch.uint8, device=DEV)
    C.csa2_build_pool(bmax2, True, n_vis, n_cap, pool, ws)
    sp = torch.empty((B, T, 16384), dtype=torch.float32, device=DEV)
    C.csa2_index_score_fp4k(C.CSA2_REINDEX, q, w, codes, scales, n_vis, pool, sp, None)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(bmax).view(np.uint32), to_np(bmax2).view(np.uint32))
    sn, spn, pn = to_np(scores), to_np(sp), to_np(pool)
    for b in range(B):
        for t in range(T):
            p = pn[b, t]
            pos_all = (np.maximum(p, 0)[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
            valid = np.repeat(p >= 0, 8) & (pos_all < nv[b, t])
            assert np.array_equal(pos_all[valid], OS.reindex_candidates(p, nv[b, t]))
            assert np.array_equal(spn[b, t][valid].view(np.uint32),
                                  sn[b, t][pos_all[valid]].view(np.uint32))
            assert np.all(np.isneginf(spn[b, t][~valid]))


def test_index_score_fp4k_reindex_vs_oracle():
    _stage("index_score_fp4k reindex")
    B, T, n_cap = 2, 2, 30000
    q, w, codes, scales, oc, os_ = _inputs(B, T, n_cap, 17)
    rng = np.random.default_rng(17)
    nb = (n_cap + 7) // 8
    pool = np.full((B, T, 2048), -1, dtype=np.int32)
    nv = np.array([[n_cap, 20001], [17, 29999]], dtype=np.int32)
    for b in range(B):
        for t in range(T):
            cnt = 2048 if (b, t) != (1, 0) else 3
            pool[b, t, :cnt] = np.sort(rng.choice(nb, cnt, replace=False))
    sp = torch.empty((B, T, 16384), dtype=torch.float32, device=DEV)
    C.csa2_index_score_fp4k(C.CSA2_REINDEX, q, w, codes, scales, torch.from_numpy(nv).to(DEV),
                            torch.from_numpy(pool).to(DEV), sp, None)
    torch.cuda.synchronize()
    qn, wn, sn = to_np(q), to_np(w), to_np(sp)
    for b in range(B):
        for t in range(T):
            p = pool[b, t]
            pos = (np.maximum(p, 0)[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
            ref = OI.index_scores(qn[b, t], wn[b, t], oc[b], nv[b, t], positions=pos,
                                  k_scales=os_[b])
            ref[np.repeat(p < 0, 8)] = -np.inf
            posc = np.minimum(pos, n_cap - 1)
            bound = _bound(qn[b, t], wn[b, t], oc[b][posc], os_[b][posc])
            assert_scores_close(sn[b, t], ref, bound, "reindex b%d t%d" % (b, t))


def test_decoder_group_fp4_keys():
    """[F, X, U, X, U, X, U] at 40,000 positions with FP4 indexer keys."""
    w = scaled(WORKLOADS["c2"], 40000, 40000, "c2_40k_fp4k")
    B = 2
    _stage("decoder group fp4 keys", w)
    inp = make_inputs(w, DEV, seed=5, keep_main_bf16=True, B=B, index_k="fp4")
    inp["main"] = [inp["main_bf16"][b].contiguous() for b in range(B)]
    n_cap = w.n_cap
    codes = torch.empty((B, n_cap, 64), dtype=torch.uint8, device=DEV)
    scales = torch.empty((B, n_cap, 4), dtype=torch.uint8, device=DEV)
    C.csa2_quantize_index_k(inp["k_bf16"].reshape(B * n_cap, 128), None, codes, scales)
    cache = torch.empty((B, n_cap, 288), dtype=torch.uint8, device=DEV)
    cs = torch.from_numpy(C.csa2_rope_table(np.arange(n_cap, dtype=np.int64) * w.m)).to(DEV)
    for b in range(B):
        C.csa2_quantize_kv(inp["main"][b], cs, None, cache[b])
    n_vis = visible_entries(inp["q_pos"], w.m).to(torch.int32)
    g = LayerGroup(w.kind, B, w.T, w.n_cap, keep_scores=True)
    g.step((codes, scales), cache, n_vis, inp["q_pos"], inp["swa_pos0"], inp["q_idx"], inp["w"],
           inp["q"], inp["swa"])
    torch.cuda.synchronize()
    samples = [(b, t) for b in range(B) for t in range(w.T)]
    checked = check_queries(w, inp, g, samples, lambda b: OracleCache(inp["main"][b], w.m),
                            log=lambda *a: None)
    print(checked.line())
    assert checked.attn == checked.queries * 7 and checked.queries == len(samples)


@pytest.mark.parametrize("B,T,n_cap", [(2, 77, 10003), (1, 64, 4096), (1, 130, 300), (1, 32, 8448),
                                         (2, 20, 12800)])
def test_index_score_fp4k_prefill_shape(B, T, n_cap):
    """From 5 queries per sequence the FP4-key scan is the prefill-shaped
    contraction (key chunks shared through LDS, the scaled FP8 x FP4 MFMA): its
    scores lie within the FP8 contraction bound of the oracle and its block
    maxima are the maxima of its own scores; the same queries scored one at a
    time by the decode-shaped kernel lie within the float32 bound. T and n_cap
    are ragged, or whole 256-key chunks."""
    from oracle import formats as OF
    from oracle import mxfp4 as OM
    from tests.helpers import fp8_contraction_bound
    _stage("index_score_fp4k prefill", B, T, n_cap)
    q, w, codes, scales, oc, os_ = _inputs(B, T, n_cap, 31 + n_cap)
    rng = np.random.default_rng(T)
    nv = np.minimum(n_cap, (np.arange(T) + n_cap - T + 1)[None, :].repeat(B, 0)).astype(np.int32)
    nv[0, 0] = 0
    nv[0, 1] = 1
    nv[-1, 2] = 33
    nv[-1, -1] = n_cap
    nv[0, 3:8] = rng.integers(0, n_cap + 1, 5)
    n_vis = torch.from_numpy(nv).to(DEV)
    nb = (n_cap + 7) // 8
    scores = torch.empty((B, T, n_cap), dtype=torch.float32, device=DEV)
    bmax = torch.empty((B, T, nb), dtype=torch.float32, device=DEV)
    C.csa2_index_score_fp4k(C.CSA2_FULL, q, w, codes, scales, n_vis, None, scores, bmax)
    torch.cuda.synchronize()
    one_s = torch.empty((1, 1, n_cap), dtype=torch.float32, device=DEV)
    one_b = torch.empty((1, 1, nb), dtype=torch.float32, device=DEV)
    sn, bn, qn, wn = to_np(scores), to_np(bmax), to_np(q), to_np(w)
    for b in range(B):
        for t in range(T):
            assert np.array_equal(bn[b, t], OI.block_max(sn[b, t], nv[b, t])), (b, t)
    for b in range(B):
        kv = OM.dequantize_index_keys(oc[b], os_[b])
        for t in sorted({0, 1, 2, T // 2, T - 1}):
            ref = OI.index_scores(qn[b, t], wn[b, t], oc[b], nv[b, t], k_scales=os_[b])
            qv = OF.e4m3_decode(qn[b, t].reshape(32, 128))
            assert_scores_close(sn[b, t], ref, fp8_contraction_bound(qv, wn[b, t], kv),
                                "prefill-shaped b%d t%d" % (b, t))
            C.csa2_index_score_fp4k(C.CSA2_FULL, q[b:b + 1, t:t + 1], w[b:b + 1, t:t + 1],
                                    codes[b:b + 1], scales[b:b + 1], n_vis[b:b + 1, t:t + 1].clone(),
                                    None, one_s, one_b)
            torch.cuda.synchronize()
            assert_scores_close(to_np(one_s)[0, 0], ref, _bound(qn[b, t], wn[b, t], oc[b], os_[b]),
                                "decode-shaped b%d t%d" % (b, t))