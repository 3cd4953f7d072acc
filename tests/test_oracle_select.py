"""Pins for the oracle's indexer scores, Top-K, pool and Reindex candidates
(CPU only): exact brute force, closed forms, hand-ranked fixtures and the
pool-contains-Top-K invariant."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as Fm
from oracle import indexer as I
from oracle import select as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _e4m3_code_of(v):
    for c in range(256):
        x = Fm.e4m3_value_of_code(c)
        if x == v and (np.signbit(x) == np.signbit(v)):
            return c
    raise ValueError(v)


def test_scores_vs_exact_brute_force():
    """Integer-valued E4M3 q, k and dyadic w: every quantity is exact, so the
    oracle must equal a pure-Python rational evaluation exactly."""
    rng = np.random.default_rng(0)
    vals = [-4.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0]
    codes = {v: _e4m3_code_of(v) for v in vals}
    q = rng.choice(vals, (32, 128))
    k = rng.choice(vals, (20, 128))
    w = (rng.integers(0, 64, 32) / 64.0).astype(np.float32)
    qc = np.vectorize(codes.get)(q).astype(np.uint8)
    kc = np.vectorize(codes.get)(k).astype(np.uint8)
    got = I.index_scores(qc, w, kc, n_vis=17)
    for n in range(20):
        if n >= 17:
            assert got[n] == -np.inf
            continue
        tot = Fraction(0)
        for h in range(32):
            d = sum(Fraction(q[h, c]) * Fraction(k[n, c]) for c in range(128))
            tot += Fraction(float(w[h])) * max(d, Fraction(0))
        assert Fraction(float(got[n])) == tot


def test_dot_products_exact_at_extremes():
    """E4M3 extremes (448 and 2^-9) in one dot product stay exact in float64."""
    q = np.zeros((32, 128), dtype=np.uint8)
    k = np.zeros((1, 128), dtype=np.uint8)
    q[:, :64] = 0x7E          # 448
    q[:, 64:] = 0x01          # 2^-9
    k[0, :] = 0x7E
    k[0, 127] = 0x01
    w = np.zeros(32, dtype=np.float32)
    w[0] = 1.0
    s = I.index_scores(q, w, k, n_vis=1)
    exact = 64 * 448 * 448 + 63 * 2.0 ** -9 * 448 + 2.0 ** -18
    assert float(s[0]) == float(np.float32(exact))


def test_closed_form_unit_vectors_and_relu():
    one, mone = _e4m3_code_of(1.0), _e4m3_code_of(-1.0)
    q = np.zeros((32, 128), dtype=np.uint8)
    q[:, 5] = one
    k = np.zeros((3, 128), dtype=np.uint8)
    k[0, 5] = one          # d_h = 1 for all h -> score = sum(w)
    k[1, 5] = mone         # d_h = -1 -> ReLU -> 0
    k[2, 6] = one          # orthogonal -> 0
    w = np.linspace(0.0, 1.0, 32).astype(np.float32)
    s = I.index_scores(q, w, k, n_vis=3)
    assert float(s[0]) == float(np.float32(np.sum(w.astype(np.float64))))
    assert s[1] == 0.0 and s[2] == 0.0


def test_block_max():
    with open(os.path.join(GOLD, "topk_worked.json")) as f:
        case = json.load(f)["pool_case"]
    s = np.array(case["scores"], dtype=np.float32)
    assert I.block_max(s, case["n_vis"]).tolist() == case["block_max"]


# ------------------------------------------------------------------ top-k -----

def test_topk_worked_examples():
    with open(os.path.join(GOLD, "topk_worked.json")) as f:
        g = json.load(f)
    for c in g["topk"]:
        sc = np.array(c["scores"], dtype=np.float32)
        got = S.topk_positions(sc, np.arange(sc.shape[0]), k=c["k"])
        assert got.tolist() == c["expect"]
    pc = g["pool_case"]
    s = np.array(pc["scores"], dtype=np.float32)
    bm = I.block_max(s, pc["n_vis"])
    for n in (2, 3, 8):
        assert S.build_pool(bm, pc["n_vis"], n_blocks=n).tolist() == pc["pool_%d" % n]
    nv = pc["n_vis"]
    for k in (3, 4):
        assert S.topk_positions(s[:nv], np.arange(nv), k=k).tolist() == pc["topk_%d" % k]


@pytest.mark.parametrize("seed", range(20))
def test_topk_vs_python_sorted(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    k = int(rng.integers(1, 20))
    sc = rng.integers(0, 5, n).astype(np.float32)          # tie-heavy
    pos = np.sort(rng.choice(1000, n, replace=False))
    ranked = sorted(range(n), key=lambda i: (-float(sc[i]), int(pos[i])))
    want = sorted(int(pos[i]) for i in ranked[:k])
    got = S.topk_positions(sc, pos, k=k)
    assert got[:len(want)].tolist() == want
    assert np.all(got[len(want):] == -1)
    assert len(want) == min(k, n)


def _brute_pool(scores, n_vis, n_blocks):
    nb = -(-n_vis // 8)
    bm = []
    for b in range(nb):
        vals = [float(scores[p]) for p in range(8 * b, min(8 * b + 8, n_vis))]
        bm.append(max(vals))
    ranked = sorted(range(nb), key=lambda b: (-bm[b], b))
    keep = sorted(ranked[:n_blocks])
    return keep + [-1] * (n_blocks - len(keep))


@pytest.mark.parametrize("seed", range(300))
def test_pool_brute_force_and_contains_topk(seed):
    """Pool equals brute force; and the Full Top-K always lies inside the pool
    when the pool has at least K blocks (each block ranked ahead of a Top-K
    position's block holds a distinct position ranked ahead of it)."""
    rng = np.random.default_rng(1000 + seed)
    n_cap = int(rng.integers(1, 120))
    n_vis = int(rng.integers(1, n_cap + 1))
    k = int(rng.integers(1, 9))
    n_blocks = int(rng.integers(k, k + 5))
    sc = rng.integers(0, 4, n_cap).astype(np.float32)
    sc[n_vis:] = 1000.0                                      # invisible poison
    masked = sc.copy()
    masked[n_vis:] = -np.inf
    pool = S.build_pool(I.block_max(masked, n_vis), n_vis, n_blocks=n_blocks)
    assert pool.tolist() == _brute_pool(sc, n_vis, n_blocks)
    top = S.topk_positions(sc[:n_vis], np.arange(n_vis), k=k)
    blocks = set(int(b) for b in pool if b >= 0)
    assert all(int(p) // 8 in blocks for p in top if p >= 0)
    # Reindex over the pool with the same scores reproduces the Full Top-K
    cand = S.reindex_candidates(pool, n_vis)
    assert S.topk_positions(sc[cand], cand, k=k).tolist() == top.tolist()


def test_small_context_pool_is_every_block():
    sc = np.arange(100, dtype=np.float32)
    pool = S.build_pool(I.block_max(sc, 100), 100)
    assert pool[:13].tolist() == list(range(13)) and np.all(pool[13:] == -1)
    assert S.POOL_BLOCKS * S.BLOCK == 16384 and S.TOPK == 512


def test_reindex_candidates_respect_visibility():
    pool = np.array([0, 2, 5, -1], dtype=np.int32)
    assert S.reindex_candidates(pool, 43).tolist() == list(range(8)) + list(range(16, 24)) + list(range(40, 43))


@pytest.mark.parametrize("seed", range(300))
def test_two_level_containment(seed):
    """The reading behind the device's hierarchical selection, pinned by brute
    force on tie-heavy inputs: with ties to the lower index at every level, the
    k best positions lie in the k best blocks of 8, and the k best blocks lie
    in the k best super-blocks of 8 blocks; so selecting inside those children
    reproduces the plain selection exactly."""
    rng = np.random.default_rng(5000 + seed)
    n_cap = int(rng.integers(1, 900))
    n_vis = int(rng.integers(1, n_cap + 1))
    k = int(rng.integers(1, 12))
    sc = rng.integers(0, 3, n_cap).astype(np.float32)
    masked = sc.copy()
    masked[n_vis:] = -np.inf
    top = S.topk_positions(sc[:n_vis], np.arange(n_vis), k=k)
    bm = I.block_max(masked, n_vis)
    n_blk = -(-n_vis // 8)
    best_blk = S.topk_positions(bm[:n_blk], np.arange(n_blk), k=k)
    # super-block maxima over blocks (a block max is -inf when invisible)
    n_sb = -(-n_blk // 8)
    pad = np.full(n_sb * 8, -np.inf, dtype=np.float32)
    pad[:n_blk] = bm[:n_blk]
    sm = pad.reshape(n_sb, 8).max(axis=1)
    best_sb = S.topk_positions(sm, np.arange(n_sb), k=k)
    assert set(int(p) // 8 for p in top if p >= 0) <= set(int(b) for b in best_blk if b >= 0)
    assert set(int(b) // 8 for b in best_blk if b >= 0) <= set(int(s) for s in best_sb if s >= 0)
    # selecting inside the children of the chosen parents gives the same result
    child_blk = np.array([8 * s + r for s in best_sb if s >= 0 for r in range(8)
                          if 8 * s + r < n_blk], dtype=np.int64)
    assert S.topk_positions(bm[child_blk], child_blk, k=k).tolist() == best_blk.tolist()
    child_pos = np.array([8 * b + r for b in best_blk if b >= 0 for r in range(8)
                          if 8 * b + r < n_vis], dtype=np.int64)
    assert S.topk_positions(sc[child_pos], child_pos, k=k).tolist() == top.tolist()
