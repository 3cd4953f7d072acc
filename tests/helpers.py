"""Shared test helpers: acceptance rules and host copies of device inputs.

The acceptance rules follow the tolerances stated for this path:
  * FP4 packing, the pool and Top-K on identical float32 scores: bit-exact;
  * scores of the decode-shaped scan (every Top-K and pool decision):
    |gpu - oracle| <= 160 * 2^-24 * sum_h w_h sum_c |q_hc k_c| (Higham's
    gamma_n for the 128 + 32 float32 additions); scores of the prefill-shaped
    FP8 contraction: fp8_contraction_bound;
  * Top-K end to end: the sets agree except for positions whose oracle score is
    within 1e-5 (relative) of the oracle's K-th score;
  * attention: max-abs <= 2e-3 and relative L2 <= 1e-3 against float64.
"""

import numpy as np
import torch

from oracle import formats as OF
from oracle import rope as OR

SCORE_GAMMA = 160.0 * 2.0 ** -24
ATTN_MAX_ABS = 2e-3
ATTN_REL_L2 = 1e-3
NEAR_TIE = 1e-5


def has_gpu():
    return torch.cuda.is_available()


def to_np(t):
    return t.detach().cpu().numpy()


def bf16_to_np_f32(t):
    return t.detach().cpu().float().numpy()


def score_bound(q_codes, w, k_codes):
    """Per-position absolute error bound of the decode-shaped scan (fp16 MFMA,
    float32 accumulation): 160 units of 2^-24 * sum_h |w_h| sum_c |q_hc k_c|."""
    q = np.abs(OF.e4m3_decode(q_codes.reshape(32, 128)))
    k = np.abs(OF.e4m3_decode(k_codes))
    return SCORE_GAMMA * (k @ q.T) @ np.abs(np.asarray(w, dtype=np.float64).reshape(32))


def fp8_contraction_bound(q_values, w, k_values):
    """Per-position absolute error bound of the prefill-shaped scan, whose FP8
    MFMA (v_mfma_f32_32x32x64_f8f6f4) truncates every product to 13 fractional
    bits below the largest product of its instruction (measured on gfx950; the
    accumulator itself is kept in float32). A head's 128-term dot product runs
    as two such instructions of 64 products, so it is off by less than
    2 * 63 * 2^-13 * max_c |q_hc k_c|; the weighted ReLU sum is 1-Lipschitz in
    each head, and the float32 epilogue adds the 160 units of score_bound.

    q_values [32,128] and k_values [n,128]: decoded values (floats)."""
    qa = np.abs(np.asarray(q_values, dtype=np.float64).reshape(32, 128))
    ka = np.abs(np.asarray(k_values, dtype=np.float64))
    wa = np.abs(np.asarray(w, dtype=np.float64).reshape(32))
    # max_c |q_hc k_nc| for every (position, head), in chunks
    mx = np.empty((ka.shape[0], 32))
    for a in range(0, ka.shape[0], 4096):
        mx[a:a + 4096] = (ka[a:a + 4096, None, :] * qa[None, :, :]).max(axis=2)
    trunc = 2.0 * 63.0 * 2.0 ** -13 * (mx @ wa)
    return trunc + SCORE_GAMMA * (ka @ qa.T) @ wa


def assert_scores_close(gpu, ref, bound, what=""):
    gpu = np.asarray(gpu, dtype=np.float32)
    ref = np.asarray(ref, dtype=np.float32)
    ninf_g, ninf_r = np.isneginf(gpu), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), "%s: -inf pattern differs" % what
    fin = ~ninf_r
    err = np.abs(gpu[fin].astype(np.float64) - ref[fin].astype(np.float64))
    assert np.all(err <= bound[fin] + 1e-30), "%s: max err %g > bound" % (what, float((err - bound[fin]).max()))


def kth_value(scores, k):
    """The k-th largest value (1-based) of a float32 array."""
    s = np.sort(np.asarray(scores, dtype=np.float32))[::-1]
    return float(s[min(k, s.shape[0]) - 1])


def assert_topk_near(gpu_idx, ref_idx, score_of_pos, k=512, extra_allowed=None, what=""):
    """Sets equal except near-ties of the K-th oracle score.

    score_of_pos: dict/callable position -> oracle float32 score."""
    g = set(int(x) for x in gpu_idx if x >= 0)
    o = set(int(x) for x in ref_idx if x >= 0)
    assert len(g) == len(o), "%s: %d vs %d selected" % (what, len(g), len(o))
    assert list(gpu_idx) == sorted(gpu_idx[gpu_idx >= 0].tolist()) + [-1] * int((gpu_idx < 0).sum())
    diff = g ^ o
    if not diff:
        return 0
    kth = min(float(score_of_pos(p)) for p in o)
    for p in diff:
        if extra_allowed is not None and extra_allowed(p):
            continue
        s = float(score_of_pos(p))
        assert abs(s - kth) <= NEAR_TIE * abs(kth), "%s: position %d score %r vs K-th %r" % (what, p, s, kth)
    return len(diff)


def assert_attn_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    rel = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30)
    assert np.all(np.isfinite(gpu)), what + ": non-finite output"
    assert err.max() <= ATTN_MAX_ABS, "%s: max-abs %g" % (what, err.max())
    assert rel <= ATTN_REL_L2, "%s: rel-L2 %g" % (what, rel)
    return float(err.max()), float(rel)


class OracleCache:
    """Oracle-side packed main-KV rows of one sequence, quantised lazily by the
    oracle from the bf16 source rows (RoPE at position j * m, then FP4)."""

    def __init__(self, main_bf16_rows, m):
        self.src = main_bf16_rows          # torch bf16 [n_cap, 512] (device or host)
        self.m = m
        self.cache = {}

    def __len__(self):
        return int(self.src.shape[0])

    def __getitem__(self, sel):
        sel = np.asarray(sel, dtype=np.int64).reshape(-1)
        need = [int(j) for j in sel if int(j) not in self.cache]
        if need:
            need = sorted(set(need))
            x = self.src[torch.tensor(need, device=self.src.device)].float().cpu().numpy()
            y = OR.apply_rope(x, [j * self.m for j in need])
            rows = OF.quantize_rows(y)
            for j, r in zip(need, rows):
                self.cache[j] = r
        return np.stack([self.cache[int(j)] for j in sel]) if sel.size else np.zeros((0, 288), np.uint8)
