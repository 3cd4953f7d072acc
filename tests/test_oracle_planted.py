"""Planted mistakes: each case swaps one oracle function for a copy with a
plausible error in it (a dropped term, a flipped sign, a transposed operand, an
off-by-one, the wrong tie rule or rounding) and requires that at least one of
the oracle's pins then fails. This shows that the pins constrain the oracle
itself, not merely agree with it (CPU only; the oracle is swapped through
pytest's monkeypatch and restored after each case)."""

import numpy as np
import pytest

from oracle import attention as A
from oracle import compress as Cm
from oracle import formats as F
from oracle import group as G
from oracle import indexer as I
from oracle import mxfp4 as M
from oracle import rope as R
from oracle import select as S
from tests import test_oracle_attention_group as TA
from tests import test_oracle_formats as TF
from tests import test_oracle_mxfp4 as TM
from tests import test_oracle_rope_compress as TR
from tests import test_oracle_select as TS


# ----------------------------------------------------------- mutant oracles --

def _scores_mutant(relu=True, vis_extra=0, transpose_q=False):
    """The indexer score with one of three mistakes switched on."""
    def index_scores(q_codes, w, k_codes, n_vis, positions=None, chunk=65536, k_scales=None):
        codes = np.asarray(q_codes)
        if transpose_q:     # heads and channels swapped when reading the query
            q = F.e4m3_decode(codes.reshape(-1)).reshape(128, 32).T
        else:
            q = F.e4m3_decode(codes.reshape(32, 128))
        w64 = np.asarray(w, dtype=np.float32).astype(np.float64).reshape(32)
        k_codes = np.asarray(k_codes)
        if positions is None:
            positions = np.arange(k_codes.shape[0], dtype=np.int64)
        positions = np.asarray(positions, dtype=np.int64)
        out = np.full(positions.shape[0], -np.inf, dtype=np.float32)
        sel = np.nonzero(positions < int(n_vis) + vis_extra)[0]
        pos = np.minimum(positions[sel], k_codes.shape[0] - 1)
        k = (F.e4m3_decode(k_codes[pos]) if k_scales is None
             else M.dequantize_index_keys(k_codes[pos], k_scales[pos]))
        d = k @ q.T
        acc = np.zeros(sel.shape[0])
        for h in range(32):
            acc = acc + w64[h] * (np.maximum(d[:, h], 0.0) if relu else d[:, h])
        out[sel] = acc.astype(np.float32)
        return out
    return index_scores


def _rope_mutant(sign=1.0, start=R.ROPE_START, base=R.ROPE_BASE, pairs_div=R.ROPE_PAIRS):
    """RoPE with a flipped rotation sense, the wrong channels or the wrong
    frequency schedule."""
    def apply_rope(x, positions):
        x = np.asarray(x, dtype=np.float32)
        pos = np.asarray(positions, dtype=np.float64).reshape(-1)
        th = base ** (-np.arange(32) / pairs_div)
        ang = pos[:, None] * th[None, :]
        c = np.cos(ang).astype(np.float32)
        s = (sign * np.sin(ang)).astype(np.float32)
        y = x.copy()
        x0, x1 = x[:, start:start + 64:2], x[:, start + 1:start + 64:2]
        y[:, start:start + 64:2] = x0 * c - x1 * s
        y[:, start + 1:start + 64:2] = x0 * s + x1 * c
        return y
    return apply_rope


def _topk_ties_to_higher(scores, cand_positions, k=S.TOPK):
    scores = np.asarray(scores, dtype=np.float32)
    pos = np.asarray(cand_positions, dtype=np.int64)
    order = np.lexsort((-pos, -scores.astype(np.float64)))
    keep = np.sort(pos[order[:k]])
    out = np.full(k, -1, dtype=np.int32)
    out[:keep.shape[0]] = keep
    return out


def _pool_floor_blocks(bmax, n_vis, n_blocks=S.POOL_BLOCKS):
    bmax = np.asarray(bmax, dtype=np.float32)
    n_blk = min(int(n_vis) // S.BLOCK, bmax.shape[0])      # a partial last block dropped
    return S.topk_positions(bmax[:n_blk], np.arange(n_blk), k=n_blocks)


def _mx_scale_minus_one(amax):
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(a)
    code = np.clip((e.astype(np.int64) - 1) - 1 + M.E8M0_BIAS, 0, 254)   # E2M1 emax read as 1
    return np.where(a > 0.0, code, 0).astype(np.uint8)


def _scale_over_four(amax):
    a = np.asarray(amax, dtype=np.float64).reshape(-1, 1)
    dist = np.abs(4.0 * F._SCALE_VALUES[None, :] - a)       # amax / 4 instead of / 6
    return F._SCALE_CODES[dist.argmin(axis=1)]


def _e2m1_ties_away(y, s):
    y = np.asarray(y, dtype=np.float32)
    mag = np.abs(y).astype(np.float64)
    s = np.asarray(s, dtype=np.float64)
    dist = np.abs(F.E2M1_GRID[None, None, :] * s[:, None, None] - mag[:, :, None])
    mcode = (7 - dist[:, :, ::-1].argmin(axis=2)).astype(np.uint8)   # ties to the larger
    mcode = np.where(s[:, None] == 0.0, np.uint8(0), mcode)
    return (mcode | (np.signbit(y).astype(np.uint8) << 3)).astype(np.uint8)


_E4M3_MAGS = np.array([F.e4m3_value_of_code(c) for c in range(127)])


def _e4m3_truncating(x):
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    mag = np.clip(np.searchsorted(_E4M3_MAGS, a, side="right") - 1, 0, 126).astype(np.uint8)
    return (mag | (np.signbit(x).astype(np.uint8) << 7)).astype(np.uint8)


def _softmax_unscaled(q, keys, scale):
    z = q @ keys.T                                           # the scale forgotten
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return (p / p.sum(axis=1, keepdims=True)) @ keys


def _n_visible_floor(t, m):
    return np.asarray(t, dtype=np.int64) // int(m)           # the token itself not counted


def _compress_sum(token_bits, m):
    x = Cm.bf16_bits_to_f32(np.asarray(token_bits, dtype=np.uint16))
    n = -(-x.shape[0] // m)
    out = np.zeros((n, x.shape[1]), dtype=np.float32)
    for j in range(n):
        out[j] = x[j * m:(j + 1) * m].sum(axis=0)           # sum, not mean
    return Cm.f32_to_bf16_bits(out)


def _window_129(t, n_win=A.N_WIN):
    return np.arange(max(0, int(t) - n_win), int(t) + 1, dtype=np.int64)


def _block_max_ignores_visibility(scores, n_vis):
    s = np.asarray(scores, dtype=np.float32)
    n_blk = -(-s.shape[0] // I.BLOCK)
    pad = np.full(n_blk * I.BLOCK, -np.inf, dtype=np.float32)
    pad[:s.shape[0]] = s
    return pad.reshape(n_blk, I.BLOCK).max(axis=1)


def _bf16_truncating(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)                      # truncation, not nearest-even


def _reindex_ignores_visibility(pool, n_vis):
    pool = np.asarray(pool, dtype=np.int64)
    b = pool[pool >= 0]
    return (b[:, None] * S.BLOCK + np.arange(S.BLOCK)[None, :]).reshape(-1)


def _e4m3_value_no_subnormals(code):
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 15 and m == 7:
        return float("nan")
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)          # exponent 0 read as normal


_E4M3_NO_SUB = np.array([_e4m3_value_no_subnormals(c) for c in range(256)])


def _e4m3_decode_no_subnormals(codes):
    return _E4M3_NO_SUB[np.asarray(codes, dtype=np.uint8)]


def _dequantize_rows_per_32(rows):
    codes, sc = F.unpack_codes(rows)
    v = F.e2m1_decode(codes)
    s = F.e4m3_decode(sc)[:, ::2]                             # one scale per 32 channels
    return v * np.repeat(s, 2 * F.GROUP, axis=1)


def _unpack_high_nibble_first(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.empty((packed.shape[0], 128), dtype=np.uint8)
    codes[:, 0::2] = packed >> 4                              # nibble order swapped
    codes[:, 1::2] = packed & 0xF
    return codes


def _mx_scale_values_bias_128(codes):
    return np.ldexp(1.0, np.asarray(codes, dtype=np.int64) - 128)


# --------------------------------------------------------------- the cases --

def _run_group_mutant(kind):
    """run_group with one per-layer routing mistake: a Reindex layer scoring
    with the first layer's indexer query, every attention reading the first
    layer's query or window, or a Reuse layer copying the first layer's
    indices."""
    def run_group(schedule, q_idx, w, q, swa, k_codes, cache_rows, n_vis, t, swa_pos0,
                  scale=1.0, with_pool=True, k_scales=None, ring=False):
        idx_of, out_of, scores_of = {}, {}, {}
        pool = None
        for li, (mode, src) in enumerate(schedule):
            if mode == "F":
                s = I.index_scores(q_idx[li], w[li], k_codes, n_vis, k_scales=k_scales)
                nv = min(int(n_vis), s.shape[0])
                idx_of[li] = S.topk_positions(s[:nv], np.arange(nv))
                if with_pool and pool is None:
                    pool = S.build_pool(I.block_max(s, n_vis), n_vis)
                scores_of[li] = s
            elif mode == "X":
                qs = 0 if kind == "reindex_q0" else li
                cand = S.reindex_candidates(pool, n_vis)
                s = I.index_scores(q_idx[qs], w[qs], k_codes, n_vis, positions=cand,
                                   k_scales=k_scales)
                idx_of[li] = S.topk_positions(s, cand)
                scores_of[li] = (cand, s)
            else:
                idx_of[li] = idx_of[0 if kind == "reuse_0" else src].copy()
            out_of[li] = A.sparse_attention(q[0 if kind == "q0" else li], cache_rows, idx_of[li],
                                            swa[0 if kind == "swa0" else li], t, swa_pos0, scale,
                                            ring=ring)
        return idx_of, out_of, pool, scores_of
    return run_group


def _window_rows_mutant(kind):
    """Window rows with a ring addressed from swa_pos0, or without the check
    that the buffer holds a token."""
    def window_rows(t, swa_pos0, S_, ring=False):
        toks = A.swa_tokens(t)
        if kind != "no_hold_check":
            toks = toks[(toks >= int(swa_pos0)) & (toks < int(swa_pos0) + int(S_))]
        if ring:
            rows = (toks - int(swa_pos0)) % int(S_) if kind == "ring_from_pos0" else toks % int(S_)
        else:
            rows = (toks - int(swa_pos0)) % int(S_)
        return toks, rows
    return window_rows


def _gather_keys_clamped(cache_rows, idx, swa_codes, t, swa_pos0, ring=False):
    """Selected indices clamped into the cache instead of skipped."""
    idx = np.asarray(idx, dtype=np.int64)
    sel = np.clip(idx[idx >= 0], 0, len(cache_rows) - 1)
    main = F.dequantize_rows(np.asarray(cache_rows[sel]))
    swa_codes = np.asarray(swa_codes)
    _, rows = A.window_rows(t, swa_pos0, swa_codes.shape[0], ring)
    return np.concatenate([main, F.e4m3_decode(swa_codes[rows])], axis=0)


_ROUTING_PINS = [TA.test_reindex_with_the_full_layers_query_reproduces_its_topk,
                 TA.test_each_reindex_layer_scores_with_its_own_indexer_query,
                 TA.test_each_layer_attends_with_its_own_query,
                 TA.test_each_layer_attends_over_its_own_window,
                 TA.test_reuse_is_byte_identical_and_sources_untouched]


CASES = [
    ("score: ReLU dropped", I, "index_scores", _scores_mutant(relu=False),
     [TS.test_scores_vs_exact_brute_force, TS.test_closed_form_unit_vectors_and_relu]),
    ("score: position n_vis visible", I, "index_scores", _scores_mutant(vis_extra=1),
     [TS.test_scores_vs_exact_brute_force]),
    ("score: query operand transposed", I, "index_scores", _scores_mutant(transpose_q=True),
     [TS.test_scores_vs_exact_brute_force, TS.test_closed_form_unit_vectors_and_relu]),
    ("rope: rotation sense flipped", R, "apply_rope", _rope_mutant(sign=-1.0),
     [TR.test_matches_complex_rotation_closed_form]),
    ("rope: first 64 channels rotated", R, "apply_rope", _rope_mutant(start=0),
     [TR.test_only_last_64_channels_move]),
    ("rope: frequencies 10000^(-2i/32)", R, "apply_rope", _rope_mutant(pairs_div=16),
     [TR.test_matches_complex_rotation_closed_form]),
    ("top-k: ties to the higher position", S, "topk_positions", _topk_ties_to_higher,
     [TS.test_topk_worked_examples] + [lambda s=s: TS.test_topk_vs_python_sorted(s)
                                       for s in range(5)]),
    ("pool: partial last block dropped", S, "build_pool", _pool_floor_blocks,
     [TS.test_topk_worked_examples, TS.test_small_context_pool_is_every_block]),
    ("fp4 keys: E8M0 scale one binade high", M, "mx_scale_codes", _mx_scale_minus_one,
     [TM.test_worked_blocks, TM.test_scale_rule_vs_exact_powers_of_two]),
    ("fp4 main KV: scale from amax/4", F, "scale_codes", _scale_over_four,
     [TF.test_worked_groups, TF.test_scale_vs_exact_rationals]),
    ("fp4 main KV: E2M1 ties away from zero", F, "e2m1_codes", _e2m1_ties_away,
     [TF.test_e2m1_codes_vs_exact_rationals, TF.test_worked_groups]),
    ("e4m3 append: truncation", F, "e4m3_encode", _e4m3_truncating,
     [TF.test_e4m3_encode_midpoints_ties_to_even_and_saturation]),
    ("attention: softmax scale forgotten", A, "softmax_attention", _softmax_unscaled,
     [TA.test_matches_torch_sdpa_on_gathered_rows]),
    ("attention: 129-token window", A, "swa_tokens", _window_129, [TA.test_window_bounds]),
    ("compressor: the current token not counted", Cm, "n_visible", _n_visible_floor,
     [TR.test_visible_count]),
    ("compressor: sum instead of mean", Cm, "compress_mean", _compress_sum,
     [TR.test_mean_matches_torch_and_closed_form]),
    ("block maxima: invisible positions counted", I, "block_max", _block_max_ignores_visibility,
     [TS.test_block_max]),
    ("compressor: bf16 by truncation", Cm, "f32_to_bf16_bits", _bf16_truncating,
     [TR.test_bf16_rounding_matches_torch]),
    ("reindex: positions past n_vis kept", S, "reindex_candidates", _reindex_ignores_visibility,
     [TS.test_reindex_candidates_respect_visibility]),
    ("e4m3 decode: subnormals read as normals", F, "e4m3_decode", _e4m3_decode_no_subnormals,
     [TF.test_e4m3_golden_points, TF.test_e4m3_decode_matches_torch]),
    ("fp4 keys: high nibble read as the even channel", M, "unpack_index_codes",
     _unpack_high_nibble_first,
     [TM.test_layout_low_nibble_even_channel_and_scale_bytes, TM.test_grid_valued_blocks_round_trip]),
    ("fp4 keys: E8M0 bias 128", M, "mx_scale_values", _mx_scale_values_bias_128,
     [TM.test_grid_valued_blocks_round_trip, TM.test_dequantised_values_are_code_times_power_of_two,
      TM.test_worked_blocks]),
    ("fp4 keys: E2M1 ties away from zero", M, "e2m1_codes", _e2m1_ties_away,
     [lambda: TM.test_elements_vs_exact_rationals(0), TM.test_worked_blocks]),
    ("main KV: one scale per 32 channels", F, "dequantize_rows", _dequantize_rows_per_32,
     [TF.test_grid_valued_group_round_trips,
      lambda: TF.test_quantize_is_nearest_over_whole_rows(0)]),
    ("group: Reindex scores with the first layer's indexer query", G, "run_group",
     _run_group_mutant("reindex_q0"), _ROUTING_PINS),
    ("group: every attention reads the first layer's query", G, "run_group",
     _run_group_mutant("q0"), _ROUTING_PINS),
    ("group: every attention reads the first layer's window", G, "run_group",
     _run_group_mutant("swa0"), _ROUTING_PINS),
    ("group: Reuse copies the first layer's indices", G, "run_group",
     _run_group_mutant("reuse_0"), _ROUTING_PINS),
    ("window: ring rows counted from swa_pos0", A, "window_rows",
     _window_rows_mutant("ring_from_pos0"),
     [TA.test_ring_window_equals_linear_window, TA.test_ring_window_closed_form_names_the_tokens_used]),
    ("window: tokens the buffer does not hold are read", A, "window_rows",
     _window_rows_mutant("no_hold_check"),
     [TA.test_out_of_range_indices_and_unheld_window_tokens_are_skipped,
      TA.test_ring_window_closed_form_names_the_tokens_used]),
    ("attention: out-of-range indices clamped into the cache", A, "gather_keys",
     _gather_keys_clamped, [TA.test_out_of_range_indices_and_unheld_window_tokens_are_skipped]),
]


@pytest.mark.parametrize("name,module,attr,mutant,pins", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_fails_a_pin(name, module, attr, mutant, pins, monkeypatch):
    monkeypatch.setattr(module, attr, mutant)
    failed = []
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed.append(getattr(pin, "__name__", "pin"))
    assert failed, "no pin caught the planted mistake: %s" % name


@pytest.mark.parametrize("name,module,attr,mutant,pins", CASES, ids=[c[0] for c in CASES])
def test_pins_pass_on_the_oracle_itself(name, module, attr, mutant, pins):
    for pin in pins:
        pin()
