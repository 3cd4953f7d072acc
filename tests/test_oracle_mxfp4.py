"""Pins for the oracle's FP4 indexer keys (E2M1 + one E8M0 scale per 32
channels) and for scores over them (CPU only): hand-worked blocks, the scale
rule against exact powers of two, element rounding against exact rationals,
round trips of grid-valued blocks, the byte layout, and scores against exact
rational brute force."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import indexer as I
from oracle import mxfp4 as M

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _block_from(d):
    v = np.zeros(32, dtype=np.float32)
    for k, x in d.items():
        v[int(k)] = np.float32(x)
    return v


def test_worked_blocks():
    with open(os.path.join(GOLD, "mxfp4_worked_blocks.json")) as f:
        blocks = json.load(f)["blocks"]
    for b in blocks:
        v = _block_from(b["values"])
        key = np.concatenate([v, np.zeros(96, dtype=np.float32)]).reshape(1, 128)
        codes, scales = M.quantize_index_keys(key)
        assert int(scales[0, 0]) == b["scale_code"], b["note"]
        assert list(scales[0, 1:]) == [0, 0, 0]
        c = M.unpack_index_codes(codes)[0, :32]
        want = np.zeros(32, dtype=np.uint8)
        for k, x in b["codes"].items():
            want[int(k)] = x
        # zero channels keep the sign of +0
        assert c.tolist() == want.tolist(), b["note"]


def _floor_log2(a):
    """floor(log2(a)) of a positive rational, by exact comparisons."""
    a = Fraction(a)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def test_scale_rule_vs_exact_powers_of_two():
    rng = np.random.default_rng(3)
    amax = np.concatenate([
        np.abs(rng.standard_normal(200)).astype(np.float32) * np.float32(3.0),
        (np.float32(2.0) ** rng.uniform(-140, 127, 200)).astype(np.float32),
        np.array([2.0 ** e for e in range(-20, 21)], dtype=np.float32),           # exact powers
        np.array([np.nextafter(np.float32(2.0 ** e), np.float32(0)) for e in range(-20, 21)],
                 dtype=np.float32),                                               # just below
        np.array([0.0, 448.0, 6.0, 3.4e38], dtype=np.float32),
    ])
    got = M.mx_scale_codes(amax)
    for a, g in zip(amax, got):
        if a == 0:
            assert g == 0
            continue
        want = min(max(_floor_log2(float(a)) - 2 + 127, 0), 254)
        assert int(g) == want, float(a)


_E2M1_CANDS = [(c, float(F.E2M1_GRID[c])) for c in range(8)]


def _nearest_even(x):
    best = min(abs(Fraction(v) - x) for _, v in _E2M1_CANDS)
    tied = [c for c, v in _E2M1_CANDS if abs(Fraction(v) - x) == best]
    ev = [c for c in tied if c % 2 == 0]
    return ev[0] if ev else tied[0]


@pytest.mark.parametrize("seed", [0, 1])
def test_elements_vs_exact_rationals(seed):
    rng = np.random.default_rng(10 + seed)
    k = (rng.standard_normal((24, 128)) * np.float32(2.0) ** rng.integers(-8, 8, (24, 1))).astype(np.float32)
    # plant exact midpoints and saturating values relative to each block's scale
    for r in range(8):
        blk = k[r, :32]
        e = math.floor(math.log2(float(np.abs(blk).max())))
        X = 2.0 ** (e - 2)
        for i, mid in enumerate([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]):
            blk[1 + i] = np.float32(mid * X) * (1 if i % 2 else -1)
        blk[0] = np.float32(7.5 * X)          # new amax, same exponent: saturates to 6
    codes, scales = M.quantize_index_keys(k)
    c = M.unpack_index_codes(codes)
    for r in range(k.shape[0]):
        for b in range(4):
            blk = k[r, 32 * b:32 * b + 32]
            X = Fraction(2) ** (int(scales[r, b]) - 127)
            for i in range(32):
                v = float(blk[i])
                mag = _nearest_even(abs(Fraction(v)) / X)
                sign = 8 if math.copysign(1.0, v) < 0 else 0
                assert int(c[r, 32 * b + i]) == (mag | sign), (r, b, i, v)


def test_grid_valued_blocks_round_trip():
    rng = np.random.default_rng(4)
    for j in range(-10, 11, 3):
        for top in (6.0, 4.0, 3.0):
            g = F.E2M1_GRID[rng.integers(0, 8, 128)] * rng.choice([-1, 1], 128)
            g[0::32] = top             # the block maximum sets the exponent
            if top == 3.0:             # grid values that stay on the grid when doubled
                g = np.clip(g, -3.0, 3.0)
            k = (g * 2.0 ** j).astype(np.float32).reshape(1, 128)
            codes, scales = M.quantize_index_keys(k)
            back = M.dequantize_index_keys(codes, scales)
            assert np.array_equal(back, k.astype(np.float64)), (j, top)


def test_layout_low_nibble_even_channel_and_scale_bytes():
    k = np.zeros((1, 128), dtype=np.float32)
    k[0, 0] = 6.0       # block 0: scale code 127 (amax 6 -> exponent 2 - 2 = 0)
    k[0, 1] = -1.0
    k[0, 64] = 0.75     # block 2: amax 0.75 -> exponent -1 - 2 -> code 124; 0.75*8 = 6
    k[0, 127] = 0.5     # block 3: exponent -1 - 2 -> 124; 0.5*8 = 4 (code 6)
    codes, scales = M.quantize_index_keys(k)
    assert scales[0].tolist() == [127, 0, 124, 124]
    assert codes[0, 0] == (7 | (10 << 4))          # 6 -> code 7 (low), -1 -> 8 | 2 (high)
    assert codes[0, 32] == 7                       # channel 64: 0.75 / 2^-3 = 6
    assert codes[0, 63] == (6 << 4)                # channel 127 (high nibble): 0.5 / 2^-3 = 4
    assert np.count_nonzero(codes) == 3


def test_scores_with_fp4_keys_vs_exact_brute_force():
    """Integer-valued E4M3 queries, FP4 keys with block scales 2^-7..2^7 and
    6-bit dyadic weights: the exact total needs at most 38 bits, so it is a
    float64 value and the oracle must return its single rounding to float32."""
    rng = np.random.default_rng(5)
    vals = [-4.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0]
    qcode = {}
    for c in range(256):
        x = F.e4m3_value_of_code(c)
        if x in vals and not (x == 0 and c != 0):
            qcode.setdefault(x, c)
    q = rng.choice(vals, (32, 128))
    qc = np.vectorize(qcode.get)(q).astype(np.uint8)
    n = 12
    codes = rng.integers(0, 256, (n, 64)).astype(np.uint8)
    scales = rng.integers(120, 135, (n, 4)).astype(np.uint8)
    kv = M.dequantize_index_keys(codes, scales)
    w = (rng.integers(0, 64, 32) / 64.0).astype(np.float32)
    got = I.index_scores(qc, w, codes, n_vis=10, k_scales=scales)
    for p in range(n):
        if p >= 10:
            assert got[p] == -np.inf
            continue
        tot = Fraction(0)
        for h in range(32):
            d = sum(Fraction(q[h, c]) * Fraction(float(kv[p, c])) for c in range(128))
            tot += Fraction(float(w[h])) * max(d, Fraction(0))
        assert Fraction(float(tot)) == tot          # exact in float64
        assert got[p] == np.float32(float(tot)), p


def test_dequantised_values_are_code_times_power_of_two():
    codes = np.arange(64, dtype=np.uint8).reshape(1, 64) * 3
    scales = np.array([[127, 100, 0, 254]], dtype=np.uint8)
    v = M.dequantize_index_keys(codes, scales)
    c = M.unpack_index_codes(codes)[0]
    for ch in range(128):
        e = int(scales[0, ch // 32]) - 127
        assert v[0, ch] == F.e2m1_decode(c[ch]) * 2.0 ** e
