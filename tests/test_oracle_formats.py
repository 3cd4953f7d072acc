"""Pins for the oracle's FP8 / FP4 codecs and the 288-byte row (CPU only).

Each test checks the oracle against something other than itself: the OCP E4M3
definition, torch's float8_e4m3fn conversion, exact rational (Fraction)
brute force, hand-worked fixtures, or closed forms."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bits_to_f32(bits):
    return np.array([int(b, 16) for b in bits], dtype=np.uint32).view(np.float32)


# ---------------------------------------------------------------- E2M1 -----

def test_e2m1_sixteen_code_points():
    """Closed form of E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa
    bit): the 16 codes enumerate +-{0, .5, 1, 1.5, 2, 3, 4, 6}."""
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1 + m / 2)
        want = -mag if s else mag
        got = float(F.e2m1_decode(np.array([code]))[0])
        assert got == want and math.copysign(1, got) == math.copysign(1, want)
    mags = sorted(set(abs(float(v)) for v in F.e2m1_decode(np.arange(16))))
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


# ---------------------------------------------------------------- E4M3 -----

def test_e4m3_golden_points():
    with open(os.path.join(GOLD, "e4m3_ocp_points.json")) as f:
        pts = json.load(f)["points"]
    for p in pts:
        got = float(F.e4m3_decode(np.array([int(p["code"], 16)]))[0])
        if p["value"] == "nan":
            assert math.isnan(got)
        else:
            assert got == p["value"]
            assert math.copysign(1, got) == math.copysign(1, p["value"])


def test_e4m3_decode_matches_torch():
    """torch's float8_e4m3fn decode of all 256 bytes (NaNs compared as NaN)."""
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert nan.sum() == 2


def test_e4m3_all_finite_codes_round_trip_as_scale():
    """A group whose amax is exactly 6 * v yields scale code v for every
    non-negative finite code v (0x00..0x7E)."""
    for code in range(127):
        v = F.e4m3_value_of_code(code)
        amax = np.float32(6.0 * v)
        assert float(amax) == 6.0 * v            # 6 v is exact in float32
        assert int(F.scale_codes(np.array([amax]))[0]) == code


def _frac_nearest_even(x, cands):
    """Exact nearest (value, code) among cands; ties to the even code."""
    best = None
    for code, v in cands:
        d = abs(Fraction(v) - x)
        key = (d, code % 2)
        if best is None or key < best[0]:
            best = (key, code)
    return best[1]


_SCALE_CANDS = [(c, F.e4m3_value_of_code(c)) for c in range(127)]


def test_scale_vs_exact_rationals():
    rng = np.random.default_rng(1)
    amax = np.concatenate([
        np.abs(rng.standard_normal(300)).astype(np.float32) * np.float32(3.0),
        (np.float32(10.0) ** rng.uniform(-5, 4, 300)).astype(np.float32),
        # exact ties: amax = 6 * (midpoint between adjacent codes)
        np.array([6.0 * (F.e4m3_value_of_code(c) + F.e4m3_value_of_code(c + 1)) / 2
                  for c in range(0, 126, 3)], dtype=np.float32),
        np.array([0.0, 1e9, 2688.0, 2880.0, 2879.0], dtype=np.float32),
    ])
    got = F.scale_codes(amax)
    for a, g in zip(amax, got):
        x = Fraction(float(a)) / 6
        assert int(g) == _frac_nearest_even(x, _SCALE_CANDS), float(a)


_E2M1_CANDS = [(c, float(F.E2M1_GRID[c])) for c in range(8)]


def test_e2m1_codes_vs_exact_rationals():
    rng = np.random.default_rng(2)
    s = np.array([F.e4m3_value_of_code(c) for c in rng.integers(1, 127, 40)])
    y = (rng.standard_normal((40, 16)) * 2.5).astype(np.float32) * s[:, None].astype(np.float32)
    # plant exact ties at every E2M1 midpoint
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for i, mid in enumerate(mids):
        y[i, 0] = np.float32(mid * s[i])
        y[i, 1] = -np.float32(mid * s[i])
    codes = F.e2m1_codes(y, s)
    for gi in range(y.shape[0]):
        for ci in range(16):
            v = float(y[gi, ci])
            x = Fraction(abs(v)) / Fraction(float(s[gi]))
            mag = _frac_nearest_even(x, _E2M1_CANDS)
            sign = 8 if math.copysign(1, v) < 0 else 0
            assert int(codes[gi, ci]) == (mag | sign)


def test_worked_groups():
    with open(os.path.join(GOLD, "fp4_worked_groups.json")) as f:
        groups = json.load(f)["groups"]
    for g in groups:
        if "y" in g:
            y = np.array(g["y"], dtype=np.float32)
        else:
            y = _bits_to_f32(g["y_bits"])
        row = np.zeros((1, 512), dtype=np.float32)
        row[0, :16] = y
        packed = F.quantize_rows(row)[0]
        codes, sc = F.unpack_codes(packed[None])
        assert list(codes[0, :16]) == g["codes"], g["name"]
        assert list(packed[:8]) == [int(b, 16) for b in g["packed"]], g["name"]
        assert int(packed[256]) == int(g["scale"], 16), g["name"]


def test_grid_valued_group_round_trips():
    """amax = 6 s with every entry on the grid times s dequantises exactly."""
    rng = np.random.default_rng(3)
    rows = np.zeros((8, 512), dtype=np.float32)
    for r in range(8):
        for g in range(32):
            s = F.e4m3_value_of_code(int(rng.integers(1, 127)))
            vals = rng.choice(F.E2M1_GRID, 16) * rng.choice([-1, 1], 16)
            vals[rng.integers(16)] = 6.0
            rows[r, g * 16:(g + 1) * 16] = (vals * s).astype(np.float32)
    deq = F.dequantize_rows(F.quantize_rows(rows))
    assert np.array_equal(deq, rows.astype(np.float64))


def test_row_layout_and_zero_scale():
    assert F.ROW_BYTES == 288
    rows = np.zeros((2, 512), dtype=np.float32)
    rows[1, :] = -0.0
    p = F.quantize_rows(rows)
    assert p.shape == (2, 288)
    assert np.all(p[0] == 0)
    assert np.all(p[1, :256] == 0x88) and np.all(p[1, 256:] == 0)


def test_products_exact_in_half_and_bf16():
    """Every E2M1 x E4M3 product is exact in fp16, bf16 and fp32."""
    e2 = F.E2M1_GRID
    e4 = np.array([F.e4m3_value_of_code(c) for c in range(127)])
    prod = (e2[:, None] * e4[None, :]).reshape(-1)
    assert np.array_equal(prod.astype(np.float16).astype(np.float64), prod)
    assert np.array_equal(prod.astype(np.float32).astype(np.float64), prod)
    t = torch.tensor(prod, dtype=torch.float64)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float64), t)


def test_threshold_times_scale_exact_in_fp32():
    """Thresholds times any E4M3 scale, and 6 x any E4M3 midpoint, are exact in
    float32 (the property a division-free quantiser relies on)."""
    e4 = np.array([F.e4m3_value_of_code(c) for c in range(127)])
    th = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    p = (th[:, None] * e4[None, :]).reshape(-1)
    assert np.array_equal(p.astype(np.float32).astype(np.float64), p)
    mids = 6.0 * (e4[:-1] + e4[1:]) / 2
    assert np.array_equal(mids.astype(np.float32).astype(np.float64), mids)


@pytest.mark.parametrize("seed", [0, 1])
def test_quantize_is_nearest_over_whole_rows(seed):
    """Dequantised values are the nearest grid-times-scale values (no closer
    representable value exists for any element), checked by brute force."""
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((4, 512)).astype(np.float32)
    y[:, rng.integers(512, size=5)] *= 8
    p = F.quantize_rows(y)
    deq = F.dequantize_rows(p)
    s = np.repeat(F.e4m3_decode(p[:, 256:]), 16, axis=1)
    cand = F.E2M1_GRID[None, None, :] * s[:, :, None]
    best = np.abs(cand - np.abs(y.astype(np.float64))[:, :, None]).min(axis=2)
    assert np.array_equal(np.abs(np.abs(deq) - np.abs(y)), best)


# ---- E4M3 encoding (window rows and FP8 indexer keys appended by the write path)

def test_e4m3_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def test_e4m3_encode_midpoints_ties_to_even_and_saturation():
    for c in range(0, 126):
        lo, hi = F.e4m3_value_of_code(c), F.e4m3_value_of_code(c + 1)
        mid = (lo + hi) / 2.0                      # exact: at most 5 significant bits
        want = c if c % 2 == 0 else c + 1
        assert int(F.e4m3_encode(np.float32(mid))) == want, c
        assert int(F.e4m3_encode(np.float32(-mid))) == want | 0x80, c
        assert int(F.e4m3_encode(np.nextafter(np.float32(mid), np.float32(0)))) == c
        assert int(F.e4m3_encode(np.nextafter(np.float32(mid), np.float32(1e9)))) == c + 1
    for big in (448.5, 463.0, 464.0, 480.0, 1e6, 3e38):
        assert int(F.e4m3_encode(np.float32(big))) == 0x7E
        assert int(F.e4m3_encode(np.float32(-big))) == 0xFE
    assert int(F.e4m3_encode(np.float32(-0.0))) == 0x80


def test_e4m3_encode_matches_torch_float8_after_clamping():
    """torch's float8_e4m3fn cast rounds to nearest even but gives NaN beyond the
    range, so on values clamped to +-448 it must agree with the oracle."""
    import torch
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 3, 20000),
                        rng.standard_normal(2000) * 600.0]).astype(np.float32)
    x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()     # bf16 values, as appended
    t = torch.from_numpy(x).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(x), t)
