"""Pins for the oracle's RoPE and sequence-compression steps (CPU only)."""

import cmath
import math

import numpy as np
import torch

from oracle import rope as R
from oracle import compress as C


def test_position_zero_is_identity():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 512)).astype(np.float32)
    assert np.array_equal(R.apply_rope(x, [0, 0, 0]), x)


def test_only_last_64_channels_move():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    y = R.apply_rope(x, [1, 7, 1000, 1048574])
    assert np.array_equal(y[:, :448], x[:, :448])
    assert not np.array_equal(y[:, 448:], x[:, 448:])


def test_matches_complex_rotation_closed_form():
    """Each adjacent pair (448+2i, 449+2i) is the complex number x0 + i x1
    multiplied by exp(i p theta_i), theta_i = 10000^(-2i/64), evaluated here via
    exp/log in float64 (a different evaluation from the oracle's)."""
    rng = np.random.default_rng(2)
    pos = [0, 1, 2, 5, 131070, 1048575]
    x = rng.standard_normal((len(pos), 512)).astype(np.float32)
    y = R.apply_rope(x, pos)
    for r, p in enumerate(pos):
        for i in range(32):
            th = math.exp(-(2 * i / 64) * math.log(10000.0))
            z = complex(float(x[r, 448 + 2 * i]), float(x[r, 449 + 2 * i])) * cmath.exp(1j * p * th)
            tol = 4e-7 * (abs(z) + 1e-30)
            assert abs(float(y[r, 448 + 2 * i]) - z.real) <= tol
            assert abs(float(y[r, 449 + 2 * i]) - z.imag) <= tol


def test_norm_preserved_per_pair():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 512)).astype(np.float32)
    pos = rng.integers(0, 1 << 20, 50)
    y = R.apply_rope(x, pos).astype(np.float64)
    a = x[:, 448:].astype(np.float64).reshape(50, 32, 2)
    b = y[:, 448:].reshape(50, 32, 2)
    na, nb = np.linalg.norm(a, axis=2), np.linalg.norm(b, axis=2)
    assert np.all(np.abs(na - nb) <= 3e-7 * na + 1e-30)


def test_relative_position_property():
    """<R_p a, R_q b> = <R_(p-r) a, R_(q-r) b> within float32 rounding."""
    rng = np.random.default_rng(4)
    a = rng.standard_normal((1, 512)).astype(np.float32)
    b = rng.standard_normal((1, 512)).astype(np.float32)
    for p, q, r in [(10, 3, 2), (1000, 999, 500), (70000, 12, 12)]:
        l = float(R.apply_rope(a, [p])[0, 448:].astype(np.float64) @ R.apply_rope(b, [q])[0, 448:].astype(np.float64))
        rr = float(R.apply_rope(a, [p - r])[0, 448:].astype(np.float64) @ R.apply_rope(b, [q - r])[0, 448:].astype(np.float64))
        assert abs(l - rr) <= 1e-5 * (np.abs(a[0, 448:]) @ np.abs(b[0, 448:]))


def test_cos_sin_rounded_once_from_float64():
    c, s = R.rope_cos_sin([3])
    for i in range(32):
        ang = 3.0 * 10000.0 ** (-i / 32)
        assert c[0, i] == np.float32(math.cos(ang))
        assert s[0, i] == np.float32(math.sin(ang))


# ------------------------------------------------------------ compress -----

def test_entry_count_is_ceil():
    for n in [1, 2, 3, 4, 5, 131072, 262144 + 4096, 1048576]:
        for m in [1, 2, 3]:
            assert C.n_entries(n, m) == math.ceil(n / m)
    rng = np.random.default_rng(5)
    for n in [1, 2, 3, 7]:
        for m in [1, 2]:
            tok = C.f32_to_bf16_bits(rng.standard_normal((n, 8)).astype(np.float32))
            assert C.compress_mean(tok, m).shape[0] == math.ceil(n / m)


def test_m1_is_identity():
    rng = np.random.default_rng(6)
    tok = C.f32_to_bf16_bits(rng.standard_normal((9, 16)).astype(np.float32))
    assert np.array_equal(C.compress_mean(tok, 1), tok)


def test_mean_matches_torch_and_closed_form():
    rng = np.random.default_rng(7)
    x = torch.randn(10, 512, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    want = ((x[0::2].float() + x[1::2].float()) / 2).to(torch.bfloat16)
    got = C.compress_mean(bits, 2)
    assert np.array_equal(got, want.view(torch.int16).numpy().view(np.uint16))
    # closed form: mean of exactly representable values
    two = C.f32_to_bf16_bits(np.array([[1.0, -3.0], [3.0, 5.0], [8.0, 0.5]], dtype=np.float32))
    out = C.bf16_bits_to_f32(C.compress_mean(two, 2))
    assert out.tolist() == [[2.0, 1.0], [8.0, 0.5]]
    del rng


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-3, 3, 100000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(C.f32_to_bf16_bits(x), want)


def test_visible_count():
    assert C.n_visible(0, 1) == 1 and C.n_visible(0, 2) == 0
    assert C.n_visible(1, 2) == 1 and C.n_visible(2, 2) == 1
    # prefill chunk: the last of 4,096 queries after 262,144 tokens sees 133,120
    assert C.n_visible(262144 + 4096 - 1, 2) == 133120
    assert C.n_visible(8191, 1) == 8192 and C.n_visible(131071, 2) == 65536
