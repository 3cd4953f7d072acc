"""RoPE on the main-KV latent (oracle; test-only).

The pages say the main KV is quantised after RoPE [P1 §三; P3 第三刀]; they give
no RoPE details. The spec of this path fixes RoPE on the last 64 of the 512
channels with base 10000. Readings taken:
  * Pairs are adjacent channels (448 + 2i, 449 + 2i), i = 0..31, with inverse
    frequency theta_i = 10000^(-i/32) (RoFormer's definition: base^(-2i/d) for a
    d = 64 rotary sub-space).
  * The position of compressed entry j is j * m, its first token.
  * cos and sin are evaluated in float64 and rounded once to float32; the
    rotation is done in float32 with every product and sum rounded separately:
        y0 = fl(fl(x0 c) - fl(x1 s)),  y1 = fl(fl(x0 s) + fl(x1 c)).
"""

import math

import numpy as np

ROPE_DIMS = 64
ROPE_PAIRS = ROPE_DIMS // 2
ROPE_BASE = 10000.0
D_MAIN = 512
ROPE_START = D_MAIN - ROPE_DIMS   # 448


def rope_cos_sin(positions):
    """float32 cos/sin per (position, pair): returns (cos, sin) each [n, 32].

    Uses Python's ``math`` (the C library's pow/cos/sin on float64) one value at a
    time: slow, but a plain evaluation of the definition."""
    positions = [int(p) for p in np.asarray(positions).reshape(-1)]
    theta = [math.pow(ROPE_BASE, -i / ROPE_PAIRS) for i in range(ROPE_PAIRS)]
    c = np.empty((len(positions), ROPE_PAIRS), dtype=np.float32)
    s = np.empty((len(positions), ROPE_PAIRS), dtype=np.float32)
    cache = {}
    for r, p in enumerate(positions):
        if p not in cache:
            ang = [float(p) * th for th in theta]
            cache[p] = ([math.cos(a) for a in ang], [math.sin(a) for a in ang])
        cc, ss = cache[p]
        c[r] = np.array(cc, dtype=np.float64).astype(np.float32)
        s[r] = np.array(ss, dtype=np.float64).astype(np.float32)
    return c, s


def apply_rope(x, positions):
    """Rotate the last 64 channels of float32 rows ``x`` [n, 512] by their
    positions; channels 0..447 pass through unchanged."""
    x = np.asarray(x, dtype=np.float32)
    c, s = rope_cos_sin(positions)
    y = x.copy()
    x0 = x[:, ROPE_START::2]
    x1 = x[:, ROPE_START + 1::2]
    # float32 NumPy arithmetic rounds every product and every sum on its own.
    y[:, ROPE_START::2] = (x0 * c) - (x1 * s)
    y[:, ROPE_START + 1::2] = (x0 * s) + (x1 * c)
    return y
