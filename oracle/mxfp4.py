"""FP4 indexer keys: E2M1 elements with one power-of-two scale per 32 channels
(oracle; test-only).

What the pages fix: an earlier model generation already trained the indexer's
query and key in FP4 ("DeepSeek V4.1 Flash vs V4 Pro", 黑科技之三), and the FP4
format the pages do describe belongs to the MXFP4 family ("DeepSeek V4.1-Flash
为什么这么强？CED 与 CSA2 架构全拆解", §三). They give no block size or scale
type for the indexer. Readings taken:
  * Indexer keys only: the 128-wide key of a position becomes 128 E2M1 codes
    plus one E8M0 scale per block of 32 consecutive channels (4 per key), the
    MX layout of the OCP Microscaling Formats specification v1.0 (its MXFP4
    element and scale types). The indexer query stays FP8 E4M3 as in every
    workload.
  * Scale of a block (that specification's conversion rule): with amax the
    largest |v| of the block, the shared exponent is floor(log2(amax)) minus 2
    (2 is the exponent of the largest E2M1 value, 6 = 1.5 * 2^2); the stored
    E8M0 code is that exponent plus the bias 127, clamped to 0..254. A block
    of zeros stores code 0.
  * Each element: the E2M1 grid point nearest to |v| / 2^(code - 127), ties to
    the even code, saturating at 6 (amax / scale lies in [4, 8), so the
    largest elements may clip); the sign bit is the sign bit of v, also when
    the magnitude is 0.
  * Layout: codes [n][64] (byte j holds channel 2j in its low nibble, 2j+1 in
    its high nibble) and scales [n][4] (byte b scales channels 32b..32b+31).
  * Scores use the dequantised key value code * 2^(scale - 127) in place of the
    E4M3 key; every product with an E4M3 query element is exact in float64, and
    so are 128-term sums whenever the four block scales of a key lie within
    2^20 of one another (they always do for rows drawn from one distribution).
"""

import numpy as np

from .formats import E2M1_GRID, e2m1_codes, e2m1_decode

D_IDX = 128
MX_BLOCK = 32                   # channels per E8M0 scale (OCP MX block size)
MX_BLOCKS = D_IDX // MX_BLOCK   # 4 scales per key
CODE_BYTES = D_IDX // 2         # 64 bytes of packed E2M1 codes per key
E8M0_BIAS = 127
E2M1_EMAX = 2                   # 6 = 1.5 * 2^2


def mx_scale_codes(amax):
    """E8M0 scale code per block from its largest magnitude (float array >= 0):
    floor(log2(amax)) - 2 + 127, clamped to [0, 254]; 0 for amax == 0.
    floor(log2(.)) is read off the binary exponent (np.frexp: amax = f * 2^E
    with f in [0.5, 1), so floor(log2(amax)) = E - 1), exact for every float."""
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(a)
    code = (e.astype(np.int64) - 1) - E2M1_EMAX + E8M0_BIAS
    code = np.clip(code, 0, 254)
    return np.where(a > 0.0, code, 0).astype(np.uint8)


def mx_scale_values(codes):
    """2^(code - 127) as float64."""
    return np.ldexp(1.0, np.asarray(codes, dtype=np.int64) - E8M0_BIAS)


def quantize_index_keys(k):
    """Float32 keys [n, 128] (bf16 values) -> (codes [n, 64] uint8, scales [n, 4] uint8)."""
    k = np.asarray(k, dtype=np.float32)
    n = k.shape[0]
    assert k.shape == (n, D_IDX)
    packed = np.empty((n, CODE_BYTES), dtype=np.uint8)
    scales = np.empty((n, MX_BLOCKS), dtype=np.uint8)
    step = 4096
    for r0 in range(0, n, step):
        blocks = k[r0:r0 + step].reshape(-1, MX_BLOCK)              # [rows*4, 32]
        sc = mx_scale_codes(np.abs(blocks).max(axis=1))             # [rows*4]
        codes = e2m1_codes(blocks, mx_scale_values(sc)).reshape(-1, D_IDX)
        packed[r0:r0 + step] = codes[:, 0::2] | (codes[:, 1::2] << 4)
        scales[r0:r0 + step] = sc.reshape(-1, MX_BLOCKS)
    return packed, scales


def unpack_index_codes(packed):
    """Packed codes [n, 64] -> E2M1 codes [n, 128]."""
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.empty((packed.shape[0], D_IDX), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    return codes


def dequantize_index_keys(packed, scales):
    """Key values float64 [n, 128]: E2M1 value times its block's 2^(scale - 127)."""
    v = e2m1_decode(unpack_index_codes(packed))
    s = mx_scale_values(np.asarray(scales, dtype=np.uint8).reshape(-1, MX_BLOCKS))
    return v * np.repeat(s, MX_BLOCK, axis=1)


__all__ = ["mx_scale_codes", "mx_scale_values", "quantize_index_keys", "unpack_index_codes",
           "dequantize_index_keys", "E2M1_GRID", "MX_BLOCK", "MX_BLOCKS", "CODE_BYTES"]
