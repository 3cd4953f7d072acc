"""Seeded synthetic inputs for the CSA2 hot path (shared by tests and the bench).

This module draws random numbers and casts them to the storage dtypes; it holds
none of the method's arithmetic. Every tensor is drawn from its own stream,
keyed by (seed, config name, tensor name, chunk), with torch's generator on the
target device, in fixed-size chunks so the values do not depend on memory
limits. Recipe (the workloads' stated distributions):
  * indexer q and k ~ N(0, 1), cast to E4M3 (round to nearest even, clamped to
    +-448 first so the cast saturates); head weights w ~ U(0, 1) / 32 (float32);
  * main-KV tokens ~ N(0, 1) -> bf16; with m = 2 each compressed entry is the
    bf16 rounding of the float32 mean of its token pair;
  * main queries ~ N(0, 1) / sqrt(512) -> bf16 (the softmax scale is folded in);
  * window rows ~ N(0, 1) -> E4M3;
  * "outliers": round(1% of the channels) (at least one) of a tensor, chosen
    once from the tensor's stream, are multiplied by 8 in every row before the
    cast.
"""

import math
import zlib

import torch

ROW_CHUNK = 1 << 16


def _seed(seed, *tags):
    h = zlib.crc32(("/".join(str(t) for t in (seed,) + tags)).encode())
    return (h * 2654435761 + int(seed)) % (1 << 62)


def _gen(device, seed, *tags):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, *tags))
    return g


def outlier_channels(width, seed, *tags):
    """The round(1%) (>= 1) channels of a `width`-wide tensor scaled by 8."""
    g = torch.Generator(device="cpu")
    g.manual_seed(_seed(seed, "outliers", *tags))
    n = max(1, int(round(0.01 * width)))
    return torch.randperm(width, generator=g)[:n]


def normal_rows(n_rows, width, device, seed, *tags, outliers=False, scale=1.0):
    """float32 [n_rows, width] ~ N(0, scale^2), drawn chunk by chunk."""
    out = torch.empty((n_rows, width), dtype=torch.float32, device=device)
    for c0 in range(0, n_rows, ROW_CHUNK):
        c1 = min(n_rows, c0 + ROW_CHUNK)
        g = _gen(device, seed, *tags, c0 // ROW_CHUNK)
        out[c0:c1] = torch.randn((c1 - c0, width), generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        out.mul_(scale)
    if outliers:
        ch = outlier_channels(width, seed, *tags).to(device)
        out[:, ch] *= 8.0
    return out


def to_e4m3(x):
    """uint8 E4M3 codes of float32 x (nearest even, saturating at +-448)."""
    return x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def e4m3_rows(n_rows, width, device, seed, *tags, outliers=False):
    out = torch.empty((n_rows, width), dtype=torch.uint8, device=device)
    for c0 in range(0, n_rows, ROW_CHUNK):
        c1 = min(n_rows, c0 + ROW_CHUNK)
        g = _gen(device, seed, *tags, c0 // ROW_CHUNK)
        x = torch.randn((c1 - c0, width), generator=g, device=device, dtype=torch.float32)
        if outliers:
            x[:, outlier_channels(width, seed, *tags).to(device)] *= 8.0
        out[c0:c1] = to_e4m3(x)
    return out


def head_weights(n_q, device, seed, *tags):
    g = _gen(device, seed, *tags)
    return torch.rand((n_q, 32), generator=g, device=device, dtype=torch.float32) / 32.0


def token_rows_bf16(n_rows, device, seed, *tags, outliers=False, first_row=0):
    """bf16 [n_rows, 512] token rows; rows are drawn per ROW_CHUNK so any
    aligned sub-range can be regenerated alone (first_row % ROW_CHUNK == 0)."""
    assert first_row % ROW_CHUNK == 0
    out = torch.empty((n_rows, 512), dtype=torch.bfloat16, device=device)
    ch = outlier_channels(512, seed, *tags).to(device) if outliers else None
    for c0 in range(0, n_rows, ROW_CHUNK):
        c1 = min(n_rows, c0 + ROW_CHUNK)
        g = _gen(device, seed, *tags, (first_row + c0) // ROW_CHUNK)
        x = torch.randn((c1 - c0, 512), generator=g, device=device, dtype=torch.float32)
        if ch is not None:
            x[:, ch] *= 8.0
        out[c0:c1] = x.to(torch.bfloat16)
    return out


def pooled_main_rows(n_entries, m, device, seed, *tags, outliers=False, first_entry=0):
    """bf16 [n_entries, 512] compressed main-KV rows: for m = 1 the token rows,
    for m > 1 the bf16 rounding of the float32 mean of m consecutive token rows
    (summed in token order)."""
    if m == 1:
        return token_rows_bf16(n_entries, device, seed, *tags, outliers=outliers,
                               first_row=first_entry)
    out = torch.empty((n_entries, 512), dtype=torch.bfloat16, device=device)
    step = ROW_CHUNK // m
    assert first_entry % step == 0
    for e0 in range(0, n_entries, step):
        e1 = min(n_entries, e0 + step)
        tok = token_rows_bf16((e1 - e0) * m, device, seed, *tags, outliers=outliers,
                              first_row=(first_entry + e0) * m).float()
        acc = tok[0::m].clone()
        for j in range(1, m):
            acc = acc + tok[j::m]
        out[e0:e1] = (acc / float(m)).to(torch.bfloat16)
    return out


def main_queries(n_q, device, seed, *tags, outliers=False):
    """bf16 [n_q, 64, 512] ~ N(0,1)/sqrt(512)."""
    x = normal_rows(n_q * 64, 512, device, seed, *tags, outliers=outliers,
                    scale=1.0 / math.sqrt(512.0))
    return x.to(torch.bfloat16).view(n_q, 64, 512)
