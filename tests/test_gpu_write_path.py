"""GPU parity of the rest of the write path against the oracle, through the C
ABI: the m-token mean compressor and the E4M3 append (window rows, FP8 indexer
keys) bit for bit, and one decode step's appends composed with the FP4 packer."""

import numpy as np
import pytest
import torch

import compressed_kv_cache_02_amd as C
from oracle import compress as OC
from oracle import formats as OF
from oracle import rope as OR
import synth
from tests.helpers import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _stage(*a):
    print("[gpu-test]", *a, flush=True)


def _bits(t):
    return to_np(t.view(torch.int16)).view(np.uint16)


def _special_rows(width, huge=True):
    """bf16 rows with -0, zeros, large and subnormal values and every E4M3 midpoint
    (``huge`` adds 3e38, whose pairwise sums would overflow the compressor)."""
    mids = []
    for c in range(126):
        mids.append((OF.e4m3_value_of_code(c) + OF.e4m3_value_of_code(c + 1)) / 2.0)
    vals = np.array(mids + [0.0, -0.0, 448.0, 449.0, 464.0, 480.0, 1e6, 2.0 ** -133, 2.0 ** -126,
                            2.0 ** -10, 3 * 2.0 ** -10] + ([3.0e38] if huge else []),
                    dtype=np.float32)
    vals = np.concatenate([vals, -vals])
    n = -(-vals.size // width)
    rows = np.zeros(n * width, dtype=np.float32)
    rows[:vals.size] = vals
    t = torch.from_numpy(rows.reshape(n, width)).to(torch.bfloat16)
    return t


@pytest.mark.parametrize("n_tok,width,m", [(4099, 512, 2), (1001, 128, 2), (777, 512, 3),
                                           (64, 512, 1), (5, 128, 4)])
def test_compress_tokens_bitexact(n_tok, width, m):
    _stage("compress", n_tok, width, m)
    x = synth.normal_rows(n_tok, width, DEV, n_tok, "tok", outliers=(width == 512)).to(torch.bfloat16)
    sp = _special_rows(width, huge=False).to(DEV)
    x = torch.cat([sp, x])[:n_tok].contiguous() if n_tok >= sp.shape[0] else x
    n_out = -(-n_tok // m)
    out = torch.empty((n_out, width), dtype=torch.bfloat16, device=DEV)
    C.csa2_compress_tokens(x, m, out)
    torch.cuda.synchronize()
    want = OC.compress_mean(_bits(x), m)
    assert np.array_equal(_bits(out), want)


@pytest.mark.parametrize("n,width", [(3001, 512), (777, 128)])
def test_quantize_e4m3_bitexact(n, width):
    _stage("quantize_e4m3", n, width)
    x = synth.normal_rows(n, width, DEV, n, "e4", scale=1.0).to(torch.bfloat16)
    x = x * torch.exp2(torch.randint(-12, 10, (n, 1), device=DEV).float()).to(torch.bfloat16)
    x = torch.cat([_special_rows(width).to(DEV), x]).contiguous()
    n = x.shape[0]
    out = torch.empty((n, width), dtype=torch.uint8, device=DEV)
    C.csa2_quantize_e4m3(x, None, out)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(out), OF.e4m3_encode(x.float().cpu().numpy()))


def test_quantize_e4m3_slots():
    _stage("quantize_e4m3 slots")
    n, rows, width = 30, 50, 512
    x = synth.normal_rows(n, width, DEV, 3, "e4s").to(torch.bfloat16)
    slot = (torch.arange(n, dtype=torch.int64, device=DEV) * 7) % rows
    slot[3] = -1
    slot[4] = rows
    out = torch.full((rows, width), 0x5A, dtype=torch.uint8, device=DEV)
    C.csa2_quantize_e4m3(x, slot, out)
    torch.cuda.synchronize()
    want = np.full((rows, width), 0x5A, np.uint8)
    codes = OF.e4m3_encode(x.float().cpu().numpy())
    for i, s in enumerate(to_np(slot)):
        if 0 <= s < rows:
            want[s] = codes[i]
    assert np.array_equal(to_np(out), want)


def test_decode_step_appends_compose():
    """One decode step at m = 2 for B sequences whose open group just completed:
    the token pair is compressed, the main-KV entry RoPE'd and packed into the
    newest cache slot, the pair's indexer key compressed and appended as E4M3,
    and the new token's window row appended as E4M3; every byte as the oracle's
    chain computes it."""
    B, m, n_cap, S = 5, 2, 100, 128
    _stage("decode step appends", B)
    tok = synth.normal_rows(B * m, 512, DEV, 8, "wtok", outliers=True).to(torch.bfloat16)
    ktok = synth.normal_rows(B * m, 128, DEV, 8, "wk").to(torch.bfloat16)
    entry = torch.empty((B, 512), dtype=torch.bfloat16, device=DEV)
    kentry = torch.empty((B, 128), dtype=torch.bfloat16, device=DEV)
    C.csa2_compress_tokens(tok, m, entry)
    C.csa2_compress_tokens(ktok, m, kentry)
    j = n_cap - 1
    slot = torch.arange(B, dtype=torch.int64, device=DEV) * n_cap + j
    cache = torch.zeros((B, n_cap, 288), dtype=torch.uint8, device=DEV)
    cs = torch.from_numpy(C.csa2_rope_table(np.full(B, j * m, dtype=np.int64))).to(DEV)
    C.csa2_quantize_kv(entry, cs, slot, cache)
    k_idx = torch.zeros((B, n_cap, 128), dtype=torch.uint8, device=DEV)
    C.csa2_quantize_e4m3(kentry, slot, k_idx)
    swa = torch.zeros((B, S, 512), dtype=torch.uint8, device=DEV)
    wslot = torch.arange(B, dtype=torch.int64, device=DEV) * S + (S - 1)
    new_tok = tok.view(B, m, 512)[:, m - 1].contiguous()
    C.csa2_quantize_e4m3(new_tok, wslot, swa)
    torch.cuda.synchronize()
    e_bits = OC.compress_mean(_bits(tok), m)                       # [B, 512]
    assert np.array_equal(_bits(entry), e_bits)
    rows = OF.quantize_rows(OR.apply_rope(OC.bf16_bits_to_f32(e_bits), [j * m] * B))
    assert np.array_equal(to_np(cache)[:, j], rows)
    k_bits = OC.compress_mean(_bits(ktok), m)
    assert np.array_equal(to_np(k_idx)[:, j], OF.e4m3_encode(OC.bf16_bits_to_f32(k_bits)))
    assert np.array_equal(to_np(swa)[:, S - 1], OF.e4m3_encode(new_tok.float().cpu().numpy()))
    assert not to_np(cache)[:, :j].any() and not to_np(swa)[:, :S - 1].any()
