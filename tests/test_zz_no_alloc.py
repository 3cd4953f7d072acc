"""The allocation-free fused scan + Top-K (csa2_index_topk_noalloc), through the
C ABI: on the GPU its indices equal csa2_index_topk's (with a caller workspace)
byte for byte, on two calls in a row (the second smaller, so stale contents of
the shared scratch from the first call would show), for a decode-shaped and a
prefill-shaped (narrowed) request; a request beyond the scratch is rejected
before anything runs."""

import ctypes

import numpy as np
import pytest
import torch

import compressed_kv_cache_02_amd as C
import synth
from tests.helpers import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(B, T, n_cap, seed, fp4=False):
    q = synth.e4m3_rows(B * T * 32, 128, DEV, seed, "naq").view(B, T, 32, 128)
    w = synth.head_weights(B * T, DEV, seed, "naw").view(B, T, 32)
    if fp4:
        kb = synth.normal_rows(B * n_cap, 128, DEV, seed, "nak4").to(torch.bfloat16)
        codes = torch.empty((B, n_cap, 64), dtype=torch.uint8, device=DEV)
        scl = torch.empty((B, n_cap, 4), dtype=torch.uint8, device=DEV)
        C.csa2_quantize_index_k(kb, None, codes, scl)
        keys = (codes, scl)
    else:
        keys = synth.e4m3_rows(B * n_cap, 128, DEV, seed, "nak").view(B, n_cap, 128)
    nv = np.minimum(n_cap, (n_cap - T + 1 + np.arange(T))[None, :].repeat(B, 0)).astype(np.int32)
    nv.flat[0] = min(n_cap, 777)
    return q, w, keys, torch.from_numpy(nv).to(DEV)


def _both(B, T, n_cap, seed, fp4=False):
    q, w, keys, n_vis = _case(B, T, n_cap, seed, fp4)
    ws = torch.empty(C.csa2_workspace_bytes(C.CSA2_OP_INDEX_TOPK, 0, B, T, n_cap),
                     dtype=torch.uint8, device=DEV)
    ref = torch.full((B, T, 512), -7, dtype=torch.int32, device=DEV)
    got = torch.full((B, T, 512), -9, dtype=torch.int32, device=DEV)
    C.csa2_index_topk(q, w, keys, n_vis, ref, ws)
    C.csa2_index_topk_noalloc(q, w, keys, n_vis, got)
    torch.cuda.synchronize()
    return to_np(got), to_np(ref)


@pytest.mark.parametrize("first,second", [
    ((2, 1, 300007, 1, False), (1, 1, 40003, 2, False)),      # decode-shaped, long then short
    ((1, 70, 60013, 3, False), (2, 5, 20011, 4, True)),       # prefill-shaped (narrowed), then FP4
])
def test_noalloc_matches_workspace_call_twice(first, second):
    print("[gpu-noalloc]", first, second, flush=True)
    for case in (first, second):
        got, ref = _both(*case)
        assert got.tobytes() == ref.tobytes(), case


def test_noalloc_rejects_requests_beyond_its_scratch():
    f = C.lib().csa2_index_topk_noalloc
    B, T, n_cap = 4096, 4, 1 << 20       # block maxima alone: 4,096 x 131,072 x 4 bytes
    assert C.csa2_workspace_bytes(C.CSA2_OP_INDEX_TOPK, 0, 1, B * T // 16, n_cap) > 0
    fake = ctypes.c_void_p(0x100000)
    status = f(fake, fake, fake, None, fake, B // 16, T, n_cap, fake, None)
    assert status == C.CSA2_EWORKSPACE
