"""The C ABI without a GPU: the library loads, exports every function
include/csa2.h declares, the host RoPE table matches the oracle bit for bit, and
every argument error is rejected before anything is launched.

Calls here that pass placeholder pointers are all ones the library must reject
during host-side validation; none of them can reach a kernel launch."""

import ctypes
import os
import re

import numpy as np
import pytest

import compressed_kv_cache_02_amd as C
from oracle import rope as OR

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

pytestmark = pytest.mark.skipif(not os.path.exists(C.lib_path()),
                                reason="libcsa2.so not built")

FAKE = 0x10000          # aligned placeholder, only used where validation must fail
FAKE_MIS = 0x10004      # misaligned placeholder


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


def test_header_functions_are_exported():
    names = declared_functions()
    assert len(names) == 16, names
    L = C.lib()
    for n in names:
        assert hasattr(L, n), n
    assert C.csa2_abi_version() == 7


def test_status_strings():
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(C.csa2_status_string(s), str)


def test_rope_table_matches_oracle_bit_for_bit():
    pos = np.array([0, 1, 2, 3, 1000, 131070, 524287 * 2, 1048575], dtype=np.int64)
    t = C.csa2_rope_table(pos)
    c, s = OR.rope_cos_sin(pos)
    assert np.array_equal(t[:, :, 0], c) and np.array_equal(t[:, :, 1], s)
    with pytest.raises(C.Csa2Error):
        C.csa2_rope_table(np.array([-1], dtype=np.int64))


def test_workspace_sizes():
    ws = C.csa2_workspace_bytes
    assert ws(C.CSA2_OP_INDEX_SCORE, 0, 8, 1, 1 << 20) == 0
    assert ws(C.CSA2_OP_TOPK, C.CSA2_REUSE, 8, 1, 1 << 20) == 0
    assert ws(C.CSA2_OP_TOPK, C.CSA2_REINDEX, 8, 1, 1 << 20) == 0
    assert ws(C.CSA2_OP_TOPK, C.CSA2_FULL, 8, 1, 16384) == 0
    assert ws(C.CSA2_OP_TOPK, C.CSA2_FULL, 8, 1, 1 << 20) > 0
    assert ws(C.CSA2_OP_BUILD_POOL, 0, 8, 1, 1 << 20) > 0
    assert ws(C.CSA2_OP_TOPK, C.CSA2_FULL, 0, 1, 100) == 0         # invalid sizes
    assert ws(C.CSA2_OP_TOPK, C.CSA2_FULL, 1, 1, 1 << 31) == 0
    for op in range(5):
        assert ws(op, 0, 3, 5, 1000) % 256 == 0
    assert ws(C.CSA2_OP_INDEX_TOPK, 0, 8, 1, 1 << 20) > ws(C.CSA2_OP_INDEX_TOPK, 0, 8, 1, 16384) > 0


def _p(x):
    return ctypes.c_void_p(x) if x else None


def test_index_score_rejects_bad_arguments():
    f = C.lib().csa2_index_score
    ok = dict(q=FAKE, w=FAKE, k=FAKE, nv=FAKE, pool=FAKE, s=FAKE, bm=None)

    def call(mode=0, B=1, T=1, n_cap=100, **kw):
        a = dict(ok)
        a.update(kw)
        return f(mode, _p(a["q"]), _p(a["w"]), _p(a["k"]), _p(a["nv"]), _p(a["pool"]), B, T,
                 n_cap, _p(a["s"]), _p(a["bm"]), None)

    assert call(mode=2) == C.CSA2_EINVAL                       # REUSE is not a scoring mode
    assert call(mode=7) == C.CSA2_EINVAL
    assert call(q=0) == C.CSA2_EINVAL
    assert call(k=FAKE_MIS) == C.CSA2_EINVAL
    assert call(mode=1, pool=0) == C.CSA2_EINVAL                # REINDEX needs a pool
    assert call(mode=1, bm=FAKE) == C.CSA2_EINVAL               # no block max in REINDEX
    assert call(s=0) == C.CSA2_EINVAL                           # FULL: nothing to write
    assert call(mode=1, s=0) == C.CSA2_EINVAL                   # REINDEX needs scores
    assert call(s=0, bm=FAKE_MIS) == C.CSA2_EINVAL
    assert call(B=0) == C.CSA2_EINVAL
    assert call(T=0) == C.CSA2_EINVAL
    assert call(n_cap=0) == C.CSA2_EINVAL
    assert call(n_cap=1 << 31) == C.CSA2_EINVAL
    assert call(B=300, T=300) == C.CSA2_EINVAL                  # too many queries


def test_topk_and_pool_reject_bad_arguments():
    # csa2_topk(mode, scores, bmax, n_vis, pool, src_idx, B, T, n_cap, idx, ws, ws_bytes, stream)
    f = C.lib().csa2_topk
    N = 1 << 20          # large enough that FULL needs a workspace
    F, M = _p(FAKE), _p(FAKE_MIS)
    assert f(0, F, None, F, None, None, 1, 1, N, F, None, 0, None) == C.CSA2_EWORKSPACE
    assert f(0, F, None, F, None, None, 1, 1, N, F, F, 16, None) == C.CSA2_EWORKSPACE
    assert f(1, F, None, F, None, None, 1, 1, 100, F, F, 1 << 30, None) == C.CSA2_EINVAL  # no pool
    assert f(1, F, F, F, F, None, 1, 1, 100, F, F, 1 << 30, None) == C.CSA2_EINVAL       # bmax
    assert f(2, None, None, None, None, None, 1, 1, 100, F, None, 0, None) == C.CSA2_EINVAL
    assert f(5, F, None, F, None, None, 1, 1, 100, F, F, 1 << 30, None) == C.CSA2_EINVAL
    assert f(0, F, None, F, None, None, 1, 1, 100, M, F, 1 << 30, None) == C.CSA2_EINVAL
    assert f(0, F, M, F, None, None, 1, 1, 100, F, F, 1 << 30, None) == C.CSA2_EINVAL
    assert f(0, F, None, F, M, None, 1, 1, 100, F, F, 1 << 30, None) == C.CSA2_EINVAL
    assert f(0, None, None, F, None, None, 1, 1, 100, F, F, 1 << 30, None) == C.CSA2_EINVAL
    g = C.lib().csa2_build_pool
    assert g(F, 1, F, 1, 1, N, F, None, 0, None) == C.CSA2_EWORKSPACE
    assert g(F, 1, F, 1, 1, N, F, F, 8, None) == C.CSA2_EWORKSPACE
    assert g(None, 1, F, 1, 1, N, F, F, 1 << 30, None) == C.CSA2_EINVAL
    assert g(F, 1, F, 1, 0, N, F, F, 1 << 30, None) == C.CSA2_EINVAL


def test_attn_and_quantize_reject_bad_arguments():
    f = C.lib().csa2_sparse_attn
    args = [_p(FAKE)] * 6
    assert f(*args, 1, 1, 100, 0, ctypes.c_float(1.0), _p(FAKE), _p(FAKE), 1 << 30, None) == C.CSA2_EINVAL
    assert f(*args, 1, 1, 100, 128, ctypes.c_float(float("nan")), _p(FAKE), _p(FAKE), 1 << 30, None) == C.CSA2_EINVAL
    bad = list(args)
    bad[2] = None
    assert f(*bad, 1, 1, 100, 128, ctypes.c_float(1.0), _p(FAKE), _p(FAKE), 1 << 30, None) == C.CSA2_EINVAL
    # up to 12 queries split their keys over slices whose partial results need
    # a workspace; without one the call is rejected before any launch
    assert C.csa2_workspace_bytes(C.CSA2_OP_SPARSE_ATTN, 0, 1, 1, 100) > 0
    assert C.csa2_workspace_bytes(C.CSA2_OP_SPARSE_ATTN, 0, 3, 4, 100) > 0
    assert C.csa2_workspace_bytes(C.CSA2_OP_SPARSE_ATTN, 0, 1, 13, 100) == 0
    assert C.csa2_workspace_bytes(C.CSA2_OP_SPARSE_ATTN, 0, 1, 64, 100) == 0
    assert C.csa2_workspace_bytes(C.CSA2_OP_SPARSE_ATTN, 0, 8, 512, 100) == 0
    assert f(*args, 1, 1, 100, 128, ctypes.c_float(1.0), _p(FAKE), None, 0, None) == C.CSA2_EWORKSPACE
    assert f(*args, 1, 1, 100, 128, ctypes.c_float(1.0), _p(FAKE), _p(FAKE), 64, None) == C.CSA2_EWORKSPACE
    r = C.lib().csa2_sparse_attn_ring
    assert r(*args, 1, 1, 100, 0, ctypes.c_float(1.0), _p(FAKE), _p(FAKE), 1 << 30, None) == C.CSA2_EINVAL
    assert r(*args, 1, 1, 100, 128, ctypes.c_float(float("inf")), _p(FAKE), _p(FAKE), 1 << 30,
             None) == C.CSA2_EINVAL
    assert r(*bad, 1, 1, 100, 128, ctypes.c_float(1.0), _p(FAKE), _p(FAKE), 1 << 30, None) == C.CSA2_EINVAL
    assert r(*args, 1, 1, 100, 128, ctypes.c_float(1.0), _p(FAKE_MIS), _p(FAKE), 1 << 30,
             None) == C.CSA2_EINVAL
    assert r(*args, 1, 1, 100, 128, ctypes.c_float(1.0), _p(FAKE), None, 0, None) == C.CSA2_EWORKSPACE
    q = C.lib().csa2_quantize_kv
    assert q(_p(FAKE), _p(FAKE), None, -1, _p(FAKE), 10, None) == C.CSA2_EINVAL
    assert q(_p(FAKE), _p(FAKE), None, 11, _p(FAKE), 10, None) == C.CSA2_EINVAL   # rows beyond the cache
    assert q(None, _p(FAKE), None, 4, _p(FAKE), 10, None) == C.CSA2_EINVAL
    assert q(_p(FAKE), _p(FAKE), _p(FAKE_MIS), 4, _p(FAKE), 10, None) == C.CSA2_EINVAL
    assert q(_p(FAKE), _p(FAKE), None, 0, _p(FAKE), 10, None) == C.CSA2_OK           # nothing to do


def test_fp4_key_calls_reject_bad_arguments():
    q = C.lib().csa2_quantize_index_k
    F, M = _p(FAKE), _p(FAKE_MIS)
    assert q(F, None, -1, F, F, 10, None) == C.CSA2_EINVAL
    assert q(F, None, 11, F, F, 10, None) == C.CSA2_EINVAL      # rows beyond the buffers
    assert q(F, None, 4, F, F, 0, None) == C.CSA2_EINVAL
    assert q(None, None, 4, F, F, 10, None) == C.CSA2_EINVAL
    assert q(F, None, 4, F, _p(FAKE + 2), 10, None) == C.CSA2_EINVAL
    assert q(F, M, 4, F, F, 10, None) == C.CSA2_EINVAL
    assert q(F, None, 0, F, F, 10, None) == C.CSA2_OK            # nothing to do
    f = C.lib().csa2_index_score_fp4k

    def call(mode=0, B=1, T=1, n_cap=100, **kw):
        a = dict(q=FAKE, w=FAKE, k=FAKE, ks=FAKE, nv=FAKE, pool=FAKE, s=FAKE, bm=None)
        a.update(kw)
        return f(mode, _p(a["q"]), _p(a["w"]), _p(a["k"]), _p(a["ks"]), _p(a["nv"]),
                 _p(a["pool"]), B, T, n_cap, _p(a["s"]), _p(a["bm"]), None)

    assert call(mode=2) == C.CSA2_EINVAL
    assert call(ks=0) == C.CSA2_EINVAL                          # scales are required
    assert call(ks=FAKE + 2) == C.CSA2_EINVAL                  # scales: 4-byte aligned
    assert call(mode=1, pool=0) == C.CSA2_EINVAL
    assert call(mode=1, bm=FAKE) == C.CSA2_EINVAL
    assert call(s=0) == C.CSA2_EINVAL
    assert call(n_cap=0) == C.CSA2_EINVAL
    assert call(B=300, T=300) == C.CSA2_EINVAL


def test_write_path_helpers_reject_bad_arguments():
    F, M = _p(FAKE), _p(FAKE_MIS)
    c = C.lib().csa2_compress_tokens
    assert c(F, 4, 512, 0, F, None) == C.CSA2_EINVAL             # m < 1
    assert c(F, 4, 512, 65, F, None) == C.CSA2_EINVAL            # m beyond the limit
    assert c(F, 4, 500, 2, F, None) == C.CSA2_EINVAL             # width not a multiple of 8
    assert c(F, 4, 16384, 2, F, None) == C.CSA2_EINVAL
    assert c(F, -1, 512, 2, F, None) == C.CSA2_EINVAL
    assert c(M, 4, 512, 2, F, None) == C.CSA2_EINVAL
    assert c(F, 4, 512, 2, None, None) == C.CSA2_EINVAL
    assert c(F, 0, 512, 2, F, None) == C.CSA2_OK                 # nothing to do
    q = C.lib().csa2_quantize_e4m3
    assert q(F, 4, 512, None, F, 3, None) == C.CSA2_EINVAL      # rows beyond the output
    assert q(F, 4, 12, None, F, 10, None) == C.CSA2_EINVAL
    assert q(F, 4, 512, M, F, 10, None) == C.CSA2_EINVAL
    assert q(None, 4, 512, None, F, 10, None) == C.CSA2_EINVAL
    assert q(F, 4, 512, None, F, 0, None) == C.CSA2_EINVAL
    assert q(F, 0, 512, None, F, 10, None) == C.CSA2_OK


def test_index_topk_rejects_bad_arguments():
    f = C.lib().csa2_index_topk
    F, M = _p(FAKE), _p(FAKE_MIS)
    need = C.csa2_workspace_bytes(C.CSA2_OP_INDEX_TOPK, 0, 1, 1, 100000)
    assert f(F, F, F, None, F, 1, 1, 100000, F, None, 0, None) == C.CSA2_EWORKSPACE
    assert f(F, F, F, None, F, 1, 1, 100000, F, F, need - 1, None) == C.CSA2_EWORKSPACE
    assert f(F, F, F, None, F, 1, 1, (1 << 20) + 1, F, F, 1 << 40, None) == C.CSA2_EUNSUPPORTED
    assert f(F, F, M, None, F, 1, 1, 100000, F, F, need, None) == C.CSA2_EINVAL
    assert f(F, F, F, _p(FAKE + 2), F, 1, 1, 100000, F, F, need, None) == C.CSA2_EINVAL
    assert f(F, F, F, None, F, 1, 1, 100000, M, F, need, None) == C.CSA2_EINVAL
    assert f(F, F, F, None, F, 0, 1, 100000, F, F, need, None) == C.CSA2_EINVAL
    assert f(F, F, F, None, F, 1, 1, 100000, F, M, need, None) == C.CSA2_EINVAL


def test_group_fuses_only_within_the_fused_entry_limit():
    """The automatic choice of the fused scan + Top-K (host logic only): long
    decode contexts, and every step whose scan is prefill-shaped (its FP8
    scores are re-scored FP32-accurately only inside the fused call)."""
    from compressed_kv_cache_02_amd.group import fused_topk_auto
    assert C.INDEX_TOPK_MAX_CAP == 1 << 20
    assert fused_topk_auto(1, 1 << 20) and fused_topk_auto(1, 524288)
    assert fused_topk_auto(4096, 133120) and fused_topk_auto(64, 1000)
    assert fused_topk_auto(63, 200000) and fused_topk_auto(4, 8192)
    assert not fused_topk_auto(1, 65536) and not fused_topk_auto(3, 200000)
    assert not fused_topk_auto(1, (1 << 20) + 8) and not fused_topk_auto(4096, 1 << 21)


def test_binding_constants_match_the_header():
    """Every numeric #define of csa2.h that the binding mirrors has the same value."""
    import re
    text = open(os.path.join(ROOT, "include", "csa2.h")).read()
    defs = {m.group(1): int(m.group(2)) for m in
            re.finditer(r"^#define CSA2_([A-Z0-9_]+)\s+(-?\d+)\b", text, re.M)}
    mirrored = {"IDX_FP4_CODE_BYTES": C.IDX_FP4_CODE_BYTES, "IDX_FP4_SCALES": C.IDX_FP4_SCALES,
                "INDEX_TOPK_MAX_CAP": C.INDEX_TOPK_MAX_CAP,
                "NOALLOC_SCRATCH_BYTES": C.NOALLOC_SCRATCH_BYTES,
                "PREFILL_MIN_T_FP8": C.PREFILL_MIN_T_FP8, "PREFILL_MIN_T_FP4": C.PREFILL_MIN_T_FP4}
    for k, v in mirrored.items():
        assert defs[k] == v, k
    for k in ("IDX_HEADS", "IDX_DIM", "HEADS", "DIM", "ROW_BYTES", "TOPK", "POOL_BLOCKS", "BLOCK",
              "POOL_CAND", "WINDOW"):
        if k in defs:
            assert defs[k] == getattr(C, k), k


def test_zero_rows_are_a_no_op():
    """Appending no rows is valid and launches nothing (no pointer is read), while
    negative counts and empty destinations stay errors."""
    L = C.lib()
    assert L.csa2_quantize_kv(None, None, None, 0, None, 1, None) == C.CSA2_OK
    assert L.csa2_quantize_kv(None, None, None, -1, None, 1, None) == C.CSA2_EINVAL
    assert L.csa2_quantize_kv(None, None, None, 0, None, 0, None) == C.CSA2_EINVAL
    assert L.csa2_quantize_e4m3(None, 0, 512, None, None, 1, None) == C.CSA2_OK
    assert L.csa2_quantize_e4m3(None, 0, 500, None, None, 1, None) == C.CSA2_EINVAL
    assert L.csa2_quantize_index_k(None, None, 0, None, None, 1, None) == C.CSA2_OK
    assert L.csa2_quantize_index_k(None, None, -2, None, None, 1, None) == C.CSA2_EINVAL
    assert L.csa2_compress_tokens(None, 0, 512, 2, None, None) == C.CSA2_OK
