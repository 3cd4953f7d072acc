"""Python binding of libcsa2 (the CSA2 per-layer hot path on MI355X / gfx950).

Argument marshalling only: every function below takes torch tensors that live
on the GPU, checks dtypes/shapes, and passes their device pointers and sizes to
the C function of the same name in libcsa2.so (see include/csa2.h for the
contract). All computation happens in the library's HIP kernels; there is no
fallback. If the library is missing, importing works but the first call raises.
"""

import ctypes
import os

import numpy as np

__all__ = [
    "CSA2_FULL", "CSA2_REINDEX", "CSA2_REUSE", "CSA2_OP_INDEX_SCORE", "CSA2_OP_BUILD_POOL",
    "CSA2_OP_TOPK", "CSA2_OP_SPARSE_ATTN", "Csa2Error", "lib", "lib_path",
    "csa2_abi_version", "csa2_status_string", "csa2_workspace_bytes", "csa2_rope_table",
    "csa2_quantize_kv", "csa2_index_score", "csa2_build_pool", "csa2_topk",
    "csa2_sparse_attn", "csa2_quantize_index_k", "csa2_index_score_fp4k",
    "csa2_compress_tokens", "csa2_quantize_e4m3", "csa2_index_topk", "CSA2_OP_INDEX_TOPK",
    "csa2_sparse_attn_ring", "csa2_index_topk_noalloc", "NOALLOC_SCRATCH_BYTES",
]

CSA2_FULL, CSA2_REINDEX, CSA2_REUSE = 0, 1, 2
CSA2_OP_INDEX_SCORE, CSA2_OP_BUILD_POOL, CSA2_OP_TOPK, CSA2_OP_SPARSE_ATTN = 0, 1, 2, 3
CSA2_OP_INDEX_TOPK = 4
CSA2_OK, CSA2_EINVAL, CSA2_EUNSUPPORTED, CSA2_EWORKSPACE, CSA2_EHIP = 0, -1, -2, -3, -4

IDX_HEADS, IDX_DIM, HEADS, DIM = 32, 128, 64, 512
ROW_BYTES, TOPK, POOL_BLOCKS, BLOCK, POOL_CAND, WINDOW = 288, 512, 2048, 8, 16384, 128
IDX_FP4_CODE_BYTES, IDX_FP4_SCALES = 64, 4
INDEX_TOPK_MAX_CAP = 1 << 20        # longest context csa2_index_topk serves
NOALLOC_SCRATCH_BYTES = 32 << 20    # library-owned scratch of csa2_index_topk_noalloc
# query tokens per sequence from which a Full scan is prefill-shaped (E4M3 / FP4 keys)
PREFILL_MIN_T_FP8, PREFILL_MIN_T_FP4 = 4, 5

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_f32 = ctypes.c_float

_SIGS = {
    "csa2_abi_version": (_i32, []),
    "csa2_status_string": (ctypes.c_char_p, [_i32]),
    "csa2_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i64]),
    "csa2_rope_table": (_i32, [_vp, _i64, _vp]),
    "csa2_quantize_kv": (_i32, [_vp, _vp, _vp, _i64, _vp, _i64, _vp]),
    "csa2_index_score": (_i32, [_i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _vp, _vp, _vp]),
    "csa2_index_topk": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _vp, _vp, _sz, _vp]),
    "csa2_index_topk_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _vp, _vp]),
    "csa2_compress_tokens": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp]),
    "csa2_quantize_e4m3": (_i32, [_vp, _i64, _i32, _vp, _vp, _i64, _vp]),
    "csa2_quantize_index_k": (_i32, [_vp, _vp, _i64, _vp, _vp, _i64, _vp]),
    "csa2_index_score_fp4k": (_i32, [_i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _vp, _vp,
                                     _vp]),
    "csa2_build_pool": (_i32, [_vp, _i32, _vp, _i32, _i32, _i64, _vp, _vp, _sz, _vp]),
    "csa2_topk": (_i32, [_i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _vp, _vp, _sz, _vp]),
    "csa2_sparse_attn": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i32, _f32,
                                _vp, _vp, _sz, _vp]),
    "csa2_sparse_attn_ring": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i32, _f32,
                                     _vp, _vp, _sz, _vp]),
}


class Csa2Error(RuntimeError):
    def __init__(self, name, status):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (name, csa2_status_string(status), status))


def lib_path():
    return os.environ.get("CSA2_LIB", os.path.join(_HERE, "libcsa2.so"))


def lib():
    """The loaded libcsa2.so (ctypes). Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError("libcsa2.so not found at %s; build it with "
                               "`python -m compressed_kv_cache_02_amd.build`" % path)
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _check(name, status):
    if status != CSA2_OK:
        raise Csa2Error(name, status)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _expect(t, name, dtype, shape=None, ndim=None):
    import torch
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims" % (name, ndim))
    del torch


def csa2_abi_version():
    return lib().csa2_abi_version()


def csa2_status_string(status):
    return lib().csa2_status_string(status).decode()


def csa2_workspace_bytes(op, mode, B, T, n_cap):
    return int(lib().csa2_workspace_bytes(op, mode, B, T, n_cap))


def csa2_rope_table(positions):
    """Host RoPE table: float32 [n, 32, 2] (cos, sin) for int64 positions."""
    pos = np.ascontiguousarray(positions, dtype=np.int64).reshape(-1)
    out = np.empty((pos.shape[0], 32, 2), dtype=np.float32)
    _check("csa2_rope_table", lib().csa2_rope_table(pos.ctypes.data_as(_vp), pos.shape[0],
                                                    out.ctypes.data_as(_vp)))
    return out


def csa2_quantize_kv(kv_bf16, cos_sin, dst_slot, cache, stream=None):
    """kv_bf16 [n,512] bf16, cos_sin [n,32,2] f32, dst_slot [n] int64 or None,
    cache [rows,288] uint8 (any leading dims flattened)."""
    import torch
    n = kv_bf16.shape[0]
    _expect(kv_bf16, "kv_bf16", torch.bfloat16, (n, DIM))
    _expect(cos_sin, "cos_sin", torch.float32, (n, 32, 2))
    if dst_slot is not None:
        _expect(dst_slot, "dst_slot", torch.int64, (n,))
    _expect(cache, "cache", torch.uint8)
    rows = cache.numel() // ROW_BYTES
    _check("csa2_quantize_kv", lib().csa2_quantize_kv(_p(kv_bf16), _p(cos_sin), _p(dst_slot), n,
                                                      _p(cache), rows, _stream(stream)))


def csa2_index_score(mode, q_idx, w, k_idx, n_vis, pool, scores, bmax=None, stream=None):
    """q_idx [B,T,32,128] uint8, w [B,T,32] f32, k_idx [B,n_cap,128] uint8,
    n_vis [B,T] int32, pool [B,T,2048] int32 (REINDEX), scores f32
    ([B,T,n_cap] FULL / [B,T,16384] REINDEX; None in FULL mode writes only
    the block maxima), bmax [B,T,ceil(n_cap/8)] f32 or None."""
    import torch
    B, T = q_idx.shape[0], q_idx.shape[1]
    n_cap = k_idx.shape[1]
    _expect(q_idx, "q_idx", torch.uint8, (B, T, IDX_HEADS, IDX_DIM))
    _expect(w, "w", torch.float32, (B, T, IDX_HEADS))
    _expect(k_idx, "k_idx", torch.uint8, (B, n_cap, IDX_DIM))
    _expect(n_vis, "n_vis", torch.int32, (B, T))
    n_items = n_cap if mode == CSA2_FULL else POOL_CAND
    if scores is not None or mode != CSA2_FULL:
        _expect(scores, "scores", torch.float32, (B, T, n_items))
    if pool is not None:
        _expect(pool, "pool", torch.int32, (B, T, POOL_BLOCKS))
    if bmax is not None:
        _expect(bmax, "bmax", torch.float32, (B, T, (n_cap + BLOCK - 1) // BLOCK))
    _check("csa2_index_score", lib().csa2_index_score(mode, _p(q_idx), _p(w), _p(k_idx),
                                                      _p(n_vis), _p(pool), B, T, n_cap,
                                                      _p(scores), _p(bmax), _stream(stream)))


def csa2_index_topk(q_idx, w, keys, n_vis, idx, ws, stream=None):
    """Fused Full scan + Top-512. keys: FP8 keys [B,n_cap,128] uint8, or a pair
    (codes [B,n_cap,64], scales [B,n_cap,4]) of FP4 keys; idx [B,T,512] int32;
    ws a uint8 device tensor of csa2_workspace_bytes(CSA2_OP_INDEX_TOPK, ...) bytes."""
    import torch
    B, T = q_idx.shape[0], q_idx.shape[1]
    if isinstance(keys, tuple):
        k, ks = keys
        n_cap = k.shape[1]
        _expect(k, "k_codes", torch.uint8, (B, n_cap, IDX_FP4_CODE_BYTES))
        _expect(ks, "k_scales", torch.uint8, (B, n_cap, IDX_FP4_SCALES))
    else:
        k, ks = keys, None
        n_cap = k.shape[1]
        _expect(k, "k_idx", torch.uint8, (B, n_cap, IDX_DIM))
    _expect(q_idx, "q_idx", torch.uint8, (B, T, IDX_HEADS, IDX_DIM))
    _expect(w, "w", torch.float32, (B, T, IDX_HEADS))
    _expect(n_vis, "n_vis", torch.int32, (B, T))
    _expect(idx, "idx", torch.int32, (B, T, TOPK))
    _expect(ws, "ws", torch.uint8)
    _check("csa2_index_topk", lib().csa2_index_topk(_p(q_idx), _p(w), _p(k), _p(ks), _p(n_vis), B,
                                                    T, n_cap, _p(idx), _p(ws), ws.numel(),
                                                    _stream(stream)))


def csa2_index_topk_noalloc(q_idx, w, keys, n_vis, idx, stream=None):
    """csa2_index_topk with the library's own scratch (no workspace argument;
    allocates nothing). Calls that overlap on one GPU race."""
    import torch
    B, T = q_idx.shape[0], q_idx.shape[1]
    if isinstance(keys, tuple):
        k, ks = keys
        n_cap = k.shape[1]
        _expect(k, "k_codes", torch.uint8, (B, n_cap, IDX_FP4_CODE_BYTES))
        _expect(ks, "k_scales", torch.uint8, (B, n_cap, IDX_FP4_SCALES))
    else:
        k, ks = keys, None
        n_cap = k.shape[1]
        _expect(k, "k_idx", torch.uint8, (B, n_cap, IDX_DIM))
    _expect(q_idx, "q_idx", torch.uint8, (B, T, IDX_HEADS, IDX_DIM))
    _expect(w, "w", torch.float32, (B, T, IDX_HEADS))
    _expect(n_vis, "n_vis", torch.int32, (B, T))
    _expect(idx, "idx", torch.int32, (B, T, TOPK))
    _check("csa2_index_topk_noalloc", lib().csa2_index_topk_noalloc(
        _p(q_idx), _p(w), _p(k), _p(ks), _p(n_vis), B, T, n_cap, _p(idx), _stream(stream)))


def csa2_compress_tokens(tokens_bf16, m, out_bf16, stream=None):
    """tokens_bf16 [n_tok, width] bf16 -> out_bf16 [ceil(n_tok/m), width] bf16
    (mean of every m consecutive rows)."""
    import torch
    n_tok, width = tokens_bf16.shape
    _expect(tokens_bf16, "tokens_bf16", torch.bfloat16, (n_tok, width))
    _expect(out_bf16, "out_bf16", torch.bfloat16, ((n_tok + m - 1) // m, width))
    _check("csa2_compress_tokens", lib().csa2_compress_tokens(_p(tokens_bf16), n_tok, width, m,
                                                              _p(out_bf16), _stream(stream)))


def csa2_quantize_e4m3(rows_bf16, dst_slot, out, stream=None):
    """rows_bf16 [n, width] bf16 -> E4M3 codes in out [rows, width] uint8 (any
    leading dims of out flattened) at dst_slot [n] int64 (None: row r -> r)."""
    import torch
    n, width = rows_bf16.shape
    _expect(rows_bf16, "rows_bf16", torch.bfloat16, (n, width))
    if dst_slot is not None:
        _expect(dst_slot, "dst_slot", torch.int64, (n,))
    _expect(out, "out", torch.uint8)
    if out.shape[-1] != width:
        raise ValueError("out rows must be %d wide" % width)
    _check("csa2_quantize_e4m3", lib().csa2_quantize_e4m3(_p(rows_bf16), n, width, _p(dst_slot),
                                                          _p(out), out.numel() // width,
                                                          _stream(stream)))


def csa2_quantize_index_k(k_bf16, dst_slot, codes, scales, stream=None):
    """k_bf16 [n,128] bf16, dst_slot [n] int64 or None, codes [rows,64] uint8,
    scales [rows,4] uint8 (any leading dims of codes/scales flattened)."""
    import torch
    n = k_bf16.shape[0]
    _expect(k_bf16, "k_bf16", torch.bfloat16, (n, IDX_DIM))
    if dst_slot is not None:
        _expect(dst_slot, "dst_slot", torch.int64, (n,))
    _expect(codes, "codes", torch.uint8)
    _expect(scales, "scales", torch.uint8)
    rows = codes.numel() // IDX_FP4_CODE_BYTES
    if codes.shape[-1] != IDX_FP4_CODE_BYTES or scales.shape[-1] != IDX_FP4_SCALES or \
            scales.numel() // IDX_FP4_SCALES != rows:
        raise ValueError("codes must be [..., 64] and scales [..., 4] with the same rows")
    _check("csa2_quantize_index_k", lib().csa2_quantize_index_k(_p(k_bf16), _p(dst_slot), n,
                                                                _p(codes), _p(scales), rows,
                                                                _stream(stream)))


def csa2_index_score_fp4k(mode, q_idx, w, k_codes, k_scales, n_vis, pool, scores, bmax=None,
                          stream=None):
    """As csa2_index_score with FP4 indexer keys: k_codes [B,n_cap,64] uint8,
    k_scales [B,n_cap,4] uint8."""
    import torch
    B, T = q_idx.shape[0], q_idx.shape[1]
    n_cap = k_codes.shape[1]
    _expect(q_idx, "q_idx", torch.uint8, (B, T, IDX_HEADS, IDX_DIM))
    _expect(w, "w", torch.float32, (B, T, IDX_HEADS))
    _expect(k_codes, "k_codes", torch.uint8, (B, n_cap, IDX_FP4_CODE_BYTES))
    _expect(k_scales, "k_scales", torch.uint8, (B, n_cap, IDX_FP4_SCALES))
    _expect(n_vis, "n_vis", torch.int32, (B, T))
    n_items = n_cap if mode == CSA2_FULL else POOL_CAND
    if scores is not None or mode != CSA2_FULL:
        _expect(scores, "scores", torch.float32, (B, T, n_items))
    if pool is not None:
        _expect(pool, "pool", torch.int32, (B, T, POOL_BLOCKS))
    if bmax is not None:
        _expect(bmax, "bmax", torch.float32, (B, T, (n_cap + BLOCK - 1) // BLOCK))
    _check("csa2_index_score_fp4k", lib().csa2_index_score_fp4k(
        mode, _p(q_idx), _p(w), _p(k_codes), _p(k_scales), _p(n_vis), _p(pool), B, T, n_cap,
        _p(scores), _p(bmax), _stream(stream)))


def csa2_build_pool(src, is_bmax, n_vis, n_cap, pool, ws, stream=None):
    """src: block maxima [B,T,ceil(n_cap/8)] (is_bmax) or scores [B,T,n_cap];
    pool [B,T,2048] int32; ws a uint8 device tensor."""
    import torch
    B, T = n_vis.shape
    _expect(src, "src", torch.float32, (B, T, (n_cap + BLOCK - 1) // BLOCK if is_bmax else n_cap))
    _expect(n_vis, "n_vis", torch.int32, (B, T))
    _expect(pool, "pool", torch.int32, (B, T, POOL_BLOCKS))
    _check("csa2_build_pool", lib().csa2_build_pool(_p(src), 1 if is_bmax else 0, _p(n_vis), B,
                                                    T, n_cap, _p(pool), _p(ws),
                                                    0 if ws is None else ws.numel(),
                                                    _stream(stream)))


def csa2_topk(mode, scores, n_vis, pool, src_idx, n_cap, idx, ws, stream=None, bmax=None):
    """idx [B,T,512] int32 written; FULL scores [B,T,n_cap] (optional helpers:
    bmax [B,T,ceil(n_cap/8)] and the pool [B,T,2048] built from the same
    scores), REINDEX scores [B,T,16384] with pool [B,T,2048]; REUSE copies
    src_idx [B,T,512]."""
    import torch
    B, T = idx.shape[0], idx.shape[1]
    _expect(idx, "idx", torch.int32, (B, T, TOPK))
    if mode == CSA2_REUSE:
        _expect(src_idx, "src_idx", torch.int32, (B, T, TOPK))
    else:
        _expect(scores, "scores", torch.float32,
                (B, T, n_cap if mode == CSA2_FULL else POOL_CAND))
        _expect(n_vis, "n_vis", torch.int32, (B, T))
        if pool is not None:
            _expect(pool, "pool", torch.int32, (B, T, POOL_BLOCKS))
        if bmax is not None:
            _expect(bmax, "bmax", torch.float32, (B, T, (n_cap + BLOCK - 1) // BLOCK))
    _check("csa2_topk", lib().csa2_topk(mode, _p(scores), _p(bmax), _p(n_vis), _p(pool),
                                        _p(src_idx), B, T, n_cap, _p(idx), _p(ws),
                                        0 if ws is None else ws.numel(), _stream(stream)))


def _attn_args(q, cache, idx, swa, q_pos, swa_pos0, out):
    import torch
    B, T = q.shape[0], q.shape[1]
    n_cap = cache.shape[1]
    S = swa.shape[1]
    _expect(q, "q", torch.bfloat16, (B, T, HEADS, DIM))
    _expect(cache, "cache", torch.uint8, (B, n_cap, ROW_BYTES))
    _expect(idx, "idx", torch.int32, (B, T, TOPK))
    _expect(swa, "swa", torch.uint8, (B, S, DIM))
    _expect(q_pos, "q_pos", torch.int64, (B, T))
    _expect(swa_pos0, "swa_pos0", torch.int64, (B,))
    _expect(out, "out", torch.float32, (B, T, HEADS, DIM))
    return B, T, n_cap, S


def csa2_sparse_attn(q, cache, idx, swa, q_pos, swa_pos0, scale, out, ws=None, stream=None):
    """q [B,T,64,512] bf16, cache [B,n_cap,288] uint8, idx [B,T,512] int32,
    swa [B,S,512] uint8 (row s = token swa_pos0 + s), q_pos [B,T] int64,
    swa_pos0 [B] int64, out [B,T,64,512] f32; ws: uint8 device workspace of
    csa2_workspace_bytes(CSA2_OP_SPARSE_ATTN, ...) bytes (None when that is 0)."""
    B, T, n_cap, S = _attn_args(q, cache, idx, swa, q_pos, swa_pos0, out)
    _check("csa2_sparse_attn", lib().csa2_sparse_attn(_p(q), _p(cache), _p(idx), _p(swa),
                                                      _p(q_pos), _p(swa_pos0), B, T, n_cap, S,
                                                      float(scale), _p(out), _p(ws),
                                                      0 if ws is None else ws.numel(),
                                                      _stream(stream)))


def csa2_sparse_attn_ring(q, cache, idx, swa, q_pos, swa_pos0, scale, out, ws=None, stream=None):
    """csa2_sparse_attn over a ring-buffer window: token t of sequence b in row
    t mod S of swa [B,S,512]; rows hold tokens [swa_pos0, swa_pos0 + S)."""
    B, T, n_cap, S = _attn_args(q, cache, idx, swa, q_pos, swa_pos0, out)
    _check("csa2_sparse_attn_ring", lib().csa2_sparse_attn_ring(
        _p(q), _p(cache), _p(idx), _p(swa), _p(q_pos), _p(swa_pos0), B, T, n_cap, S,
        float(scale), _p(out), _p(ws), 0 if ws is None else ws.numel(), _stream(stream)))
