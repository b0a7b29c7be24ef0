"""Python binding of the C ABI in ``include/csa.h`` (``libcsa.so``, built in-tree).

Argument marshalling only: each function takes torch tensors that already live on
the GPU, passes their device pointers, sizes and the current HIP stream to the C
entry point of the same name, and raises ``CSAError`` on a non-zero status.  All
arithmetic runs in the library's HIP kernels.  There is no fallback: if the
library is missing, importing this module raises.

Tensor dtypes: fp32 -> CSA_F32, bfloat16 -> CSA_BF16, uint8 or float8_e4m3fn codes
-> CSA_FP8_E4M3.  Workspaces are sized with the library's own queries and, when
the caller passes none, allocated with torch (device memory plumbing).
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")

CSA_F32, CSA_BF16, CSA_FP8_E4M3, CSA_FP4_E2M1, CSA_PACKED_FP4_E4M3, CSA_PACKED_FP8_ROPE = 0, 1, 2, 3, 4, 5
CSA_LAYOUT_ROWS, CSA_LAYOUT_B16 = 0, 1
CSA_KV_BF16, CSA_KV_FP4_E4M3, CSA_KV_FP8_ROPE_BF16 = 0, 1, 2
STATUS = {0: "CSA_OK", 1: "CSA_ERR_INVALID_ARG", 2: "CSA_ERR_UNSUPPORTED", 3: "CSA_ERR_WORKSPACE",
          4: "CSA_ERR_HIP", 5: "CSA_ERR_SCRATCH"}

EXPORTS = ("csa_status_string", "csa_version", "csa_compress_workspace_size", "csa_compress",
           "csa_compress_state_size", "csa_compress_decode_workspace_size", "csa_compress_decode",
           "csa_compress_decode_many_workspace_size", "csa_compress_decode_many",
           "csa2_compress_workspace_size", "csa2_compress",
           "csa_index_score", "csa_index_topk_workspace_size", "csa_index_topk",
           "csa_index_segments_size", "csa_index_score_segments", "csa_topk_merge",
           "csa_index_keys_b16_size", "csa_index_keys_b16", "csa_index_score_segments_b16",
           "csa_index_score_segments_bmax", "csa_index_pool_segments_size", "csa_index_score_pool",
           "csa_index_score_mx",
           "csa_topk_workspace_size", "csa_topk", "csa_topk_algo",
           "csa_attn_workspace_size", "csa_sparse_attn", "csa_topk_sparse_attn", "hca_dense_attn",
           "csa_sparse_attn_noalloc_max_bytes", "csa_sparse_attn_noalloc")


class DecodeCompressor(ctypes.Structure):
    """csa_decode_compressor: the per-compressor arguments of csa_compress_decode_many."""
    _fields_ = [("w_proj", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("overlap", ctypes.c_int),
                ("online", ctypes.c_int), ("m", ctypes.c_int), ("c", ctypes.c_int), ("d_rope", ctypes.c_int),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("state", ctypes.c_void_p),
                ("cache", ctypes.c_void_p), ("cache_scale", ctypes.c_void_p), ("out_dtype", ctypes.c_int),
                ("out_layout", ctypes.c_int), ("Nc_max", ctypes.c_int)]


class CSAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m compressed_sparse_kv_amd.build` "
                          "(hipcc, gfx950).  There is no fallback path.")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    i64 = ctypes.c_int64
    sig = {
        "csa_status_string": ([i], ctypes.c_char_p),
        "csa_version": ([], i),
        "csa_compress_workspace_size": ([i, i, i, i, i, i], sz),
        "csa_compress": ([vp, vp, i, vp, vp, i, i, i, i, i, i, i, f, f, i64, vp, vp, i, i, i, vp, sz, vp], i),
        "csa_compress_state_size": ([i, i, i, i, i], sz),
        "csa2_compress_workspace_size": ([i, i, i, i], sz),
        "csa2_compress": ([vp, i, vp, vp, i, i, i, i, i, i, i, f, f, f, i64, vp, vp, i, vp, vp, i, vp, sz, vp], i),
        "csa_compress_decode_workspace_size": ([i, i, i, i, i], sz),
        "csa_compress_decode": ([vp, i, vp, vp, i, i, i, i, i, i, i, f, f, vp, i, vp, vp, vp, i, i, i, vp, sz, vp], i),
        "csa_compress_decode_many_workspace_size": ([i, i, i, i, ctypes.POINTER(DecodeCompressor)], sz),
        "csa_compress_decode_many": ([vp, i, i, i, vp, i, i, ctypes.POINTER(DecodeCompressor), vp, sz, vp], i),
        "csa_index_score": ([vp, vp, vp, vp, vp, i, vp, i, i, i, i, i, i, vp, vp], i),
        "csa_index_topk_workspace_size": ([i, i, i, i], sz),
        "csa_index_topk": ([vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, vp, vp, sz, vp], i),
        "csa_index_segments_size": ([i, i, i, i], sz),
        "csa_index_score_segments": ([vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, vp, sz, vp], i),
        "csa_index_keys_b16_size": ([i, i], sz),
        "csa_index_keys_b16": ([vp, vp, i, i, vp], i),
        "csa_index_score_segments_b16": ([vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, vp, sz, vp], i),
        "csa_topk_merge": ([vp, sz, i, i, i, i, vp, vp], i),
        "csa_index_score_segments_bmax": ([vp, vp, vp, vp, i, vp, vp, i, i, i, i, i, i, i, vp, vp, sz, vp, vp], i),
        "csa_index_pool_segments_size": ([i, i, i, i], sz),
        "csa_index_score_mx": ([vp, vp, vp, vp, vp, i, vp, i, i, i, i, i, i, i, vp, i, vp, sz, vp], i),
        "csa_index_score_pool": ([vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, sz, vp], i),
        "csa_topk_workspace_size": ([i, i, i], sz),
        "csa_topk": ([vp, i, i, i, i, vp, vp, sz, vp], i),
        "csa_topk_algo": ([vp, i, i, i, i, vp, vp, sz, i, vp], i),
        "csa_attn_workspace_size": ([i, i, i, i, i, i], sz),
        "csa_sparse_attn": ([vp, vp, vp, vp, vp, vp, i, i, f, i, i, i, i, i, i, i, i, i, f, vp, vp, vp, sz, vp], i),
        "csa_topk_sparse_attn": ([vp, vp, vp, sz, vp, vp, vp, i, i, f, i, i, i, i, i, i, i, i, i, f, vp, vp, vp, vp, sz,
                                  vp], i),
        "hca_dense_attn": ([vp, vp, vp, i, vp, vp, i, i, f, i, i, i, i, i, i, i, i, f, vp, vp, vp, sz, vp], i),
        "csa_sparse_attn_noalloc_max_bytes": ([], sz),
        "csa_sparse_attn_noalloc": ([vp, vp, vp, vp, vp, vp, i, i, f, i, i, i, i, i, i, i, i, i, f, vp, vp, vp], i),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _check(fn: str, st: int):
    if st != 0:
        raise CSAError(fn, st, _lib.csa_status_string(st).decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return CSA_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _ws(nbytes: int, ws, device):
    if nbytes == 0:
        return ws, (0 if ws is None else ws.numel() * ws.element_size())
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


# ---------------------------------------------------------------------------------------
# Stage 1
# ---------------------------------------------------------------------------------------

def compress_workspace_size(B, T, m, c, overlap, has_prev) -> int:
    return int(_lib.csa_compress_workspace_size(B, T, m, c, int(overlap), int(has_prev)))


def csa_compress(hidden, hidden_prev, w_proj, bias, *, overlap: bool, m: int, c: int, d_rope: int,
                 rope_theta: float, rms_eps: float, p0: int, out, out_scale=None, out_dtype: int | None = None,
                 layout: int = CSA_LAYOUT_ROWS, Nc_max: int | None = None, ws=None, stream=None):
    """hidden [B,T,d], hidden_prev [B,m,d] or None, w_proj [S*c, d], bias [S/2,m,c] fp32,
    out [B,T/m,c] (fp32 / bf16 / uint8 codes with out_scale [B,T/m]); out_dtype (default:
    from out's dtype) selects the low-precision types: CSA_FP4_E2M1 (codes [B,T/m,c/2],
    out_scale uint8 [B,T/m,c/32]), CSA_PACKED_FP4_E4M3 / CSA_PACKED_FP8_ROPE (uint8 rows).
    layout=CSA_LAYOUT_B16 (FP8, c = 128): out is the 16-entry blocked cache of Nc_max
    entries per sequence and out_scale [B,Nc_max]; the chunk's entries land at p0/m on."""
    _dev(hidden, hidden_prev, w_proj, bias, out, out_scale)
    B, T, d = hidden.shape
    if layout != CSA_LAYOUT_ROWS:
        if Nc_max is None:
            raise ValueError("Nc_max is required for the blocked layout")
        out_dtype = CSA_FP8_E4M3
    ws, wsb = _ws(compress_workspace_size(B, T, m, c, overlap, hidden_prev is not None), ws, hidden.device)
    _check("csa_compress", _lib.csa_compress(
        _p(hidden), _p(hidden_prev), _dtype(hidden), _p(w_proj), _p(bias), int(overlap), B, T, d, m, c,
        d_rope, float(rope_theta), float(rms_eps), int(p0), _p(out), _p(out_scale),
        _dtype(out) if out_dtype is None else int(out_dtype), int(layout), int(Nc_max or 0), _p(ws), wsb,
        _stream(stream)))
    return out


def csa2_compress(hidden, w_proj, w_k, *, m: int, d_rope: int, theta_kv: float, theta_k: float, rms_eps: float,
                  p0: int, kv_out, k_out, kv_scale=None, k_scale=None, kv_dtype: int | None = None,
                  k_dtype: int | None = None, ws=None, stream=None):
    """CSA2 compressor: hidden [B,T,d], w_proj [(2 if m > 1 else 1)*c, d], w_k [d_I, c] ->
    kv_out [B,T/m,c] and k_out [B,T/m,d_I] (fp32 / bf16 / uint8 codes with their scales);
    kv_dtype / k_dtype (default: from the tensors) select the low-precision types as in
    csa_compress (c = w_k.shape[1], d_I = w_k.shape[0])."""
    _dev(hidden, w_proj, w_k, kv_out, k_out, kv_scale, k_scale, ws)
    B, T, d = hidden.shape
    dI, c = w_k.shape
    ws, wsb = _ws(int(_lib.csa2_compress_workspace_size(B, T, m, c)), ws, hidden.device)
    _check("csa2_compress", _lib.csa2_compress(
        _p(hidden), _dtype(hidden), _p(w_proj), _p(w_k), B, T, d, m, c, dI, d_rope, float(theta_kv), float(theta_k),
        float(rms_eps), int(p0), _p(kv_out), _p(kv_scale), _dtype(kv_out) if kv_dtype is None else int(kv_dtype),
        _p(k_out), _p(k_scale), _dtype(k_out) if k_dtype is None else int(k_dtype), _p(ws), wsb, _stream(stream)))
    return kv_out, k_out


def compress_state_size(B, m, c, overlap, online=False) -> int:
    return int(_lib.csa_compress_state_size(B, m, c, int(overlap), int(online)))


def compress_decode_workspace_size(B, d, c, overlap, in_dtype=CSA_BF16) -> int:
    return int(_lib.csa_compress_decode_workspace_size(B, d, c, int(overlap), int(in_dtype)))


def csa_compress_decode(hidden, w_proj, bias, pos, state, cache, *, overlap: bool, m: int, c: int, d_rope: int,
                        rope_theta: float, rms_eps: float, online: bool = False, emit: bool = True,
                        cache_scale=None, layout: int = CSA_LAYOUT_ROWS, Nc_max: int | None = None, ws=None,
                        out_dtype: int | None = None, stream=None):
    """One decode token per sequence: hidden [B,d], pos [B] int64, state (uint8 or fp32,
    compress_state_size bytes); a completed block's entry goes to cache ([B,Nc_max,c] rows,
    or the 16-entry blocked FP8 layout with layout=CSA_LAYOUT_B16, Nc_max given)."""
    _dev(hidden, w_proj, bias, pos, state, cache, cache_scale)
    B, d = hidden.shape
    if Nc_max is None:
        if layout != CSA_LAYOUT_ROWS:
            raise ValueError("Nc_max is required for the blocked layout")
        Nc_max = cache.shape[1]
    if state.numel() * state.element_size() < compress_state_size(B, m, c, overlap, online):
        raise ValueError("state smaller than compress_state_size")
    ws, wsb = _ws(compress_decode_workspace_size(B, d, c, overlap, _dtype(hidden)), ws, hidden.device)
    out_dt = CSA_FP8_E4M3 if layout == CSA_LAYOUT_B16 else _dtype(cache) if out_dtype is None else int(out_dtype)
    _check("csa_compress_decode", _lib.csa_compress_decode(
        _p(hidden), _dtype(hidden), _p(w_proj), _p(bias), int(overlap), int(online), B, d, m, c, d_rope,
        float(rope_theta), float(rms_eps), _p(pos), int(emit), _p(state), _p(cache), _p(cache_scale), out_dt,
        int(layout), int(Nc_max), _p(ws), wsb, _stream(stream)))
    return cache


def _decode_comp(B, w_proj, bias, state, cache, *, overlap: bool, m: int, c: int, d_rope: int, rope_theta: float,
                 rms_eps: float, online: bool = False, cache_scale=None, layout: int = CSA_LAYOUT_ROWS,
                 Nc_max: int | None = None, out_dtype: int | None = None) -> DecodeCompressor:
    _dev(w_proj, bias, state, cache, cache_scale)
    if Nc_max is None:
        if layout != CSA_LAYOUT_ROWS:
            raise ValueError("Nc_max is required for the blocked layout")
        Nc_max = cache.shape[1]
    if state.numel() * state.element_size() < compress_state_size(B, m, c, overlap, online):
        raise ValueError("state smaller than compress_state_size")
    out_dt = CSA_FP8_E4M3 if layout == CSA_LAYOUT_B16 else _dtype(cache) if out_dtype is None else int(out_dtype)
    return DecodeCompressor(_p(w_proj), _p(bias), int(overlap), int(online), m, c, d_rope, float(rope_theta),
                            float(rms_eps), _p(state), _p(cache), _p(cache_scale), out_dt, int(layout), int(Nc_max))


def decode_compressors(B, comps):
    """The csa_decode_compressor array for comps (dicts of csa_compress_decode's
    per-compressor keywords), to build once and pass to csa_compress_decode_many on every
    step; the caller keeps the tensors it points to alive."""
    if isinstance(comps, ctypes.Array):
        return comps
    structs = [_decode_comp(B, **k) for k in comps]
    return (DecodeCompressor * len(structs))(*structs)


def compress_decode_many_workspace_size(B, d, in_dtype, comps) -> int:
    arr = decode_compressors(B, comps)
    return int(_lib.csa_compress_decode_many_workspace_size(B, d, int(in_dtype), len(arr), arr))


def csa_compress_decode_many(hidden, pos, comps, *, emit: bool = True, ws=None, stream=None):
    """The decode step of 1 or 2 compressors over the same new tokens (hidden [B,d], pos [B]
    int64): comps are dicts of csa_compress_decode's per-compressor keywords (w_proj, bias,
    state, cache, overlap, m, c, d_rope, rope_theta, rms_eps, and optionally online,
    cache_scale, layout, Nc_max, out_dtype), or the array decode_compressors made of them.
    Same results as one csa_compress_decode per compressor, in order."""
    _dev(hidden, pos)
    B, d = hidden.shape
    arr = decode_compressors(B, comps)
    ws, wsb = _ws(compress_decode_many_workspace_size(B, d, _dtype(hidden), arr), ws, hidden.device)
    _check("csa_compress_decode_many", _lib.csa_compress_decode_many(
        _p(hidden), _dtype(hidden), B, d, _p(pos), int(emit), len(arr), arr, _p(ws), wsb, _stream(stream)))


# ---------------------------------------------------------------------------------------
# Stage 2
# ---------------------------------------------------------------------------------------

def csa_index_score(q, q_scale, w, k, k_scale, q_pos, *, m: int, scores, stream=None):
    """q [B,S,H_I,d_I], k [B,Nc,d_I] (fp8 codes + scales, or fp32 with scales None),
    w [B,S,H_I], q_pos [B,S] int64 -> scores [B,S,Nc] fp32."""
    _dev(q, q_scale, w, k, k_scale, q_pos, scores)
    B, S, H, D = q.shape
    Nc = k.shape[1]
    _check("csa_index_score", _lib.csa_index_score(
        _p(q), _p(q_scale), _p(w), _p(k), _p(k_scale), _dtype(q), _p(q_pos), B, S, H, D, Nc, m,
        _p(scores), _stream(stream)))
    return scores


# ---------------------------------------------------------------------------------------
# Stages 2 + 3 in one call
# ---------------------------------------------------------------------------------------

def index_topk_workspace_size(B, S, Nc, k) -> int:
    return int(_lib.csa_index_topk_workspace_size(B, S, Nc, k))


def csa_index_topk(q, q_scale, w, k_codes, k_scale, q_pos, *, m: int, k: int, idx, scores=None, ws=None,
                   stream=None):
    """FP8 q [B,S,64,128] + q_scale [B,S,64], w [B,S,64], k_codes [B,Nc,128] + k_scale [B,Nc],
    q_pos [B,S] -> idx [B,S,k] int32 (and scores [B,S,Nc] fp32 when given)."""
    _dev(q, q_scale, w, k_codes, k_scale, q_pos, idx, scores, ws)
    B, S, H, D = q.shape
    Nc = k_codes.shape[1]
    need = index_topk_workspace_size(B, S, Nc, k)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check("csa_index_topk", _lib.csa_index_topk(
        _p(q), _p(q_scale), _p(w), _p(k_codes), _p(k_scale), _p(q_pos), B, S, H, D, Nc, m, k, _p(scores), _p(idx),
        _p(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return idx


def index_segments_size(B, S, Nc, k) -> int:
    return int(_lib.csa_index_segments_size(B, S, Nc, k))


def index_keys_b16_size(B, Nc) -> int:
    return int(_lib.csa_index_keys_b16_size(B, Nc))


def csa_index_keys_b16(k_codes, k_blocks, stream=None):
    """k_blocks (uint8, index_keys_b16_size bytes) = k_codes [B,Nc,128] in 16-entry blocks."""
    _dev(k_codes, k_blocks)
    B, Nc, D = k_codes.shape
    if k_blocks.numel() * k_blocks.element_size() < index_keys_b16_size(B, Nc):
        raise ValueError("k_blocks smaller than index_keys_b16_size")
    _check("csa_index_keys_b16", _lib.csa_index_keys_b16(_p(k_codes), _p(k_blocks), B, Nc, _stream(stream)))
    return k_blocks


def csa_index_score_segments_b16(q, q_scale, w, k_blocks, k_scale, q_pos, *, m: int, k: int, cand, scores=None,
                                 stream=None):
    """csa_index_score_segments with the keys in 16-entry blocks (csa_index_keys_b16)."""
    _dev(q, q_scale, w, k_blocks, k_scale, q_pos, cand, scores)
    B, S, H, D = q.shape
    Nc = k_scale.shape[1]
    if k_blocks.numel() * k_blocks.element_size() < index_keys_b16_size(B, Nc):
        raise ValueError("k_blocks smaller than index_keys_b16_size")
    _check("csa_index_score_segments_b16", _lib.csa_index_score_segments_b16(
        _p(q), _p(q_scale), _p(w), _p(k_blocks), _p(k_scale), _p(q_pos), B, S, H, D, Nc, m, k, _p(scores),
        _p(cand), cand.numel() * cand.element_size(), _stream(stream)))
    return cand


def csa_index_score_segments(q, q_scale, w, k_codes, k_scale, q_pos, *, m: int, k: int, cand, scores=None,
                             stream=None):
    """Decode shapes: scores (when given) and every 4096-entry segment's top-k as (key, entry)
    uint32 pairs in cand (a uint8 tensor of index_segments_size bytes)."""
    _dev(q, q_scale, w, k_codes, k_scale, q_pos, cand, scores)
    B, S, H, D = q.shape
    Nc = k_codes.shape[1]
    _check("csa_index_score_segments", _lib.csa_index_score_segments(
        _p(q), _p(q_scale), _p(w), _p(k_codes), _p(k_scale), _p(q_pos), B, S, H, D, Nc, m, k, _p(scores),
        _p(cand), cand.numel() * cand.element_size(), _stream(stream)))
    return cand


def csa_index_score_segments_bmax(q, q_scale, w, k_keys, k_scale, q_pos, *, m: int, k: int, cand, block_max,
                                  Nc: int, layout: int = CSA_LAYOUT_ROWS, scores=None, stream=None):
    """The Full layer of the hierarchical indexer: segment candidates (and scores) plus the
    block-of-8 maxima block_max [B,S,ceil(Nc/8)] fp32."""
    _dev(q, q_scale, w, k_keys, k_scale, q_pos, cand, block_max, scores)
    B, S, H, D = q.shape
    _check("csa_index_score_segments_bmax", _lib.csa_index_score_segments_bmax(
        _p(q), _p(q_scale), _p(w), _p(k_keys), int(layout), _p(k_scale), _p(q_pos), B, S, H, D, Nc, m, k, _p(scores),
        _p(cand), cand.numel() * cand.element_size(), _p(block_max), _stream(stream)))
    return cand


def csa_index_score_mx(q, q_scale, w, k_codes, k_scale, q_pos, *, fp4: bool, m: int, scores=None, k: int = 0,
                       cand=None, score_bf16: bool = False, stream=None):
    """Index scores over MX caches: q [B,S,64,64 (FP4) or 128 (FP8)] uint8, q_scale [B,S,64,4]
    E8M0, w [B,S,64], k_codes [B,Nc,64 or 128], k_scale [B,Nc,4]; scores [B,S,Nc] and/or the
    segment top-k pairs in cand (decode shapes)."""
    _dev(q, q_scale, w, k_codes, k_scale, q_pos, scores, cand)
    B, S, H = q.shape[:3]
    Nc = k_codes.shape[1]
    _check("csa_index_score_mx", _lib.csa_index_score_mx(
        _p(q), _p(q_scale), _p(w), _p(k_codes), _p(k_scale), CSA_FP4_E2M1 if fp4 else CSA_FP8_E4M3, _p(q_pos), B, S,
        H, 128, Nc, m, int(score_bf16), _p(scores), int(k), _p(cand),
        0 if cand is None else cand.numel() * cand.element_size(), _stream(stream)))
    return scores if cand is None else cand


def index_pool_segments_size(B, S, n_blocks, k) -> int:
    return int(_lib.csa_index_pool_segments_size(B, S, n_blocks, k))


def csa_index_score_pool(q, q_scale, w, k_codes, k_scale, q_pos, blocks, *, m: int, k: int, cand, scores=None,
                         stream=None):
    """A Reindex layer over the pool blocks [B,S,n_blocks] int32: segment candidates (key,
    position) of the pool's 8*n_blocks entries (and their scores in pool order)."""
    _dev(q, q_scale, w, k_codes, k_scale, q_pos, blocks, cand, scores)
    B, S, H, D = q.shape
    Nc, n_blocks = k_codes.shape[1], blocks.shape[-1]
    _check("csa_index_score_pool", _lib.csa_index_score_pool(
        _p(q), _p(q_scale), _p(w), _p(k_codes), _p(k_scale), _p(q_pos), _p(blocks), n_blocks, B, S, H, D, Nc, m, k,
        _p(scores), _p(cand), cand.numel() * cand.element_size(), _stream(stream)))
    return cand


def csa_topk_merge(cand, B, S, Nc, k, idx, stream=None):
    """idx [B,S,k] int32 = the k best of each row's segment candidates, as csa_topk returns them."""
    _dev(cand, idx)
    _check("csa_topk_merge", _lib.csa_topk_merge(_p(cand), cand.numel() * cand.element_size(), B, S, Nc, k, _p(idx),
                                                 _stream(stream)))
    return idx


# ---------------------------------------------------------------------------------------
# Stage 3
# ---------------------------------------------------------------------------------------

def topk_workspace_size(rows, Nc, k) -> int:
    return int(_lib.csa_topk_workspace_size(rows, Nc, k))


def csa_topk(scores, k: int, idx, *, ws=None, algo: int = 0, stream=None):
    """scores [B,S,Nc] fp32 -> idx [B,S,k] int32."""
    _dev(scores, idx, ws)
    B, S, Nc = scores.shape
    ws, wsb = _ws(topk_workspace_size(B * S, Nc, k), ws, scores.device)
    _check("csa_topk", _lib.csa_topk_algo(_p(scores), B, S, Nc, k, _p(idx), _p(ws), wsb, algo,
                                          _stream(stream)))
    return idx


# ---------------------------------------------------------------------------------------
# Stage 4
# ---------------------------------------------------------------------------------------

def attn_workspace_size(B, S, H, c, max_rows, dtype) -> int:
    return int(_lib.csa_attn_workspace_size(B, S, H, c, max_rows, dtype))


KV_ROW_BYTES = {CSA_KV_BF16: 1024, CSA_KV_FP4_E4M3: 288, CSA_KV_FP8_ROPE_BF16: 584}


def _kv_entries(kv_comp, kv_format: int, c: int) -> int:
    """Nc of a compressed cache: [B,Nc,c] in the query dtype, or for the packed formats
    [B,Nc,row bytes] uint8 (c = 512)."""
    if kv_format == CSA_KV_BF16:
        return kv_comp.shape[1]
    if kv_format not in KV_ROW_BYTES or c != 512:
        raise CSAError("attention", 2, f"kv_format {kv_format} with c = {c} is not supported")
    if kv_comp.dtype != torch.uint8 or kv_comp.dim() != 3 or kv_comp.shape[2] != KV_ROW_BYTES[kv_format]:
        raise CSAError("attention", 1, f"kv_comp of kv_format {kv_format} must be uint8 [B,Nc,{KV_ROW_BYTES[kv_format]}]")
    return kv_comp.shape[1]


def csa_sparse_attn(q, kv_comp, idx, swa, sink, *, W: int, out, lse=None, scale=None, q_pos=None, ws=None,
                    inv_rope_d: int = 0, rope_theta: float = 1e4, kv_format: int = 0, stream=None):
    """q [B,S,H,c], kv_comp [B,Nc,c] (or a packed cache of kv_format), idx [B,S,k] int32,
    swa [B,Ls,c], sink [H] fp32; q_pos [B,S] int64 (optional) leaves out window rows of
    negative positions; inv_rope_d > 0 (needs q_pos) rotates the output's last inv_rope_d
    channels back by the query position."""
    _dev(q, kv_comp, idx, swa, sink, out, lse, ws, q_pos)
    B, S, H, c = q.shape
    Nc, Ls, k = _kv_entries(kv_comp, kv_format, c), swa.shape[1], idx.shape[-1]
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    dt = _dtype(q)
    ws, wsb = _ws(attn_workspace_size(B, S, H, c, min(W, Ls) + k, dt), ws, q.device)
    _check("csa_sparse_attn", _lib.csa_sparse_attn(
        _p(q), _p(kv_comp), _p(idx), _p(q_pos), _p(swa), _p(sink), dt, int(kv_format), float(scale), B, S, H, c, Nc,
        k, Ls, W, int(inv_rope_d), float(rope_theta), _p(out), _p(lse), _p(ws), wsb, _stream(stream)))
    return out


def sparse_attn_noalloc_max_bytes() -> int:
    return int(_lib.csa_sparse_attn_noalloc_max_bytes())


def csa_sparse_attn_noalloc(q, kv_comp, idx, swa, sink, *, W: int, out, lse=None, scale=None, q_pos=None,
                            inv_rope_d: int = 0, rope_theta: float = 1e4, kv_format: int = 0, stream=None):
    """csa_sparse_attn with the split partials in the library's fixed scratch (no workspace)."""
    _dev(q, kv_comp, idx, swa, sink, out, lse, q_pos)
    B, S, H, c = q.shape
    Nc, Ls, k = _kv_entries(kv_comp, kv_format, c), swa.shape[1], idx.shape[-1]
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    _check("csa_sparse_attn_noalloc", _lib.csa_sparse_attn_noalloc(
        _p(q), _p(kv_comp), _p(idx), _p(q_pos), _p(swa), _p(sink), _dtype(q), int(kv_format), float(scale), B, S, H,
        c, Nc, k, Ls, W, int(inv_rope_d), float(rope_theta), _p(out), _p(lse), _stream(stream)))
    return out


def csa_topk_sparse_attn(q, kv_comp, cand, swa, sink, *, k: int, W: int, out, q_pos=None, lse=None, idx=None,
                         scale=None, ws=None, inv_rope_d: int = 0, rope_theta: float = 1e4, kv_format: int = 0,
                         stream=None):
    """The k best of each query's segment candidates (cand from csa_index_score_segments),
    then csa_sparse_attn over them; idx [B,S,k] int32 (optional) receives the selection."""
    _dev(q, kv_comp, cand, swa, sink, out, lse, idx, ws, q_pos)
    B, S, H, c = q.shape
    Nc, Ls = _kv_entries(kv_comp, kv_format, c), swa.shape[1]
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    dt = _dtype(q)
    ws, wsb = _ws(attn_workspace_size(B, S, H, c, min(W, Ls) + k, dt), ws, q.device)
    _check("csa_topk_sparse_attn", _lib.csa_topk_sparse_attn(
        _p(q), _p(kv_comp), _p(cand), cand.numel() * cand.element_size(), _p(q_pos), _p(swa), _p(sink), dt,
        int(kv_format), float(scale), B, S, H, c, Nc, k, Ls, W, int(inv_rope_d), float(rope_theta), _p(out), _p(lse), _p(idx), _p(ws),
        wsb, _stream(stream)))
    return out


def hca_dense_attn(q, kv_comp, q_pos, swa, sink, *, m: int, W: int, out, lse=None, scale=None, ws=None,
                   inv_rope_d: int = 0, rope_theta: float = 1e4, kv_format: int = 0, stream=None):
    """q [B,S,H,c], kv_comp [B,Nc,c] (or a packed cache of kv_format), q_pos [B,S] int64,
    swa [B,Ls,c], sink [H] fp32."""
    _dev(q, kv_comp, q_pos, swa, sink, out, lse, ws)
    B, S, H, c = q.shape
    Nc, Ls = _kv_entries(kv_comp, kv_format, c), swa.shape[1]
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    dt = _dtype(q)
    ws, wsb = _ws(attn_workspace_size(B, S, H, c, min(W, Ls) + Nc, dt), ws, q.device)
    _check("hca_dense_attn", _lib.hca_dense_attn(
        _p(q), _p(kv_comp), _p(q_pos), m, _p(swa), _p(sink), dt, int(kv_format), float(scale), B, S, H, c, Nc, Ls, W,
        int(inv_rope_d), float(rope_theta), _p(out), _p(lse), _p(ws), wsb, _stream(stream)))
    return out
