"""The C ABI library loads and exports every symbol include/csa.h declares; host-side
argument checks return their status without touching a GPU (CPU only)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")
LIB = os.path.join(ROOT, "compressed_sparse_kv_amd", "libcsa.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    assert os.path.exists(LIB), "libcsa.so not built"
    lib = ctypes.CDLL(LIB)
    names = declared_functions()
    assert {"csa_compress", "csa_index_score", "csa_topk", "csa_sparse_attn", "hca_dense_attn"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_covers_every_declared_symbol():
    from compressed_sparse_kv_amd import binding
    assert set(declared_functions()) == set(binding.EXPORTS)


def test_status_strings_and_version():
    from compressed_sparse_kv_amd import binding
    lib = binding.lib()
    assert lib.csa_version() >= 200
    for st in range(5):
        assert lib.csa_status_string(st)
    assert b"unknown" in lib.csa_status_string(99)


def test_invalid_arguments_are_rejected_before_launch():
    from compressed_sparse_kv_amd import binding
    lib = binding.lib()
    fake = ctypes.c_void_p(0x1000)       # never dereferenced: the checks fail first
    # null pointers
    assert lib.csa_index_score(None, None, None, None, None, 2, None, 1, 1, 64, 128, 10, 4, None, None) == 1
    # unsupported FP8 head shape
    assert lib.csa_index_score(fake, fake, fake, fake, fake, 2, fake, 1, 1, 32, 128, 10, 4, fake, None) == 2
    # fp32 path must not get scales
    assert lib.csa_index_score(fake, fake, fake, fake, None, 0, fake, 1, 1, 4, 32, 10, 4, fake, None) == 1
    # top-k: k out of range, bad algo, algo 2 without workspace
    assert lib.csa_topk(fake, 1, 1, 10, 0, fake, None, 0, None) == 1
    assert lib.csa_topk(fake, 1, 1, 10, 4096, fake, None, 0, None) == 1
    assert lib.csa_topk_algo(fake, 1, 1, 10, 4, fake, None, 0, 7, None) == 1
    assert lib.csa_topk_algo(fake, 1, 1, 10, 4, fake, None, 0, 2, None) == 3
    # top-k: workspace given but too small; a row longer than one workgroup holds, no workspace
    assert lib.csa_topk(fake, 4, 1, 100000, 512, fake, fake, 16, None) == 3
    assert lib.csa_topk(fake, 4, 1, 36865, 512, fake, None, 0, None) == 3
    # top-k: a row too long for one level of segments
    assert lib.csa_topk(fake, 1, 1, 36864 * 18 + 1, 2048, fake, fake, 1 << 40, None) == 2
    # compressor: T not a multiple of m, p0 > 0 with overlap and no previous block, bf16 d % 64
    args = dict(hidden=fake, prev=None, dt=0, w=fake, bias=fake, ov=1, B=1, T=10, d=64, m=4, c=8, dr=4)
    call = lambda **kw: lib.csa_compress(kw["hidden"], kw["prev"], kw["dt"], kw["w"], kw["bias"], kw["ov"],
                                         kw["B"], kw["T"], kw["d"], kw["m"], kw["c"], kw["dr"], 1e4, 1e-6,
                                         kw.get("p0", 0), fake, None, 0, 0, 0, fake, 1 << 30, None)
    assert call(**args) == 1
    assert call(**{**args, "T": 8, "p0": 4}) == 1
    assert call(**{**args, "T": 8, "dt": 1, "d": 96}) == 2
    # compressor workspace too small
    assert lib.csa_compress(fake, None, 0, fake, fake, 1, 1, 8, 64, 4, 8, 4, 1e4, 1e-6, 0, fake, None, 0, 0, 0,
                            fake, 8, None) == 3
    # low-precision entry types: packed rows need c = 512 (FP8 + RoPE also d_rope = 64), MXFP4
    # needs its scale bytes and c % 32 == 0, unknown types are invalid
    comp = lambda c, d_rope, dt, scale: lib.csa_compress(fake, None, 0, fake, fake, 1, 1, 8, 64, 4, c, d_rope, 1e4,
                                                         1e-6, 0, fake, scale, dt, 0, 0, fake, 1 << 30, None)
    assert comp(256, 64, 4, None) == 2
    assert comp(512, 32, 5, None) == 2
    assert comp(128, 64, 3, None) == 1
    assert comp(48, 16, 3, fake) == 2
    assert comp(512, 64, 6, None) == 1
    # the blocked key layout: FP8 codes of c = 128 only, a cache that holds the chunk's entries
    blk = lambda c, dt, p0, Nc_max, layout=1: lib.csa_compress(fake, fake, 1, fake, fake, 1, 1, 64, 64, 4, c, 64, 1e4,
                                                               1e-6, p0, fake, fake, dt, layout, Nc_max, fake, 1 << 30,
                                                               None)
    assert blk(128, 2, 0, 16, layout=2) == 1
    assert blk(512, 2, 0, 16) == 2
    assert blk(128, 1, 0, 16) == 2
    assert blk(128, 2, 16, 19) == 1                                   # entries 4 .. 19 do not fit 19
    assert blk(128, 2, 0, 0) == 1
    # segment candidates: shape outside the decode path, candidate buffer too small, null idx
    assert lib.csa_index_score_segments(fake, fake, fake, fake, fake, fake, 1, 8, 64, 128, 3000, 4, 128, None,
                                        fake, 1 << 30, None) == 2
    assert lib.csa_index_score_segments(fake, fake, fake, fake, fake, fake, 32, 1, 64, 128, 32768, 4, 512, None,
                                        fake, 1024, None) == 3
    assert lib.csa_topk_merge(fake, 1 << 30, 32, 1, 32768, 512, None, None) == 1
    assert lib.csa_topk_merge(fake, 1024, 32, 1, 32768, 512, fake, None) == 3     # cand smaller than its size query
    assert lib.csa_index_segments_size(32, 1, 32768, 512) == 32 * 8 * 512 * 8
    assert lib.csa_index_segments_size(1, 8, 3000, 128) == 0
    # Pro shape: 64 segment lists of 1024 merge in two levels (groups of 8): room for both
    assert lib.csa_index_segments_size(4, 1, 262144, 1024) == 4 * (64 + 8) * 1024 * 8
    # attention: Ls < S, unsupported bf16 shape, non-positive scale
    assert lib.csa_sparse_attn(fake, fake, fake, None, fake, fake, 1, 0, 0.1, 1, 4, 64, 512, 10, 8, 2, 128, 0, 1e4,
                               fake, None, None, 0, None) == 1
    assert lib.csa_sparse_attn(fake, fake, fake, None, fake, fake, 1, 0, 0.1, 1, 1, 32, 512, 10, 8, 8, 128, 0, 1e4,
                               fake, None, None, 0, None) == 2
    assert lib.hca_dense_attn(fake, fake, fake, 128, fake, fake, 1, 0, 0.0, 1, 1, 64, 512, 10, 8, 128, 0, 1e4,
                              fake, None, None, 0, None) == 1
    # packed main-KV formats: only with the bf16 kernel, a known format, a 16-byte aligned cache
    assert lib.csa_sparse_attn(fake, fake, fake, None, fake, fake, 0, 1, 0.1, 1, 1, 64, 512, 10, 8, 8, 128, 0, 1e4,
                               fake, None, None, 0, None) == 2
    assert lib.csa_sparse_attn(fake, fake, fake, None, fake, fake, 1, 3, 0.1, 1, 1, 64, 512, 10, 8, 8, 128, 0, 1e4,
                               fake, None, None, 0, None) == 1
    assert lib.hca_dense_attn(fake, ctypes.c_void_p(0x1008), fake, 128, fake, fake, 1, 2, 0.1, 1, 1, 64, 512, 10,
                              128, 128, 0, 1e4, fake, None, None, 0, None) == 1
    # inverse RoPE of the output: needs the query positions, an even width <= c
    assert lib.csa_sparse_attn(fake, fake, fake, None, fake, fake, 1, 0, 0.1, 1, 1, 64, 512, 10, 8, 128, 128, 64, 1e4,
                               fake, None, None, 0, None) == 1
    assert lib.csa_sparse_attn(fake, fake, fake, fake, fake, fake, 1, 0, 0.1, 1, 1, 64, 512, 10, 8, 128, 128, 63, 1e4,
                               fake, None, None, 0, None) == 1
    assert lib.hca_dense_attn(fake, fake, fake, 128, fake, fake, 1, 0, 0.1, 1, 1, 64, 512, 10, 128, 128, 1024, 1e4,
                              fake, None, None, 0, None) == 1
    # the decode compressor: online needs overlap 0; the blocked layout needs FP8 codes of c = 128
    dec = lambda ov, on, c, dt, layout: lib.csa_compress_decode(
        fake, 1, fake, fake, ov, on, 2, 256, 4, c, 64, 1e4, 1e-6, fake, 1, fake, fake, fake, dt, layout, 16, fake,
        1 << 30, None)
    assert dec(1, 1, 512, 1, 0) == 1
    assert dec(1, 0, 512, 1, 1) == 2
    assert dec(1, 0, 512, 2, 1) == 2
    assert lib.csa_compress_decode(fake, 1, fake, fake, 1, 0, 2, 200, 4, 128, 64, 1e4, 1e-6, fake, 1, fake, fake, fake,
                                   1, 0, 16, fake, 1 << 30, None) == 2       # bf16 hidden: d % 128 != 0
    assert lib.csa_compress_decode(fake, 1, fake, fake, 1, 0, 2, 256, 4, 128, 64, 1e4, 1e-6, fake, 1, fake, fake, fake,
                                   1, 0, 16, fake, 8, None) == 3             # workspace too small
    assert lib.csa_compress_state_size(32, 4, 512, 1, 0) == 32 * 8 * 2048 * 4
    assert lib.csa_compress_state_size(64, 128, 512, 0, 0) == 64 * 128 * 1024 * 4
    assert lib.csa_compress_state_size(64, 128, 512, 0, 1) == 64 * 3 * 512 * 4
    # fused selection + attention: null candidates, fp32 dtype, too many candidates per
    # query after the first merge level (21 segments x 2048 -> 5 x 2048), workspace too
    # small for the split partials (also with two merge levels: V4-Pro, 64 segments x 1024)
    fused = lambda cand, dt, Nc, k, ws_bytes, cand_bytes=1 << 40: lib.csa_topk_sparse_attn(
        fake, fake, cand, cand_bytes, None, fake, fake, dt, 0, 0.1, 32, 1, 64, 512, Nc, k, 128, 128, 0, 1e4, fake, None,
        None, fake, ws_bytes, None)
    assert fused(None, 1, 32768, 512, 1 << 40) == 1
    assert fused(fake, 0, 32768, 512, 1 << 40) == 2
    assert fused(fake, 1, 86000, 2048, 1 << 40) == 2
    assert fused(fake, 1, 32768, 512, 16) == 3
    assert fused(fake, 1, 262144, 1024, 16) == 3
    assert fused(fake, 1, 32768, 512, 1 << 40, cand_bytes=1024) == 3     # cand smaller than its size query


def test_workspace_queries():
    from compressed_sparse_kv_amd import binding as b
    assert b.compress_workspace_size(1, 8192, 4, 512, True, True) == (8192 + 4) * 2048 * 4
    assert b.compress_workspace_size(1, 8192, 4, 128, False, False) == 8192 * 256 * 4
    assert b.topk_workspace_size(32, 32768, 512) > 0
    assert b.attn_workspace_size(32, 1, 64, 512, 640, 1) > 0           # split rows need partials
    assert b.attn_workspace_size(1, 1, 8, 64, 160, 0) == 8 * 66 * 4    # fp32 path: one partial


def test_compress_decode_many_checks_and_workspace():
    """csa_compress_decode_many: arguments of every compressor are checked before anything
    is enqueued, and its workspace is the single call's for one compressor, the 256-aligned
    first share plus the second for two."""
    from compressed_sparse_kv_amd import binding as b
    lib = b.lib()
    fake = 0x1000                         # 16-byte aligned, never dereferenced: checks fail first
    D = b.DecodeCompressor
    main = D(fake, fake, 1, 0, 4, 512, 64, 1e4, 1e-6, fake, fake, None, b.CSA_BF16, b.CSA_LAYOUT_ROWS, 64)
    idx = D(fake, fake, 1, 0, 4, 128, 64, 1e4, 1e-6, fake, fake, fake, b.CSA_FP8_E4M3, b.CSA_LAYOUT_B16, 64)
    two = (D * 2)(main, idx)
    single_main = lib.csa_compress_decode_workspace_size(32, 5120, 512, 1, b.CSA_BF16)
    single_idx = lib.csa_compress_decode_workspace_size(32, 5120, 128, 1, b.CSA_BF16)
    assert lib.csa_compress_decode_many_workspace_size(32, 5120, b.CSA_BF16, 1, two) == single_main
    assert lib.csa_compress_decode_many_workspace_size(32, 5120, b.CSA_BF16, 2, two) == \
        (single_main + 255) // 256 * 256 + single_idx
    assert lib.csa_compress_decode_many_workspace_size(32, 5120, b.CSA_BF16, 3, two) == 0
    ws_ok = (single_main + 255) // 256 * 256 + single_idx
    # n out of range, no compressors
    assert lib.csa_compress_decode_many(fake, b.CSA_BF16, 32, 5120, fake, 1, 0, two, fake, ws_ok, None) == 1
    assert lib.csa_compress_decode_many(fake, b.CSA_BF16, 32, 5120, fake, 1, 3, two, fake, ws_ok, None) == 1
    assert lib.csa_compress_decode_many(fake, b.CSA_BF16, 32, 5120, fake, 1, 2, None, fake, ws_ok, None) == 1
    # the second compressor's blocked layout needs FP8 codes of c = 128
    bad = (D * 2)(main, D(fake, fake, 1, 0, 4, 256, 64, 1e4, 1e-6, fake, fake, fake, b.CSA_FP8_E4M3,
                          b.CSA_LAYOUT_B16, 64))
    assert lib.csa_compress_decode_many(fake, b.CSA_BF16, 32, 5120, fake, 1, 2, bad, fake, ws_ok, None) == 2
    # odd c in the second compressor; workspace one byte short
    bad2 = (D * 2)(main, D(fake, fake, 1, 0, 4, 127, 64, 1e4, 1e-6, fake, fake, fake, b.CSA_FP8_E4M3,
                           b.CSA_LAYOUT_ROWS, 64))
    assert lib.csa_compress_decode_many(fake, b.CSA_BF16, 32, 5120, fake, 1, 2, bad2, fake, ws_ok, None) == 1
    assert lib.csa_compress_decode_many(fake, b.CSA_BF16, 32, 5120, fake, 1, 2, two, fake, ws_ok - 1, None) == 3
