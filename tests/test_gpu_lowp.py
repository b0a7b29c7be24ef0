"""Low-precision cache rows through the C ABI against the oracle: index scores over MXFP4
queries and keys (E2M1 + E8M0 per 32) on the scaled MFMA, their bf16 cast before the
top-k, and the measured precision of the FP8 form of the same unit (the reason the exact
FP8 path contracts on bf16 MFMA after an exact conversion)."""

import math

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from synthetic import inputs as I
from tests.parity import TOL_F32, assert_close, assert_topk_equal, dev

pytestmark = pytest.mark.gpu


def pack_nibbles(codes):
    """Two E2M1 codes per byte, the even element in the low nibble (the library's layout)."""
    c = np.asarray(codes, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def _mx_inputs(seed, B, S, Nc, fp4=True):
    rs = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3)]
    K = I.unit_rms_rows(rs[0], (B, Nc, 128)).astype(np.float64)
    q = rs[1].standard_normal((B, S, 64, 128))
    w = (rs[2].standard_normal((B, S, 64)) / np.sqrt(128 * 64)).astype(np.float32)
    if fp4:
        kc, ks = O.quantize_mxfp4(K)
        qc, qsc = O.quantize_mxfp4(q)
        kd, qd = O.dequant_mxfp4(kc, ks), O.dequant_mxfp4(qc, qsc)
        kc, qc = pack_nibbles(kc), pack_nibbles(qc)
    else:
        # MXFP8: E4M3 values with the same E8M0 block scales (exponent floor(log2 amax) - 8)
        def q8(x):
            xb = x.reshape(x.shape[:-1] + (4, 32))
            ex = np.floor(np.log2(np.abs(xb).max(axis=-1))) - 8.0
            codes = O.f64_to_e4m3fn(xb / np.exp2(ex)[..., None]).reshape(x.shape)
            return codes, (ex + 127).astype(np.uint8), O.e4m3fn_to_f64(codes) * np.repeat(np.exp2(ex), 32, axis=-1)
        kc, ks, kd = q8(K)
        qc, qsc, qd = q8(q)
    return dict(kc=kc, ks=ks, qc=qc, qs=qsc, w=w, kd=kd, qd=qd)


@pytest.mark.parametrize("B,S,Nc,t", [(2, 1, 5000, 4 * 5000 + 3), (3, 2, 9001, 4 * 7000 + 1), (1, 37, 700, 4 * 700)])
def test_index_score_mxfp4(lib, B, S, Nc, t):
    a = _mx_inputs(1000 + Nc, B, S, Nc)
    pos = (t - S + 1 + np.arange(S, dtype=np.int64))[None].repeat(B, 0)
    sc = torch.empty(B, S, Nc, device="cuda")
    lib.csa_index_score_mx(dev(a["qc"]), dev(a["qs"]), dev(a["w"]), dev(a["kc"]), dev(a["ks"]), dev(pos), fp4=True,
                           m=4, scores=sc)
    torch.cuda.synchronize()
    ref = O.index_scores(a["qd"], a["w"], a["kd"], pos, 4)
    assert_close(sc.cpu().numpy(), ref, TOL_F32, "MXFP4 index scores")


@pytest.mark.parametrize("bf16", [False, True])
def test_index_topk_mxfp4_segments(lib, bf16):
    B, Nc, k = 3, 32768, 512
    t = 4 * Nc - 1
    a = _mx_inputs(1100 + bf16, B, 1, Nc)
    pos = np.full((B, 1), t, np.int64)
    cand = torch.empty(lib.index_segments_size(B, 1, Nc, k), dtype=torch.uint8, device="cuda")
    sc = torch.empty(B, 1, Nc, device="cuda")
    lib.csa_index_score_mx(dev(a["qc"]), dev(a["qs"]), dev(a["w"]), dev(a["kc"]), dev(a["ks"]), dev(pos), fp4=True,
                           m=4, scores=sc, k=k, cand=cand, score_bf16=bf16)
    idx = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    lib.csa_topk_merge(cand, B, 1, Nc, k, idx)
    torch.cuda.synchronize()
    g, got = sc.cpu().numpy(), idx.cpu().numpy()
    # the selection is exactly the top-k of the GPU's own (rounded) scores
    assert np.array_equal(got, O.topk_indices(g, k)), "segment top-k + merge over the MXFP4 scores"
    ref = O.index_scores(a["qd"], a["w"], a["kd"], pos, 4)
    if not bf16:
        assert_close(g, ref, TOL_F32, "MXFP4 scores (segment pass)")
        assert_topk_equal(got, O.topk_indices(ref, k), ref, k, "MXFP4 top-k vs oracle")
        return
    # bf16 scores: the pages' cast of the fp32 score; the two sides' fp32 scores differ by at
    # most the fp32 bound (1e-5, checked above for the unrounded scores), so a bf16 value may
    # differ only where the oracle's score lies within 1e-5 of a bf16 rounding midpoint
    rb = O.round_bf16(ref)
    diff = (g != rb) & np.isfinite(ref)
    if diff.any():
        r = ref[diff]
        e = np.floor(np.log2(np.abs(r)))
        half = 2.0 ** (e - 8)
        frac = np.abs(r) / (2 * half)
        dist = np.abs(frac - (np.floor(frac) + 0.5)) * 2 * half
        assert np.all(dist <= TOL_F32), "bf16 scores differ away from a rounding midpoint"
    assert_topk_equal(got, O.topk_indices(rb, k), rb, k, "bf16-score top-k vs oracle", rel=2 ** -7)
    # bf16 ties are common: every tie inside the selection is broken towards the lower entry
    ties = int(np.sum([len(r) - len(np.unique(r)) for r in np.sort(g.reshape(B, -1), axis=1)]))
    assert ties > 0


def test_fp8_block_products_are_not_exact_on_the_scaled_mfma(lib):
    # MXFP8 queries and keys through the same unit: its block sums keep only part of the
    # products' bits, so the scores miss the fp32 bound the exact paths meet
    B, S, Nc = 2, 1, 4000
    a = _mx_inputs(1200, B, S, Nc, fp4=False)
    pos = np.full((B, S), 4 * Nc - 1, np.int64)
    sc = torch.empty(B, S, Nc, device="cuda")
    lib.csa_index_score_mx(dev(a["qc"]), dev(a["qs"]), dev(a["w"]), dev(a["kc"]), dev(a["ks"]), dev(pos), fp4=False,
                           m=4, scores=sc)
    torch.cuda.synchronize()
    ref = O.index_scores(a["qd"], a["w"], a["kd"], pos, 4)
    err = float(np.abs(sc.cpu().numpy() - ref).max())
    scale = float(np.abs(ref).max())
    print(f"MXFP8 on the scaled MFMA: max |score error| {err:.3e} (max |score| {scale:.3f})")
    assert err > TOL_F32, "FP8 block sums came out exact: the bf16-MFMA detour of the FP8 path could be dropped"
    assert err < 1e-2 * scale


# ---------------------------------------------------------------------------------------
# Packed main-KV caches read by the attention kernels (CSA_KV_FP4_E4M3: E2M1 + E4M3 per 16,
# 288-byte rows; CSA_KV_FP8_ROPE_BF16: e4m3 with a power-of-two row scale + bf16 RoPE
# channels, 584-byte rows).  The oracle quantises the rows; the test lays the codes out as
# the header documents; the attention result must be the oracle's attention over the
# dequantised rows, and (the decode being exact) bit-equal to the bf16 kernel's over them.
# ---------------------------------------------------------------------------------------

FMT_FP4, FMT_FP8_ROPE = 1, 2


def pack_kv(kv, fmt):
    """kv [B,Nc,512] float64 -> (packed uint8 [B,Nc,row bytes], dequantised float64 rows)."""
    if fmt == FMT_FP4:
        codes, sc = O.quantize_fp4_e4m3(kv)
        rows = np.concatenate([pack_nibbles(codes), sc.astype(np.uint8)], axis=-1)
        return rows, O.dequant_fp4_e4m3(codes, sc)
    codes, ex, rope_bits = O.quantize_fp8_rope_split(kv, 64)
    assert ex.min() >= -126 and ex.max() <= 127
    tail = np.zeros(kv.shape[:-1] + (8,), np.uint8)
    tail[..., 0] = (ex + 127).astype(np.uint8)
    rows = np.concatenate([codes.astype(np.uint8), rope_bits.astype("<u2").view(np.uint8), tail], axis=-1)
    return rows, O.dequant_fp8_rope_split(codes, ex, rope_bits)


def _fmt_attn_case(lib, fmt, B, S, Nc, k, W, seed, n_valid, dense=False, m=128, inv_rope_d=0):
    from tests.parity import assert_bf16_output, bf16_f64, dev_bf16, host_bits
    Ls = S + W - 1
    a = I.attention_inputs(seed, B, S, Nc, Ls)
    q_pos = np.tile(10 ** 6 - S + 1 + np.arange(S), (B, 1)).astype(np.int64)
    rows, kv_d = pack_kv(bf16_f64(a["kv_comp_bf16"]), fmt)
    kv_bits = I.to_bf16_bits(kv_d)
    assert np.array_equal(bf16_f64(kv_bits), kv_d), "dequantised rows are bf16 numbers"
    q_f, swa_f = bf16_f64(a["q_bf16"]), bf16_f64(a["swa_bf16"])
    out = torch.empty(B, S, 64, 512, dtype=torch.bfloat16, device="cuda")
    out_b = torch.empty_like(out)
    lse = torch.empty(B, S, 64, device="cuda")
    lse_b = torch.empty_like(lse)
    kw = dict(W=W, inv_rope_d=inv_rope_d, q_pos=dev(q_pos))
    common = (dev_bf16(a["q_bf16"]),)
    if dense:
        for kv, o, l, f in ((dev(rows), out, lse, fmt), (dev_bf16(kv_bits), out_b, lse_b, 0)):
            lib.hca_dense_attn(*common, kv, kw["q_pos"], dev_bf16(a["swa_bf16"]), dev(a["sink"]), m=m, W=W, out=o,
                               lse=l, inv_rope_d=inv_rope_d, kv_format=f)
        o_ref, l_ref = O.dense_attention(q_f, kv_d, q_pos, m, swa_f, a["sink"], 1 / math.sqrt(512), W)
    else:
        idx = dev(I.random_selection(seed, B, S, Nc, k, n_valid))
        for kv, o, l, f in ((dev(rows), out, lse, fmt), (dev_bf16(kv_bits), out_b, lse_b, 0)):
            lib.csa_sparse_attn(*common, kv, idx, dev_bf16(a["swa_bf16"]), dev(a["sink"]), out=o, lse=l,
                                kv_format=f, **kw)
        o_ref, l_ref = O.sparse_attention(q_f, kv_d, idx.cpu().numpy(), swa_f, a["sink"], 1 / math.sqrt(512),
                                          q_pos, W)
    if inv_rope_d:
        o_ref = O.inverse_rope(o_ref, q_pos[..., None], inv_rope_d, 1e4)
    torch.cuda.synchronize()
    assert_bf16_output(bf16_f64(host_bits(out)), o_ref, f"attention over packed rows (format {fmt})")
    assert_close(lse.cpu().numpy(), l_ref, TOL_F32, f"lse over packed rows (format {fmt})")
    if B * S < 64:
        # the same kernel reads both (packed rows decoded exactly while staged): bit-equal
        assert torch.equal(out, out_b) and torch.equal(lse, lse_b), "packed rows differ from their bf16 decode"
    else:
        # 64+ queries: bf16 rows go to the two-set kernel, packed rows to the staging one
        # (another summation order); the bf16 decode meets the same bound
        assert_bf16_output(bf16_f64(host_bits(out_b)), o_ref, "attention over the bf16 decode")
        assert_close(lse_b.cpu().numpy(), l_ref, TOL_F32, "lse over the bf16 decode")


@pytest.mark.parametrize("fmt", [FMT_FP4, FMT_FP8_ROPE])
def test_packed_kv_sparse_decode_split_rows(lib, fmt):
    _fmt_attn_case(lib, fmt, B=3, S=1, Nc=2000, k=512, W=128, seed=61, n_valid=np.array([[512], [300], [0]]))


@pytest.mark.parametrize("fmt", [FMT_FP4, FMT_FP8_ROPE])
def test_packed_kv_sparse_prefill_inverse_rope(lib, fmt):
    _fmt_attn_case(lib, fmt, B=2, S=40, Nc=900, k=64, W=128, seed=62, n_valid=np.array([[64], [17]]),
                   inv_rope_d=64)


@pytest.mark.parametrize("fmt", [FMT_FP4, FMT_FP8_ROPE])
def test_packed_kv_dense_hca(lib, fmt):
    _fmt_attn_case(lib, fmt, B=2, S=3, Nc=700, k=0, W=128, seed=63, n_valid=0, dense=True)


@pytest.mark.parametrize("fmt", [FMT_FP4, FMT_FP8_ROPE])
def test_packed_kv_fused_selection_and_noalloc(lib, fmt):
    # the fused selection + attention and the allocation-free entry point read packed rows
    # with the same kernels: bit-equal to csa_sparse_attn over the merged selection
    from tests.parity import assert_bf16_output, bf16_f64, dev_bf16, host_bits
    B, Nc, k, W = 3, 9000, 512, 128
    t = 4 * Nc - 1
    a = I.indexer_inputs(64, B, 1, Nc)
    at = I.attention_inputs(65, B, 1, Nc, W)
    rows, kv_d = pack_kv(bf16_f64(at["kv_comp_bf16"]), fmt)
    qpos = dev(np.full((B, 1), t, np.int64))
    cand = torch.empty(lib.index_segments_size(B, 1, Nc, k), dtype=torch.uint8, device="cuda")
    lib.csa_index_score_segments(dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), dev(a["kI_fp8"]),
                                 dev(a["kI_scale"]), qpos, m=4, k=k, cand=cand)
    idx = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    lib.csa_topk_merge(cand, B, 1, Nc, k, idx)
    q, kv, swa, sink = dev_bf16(at["q_bf16"]), dev(rows), dev_bf16(at["swa_bf16"]), dev(at["sink"])
    o1 = torch.empty(B, 1, 64, 512, dtype=torch.bfloat16, device="cuda")
    o2, o3 = torch.empty_like(o1), torch.empty_like(o1)
    lib.csa_sparse_attn(q, kv, idx, swa, sink, W=W, out=o1, q_pos=qpos, inv_rope_d=64, kv_format=fmt)
    lib.csa_topk_sparse_attn(q, kv, cand, swa, sink, k=k, W=W, out=o2, q_pos=qpos, inv_rope_d=64, kv_format=fmt)
    lib.csa_sparse_attn_noalloc(q, kv, idx, swa, sink, W=W, out=o3, q_pos=qpos, inv_rope_d=64, kv_format=fmt)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "fused selection + attention over packed rows differs"
    assert torch.equal(o1, o3), "allocation-free attention over packed rows differs"
    o_ref, _ = O.sparse_attention(bf16_f64(at["q_bf16"]), kv_d, idx.cpu().numpy(), bf16_f64(at["swa_bf16"]),
                                  at["sink"], 1 / math.sqrt(512), np.full((B, 1), t), W)
    o_ref = O.inverse_rope(o_ref, np.full((B, 1, 1), t), 64, 1e4)
    assert_bf16_output(bf16_f64(host_bits(o1)), o_ref, f"fused attention over packed rows (format {fmt})")


def test_packed_kv_rejected_with_fp32(lib):
    from compressed_sparse_kv_amd.binding import CSAError
    q = torch.zeros(1, 1, 8, 512, device="cuda")
    kv = torch.zeros(1, 10, 288, dtype=torch.uint8, device="cuda")
    idx = torch.zeros(1, 1, 4, dtype=torch.int32, device="cuda")
    swa = torch.zeros(1, 4, 512, device="cuda")
    with pytest.raises(CSAError):
        lib.csa_sparse_attn(q, kv, idx, swa, torch.zeros(8, device="cuda"), W=4, out=torch.empty_like(q),
                            kv_format=FMT_FP4)
