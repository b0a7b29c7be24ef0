"""Low-precision caches written by the compressors through the C ABI: MXFP4 indexer keys
(E2M1 + E8M0 per 32), packed FP4 main-KV rows (E2M1 + E4M3 per 16) and packed FP8 rows with
bf16 RoPE channels, from the prefill compressor, the decode step and the CSA2 compressor.
Every scale and code is the oracle's quantisation of the oracle's row, except next to a
rounding boundary (the GPU quantises its fp32 row); then the CSA2 chain runs on those caches
alone: MXFP4 index scores, top-k, and attention reading the packed FP4 rows, against the
oracle on the dequantised caches."""

import math

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from synthetic import inputs as I
from tests.parity import (TOL_F32, assert_bf16_output, assert_close, assert_mxfp4_rows, assert_packed_fp4_rows,
                          assert_packed_fp8_rope_rows, assert_topk_equal, bf16_f64, dev, dev_bf16, host_bits,
                          unpack_nibbles)

pytestmark = pytest.mark.gpu

PACKED_BYTES = {4: 288, 5: 584}


def _out(lib, dtype, B, n, c):
    """(out, scale) buffers of a low-precision entry type."""
    if dtype == lib.CSA_FP4_E2M1:
        return (torch.zeros(B, n, c // 2, dtype=torch.uint8, device="cuda"),
                torch.zeros(B, n, c // 32, dtype=torch.uint8, device="cuda"))
    return torch.zeros(B, n, PACKED_BYTES[dtype], dtype=torch.uint8, device="cuda"), None


def _check(lib, dtype, out, scale, ref, what):
    o = out.cpu().numpy()
    if dtype == lib.CSA_FP4_E2M1:
        return assert_mxfp4_rows(o, scale.cpu().numpy(), ref, what)
    if dtype == lib.CSA_PACKED_FP4_E4M3:
        return assert_packed_fp4_rows(o, ref, what)
    return assert_packed_fp8_rope_rows(o, ref, what)


@pytest.mark.parametrize("c,dtype", [(512, 4), (512, 5), (128, 3)])
def test_prefill_compressor_lowp_entries(lib, c, dtype):
    B, T, d, m = 2, 64, 256, 4
    a = I.compressor_inputs(1200 + c + dtype, B, T, d, m, c, True, 0.05, True)
    kw = dict(overlap=True, m=m, c=c, d_rope=64, rope_theta=1e4, rms_eps=1e-6, p0=4096)
    ref = O.csa_compress(bf16_f64(a["hidden_bf16"]), bf16_f64(a["W_bf16"]), a["bias"],
                         hidden_prev=bf16_f64(a["hidden_prev_bf16"]), **kw)
    out, sc = _out(lib, dtype, B, T // m, c)
    lib.csa_compress(dev_bf16(a["hidden_bf16"]), dev_bf16(a["hidden_prev_bf16"]),
                     dev_bf16(np.ascontiguousarray(a["W_bf16"].T)), dev(a["bias"]), out=out, out_scale=sc,
                     out_dtype=dtype, **kw)
    torch.cuda.synchronize()
    _check(lib, dtype, out, sc, ref, f"prefill compressor entries (type {dtype})")


@pytest.mark.parametrize("c,dtype", [(512, 4), (512, 5), (128, 3)])
def test_decode_compressor_lowp_cache(lib, c, dtype):
    m, d, B, T, Nc_max = 4, 256, 2, 24, 9
    a = I.compressor_inputs(1300 + c + dtype, B, T, d, m, c, True, 0.05, False)
    kw = dict(overlap=True, m=m, c=c, d_rope=64, rope_theta=1e4, rms_eps=1e-6)
    state = torch.empty(lib.compress_state_size(B, m, c, True), dtype=torch.uint8, device="cuda")
    cache, sc = _out(lib, dtype, B, Nc_max, c)
    W = dev_bf16(np.ascontiguousarray(a["W_bf16"].T))
    for s in range(T):
        lib.csa_compress_decode(dev_bf16(np.ascontiguousarray(a["hidden_bf16"][:, s])), W, dev(a["bias"]),
                                dev(np.full(B, s, np.int64)), state, cache, cache_scale=sc, Nc_max=Nc_max,
                                out_dtype=dtype, **kw)
    torch.cuda.synchronize()
    n = T // m
    for b in range(B):
        ref = O.decode_compress(bf16_f64(a["hidden_bf16"][b]), bf16_f64(a["W_bf16"]), a["bias"], p0=0, **kw)
        v = np.stack([ref[i] for i in range(n)])[None]
        _check(lib, dtype, cache[b:b + 1, :n], None if sc is None else sc[b:b + 1, :n], v,
               f"decode cache (type {dtype}), sequence {b}")
        assert not cache[b, n:].any(), "rows of blocks not completed stay untouched"


@pytest.mark.parametrize("m", [4, 1])
def test_csa2_compressor_fp4_caches(lib, m):
    B, T, d, c, dI = 2, 64, 256, 512, 128
    a = I.csa2_inputs(1400 + m, B, T, d, m, c, dI)
    kw = dict(m=m, d_rope=64, theta_kv=1e4, theta_k=1.6e5, rms_eps=1e-6, p0=8192)
    W = a["W_kv"] if a["W_gate"] is None else np.concatenate([a["W_kv"], a["W_gate"]], axis=1)
    kv_ref, kI_ref = O.csa2_compress(bf16_f64(a["hidden"]), bf16_f64(a["W_kv"]),
                                     None if a["W_gate"] is None else bf16_f64(a["W_gate"]), bf16_f64(a["W_k"]), **kw)
    n = T // m
    kv, _ = _out(lib, lib.CSA_PACKED_FP4_E4M3, B, n, c)
    kI, kIs = _out(lib, lib.CSA_FP4_E2M1, B, n, dI)
    lib.csa2_compress(dev_bf16(a["hidden"]), dev_bf16(np.ascontiguousarray(W.T)),
                      dev_bf16(np.ascontiguousarray(a["W_k"].T)), kv_out=kv, k_out=kI, k_scale=kIs,
                      kv_dtype=lib.CSA_PACKED_FP4_E4M3, k_dtype=lib.CSA_FP4_E2M1, **kw)
    torch.cuda.synchronize()
    assert_packed_fp4_rows(kv.cpu().numpy(), kv_ref, f"CSA2 FP4 main KV (m={m})")
    assert_mxfp4_rows(kI.cpu().numpy(), kIs.cpu().numpy(), kI_ref, f"CSA2 MXFP4 indexer K (m={m})")


def test_csa2_fp4_chain_on_gpu_caches(lib):
    """CSA2 prefill compressor -> FP4 caches -> MXFP4 index scores -> top-k -> attention over
    the packed FP4 rows, for decode queries; each stage against the oracle fed with the
    dequantised GPU caches."""
    B, m, d, c, dI, k, W = 2, 4, 256, 512, 128, 64, 128
    T = 4096                                             # 1024 entries
    Nc = T // m
    a = I.csa2_inputs(1500, B, T, d, m, c, dI)
    Wp = np.concatenate([a["W_kv"], a["W_gate"]], axis=1)
    kv, _ = _out(lib, lib.CSA_PACKED_FP4_E4M3, B, Nc, c)
    kI, kIs = _out(lib, lib.CSA_FP4_E2M1, B, Nc, dI)
    lib.csa2_compress(dev_bf16(a["hidden"]), dev_bf16(np.ascontiguousarray(Wp.T)),
                      dev_bf16(np.ascontiguousarray(a["W_k"].T)), kv_out=kv, k_out=kI, k_scale=kIs,
                      kv_dtype=lib.CSA_PACKED_FP4_E4M3, k_dtype=lib.CSA_FP4_E2M1, m=m, d_rope=64, theta_kv=1e4,
                      theta_k=1.6e5, rms_eps=1e-6, p0=0)
    # decode queries at t = T - 1 (every entry visible) and T - 7 (the last 2 blocks not yet)
    pos = np.array([[T - 1], [T - 7]], np.int64)
    rs = np.random.default_rng(1501)
    q_idx = rs.standard_normal((B, 1, 64, dI))
    qc, qsc = O.quantize_mxfp4(q_idx)
    wts = (rs.standard_normal((B, 1, 64)) / math.sqrt(dI * 64)).astype(np.float32)
    scores = torch.empty(B, 1, Nc, device="cuda")
    lib.csa_index_score_mx(dev(np.ascontiguousarray((qc[..., 0::2] | (qc[..., 1::2] << 4)).astype(np.uint8))),
                           dev(qsc), dev(wts), kI, kIs, dev(pos), fp4=True, m=m, scores=scores)
    idx = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    lib.csa_topk(scores, k, idx)
    at = I.attention_inputs(1502, B, 1, Nc, W)
    out = torch.empty(B, 1, 64, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, 1, 64, device="cuda")
    lib.csa_sparse_attn(dev_bf16(at["q_bf16"]), kv, idx, dev_bf16(at["swa_bf16"]), dev(at["sink"]), W=W, out=out,
                        lse=lse, q_pos=dev(pos), inv_rope_d=64, kv_format=lib.CSA_KV_FP4_E4M3)
    torch.cuda.synchronize()
    # the oracle on the GPU's caches, dequantised
    rows = kv.cpu().numpy()
    kv_d = O.dequant_fp4_e4m3(unpack_nibbles(rows[..., :256]), rows[..., 256:288])
    kI_d = O.dequant_mxfp4(unpack_nibbles(kI.cpu().numpy()), kIs.cpu().numpy())
    s_ref = O.index_scores(O.dequant_mxfp4(qc, qsc), wts, kI_d, pos, m)
    assert_close(scores.cpu().numpy(), s_ref, TOL_F32, "MXFP4 scores over the compressor's keys")
    idx_ref = O.topk_indices(s_ref, k)
    assert_topk_equal(idx.cpu().numpy(), idx_ref, s_ref, k, "top-k over the compressor's keys")
    o_ref, l_ref = O.sparse_attention(bf16_f64(at["q_bf16"]), kv_d, idx.cpu().numpy(), bf16_f64(at["swa_bf16"]),
                                      at["sink"], 1 / math.sqrt(512), pos, W)
    o_ref = O.inverse_rope(o_ref, pos[..., None], 64, 1e4)
    assert_bf16_output(bf16_f64(host_bits(out)), o_ref, "attention over the compressor's FP4 rows")
    assert_close(lse.cpu().numpy(), l_ref, TOL_F32, "lse over the compressor's FP4 rows")


def test_lowp_entry_types_rejected_where_unsupported(lib):
    from compressed_sparse_kv_amd.binding import CSAError
    B, T, d, m = 1, 16, 256, 4
    h = torch.zeros(B, T, d, dtype=torch.bfloat16, device="cuda")
    Wt = torch.zeros(4 * 256, d, dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros(2, m, 256, device="cuda")
    out = torch.zeros(B, T // m, 288, dtype=torch.uint8, device="cuda")
    with pytest.raises(CSAError):                          # packed rows need c = 512
        lib.csa_compress(h, None, Wt, bias, overlap=True, m=m, c=256, d_rope=64, rope_theta=1e4, rms_eps=1e-6,
                         p0=0, out=out, out_dtype=lib.CSA_PACKED_FP4_E4M3)
    with pytest.raises(CSAError):                          # MXFP4 needs its scale bytes
        lib.csa_compress(h, None, Wt, bias, overlap=True, m=m, c=256, d_rope=64, rope_theta=1e4, rms_eps=1e-6,
                         p0=0, out=out, out_dtype=lib.CSA_FP4_E2M1)
