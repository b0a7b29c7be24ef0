"""CSA2 (DeepSeek-V4.1) rows through the C ABI against the oracle: the compressor (single
stream, no bias, ratio 1, indexer key from the main latent) and the hierarchical indexer
(block candidates of the Full layer, gather-then-score Reindex)."""

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from synthetic import inputs as I
from tests.parity import (TOL_F32, assert_bf16_output, assert_bf16_within_one_step, assert_close, assert_fp8_rows,
                          assert_topk_equal, bf16_f64, dev, dev_bf16, host_bits)

pytestmark = pytest.mark.gpu


def _w_proj(a, to_dev, conv):
    W = a["W_kv"] if a["W_gate"] is None else np.concatenate([a["W_kv"], a["W_gate"]], axis=1)
    return to_dev(np.ascontiguousarray(W.T)), conv(a["W_kv"]), None if a["W_gate"] is None else conv(a["W_gate"])


@pytest.mark.parametrize("m", [4, 2, 1])
def test_csa2_compress_bf16(lib, m):
    B, T, d, c, dI = 2, 64, 256, 512, 128
    a = I.csa2_inputs(800 + m, B, T, d, m, c, dI)
    kw = dict(m=m, d_rope=64, theta_kv=1e4, theta_k=1.6e5, rms_eps=1e-6, p0=4096)
    wp, Wkv, Wg = _w_proj(a, dev_bf16, bf16_f64)
    Wk = bf16_f64(a["W_k"])
    kv_ref, kI_ref = O.csa2_compress(bf16_f64(a["hidden"]), Wkv, Wg, Wk, **kw)
    n = T // m
    kv = torch.empty(B, n, c, dtype=torch.bfloat16, device="cuda")
    kI = torch.empty(B, n, dI, dtype=torch.uint8, device="cuda")
    kIs = torch.empty(B, n, device="cuda")
    lib.csa2_compress(dev_bf16(a["hidden"]), wp, dev_bf16(np.ascontiguousarray(a["W_k"].T)), kv_out=kv, k_out=kI,
                      k_scale=kIs, **kw)
    torch.cuda.synchronize()
    assert_bf16_within_one_step(host_bits(kv), kv_ref, f"CSA2 main KV (m={m})")
    assert_fp8_rows(kI.cpu().numpy(), kIs.cpu().numpy(), kI_ref, f"CSA2 indexer K (m={m})")
    # the same call with fp32 outputs: the latent and key before their casts
    kv32 = torch.empty(B, n, c, device="cuda")
    kI32 = torch.empty(B, n, dI, device="cuda")
    lib.csa2_compress(dev_bf16(a["hidden"]), wp, dev_bf16(np.ascontiguousarray(a["W_k"].T)), kv_out=kv32, k_out=kI32,
                      **kw)
    torch.cuda.synchronize()
    assert_close(kv32.cpu().numpy(), kv_ref, TOL_F32, f"CSA2 main KV fp32 (m={m})")
    assert_close(kI32.cpu().numpy(), kI_ref, TOL_F32, f"CSA2 indexer K fp32 (m={m})")


def test_csa2_compress_fp32_tiny(lib):
    B, T, d, c, dI, m = 1, 256, 256, 64, 32, 4
    a = I.csa2_inputs(810, B, T, d, m, c, dI, bf16=False)
    kw = dict(m=m, d_rope=16, theta_kv=1e4, theta_k=1.6e5, rms_eps=1e-6, p0=0)
    wp, Wkv, Wg = _w_proj(a, dev, lambda x: x.astype(np.float64))
    kv_ref, kI_ref = O.csa2_compress(a["hidden"], Wkv, Wg, a["W_k"], **kw)
    kv = torch.empty(B, T // m, c, device="cuda")
    kI = torch.empty(B, T // m, dI, device="cuda")
    lib.csa2_compress(dev(a["hidden"]), wp, dev(np.ascontiguousarray(a["W_k"].T)), kv_out=kv, k_out=kI, **kw)
    torch.cuda.synchronize()
    assert_close(kv.cpu().numpy(), kv_ref, TOL_F32, "CSA2 main KV (fp32)")
    assert_close(kI.cpu().numpy(), kI_ref, TOL_F32, "CSA2 indexer K (fp32)")


# ---------------------------------------------------------------------------------------
# Hierarchical indexer: Full layer (scores, own top-k, block maxima -> 2048 blocks) and a
# Reindex layer over the pool (gather, score with its own query, top-k)
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("B,Nc,t,n_blocks,layout", [
    (2, 32768, 4 * 32768 - 1, 2048, 1),       # V4-Flash-sized: 4096 blocks, 2048 chosen; blocked keys
    (2, 20011, 4 * 20003 + 1, 2048, 0),       # causal limit inside a block of 8, ragged Nc; row-major keys
    (1, 9000, 4 * 9000 - 1, 512, 0),          # a pool of exactly k = 512 blocks
])
def test_hierarchical_indexer(lib, B, Nc, t, n_blocks, layout):
    import math
    k, m = 512, 4
    a = I.indexer_inputs(900 + Nc, B, 1, Nc)
    a2 = I.indexer_inputs(901 + Nc, B, 1, Nc)                # the Reindex layer's own query and weights
    pos = np.full((B, 1), t, np.int64)
    qpos = dev(pos)
    k8, ks = dev(a["kI_fp8"]), dev(a["kI_scale"])
    keys = k8 if layout == 0 else lib.csa_index_keys_b16(k8, torch.empty(lib.index_keys_b16_size(B, Nc),
                                                                         dtype=torch.uint8, device="cuda"))
    # ---- Full layer
    cand = torch.empty(lib.index_segments_size(B, 1, Nc, k), dtype=torch.uint8, device="cuda")
    scores = torch.empty(B, 1, Nc, device="cuda")
    nb8 = -(-Nc // 8)
    bmax = torch.full((B, 1, nb8), 7.0, device="cuda")
    lib.csa_index_score_segments_bmax(dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), keys, ks, qpos, m=m, k=k,
                                      cand=cand, block_max=bmax, Nc=Nc, layout=layout, scores=scores)
    idx_full = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    lib.csa_topk_merge(cand, B, 1, Nc, k, idx_full)
    blocks = torch.empty(B, 1, n_blocks, dtype=torch.int32, device="cuda")
    lib.csa_topk(bmax, n_blocks, blocks)
    torch.cuda.synchronize()
    sc, bm, blk = scores.cpu().numpy(), bmax.cpu().numpy(), blocks.cpu().numpy()
    KI = O.dequant_rows(a["kI_fp8"], a["kI_scale"])
    sc_o = O.index_scores(O.dequant_rows(a["qI_fp8"], a["qI_scale"]), a["w"], KI, pos, m)
    assert_close(sc, sc_o, TOL_F32, "Full layer scores")
    assert np.array_equal(bm, O.block_scores(sc, 8).astype(np.float32)), "block maxima of the GPU's scores"
    blk_o, pool_o = O.candidate_pool(sc, 8, n_blocks)            # the pool from the GPU's own scores
    assert np.array_equal(blk, blk_o), "chosen blocks"
    # ---- Reindex layer with its own query
    cand2 = torch.empty(lib.index_pool_segments_size(B, 1, n_blocks, k), dtype=torch.uint8, device="cuda")
    psc = torch.full((B, 1, 8 * n_blocks), 7.0, device="cuda")
    lib.csa_index_score_pool(dev(a2["qI_fp8"]), dev(a2["qI_scale"]), dev(a2["w"]), k8, ks, qpos, blocks, m=m, k=k,
                             cand=cand2, scores=psc)
    idx2 = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    lib.csa_topk_merge(cand2, B, 1, 8 * n_blocks, k, idx2)
    # the same Reindex with the Full layer's query: the Full layer's own top-k (n_blocks >= k)
    cand3 = torch.empty_like(cand2)
    lib.csa_index_score_pool(dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), k8, ks, qpos, blocks, m=m, k=k,
                             cand=cand3)
    idx3 = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    lib.csa_topk_merge(cand3, B, 1, 8 * n_blocks, k, idx3)
    torch.cuda.synchronize()
    assert torch.equal(idx3, idx_full), "Reindex with the Full layer's query differs from its top-k"
    q2 = O.dequant_rows(a2["qI_fp8"], a2["qI_scale"])
    psc_o = O.pool_scores(q2, a2["w"], KI, pool_o, pos, m)
    assert_close(psc.cpu().numpy(), psc_o, TOL_F32, "Reindex pool scores")
    # positions: bit-exact against the selection over the GPU's pool scores, tie-tolerant against the oracle's
    got = idx2.cpu().numpy()
    sel_g = O.topk_indices(psc.cpu().numpy(), k)
    want_g = np.where(sel_g >= 0, np.take_along_axis(pool_o, np.maximum(sel_g, 0), axis=-1), -1)
    assert np.array_equal(got, want_g), "Reindex top-k over the GPU's pool scores"
    want_o = O.reindex_topk(q2, a2["w"], KI, pool_o, pos, m, k)
    full_o = np.full((B, 1, Nc), -np.inf)
    for b in range(B):
        v = pool_o[b, 0] >= 0
        full_o[b, 0, pool_o[b, 0][v]] = psc_o[b, 0][v]
    assert_topk_equal(got, want_o, full_o, k, "Reindex top-k vs oracle")
    # attention over the Reindex layer's selection (positions index the shared main KV)
    at = I.attention_inputs(902 + Nc, B, 1, Nc, 128)
    out = torch.empty(B, 1, 64, 512, dtype=torch.bfloat16, device="cuda")
    lib.csa_sparse_attn(dev_bf16(at["q_bf16"]), dev_bf16(at["kv_comp_bf16"]), idx2, dev_bf16(at["swa_bf16"]),
                        dev(at["sink"]), W=128, out=out, q_pos=qpos)
    torch.cuda.synchronize()
    o_o, _ = O.sparse_attention(bf16_f64(at["q_bf16"]), bf16_f64(at["kv_comp_bf16"]), got, bf16_f64(at["swa_bf16"]),
                                at["sink"], 1 / math.sqrt(512), pos, 128)
    assert_bf16_output(bf16_f64(host_bits(out)), o_o, "attention over the Reindex selection")
