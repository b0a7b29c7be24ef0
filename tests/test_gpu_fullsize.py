"""Parity at the full workload sizes, in the launch configuration the bench times.

Every stage runs on the whole batch through the C ABI exactly as in a decode / prefill
step; the oracle then checks sampled outputs (queries, entries) one by one, and the
integer stage (top-k) is checked on every row against the oracle's selection over the
GPU's own scores (bit-exact), besides the tie-tolerant check against oracle scores."""

import math

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from synthetic import inputs as I
from tests.parity import (TOL_F32, assert_bf16_output, assert_bf16_within_one_step, assert_close, assert_fp8_rows,
                          assert_topk_equal, bf16_f64, dev, dev_bf16, host_bits)

pytestmark = pytest.mark.gpu


def _decode_chain(lib, sh, a):
    """index score -> top-k -> sparse attention for one decode step of the whole batch."""
    B, Nc, k = sh.B, sh.n_c, sh.k
    scores = torch.empty(B, 1, Nc, device="cuda")
    lib.csa_index_score(dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), dev(a["kI_fp8"]), dev(a["kI_scale"]),
                        dev(a["q_pos"]), m=sh.m, scores=scores)
    idx = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    lib.csa_topk(scores, k, idx)
    out = torch.empty(B, 1, sh.H, sh.c, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, 1, sh.H, device="cuda")
    lib.csa_sparse_attn(dev_bf16(a["q_bf16"]), dev_bf16(a["kv_comp_bf16"]), idx, dev_bf16(a["swa_bf16"]),
                        dev(a["sink"]), W=sh.W, out=out, lse=lse)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), idx.cpu().numpy(), out, lse.cpu().numpy()


def _check_decode(sh, a, scores, idx, out, lse, sample):
    k = sh.k
    # top-k, every row: bit-exact against the oracle's selection over the GPU's scores
    assert_topk_equal(idx, O.topk_indices(scores, k), scores, k, "top-k of GPU scores (all rows)", exact=True)
    out_bits = host_bits(out)
    for b in sample:
        sl = slice(b, b + 1)
        qI = O.dequant_rows(a["qI_fp8"][sl], a["qI_scale"][sl])
        KI = O.dequant_rows(a["kI_fp8"][sl], a["kI_scale"][sl])
        sc_o = O.index_scores(qI, a["w"][sl], KI, a["q_pos"][sl], sh.m)
        assert_close(scores[sl], sc_o, TOL_F32, f"index scores, sequence {b}")
        assert_topk_equal(idx[sl], O.topk_indices(sc_o, k), sc_o, k, f"top-k vs oracle scores, sequence {b}")
        o_o, lse_o = O.sparse_attention(bf16_f64(a["q_bf16"][sl]), bf16_f64(a["kv_comp_bf16"][sl]), idx[sl],
                                        bf16_f64(a["swa_bf16"][sl]), a["sink"], 1 / math.sqrt(sh.c),
                                        a["q_pos"][sl], sh.W)
        assert_bf16_output(bf16_f64(out_bits[sl]), o_o, f"attention, sequence {b}")
        assert_close(lse[sl], lse_o, TOL_F32, f"lse, sequence {b}")


def _decode_step_fused(lib, sh, a):
    """The decode step as the bench times it: scores with each segment's top-k, then the
    selection and the sparse attention in one call."""
    B, Nc, k = sh.B, sh.n_c, sh.k
    cand = torch.empty(lib.index_segments_size(B, 1, Nc, k), dtype=torch.uint8, device="cuda")
    lib.csa_index_score_segments(dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), dev(a["kI_fp8"]),
                                 dev(a["kI_scale"]), dev(a["q_pos"]), m=sh.m, k=k, cand=cand)
    idx = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    out = torch.empty(B, 1, sh.H, sh.c, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, 1, sh.H, device="cuda")
    lib.csa_topk_sparse_attn(dev_bf16(a["q_bf16"]), dev_bf16(a["kv_comp_bf16"]), cand, dev_bf16(a["swa_bf16"]),
                             dev(a["sink"]), k=k, W=sh.W, out=out, lse=lse, idx=idx)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), out, lse.cpu().numpy()


def _decode_step_bench(lib, sh, a):
    """The bench's timed calls on the Flash batch: scoring over the keys in 16-entry blocks
    with each segment's top-k (the scores written too, for the check), then the selection
    and the sparse attention in one call."""
    B, Nc, k = sh.B, sh.n_c, sh.k
    k16 = lib.csa_index_keys_b16(dev(a["kI_fp8"]), torch.empty(lib.index_keys_b16_size(B, Nc), dtype=torch.uint8,
                                                                 device="cuda"))
    cand = torch.empty(lib.index_segments_size(B, 1, Nc, k), dtype=torch.uint8, device="cuda")
    scores = torch.full((B, 1, Nc), 7.0, device="cuda")
    lib.csa_index_score_segments_b16(dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), k16, dev(a["kI_scale"]),
                                     dev(a["q_pos"]), m=sh.m, k=k, cand=cand, scores=scores)
    idx = torch.full((B, 1, k), -7, dtype=torch.int32, device="cuda")
    out = torch.empty(B, 1, sh.H, sh.c, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, 1, sh.H, device="cuda")
    lib.csa_topk_sparse_attn(dev_bf16(a["q_bf16"]), dev_bf16(a["kv_comp_bf16"]), cand, dev_bf16(a["swa_bf16"]),
                             dev(a["sink"]), k=k, W=sh.W, out=out, lse=lse, idx=idx)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), idx.cpu().numpy(), out, lse.cpu().numpy()


def test_flash_decode_full(lib):
    sh = I.FLASH_DECODE
    a = I.decode_inputs(sh).arrays
    scores, idx, out, lse = _decode_chain(lib, sh, a)
    _check_decode(sh, a, scores, idx, out, lse, sample=[0, 13, 31])
    # the bench's exact calls on the full batch, against the oracle on sampled sequences
    # (scores, selection bit-exact on every row over the GPU's scores, attention, lse)
    sc_b, idx_b, out_b, lse_b = _decode_step_bench(lib, sh, a)
    _check_decode(sh, a, sc_b, idx_b, out_b, lse_b, sample=[1, 8, 19, 26, 30])
    assert np.array_equal(idx_b, idx), "the bench's step selects other entries than the stage chain"
    # the bench's two-call step on the same inputs: the same selection on every row, and
    # the same attention output bit for bit (same kernels on the same rows in the same order)
    idx2, out2, lse2 = _decode_step_fused(lib, sh, a)
    assert np.array_equal(idx2, idx), "segment top-k + fused selection differ from csa_topk (full batch)"
    assert torch.equal(out2, out), "fused selection + attention differs from csa_sparse_attn (full batch)"
    assert np.array_equal(lse2, lse), "fused lse differs (full batch)"


def test_pro_decode_full(lib):
    sh = I.PRO_DECODE
    a = I.decode_inputs(sh).arrays
    scores, idx, out, lse = _decode_chain(lib, sh, a)
    _check_decode(sh, a, scores, idx, out, lse, sample=[0, 3])
    # the bench's scoring + top-k call (segment top-k, two merge levels): the same selection
    idx2 = torch.empty(sh.B, 1, sh.k, dtype=torch.int32, device="cuda")
    ws = torch.empty(lib.index_topk_workspace_size(sh.B, 1, sh.n_c, sh.k), dtype=torch.uint8, device="cuda")
    lib.csa_index_topk(dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), dev(a["kI_fp8"]), dev(a["kI_scale"]),
                       dev(a["q_pos"]), m=sh.m, k=sh.k, idx=idx2, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), idx), "fused scoring + top-k differs from the stage chain (Pro)"
    # the bench's Pro step: segment top-k, then the first merge level, the selection from
    # its pairs and the attention in one call
    idx3, out3, lse3 = _decode_step_fused(lib, sh, a)
    assert np.array_equal(idx3, idx), "segment top-k + merge level + fused selection differ from csa_topk (Pro)"
    assert torch.equal(out3, out), "fused selection + attention differs from csa_sparse_attn (Pro)"
    assert np.array_equal(lse3, lse), "fused lse differs (Pro)"


def test_hca_decode_full(lib):
    sh = I.HCA_DECODE
    a = I.decode_inputs(sh, with_indexer=False).arrays
    out = torch.empty(sh.B, 1, sh.H, sh.c, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(sh.B, 1, sh.H, device="cuda")
    lib.hca_dense_attn(dev_bf16(a["q_bf16"]), dev_bf16(a["kv_comp_bf16"]), dev(a["q_pos"]), dev_bf16(a["swa_bf16"]),
                       dev(a["sink"]), m=sh.m, W=sh.W, out=out, lse=lse)
    torch.cuda.synchronize()
    out_bits, lse = host_bits(out), lse.cpu().numpy()
    for b in (0, 37, 63):
        sl = slice(b, b + 1)
        o_o, lse_o = O.dense_attention(bf16_f64(a["q_bf16"][sl]), bf16_f64(a["kv_comp_bf16"][sl]), a["q_pos"][sl],
                                       sh.m, bf16_f64(a["swa_bf16"][sl]), a["sink"], 1 / math.sqrt(sh.c), sh.W)
        assert_bf16_output(bf16_f64(out_bits[sl]), o_o, f"HCA attention, sequence {b}")
        assert_close(lse[sl], lse_o, TOL_F32, f"HCA lse, sequence {b}")


def test_prefill_chunk_full(lib):
    sh = I.PREFILL
    a = I.prefill_inputs(sh)
    n_ctx, n_new = sh.ctx // sh.m, sh.S // sh.m
    Nc = n_ctx + n_new
    kw = dict(overlap=True, m=sh.m, d_rope=sh.d_rope, rope_theta=sh.rope_theta, rms_eps=1e-6, p0=sh.ctx)
    # ---- compressor: main KV (bf16) and indexer K (FP8 + row scale) for the chunk's entries
    hid, prev = dev_bf16(a["hidden_bf16"]), dev_bf16(a["hidden_prev_bf16"])
    kv = torch.empty(1, Nc, sh.c, dtype=torch.bfloat16, device="cuda")
    kv[:, :n_ctx].copy_(dev_bf16(a["kv_ctx_bf16"]))
    kI = torch.empty(1, Nc, sh.d_I, dtype=torch.uint8, device="cuda")
    kI[:, :n_ctx].copy_(dev(a["kI_ctx_fp8"]))
    kIs = torch.empty(1, Nc, device="cuda")
    kIs[:, :n_ctx].copy_(dev(a["kI_ctx_scale"]))
    lib.csa_compress(hid, prev, dev_bf16(np.ascontiguousarray(a["W_main_bf16"].T)), dev(a["B_main"]), c=sh.c,
                     out=kv[:, n_ctx:], **kw)
    kI_new = torch.empty(1, n_new, sh.d_I, dtype=torch.uint8, device="cuda")
    kIs_new = torch.empty(1, n_new, device="cuda")
    lib.csa_compress(hid, prev, dev_bf16(np.ascontiguousarray(a["W_idx_bf16"].T)), dev(a["B_idx"]), c=sh.d_I,
                     out=kI_new, out_scale=kIs_new, **kw)
    kI[:, n_ctx:].copy_(kI_new)
    kIs[:, n_ctx:].copy_(kIs_new)
    # ---- index scores for all 8192 queries, top-k, attention
    qpos = dev(a["q_pos"])
    scores = torch.empty(1, sh.S, Nc, device="cuda")
    lib.csa_index_score(dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), kI, kIs, qpos, m=sh.m, scores=scores)
    idx = torch.empty(1, sh.S, sh.k, dtype=torch.int32, device="cuda")
    lib.csa_topk(scores, sh.k, idx)
    out = torch.empty(1, sh.S, sh.H, sh.c, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, sh.S, sh.H, device="cuda")
    lib.csa_sparse_attn(dev_bf16(a["q_bf16"]), kv, idx, dev_bf16(a["swa_bf16"]), dev(a["sink"]), W=sh.W, out=out,
                        lse=lse)
    torch.cuda.synchronize()

    # compressor: sampled entries of the chunk (entry i pools block i and block i-1): the
    # first and last entries and a seeded sample in between
    hid_all = np.concatenate([a["hidden_prev_bf16"], a["hidden_bf16"]], axis=1)      # rows of blocks -1 .. S/m-1
    kv_new = host_bits(kv[:, n_ctx:])
    kI_codes, kI_sc = kI_new.cpu().numpy(), kIs_new.cpu().numpy()
    rng = np.random.default_rng(sh.seed + 500)
    ents = sorted({0, 1, 2, n_new - 2, n_new - 1, *rng.choice(np.arange(3, n_new - 2), 27, replace=False).tolist()})
    W_main, W_idx = bf16_f64(a["W_main_bf16"]), bf16_f64(a["W_idx_bf16"])
    for e in ents:
        blk = bf16_f64(hid_all[:, sh.m * (e + 1): sh.m * (e + 2)])
        blk_prev = bf16_f64(hid_all[:, sh.m * e: sh.m * (e + 1)])
        pos = sh.ctx + sh.m * e
        kw_e = dict(kw, p0=pos)
        ref = O.csa_compress(blk, W_main, a["B_main"], c=sh.c, hidden_prev=blk_prev, **kw_e)
        assert_bf16_within_one_step(kv_new[:, e:e + 1], ref, f"compressed KV, entry {n_ctx + e}")
        ref_i = O.csa_compress(blk, W_idx, a["B_idx"], c=sh.d_I, hidden_prev=blk_prev, **kw_e)
        assert_fp8_rows(kI_codes[:, e:e + 1], kI_sc[:, e:e + 1], ref_i, f"indexer K, entry {n_ctx + e}")

    # scores / top-k / attention for 256 sampled queries (on the GPU's K, which is checked
    # above): the first 64 and last 64 of the chunk (the first and last workgroups of the
    # indexer, the causal tile limits at both ends) and 128 seeded ones in between
    sc = scores.cpu().numpy()
    idx_h = idx.cpu().numpy()
    out_bits, lse_h = host_bits(out), lse.cpu().numpy()
    KI = O.dequant_rows(kI.cpu().numpy(), kIs.cpu().numpy())
    kv_h = host_bits(kv)
    mid = rng.choice(np.arange(64, sh.S - 64), 128, replace=False)
    sample = np.concatenate([np.arange(64), np.sort(mid), np.arange(sh.S - 64, sh.S)])
    for c0 in range(0, len(sample), 16):
        qs = sample[c0:c0 + 16]
        qI = O.dequant_rows(a["qI_fp8"][:, qs], a["qI_scale"][:, qs])
        sc_o = O.index_scores(qI, a["w"][:, qs], KI, a["q_pos"][:, qs], sh.m)
        assert_close(sc[:, qs], sc_o, TOL_F32, f"prefill scores, queries {qs.tolist()}")
        assert_topk_equal(idx_h[:, qs], O.topk_indices(sc[:, qs], sh.k), sc[:, qs], sh.k,
                          f"prefill top-k of GPU scores, queries {qs.tolist()}", exact=True)
        assert_topk_equal(idx_h[:, qs], O.topk_indices(sc_o, sh.k), sc_o, sh.k, f"prefill top-k, queries {qs.tolist()}")
        for s in qs:
            ss = slice(s, s + 1)
            sel = idx_h[0, s]
            rows = sorted({int(j) for j in sel if j >= 0})
            kv_sel = np.zeros((1, Nc, sh.c))
            kv_sel[0, rows] = bf16_f64(kv_h[0, rows])
            o_o, lse_o = O.sparse_attention(bf16_f64(a["q_bf16"][:, ss]), kv_sel, idx_h[:, ss],
                                            bf16_f64(a["swa_bf16"][:, s: s + sh.W]), a["sink"], 1 / math.sqrt(sh.c),
                                            a["q_pos"][:, ss], sh.W)
            assert_bf16_output(bf16_f64(out_bits[:, ss]), o_o, f"prefill attention, query {s}")
            assert_close(lse_h[:, ss], lse_o, TOL_F32, f"prefill lse, query {s}")
