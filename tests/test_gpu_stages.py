"""Stage-by-stage parity of the HIP library against the CPU oracle, at sizes the
oracle finishes in seconds that still span several tiles and a ragged tail, plus the
method's edge cases.  Every call goes through the C ABI (compressed_sparse_kv_amd.binding)."""

import math

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from synthetic import inputs as I
from tests.parity import (TOL_BF16_ATTN, TOL_F32, assert_bf16_output, assert_bf16_within_one_step, assert_close,
                          assert_fp8_rows, assert_topk_equal, bf16_f64, dev, dev_bf16, host_bits)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------------------
# Tiny fp32 layer, end to end: compress (main + indexer) -> scores -> top-k -> attention
# ---------------------------------------------------------------------------------------

def test_tiny_layer_chain_fp32(lib):
    sh = I.TINY
    a = I.tiny_inputs()
    kw = dict(overlap=True, m=sh.m, d_rope=sh.d_rope, rope_theta=sh.rope_theta, rms_eps=1e-6, p0=0)
    # oracle chain
    kv_o = O.csa_compress(a["hidden"], a["W_comp"], a["B_comp"], c=sh.c, **kw)
    kI_o = O.csa_compress(a["hidden"], a["W_icomp"], a["B_icomp"], c=sh.d_I, **kw)
    sc_o = O.index_scores(a["qI"], a["w"], kI_o, a["q_pos"], sh.m)
    idx_o = O.topk_indices(sc_o, sh.k)
    o_o, lse_o = O.sparse_attention(a["q"], kv_o, idx_o, a["swa"], a["sink"], 1 / math.sqrt(sh.c), a["q_pos"], sh.W)
    # GPU chain
    hid = dev(a["hidden"])
    kv = torch.empty(1, sh.N // sh.m, sh.c, device="cuda")
    kI = torch.empty(1, sh.N // sh.m, sh.d_I, device="cuda")
    lib.csa_compress(hid, None, dev(a["W_comp"].T), dev(a["B_comp"]), c=sh.c, out=kv, **kw)
    lib.csa_compress(hid, None, dev(a["W_icomp"].T), dev(a["B_icomp"]), c=sh.d_I, out=kI, **kw)
    qpos = dev(a["q_pos"])
    sc = torch.empty(1, 1, sh.N // sh.m, device="cuda")
    lib.csa_index_score(dev(a["qI"]), None, dev(a["w"]), kI, None, qpos, m=sh.m, scores=sc)
    idx = torch.empty(1, 1, sh.k, dtype=torch.int32, device="cuda")
    lib.csa_topk(sc, sh.k, idx)
    out = torch.empty(1, 1, sh.H, sh.c, device="cuda")
    lse = torch.empty(1, 1, sh.H, device="cuda")
    lib.csa_sparse_attn(dev(a["q"]), kv, idx, dev(a["swa"]), dev(a["sink"]), W=sh.W, out=out, lse=lse)
    # the attention stage again, fed the oracle's indices and entries
    out2 = torch.empty_like(out)
    lib.csa_sparse_attn(dev(a["q"]), dev(kv_o.astype(np.float32)), dev(idx_o.astype(np.int32)), dev(a["swa"]),
                        dev(a["sink"]), W=sh.W, out=out2)
    torch.cuda.synchronize()
    assert_close(kv.cpu().numpy(), kv_o, TOL_F32, "compressed KV")
    assert_close(kI.cpu().numpy(), kI_o, TOL_F32, "indexer K")
    assert_close(sc.cpu().numpy(), sc_o, TOL_F32, "index scores")
    assert_topk_equal(idx.cpu().numpy(), idx_o, sc_o, sh.k, "top-k")
    assert_close(out2.cpu().numpy(), o_o, TOL_F32, "attention (oracle indices)")
    # end to end, always: the oracle's attention over the GPU's own entries and selection
    # (where the selections agree this is the oracle chain itself)
    idx_g = idx.cpu().numpy()
    o_g, lse_g = O.sparse_attention(a["q"], kv.cpu().numpy().astype(np.float64), idx_g, a["swa"], a["sink"],
                                    1 / math.sqrt(sh.c), a["q_pos"], sh.W)
    assert_close(out.cpu().numpy(), o_g, TOL_F32, "attention (end to end, GPU entries and selection)")
    assert_close(lse.cpu().numpy(), lse_g, TOL_F32, "lse (end to end)")
    if np.array_equal(idx_g, idx_o):
        assert_close(out.cpu().numpy(), o_o, TOL_F32, "attention (end to end, oracle chain)")
        assert_close(lse.cpu().numpy(), lse_o, TOL_F32, "lse (oracle chain)")


# ---------------------------------------------------------------------------------------
# Stage 2: FP8 index scores (decode kernel for S <= 4, prefill kernel above)
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("B,S,Nc", [(2, 1, 1000), (3, 3, 257), (2, 37, 1000), (1, 130, 700)])
def test_index_score_fp8(lib, B, S, Nc):
    a = I.indexer_inputs(11 + S, B, S, Nc)
    m = 4
    # positions: the last query sees every entry in sequence 0; fewer elsewhere (causal edge)
    pos = np.zeros((B, S), np.int64)
    for b in range(B):
        t_last = 4 * Nc - 1 - b * 37 - (0 if b == 0 else 1)
        pos[b] = t_last - (S - 1) + np.arange(S)
    pos = np.maximum(pos, 0)
    sc = torch.empty(B, S, Nc, device="cuda")
    lib.csa_index_score(dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), dev(a["kI_fp8"]), dev(a["kI_scale"]),
                        dev(pos), m=m, scores=sc)
    ref = O.index_scores(O.dequant_rows(a["qI_fp8"], a["qI_scale"]), a["w"],
                         O.dequant_rows(a["kI_fp8"], a["kI_scale"]), pos, m)
    torch.cuda.synchronize()
    assert_close(sc.cpu().numpy(), ref, TOL_F32, "fp8 index scores")


def test_index_score_fp8_nothing_visible(lib):
    a = I.indexer_inputs(5, 1, 2, 300)
    pos = np.array([[0, 2]], np.int64)                  # t < m - 1: no complete block yet
    sc = torch.empty(1, 2, 300, device="cuda")
    lib.csa_index_score(dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), dev(a["kI_fp8"]), dev(a["kI_scale"]),
                        dev(pos), m=4, scores=sc)
    assert torch.all(sc == -math.inf)


# ---------------------------------------------------------------------------------------
# Stage 3: top-k, bit-exact on identical fp32 inputs
# ---------------------------------------------------------------------------------------

TOPK_CASES = [
    # rows, Nc, k, kind, algo
    (8, 1000, 32, "gauss", 1),
    (6, 1000, 1, "ties", 1),
    (4, 5000, 2048, "gauss", 1),
    (5, 3000, 64, "const", 1),
    (5, 3000, 64, "mixed", 1),
    (3, 32768, 512, "gauss", 1),
    (3, 32768, 512, "gauss", 2),
    (3, 32768, 512, "ties", 2),
    (2, 40000, 1024, "gauss", 1),
    (2, 40000, 1024, "mixed", 2),
    (2, 70000, 1024, "const", 2),
    (3, 32768, 512, "narrow", 1),
    (3, 32768, 512, "narrow", 2),
    (2, 70000, 2048, "gauss", 2),
    (2, 262144, 1024, "gauss", 0),
    (2, 262144, 1024, "narrow", 2),
    (300, 2000, 512, "mixed", 0),
    (64, 36864, 512, "gauss", 1),
    (3, 16000, 100, "ties", 1),
    (3, 9000, 2048, "narrow", 1),
    # more rows than compute units: the persistent long-row kernel takes a second row per
    # workgroup while the first is selected; 30004 scores leave a 52-score tail outside the
    # staged pieces, 36000 exceed the staging buffer
    (600, 30004, 512, "gauss", 1),
    (520, 36000, 300, "ties", 1),
]


@pytest.mark.parametrize("rows,Nc,k,kind,algo", TOPK_CASES)
def test_topk_exact(lib, rows, Nc, k, kind, algo):
    rng = np.random.default_rng(rows * 7 + Nc + k)
    n_vis = rng.integers(0, Nc + 1, rows)
    n_vis[0] = Nc
    if rows > 2:
        n_vis[1] = 0                                   # nothing visible: all -1
        n_vis[2] = min(Nc, max(1, k // 2))             # fewer candidates than k
    s = I.score_rows(rows + Nc, rows, Nc, kind, n_vis)
    idx = torch.empty(1, rows, k, dtype=torch.int32, device="cuda")
    lib.csa_topk(dev(s[None]), k, idx, algo=algo)
    ref = O.topk_indices(s, k)
    torch.cuda.synchronize()
    assert_topk_equal(idx.cpu().numpy(), ref, s, k, f"top-k {kind}", exact=True)


# ---------------------------------------------------------------------------------------
# Stage 4: bf16 attention (CSA sparse and HCA dense)
# ---------------------------------------------------------------------------------------

def _attn_case(lib, B, S, Nc, k, W, seed, n_valid, dense=False, m=128, q_pos=None, pass_pos=False, inv_rope_d=0,
               rope_theta=1e4):
    Ls = S + W - 1
    a = I.attention_inputs(seed, B, S, Nc, Ls)
    if q_pos is None:
        q_pos = np.tile(10 ** 6 - S + 1 + np.arange(S), (B, 1)).astype(np.int64)
    q_f = bf16_f64(a["q_bf16"]); kv_f = bf16_f64(a["kv_comp_bf16"]); swa_f = bf16_f64(a["swa_bf16"])
    out = torch.empty(B, S, 64, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, S, 64, device="cuda")
    rope = dict(inv_rope_d=inv_rope_d, rope_theta=rope_theta)
    if dense:
        lib.hca_dense_attn(dev_bf16(a["q_bf16"]), dev_bf16(a["kv_comp_bf16"]), dev(q_pos), dev_bf16(a["swa_bf16"]),
                           dev(a["sink"]), m=m, W=W, out=out, lse=lse, **rope)
        o_ref, l_ref = O.dense_attention(q_f, kv_f, q_pos, m, swa_f, a["sink"], 1 / math.sqrt(512), W)
    else:
        idx = I.random_selection(seed, B, S, Nc, k, n_valid)
        lib.csa_sparse_attn(dev_bf16(a["q_bf16"]), dev_bf16(a["kv_comp_bf16"]), dev(idx), dev_bf16(a["swa_bf16"]),
                            dev(a["sink"]), W=W, out=out, lse=lse, q_pos=dev(q_pos) if pass_pos or inv_rope_d else None,
                            **rope)
        o_ref, l_ref = O.sparse_attention(q_f, kv_f, idx, swa_f, a["sink"], 1 / math.sqrt(512), q_pos, W)
    if inv_rope_d:
        o_ref = O.inverse_rope(o_ref, q_pos[..., None], inv_rope_d, rope_theta)
    torch.cuda.synchronize()
    assert_bf16_output(bf16_f64(host_bits(out)), o_ref, "attention output")
    assert_close(lse.cpu().numpy(), l_ref, TOL_F32, "lse")


def test_sparse_attn_decode_split_rows(lib):
    # 3 queries -> several workgroups per query (LSE merge); idx with -1 padding
    _attn_case(lib, B=3, S=1, Nc=2000, k=512, W=128, seed=1, n_valid=np.array([[512], [300], [0]]))


def test_sparse_attn_prefill_windows(lib):
    # consecutive queries, each with its own sliding window; many queries -> one workgroup per query
    _attn_case(lib, B=2, S=40, Nc=900, k=64, W=128, seed=2, n_valid=64)


def test_sparse_attn_many_queries_single_split(lib):
    _attn_case(lib, B=8, S=64, Nc=600, k=96, W=128, seed=3, n_valid=90)


def test_sparse_attn_full_channel_splits(lib):
    # 64 queries: full-channel workgroups, 4 splits per query (merge); padded selections,
    # one query with nothing selected (window rows and sink only)
    n_valid = np.linspace(2048, 0, 64).astype(np.int64)[:, None]
    _attn_case(lib, B=64, S=1, Nc=5000, k=2048, W=128, seed=7, n_valid=n_valid)


def test_hca_dense_attn_full_channel_splits(lib):
    # 64 queries over 2100 entries: full-channel workgroups, 4 splits; causal bounds from
    # every entry down to none (query 63 sees window rows only)
    q_pos = (128 * (2100 - 33 * np.arange(64)) - 1).astype(np.int64)[:, None]
    q_pos[63, 0] = 100
    _attn_case(lib, B=64, S=1, Nc=2100, k=0, W=128, seed=8, n_valid=0, dense=True, q_pos=q_pos)


def test_sparse_attn_short_sequences(lib):
    # sequences shorter than the window tensor (positions 0 .. t only): rows of negative
    # positions are left out when q_pos is given; a sequence at position 0 sees one row
    q_pos = np.array([[0], [50], [126], [127], [10 ** 6]], np.int64)
    _attn_case(lib, B=5, S=1, Nc=300, k=64, W=128, seed=9, n_valid=np.array([[0], [3], [64], [64], [64]]),
               q_pos=q_pos, pass_pos=True)


def test_sparse_attn_short_prefill(lib):
    # 70 consecutive queries from position 0: full-channel kernel, windows cut at position 0
    q_pos = np.arange(70, dtype=np.int64)[None]
    _attn_case(lib, B=1, S=70, Nc=40, k=16, W=128, seed=10, n_valid=np.minimum(np.arange(70) // 4, 16)[None],
               q_pos=q_pos, pass_pos=True)


def test_hca_dense_attn_many_splits_narrow(lib):
    # 2 queries over 20736 entries: 64 splits per query (merge over more than 8 partials)
    q_pos = np.array([[128 * 20736 - 1], [128 * 20000 + 5]], np.int64)
    _attn_case(lib, B=2, S=1, Nc=20736, k=0, W=128, seed=11, n_valid=0, dense=True, q_pos=q_pos)


def test_hca_dense_attn_many_splits_wide(lib):
    # 64 consecutive queries over 20736 entries: the 64-head shape, 10 splits (row tables
    # of at most 72 chunks), merge over more than 8 partials
    S = 64
    q_pos = (128 * 20736 - S + np.arange(S, dtype=np.int64))[None]
    _attn_case(lib, B=1, S=S, Nc=20736, k=0, W=128, seed=12, n_valid=0, dense=True, q_pos=q_pos)


def test_hca_dense_attn(lib):
    # sequence 0 sees all 300 entries, sequence 1 only the first 200 (causal bound)
    q_pos = np.array([[128 * 300 - 1], [128 * 200 + 126]], np.int64)
    _attn_case(lib, B=2, S=1, Nc=300, k=0, W=128, seed=4, n_valid=0, dense=True, q_pos=q_pos)


def test_hca_dense_attn_prefill_rows(lib):
    S = 24
    q_pos = np.tile(128 * 40 - S + np.arange(S), (1, 1)).astype(np.int64)   # crosses an entry boundary
    _attn_case(lib, B=1, S=S, Nc=64, k=0, W=128, seed=5, n_valid=0, dense=True, q_pos=q_pos)


# inverse RoPE of the output, fused with the cast in each place an output is written: the
# attention kernel itself (one split), the tiled merge (several splits; 64-head and
# 32-head shapes) and the fp32 path
@pytest.mark.parametrize("case", ["single_split", "merge_narrow", "merge_wide", "hca_merge"])
def test_attention_inverse_rope(lib, case):
    if case == "single_split":
        _attn_case(lib, B=8, S=64, Nc=600, k=96, W=128, seed=31, n_valid=90, inv_rope_d=64)
    elif case == "merge_narrow":
        _attn_case(lib, B=3, S=1, Nc=2000, k=512, W=128, seed=32, n_valid=512, inv_rope_d=64, rope_theta=1.6e5)
    elif case == "merge_wide":
        _attn_case(lib, B=64, S=1, Nc=3000, k=1024, W=128, seed=33, n_valid=1024, inv_rope_d=128)
    else:
        # 2 queries over 3000 entries: more than four splits (the one-tile merge)
        q_pos = np.array([[128 * 3000 - 1], [128 * 2000 + 126]], np.int64)
        _attn_case(lib, B=2, S=1, Nc=3000, k=0, W=128, seed=34, n_valid=0, dense=True, q_pos=q_pos, inv_rope_d=64)


def test_attention_inverse_rope_fp32_and_fused(lib):
    # fp32 kernel (tiny shape) against the oracle
    rng = np.random.default_rng(35)
    B, Nc, k, H, c, W = 2, 200, 32, 8, 64, 128
    q = rng.standard_normal((B, 1, H, c)).astype(np.float32)
    kv = rng.standard_normal((B, Nc, c)).astype(np.float32)
    swa = rng.standard_normal((B, W, c)).astype(np.float32)
    sink = rng.standard_normal(H).astype(np.float32)
    idx = np.sort(np.stack([rng.choice(Nc, k, replace=False) for _ in range(B)]), axis=1)[:, None].astype(np.int32)
    pos = np.array([[1023], [70000]], np.int64)
    out = torch.empty(B, 1, H, c, device="cuda")
    lib.csa_sparse_attn(dev(q), dev(kv), dev(idx), dev(swa), dev(sink), W=W, out=out, q_pos=dev(pos), inv_rope_d=16)
    o_ref, _ = O.sparse_attention(q, kv, idx, swa, sink, 1 / math.sqrt(c), pos, W)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), O.inverse_rope(o_ref, pos[..., None], 16, 1e4), TOL_F32, "fp32 inverse RoPE")
    # the fused selection + attention applies the same epilogue as csa_sparse_attn, bit for bit
    B, Nc, k = 3, 9000, 512
    t = 4 * Nc - 1
    a = I.indexer_inputs(36, B, 1, Nc)
    at = I.attention_inputs(37, B, 1, Nc, W)
    qpos = dev(np.full((B, 1), t, np.int64))
    cand = torch.empty(lib.index_segments_size(B, 1, Nc, k), dtype=torch.uint8, device="cuda")
    lib.csa_index_score_segments(dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), dev(a["kI_fp8"]),
                                 dev(a["kI_scale"]), qpos, m=4, k=k, cand=cand)
    args = (dev_bf16(at["q_bf16"]), dev_bf16(at["kv_comp_bf16"]))
    idx_ref = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    lib.csa_topk_merge(cand, B, 1, Nc, k, idx_ref)
    o1 = torch.empty(B, 1, 64, 512, dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty_like(o1)
    lib.csa_sparse_attn(*args, idx_ref, dev_bf16(at["swa_bf16"]), dev(at["sink"]), W=W, out=o1, q_pos=qpos,
                        inv_rope_d=64)
    lib.csa_topk_sparse_attn(*args, cand, dev_bf16(at["swa_bf16"]), dev(at["sink"]), k=k, W=W, out=o2, q_pos=qpos,
                             inv_rope_d=64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "fused selection + attention: inverse RoPE epilogue differs"
    o_ref, _ = O.sparse_attention(bf16_f64(at["q_bf16"]), bf16_f64(at["kv_comp_bf16"]), idx_ref.cpu().numpy(),
                                  bf16_f64(at["swa_bf16"]), at["sink"], 1 / math.sqrt(512), np.full((B, 1), t), W)
    assert_bf16_output(bf16_f64(host_bits(o2)), O.inverse_rope(o_ref, t, 64, 1e4), "fused attention, inverse RoPE")


def test_attention_sink_only_limit(lib):
    a = I.attention_inputs(6, 1, 1, 100, 128)
    idx = I.random_selection(6, 1, 1, 100, 32, 32)
    out = torch.empty(1, 1, 64, 512, dtype=torch.bfloat16, device="cuda")
    lib.csa_sparse_attn(dev_bf16(a["q_bf16"]), dev_bf16(a["kv_comp_bf16"]), dev(idx), dev_bf16(a["swa_bf16"]),
                        dev(np.full(64, 1e4, np.float32)), W=128, out=out)
    assert torch.all(out.float().abs() == 0)


# ---------------------------------------------------------------------------------------
# Stage 1: compressor (bf16 MFMA projection)
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("overlap,m,c,T,with_prev,out_kind", [
    (True, 4, 512, 256, True, "bf16"),
    (True, 4, 128, 200, True, "fp8"),
    (True, 4, 512, 64, False, "bf16"),
    (False, 128, 512, 512, False, "bf16"),
    (False, 128, 512, 8192, False, "bf16"),          # the HCA compressor over 8192 tokens: 64 entries
])
def test_compress_bf16(lib, overlap, m, c, T, with_prev, out_kind):
    B, d = (1, 256) if T >= 4096 else (2, 256)
    a = I.compressor_inputs(20 + m + c, B, T, d, m, c, overlap, 0.05, with_prev)
    p0 = 4096 if with_prev else 0
    kw = dict(overlap=overlap, m=m, c=c, d_rope=64, rope_theta=1e4, rms_eps=1e-6, p0=p0)
    hp = a.get("hidden_prev_bf16")
    ref = O.csa_compress(bf16_f64(a["hidden_bf16"]), bf16_f64(a["W_bf16"]), a["bias"],
                         hidden_prev=None if hp is None else bf16_f64(hp), **kw)
    Wt = np.ascontiguousarray(a["W_bf16"].T)
    n = T // m
    if out_kind == "bf16":
        out = torch.empty(B, n, c, dtype=torch.bfloat16, device="cuda")
        lib.csa_compress(dev_bf16(a["hidden_bf16"]), None if hp is None else dev_bf16(hp), dev_bf16(Wt),
                         dev(a["bias"]), out=out, **kw)
        torch.cuda.synchronize()
        assert_bf16_within_one_step(host_bits(out), ref, "compressed KV (bf16)")
    else:
        out = torch.empty(B, n, c, dtype=torch.uint8, device="cuda")
        sc = torch.empty(B, n, device="cuda")
        lib.csa_compress(dev_bf16(a["hidden_bf16"]), None if hp is None else dev_bf16(hp), dev_bf16(Wt),
                         dev(a["bias"]), out=out, out_scale=sc, **kw)
        torch.cuda.synchronize()
        assert_fp8_rows(out.cpu().numpy(), sc.cpu().numpy(), ref, "indexer K (fp8)")


# ---------------------------------------------------------------------------------------
# The decode chain captured in a HIP graph: every replay equals the eager result
# ---------------------------------------------------------------------------------------

def test_decode_chain_graph_replay(lib):
    B, Nc, k, m, W = 4, 5000, 256, 4, 128
    a = I.indexer_inputs(41, B, 1, Nc)
    at = I.attention_inputs(42, B, 1, Nc, W)
    qpos = dev(np.full((B, 1), 4 * Nc + 3, np.int64))
    q8, qs, w, k8, ks = dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), dev(a["kI_fp8"]), dev(a["kI_scale"])
    q, kv, swa, sink = dev_bf16(at["q_bf16"]), dev_bf16(at["kv_comp_bf16"]), dev_bf16(at["swa_bf16"]), dev(at["sink"])
    scores = torch.empty(B, 1, Nc, device="cuda")
    idx = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    out = torch.empty(B, 1, 64, 512, dtype=torch.bfloat16, device="cuda")
    tk_ws = torch.empty(max(1, lib.topk_workspace_size(B, Nc, k)), dtype=torch.uint8, device="cuda")
    at_ws = torch.empty(max(1, lib.attn_workspace_size(B, 1, 64, 512, W + k, lib.CSA_BF16)), dtype=torch.uint8,
                        device="cuda")

    cand = torch.empty(lib.index_segments_size(B, 1, Nc, k), dtype=torch.uint8, device="cuda")

    def step():
        lib.csa_index_score(q8, qs, w, k8, ks, qpos, m=m, scores=scores)
        lib.csa_topk(scores, k, idx, ws=tk_ws)
        lib.csa_sparse_attn(q, kv, idx, swa, sink, W=W, out=out, ws=at_ws)

    def step_segments():
        lib.csa_index_score_segments(q8, qs, w, k8, ks, qpos, m=m, k=k, cand=cand, scores=scores)
        lib.csa_topk_merge(cand, B, 1, Nc, k, idx)
        lib.csa_sparse_attn(q, kv, idx, swa, sink, W=W, out=out, ws=at_ws)

    def step_fused():
        lib.csa_index_score_segments(q8, qs, w, k8, ks, qpos, m=m, k=k, cand=cand, scores=scores)
        lib.csa_topk_sparse_attn(q, kv, cand, swa, sink, k=k, W=W, out=out, idx=idx, ws=at_ws)

    step()
    torch.cuda.synchronize()
    ref = (scores.clone(), idx.clone(), out.clone())
    for fn in (step, step_segments, step_fused):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for r in range(3):
            scores.fill_(7.0)
            idx.fill_(-7)
            out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(scores, ref[0]), f"{fn.__name__}: scores differ on replay {r}"
            assert torch.equal(idx, ref[1]), f"{fn.__name__}: indices differ on replay {r}"
            assert torch.equal(out, ref[2]), f"{fn.__name__}: attention differs on replay {r}"
            fn()                                   # eager work between the replays
            torch.cuda.synchronize()


# ---------------------------------------------------------------------------------------
# Stages 2 + 3 in one call: identical to csa_index_score followed by csa_topk
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("B,S,Nc,k,t,with_scores", [
    (3, 1, 32768, 512, 4 * 32768 - 1, True),       # decode, fused path
    (2, 1, 5000, 256, 4 * 5000 + 7, False),        # ragged last segment, no score output
    (2, 2, 9000, 300, 4 * 2500 + 2, True),         # causal limit inside the row, 2 queries
    (1, 1, 3000, 2048, 4 * 3000 - 1, True),        # k above the visible count
    (2, 8, 3000, 128, 4 * 3000 + 40, True),        # prefill shape: the two stages back to back
    (1, 1, 262144, 1024, 4 * 262144 - 1, False),   # Pro shape: 64 x 1024 candidates, two merge levels
    (2, 1, 86000, 2048, 4 * 86000 - 1, True),      # two levels, the last group of segments ragged
    (1, 1, 150000, 1024, 4 * 100000 + 1, False),   # two levels, segments past the causal limit empty
    (32, 1, 32768, 512, 4 * 32768 - 1, False),     # V4-Flash decode batch
    (2, 1, 20000, 512, 4 * 20000 - 1, True),       # five segments, the last ragged
])
def test_index_topk_fused(lib, B, S, Nc, k, t, with_scores):
    a = I.indexer_inputs(B * 1000 + Nc + k, B, S, Nc)
    pos = (t - S + 1 + np.arange(S, dtype=np.int64))[None].repeat(B, 0)
    args = (dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), dev(a["kI_fp8"]), dev(a["kI_scale"]), dev(pos))
    sc_ref = torch.empty(B, S, Nc, device="cuda")
    lib.csa_index_score(*args[:5], args[5], m=4, scores=sc_ref)
    idx_ref = torch.empty(B, S, k, dtype=torch.int32, device="cuda")
    lib.csa_topk(sc_ref, k, idx_ref)
    idx = torch.empty(B, S, k, dtype=torch.int32, device="cuda")
    sc = torch.empty(B, S, Nc, device="cuda") if with_scores else None
    lib.csa_index_topk(*args, m=4, k=k, idx=idx, scores=sc)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_ref), "fused top-k differs from csa_index_score + csa_topk"
    if with_scores:
        assert torch.equal(sc, sc_ref), "fused scores differ from csa_index_score"
    # the same path as two calls (segment candidates, then the merge), where it applies
    nbytes = lib.index_segments_size(B, S, Nc, k)
    if nbytes:
        cand = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        sc2 = torch.empty(B, S, Nc, device="cuda") if with_scores else None
        lib.csa_index_score_segments(*args, m=4, k=k, cand=cand, scores=sc2)
        idx2 = torch.empty(B, S, k, dtype=torch.int32, device="cuda")
        lib.csa_topk_merge(cand, B, S, Nc, k, idx2)
        torch.cuda.synchronize()
        assert torch.equal(idx2, idx_ref), "segments + merge differ from csa_index_score + csa_topk"
        if with_scores:
            assert torch.equal(sc2, sc_ref), "segment pass scores differ from csa_index_score"
    # and against the oracle, on the first query
    qI = O.dequant_rows(a["qI_fp8"][:1, :1], a["qI_scale"][:1, :1])
    KI = O.dequant_rows(a["kI_fp8"][:1], a["kI_scale"][:1])
    sc_o = O.index_scores(qI, a["w"][:1, :1], KI, pos[:1, :1], 4)
    assert_topk_equal(idx[:1, :1].cpu().numpy(), O.topk_indices(sc_o, k), sc_o, k, "fused top-k vs oracle")


# ---------------------------------------------------------------------------------------
# Stages 3 + 4a in one call: identical to csa_topk_merge followed by csa_sparse_attn
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("B,S,Nc,k,t", [
    (3, 1, 32768, 512, 4 * 32768 - 1),     # decode: 8 segments, 4096 candidates per query
    (2, 1, 5000, 256, 4 * 5000 + 7),       # ragged last segment
    (2, 2, 9000, 301, 4 * 2500 + 2),       # causal limit inside the row; odd candidate count
    (1, 1, 1500, 2048, 4 * 1500 - 1),      # k above the visible count: -1 padding
    (2, 4, 6000, 512, 4 * 6000 - 1),       # four queries per sequence
    (64, 1, 4096, 512, 4 * 4096 - 1),      # many queries: the 64-head workgroup shape
    (16, 4, 17000, 1024, 4 * 17000 - 1),   # 64 queries, 5 x 1024 candidates: 16 per thread, 64-head shape
    (1, 1, 8192, 2048, 4 * 8192 - 1),      # the largest selection: 2 x 2048 candidates, k = 2048
    (2, 1, 65536, 512, 4 * 65536 - 1),     # 16 segments: 8192 candidates, 16 per thread, one level
    (1, 1, 36000, 901, 4 * 36000 - 1),     # 9 segments x 901: an odd count of 16-per-thread candidates
    (1, 1, 150000, 1024, 4 * 100000 + 1),  # 37 segments: first merge level (7 x 1024) in the call; empty tail
])
def test_topk_sparse_attn_fused(lib, B, S, Nc, k, t):
    a = I.indexer_inputs(7000 + B + Nc + k, B, S, Nc)
    W = 128
    Ls = S + W - 1
    at = I.attention_inputs(8000 + B + Nc, B, S, Nc, Ls)
    pos = (t - S + 1 + np.arange(S, dtype=np.int64))[None].repeat(B, 0)
    qpos = dev(pos)
    cand = torch.empty(lib.index_segments_size(B, S, Nc, k), dtype=torch.uint8, device="cuda")
    lib.csa_index_score_segments(dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]), dev(a["kI_fp8"]),
                                 dev(a["kI_scale"]), qpos, m=4, k=k, cand=cand)
    q, kv, swa, sink = dev_bf16(at["q_bf16"]), dev_bf16(at["kv_comp_bf16"]), dev_bf16(at["swa_bf16"]), dev(at["sink"])
    idx_ref = torch.empty(B, S, k, dtype=torch.int32, device="cuda")
    lib.csa_topk_merge(cand, B, S, Nc, k, idx_ref)
    out_ref = torch.empty(B, S, 64, 512, dtype=torch.bfloat16, device="cuda")
    lse_ref = torch.empty(B, S, 64, device="cuda")
    lib.csa_sparse_attn(q, kv, idx_ref, swa, sink, W=W, out=out_ref, lse=lse_ref, q_pos=qpos)
    out = torch.full_like(out_ref, 7.0)
    lse = torch.full_like(lse_ref, 7.0)
    idx = torch.full_like(idx_ref, -7)
    lib.csa_topk_sparse_attn(q, kv, cand, swa, sink, k=k, W=W, out=out, lse=lse, idx=idx, q_pos=qpos)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_ref), "fused selection differs from csa_topk_merge"
    assert torch.equal(out, out_ref), "fused attention differs from csa_sparse_attn"
    assert torch.equal(lse, lse_ref), "fused lse differs from csa_sparse_attn"
    # without the index output, the same attention
    out2 = torch.zeros_like(out_ref)
    lib.csa_topk_sparse_attn(q, kv, cand, swa, sink, k=k, W=W, out=out2, q_pos=qpos)
    torch.cuda.synchronize()
    assert torch.equal(out2, out_ref), "fused attention without idx output differs"
    # without q_pos (every window row a real position), as csa_sparse_attn without it
    out3 = torch.zeros_like(out_ref)
    out3_ref = torch.zeros_like(out_ref)
    lib.csa_sparse_attn(q, kv, idx_ref, swa, sink, W=W, out=out3_ref)
    lib.csa_topk_sparse_attn(q, kv, cand, swa, sink, k=k, W=W, out=out3)
    torch.cuda.synchronize()
    assert torch.equal(out3, out3_ref), "fused attention without q_pos differs"
    # and the first query against the oracle: its own scores, top-k and attention
    qI = O.dequant_rows(a["qI_fp8"][:1, :1], a["qI_scale"][:1, :1])
    KI = O.dequant_rows(a["kI_fp8"][:1], a["kI_scale"][:1])
    sc_o = O.index_scores(qI, a["w"][:1, :1], KI, pos[:1, :1], 4)
    assert_topk_equal(idx[:1, :1].cpu().numpy(), O.topk_indices(sc_o, k), sc_o, k, "fused selection vs oracle")
    o_ref, l_ref = O.sparse_attention(bf16_f64(at["q_bf16"][:1]), bf16_f64(at["kv_comp_bf16"][:1]),
                                      idx[:1].cpu().numpy(), bf16_f64(at["swa_bf16"][:1]), at["sink"],
                                      1 / math.sqrt(512), pos[:1], W)
    assert_bf16_output(bf16_f64(host_bits(out[:1])), o_ref, "fused attention vs oracle")
    assert_close(lse[:1].cpu().numpy(), l_ref, TOL_F32, "fused lse vs oracle")


# ---------------------------------------------------------------------------------------
# Stages 3 + 4a in one call on crafted candidate sets: equal keys (ties decided by the
# lower entry), few distinct keys (the exact radix path of the selection core), and
# segments with empty slots; 8 per thread, 16 per thread, and a first merge level
# ---------------------------------------------------------------------------------------

def _crafted_pairs(rng, rows, G, k, Nc, per_row, kind):
    """rows x per_row (key, entry) uint32 pairs: segment g's k slots hold entries of
    [4096 g, 4096 (g + 1)) in ascending order (key 0 = empty slot, entry 0)."""
    pairs = np.zeros((rows, per_row, 2), np.uint32)
    for r in range(rows):
        for g in range(G):
            lo, hi = 4096 * g, min(4096 * (g + 1), Nc)
            n = min(k, hi - lo)
            if kind == "sparse":
                n = int(rng.integers(0, n + 1))
            ent = np.sort(rng.choice(np.arange(lo, hi), size=n, replace=False)).astype(np.uint32)
            if kind == "equal":
                key = np.full(n, 0xBF800000, np.uint32)
            elif kind == "few":
                key = rng.choice(np.array([0xBF000000, 0xC0000000, 0xC0400000], np.uint32), size=n)
            else:
                key = rng.integers(1, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
            pairs[r, g * k:g * k + n, 0] = key
            pairs[r, g * k:g * k + n, 1] = ent
    return pairs


def _select_pairs(pairs_row, k):
    """The k best valid pairs (key descending, then lower entry), entries ascending, -1 padded."""
    valid = pairs_row[pairs_row[:, 0] != 0]
    order = np.lexsort((valid[:, 1], -valid[:, 0].astype(np.int64)))
    sel = np.sort(valid[order[:k], 1].astype(np.int64))
    return np.concatenate([sel, np.full(k - len(sel), -1, np.int64)])


@pytest.mark.parametrize("B,S,G,k,kind", [
    (2, 1, 8, 512, "equal"), (2, 1, 8, 512, "few"), (2, 1, 8, 512, "sparse"),
    (2, 1, 16, 512, "equal"), (2, 1, 16, 512, "few"), (2, 1, 16, 512, "sparse"),
    (1, 1, 37, 1024, "few"), (1, 1, 37, 1024, "sparse"),
    (1, 3, 16, 512, "rand"),                # several queries per sequence, 16 per thread
    (1, 2, 37, 1024, "equal"),              # several queries per sequence, first merge level
])
def test_topk_sparse_attn_fused_crafted(lib, B, S, G, k, kind):
    rng = np.random.default_rng(9100 + 7 * G + k + len(kind) + S)
    Nc = 4096 * G - 1000                    # ragged last segment
    W = 128
    Ls = W + S - 1
    per_row = lib.index_segments_size(B, S, Nc, k) // (8 * B * S)
    pairs = _crafted_pairs(rng, B * S, G, k, Nc, per_row, kind)
    cand = torch.from_numpy(pairs.view(np.uint8).reshape(-1).copy()).cuda()
    at = I.attention_inputs(9200 + G, B, S, Nc, Ls)
    q, kv, swa, sink = dev_bf16(at["q_bf16"]), dev_bf16(at["kv_comp_bf16"]), dev_bf16(at["swa_bf16"]), dev(at["sink"])
    idx_ref = torch.empty(B, S, k, dtype=torch.int32, device="cuda")
    lib.csa_topk_merge(cand, B, S, Nc, k, idx_ref)
    torch.cuda.synchronize()
    want = np.stack([_select_pairs(pairs[r, :G * k], k) for r in range(B * S)]).reshape(B, S, k)
    assert np.array_equal(idx_ref.cpu().numpy(), want), f"csa_topk_merge on {kind} candidates"
    out_ref = torch.empty(B, S, 64, 512, dtype=torch.bfloat16, device="cuda")
    lse_ref = torch.empty(B, S, 64, device="cuda")
    lib.csa_sparse_attn(q, kv, idx_ref, swa, sink, W=W, out=out_ref, lse=lse_ref)
    idx = torch.full_like(idx_ref, -7)
    out = torch.full_like(out_ref, 7.0)
    lse = torch.full_like(lse_ref, 7.0)
    lib.csa_topk_sparse_attn(q, kv, cand, swa, sink, k=k, W=W, out=out, lse=lse, idx=idx)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_ref), f"fused selection on {kind} candidates"
    assert torch.equal(out, out_ref), f"fused attention on {kind} candidates"
    assert torch.equal(lse, lse_ref), f"fused lse on {kind} candidates"


# ---------------------------------------------------------------------------------------
# The indexer keys in 16-entry blocks: the copy against its definition, and the scores and
# segment candidates identical to the row-major path's
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("B,S,Nc,k,t", [
    (3, 1, 32768, 512, 4 * 32768 - 1),     # decode: 8 segments
    (2, 1, 5000, 256, 4 * 5000 + 7),       # ragged last segment, Nc not a multiple of 16
    (2, 2, 9001, 301, 4 * 2500 + 2),       # causal limit inside the row; odd Nc and k
    (1, 1, 150000, 1024, 4 * 100000 + 1),  # 37 segments, empty tail
])
def test_index_segments_b16(lib, B, S, Nc, k, t):
    a = I.indexer_inputs(7100 + B + Nc + k, B, S, Nc)
    pos = dev((t - S + 1 + np.arange(S, dtype=np.int64))[None].repeat(B, 0))
    k8 = dev(a["kI_fp8"])
    blocks = torch.full((lib.index_keys_b16_size(B, Nc),), 0x5A, dtype=torch.uint8, device="cuda")
    lib.csa_index_keys_b16(k8, blocks)
    torch.cuda.synchronize()
    # the blocked copy against its definition (numpy re-ordering of the same codes)
    nblk = -(-Nc // 16)
    rows = np.zeros((B, nblk * 16, 128), np.uint8)
    rows[:, :Nc] = a["kI_fp8"].reshape(B, Nc, 128)
    want = rows.reshape(B, nblk, 16, 4, 32).transpose(0, 1, 3, 2, 4).reshape(-1)
    assert np.array_equal(blocks.cpu().numpy(), want), "csa_index_keys_b16 layout"
    args = (dev(a["qI_fp8"]), dev(a["qI_scale"]), dev(a["w"]))
    n = lib.index_segments_size(B, S, Nc, k)
    cand = torch.zeros(n, dtype=torch.uint8, device="cuda")
    cand16 = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    sc = torch.empty(B, S, Nc, device="cuda")
    sc16 = torch.full_like(sc, 7.0)
    lib.csa_index_score_segments(*args, k8, dev(a["kI_scale"]), pos, m=4, k=k, cand=cand, scores=sc)
    lib.csa_index_score_segments_b16(*args, blocks, dev(a["kI_scale"]), pos, m=4, k=k, cand=cand16, scores=sc16)
    torch.cuda.synchronize()
    G = -(-Nc // 4096)
    seg = B * S * G * k * 8                 # the segment pairs (the rest of each share is merge space)
    per_row = n // (B * S)
    c0 = cand.view(B * S, per_row)[:, :G * k * 8]
    c1 = cand16.view(B * S, per_row)[:, :G * k * 8]
    assert seg == c0.numel()
    assert torch.equal(c0, c1), "blocked keys: segment candidates differ"
    assert torch.equal(sc, sc16), "blocked keys: scores differ"


def test_topk_long_rows_unaligned_base(lib):
    """Scores whose base is 4- but not 16-byte aligned take the one-workgroup-per-row kernel
    (the persistent long-row kernel streams 16-byte pieces): the same selection as from an
    aligned copy, and the oracle's on sampled rows."""
    rows, Nc, k = 300, 20000, 256
    rng = np.random.default_rng(77)
    s = I.score_rows(rows + Nc + k, rows, Nc, "ties", rng.integers(Nc // 2, Nc + 1, rows))
    flat = torch.empty(rows * Nc + 4, device="cuda")
    flat[1:1 + rows * Nc] = torch.from_numpy(s.reshape(-1)).cuda()
    view = flat[1:1 + rows * Nc].view(1, rows, Nc)
    assert view.data_ptr() % 16 == 4
    idx_u = torch.empty(1, rows, k, dtype=torch.int32, device="cuda")
    idx_a = torch.empty(1, rows, k, dtype=torch.int32, device="cuda")
    lib.csa_topk(view, k, idx_u, algo=1)
    lib.csa_topk(dev(s[None]), k, idx_a, algo=1)
    torch.cuda.synchronize()
    assert torch.equal(idx_u, idx_a), "unaligned scores select differently"
    sample = [0, 1, 150, rows - 1]
    ref = O.topk_indices(s[sample], k)
    assert_topk_equal(idx_u[0, sample].cpu().numpy(), ref, s[sample], k, "top-k, unaligned base", exact=True)
