"""Pins of the CPU oracle to facts other than itself (CPU only).

Each test states what fixes the expected value: a hand-computed case, a closed
form, an invariant of the method, a library routine, or brute force.  They are
chosen so that a plausible slip in the oracle (a dropped term, a wrong sign, a
shifted block, a transposed operand, a swapped stream) fails at least one.
"""

import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def test_e4m3_decode_matches_library_dtype_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.e4m3fn_to_f64(codes)
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], ours[ok])


def test_e4m3_decode_hand_values():
    # OCP 8-bit float spec, E4M3 row: bias 7, max normal 448, min subnormal 2^-9, NaN = S.1111.111
    table = {0x38: 1.0, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6, 0xB8: -1.0, 0x00: 0.0}
    for code, val in table.items():
        assert O.e4m3fn_to_f64(np.array([code]))[0] == val
    assert np.isnan(O.e4m3fn_to_f64(np.array([0x7F, 0xFF]))).all()


def test_e4m3_encode_round_to_nearest_even():
    assert O.f64_to_e4m3fn(np.array([1.0625]))[0] == 0x38      # midpoint 1 | 1.125 -> even (1.0)
    assert O.f64_to_e4m3fn(np.array([1.1875]))[0] == 0x3A      # midpoint 1.125 | 1.25 -> even (1.25)
    assert O.f64_to_e4m3fn(np.array([-448.0]))[0] == 0xFE
    assert O.f64_to_e4m3fn(np.array([1000.0]))[0] == 0x7E      # saturates
    assert O.f64_to_e4m3fn(np.array([np.nan]))[0] == 0x7F


def test_e4m3_encode_matches_library_cast():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.normal(0, 60, 20000), rng.normal(0, 0.01, 5000),
                        rng.uniform(-448, 448, 5000)])
    # every midpoint between neighbouring codes, where the tie rule decides
    vals = O.e4m3fn_to_f64(np.arange(0x7F))
    mids = (vals[1:] + vals[:-1]) / 2
    x = np.concatenate([x, mids, -mids]).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = O.f64_to_e4m3fn(x.astype(np.float64))
    assert np.array_equal(lib, ours)


def test_bf16_decode_matches_library():
    rng = np.random.default_rng(1)
    x = torch.from_numpy(rng.normal(0, 3, 4096).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits_to_f64(bits), x.to(torch.float64).numpy())


def test_row_quantisation_bounds():
    rng = np.random.default_rng(2)
    x = rng.normal(0, 1, (64, 128))
    codes, scale = O.quantize_rows_e4m3(x)
    # the row's largest magnitude lands exactly on the largest code
    amax_pos = np.argmax(np.abs(x), axis=1)
    assert np.all(codes[np.arange(64), amax_pos] & 0x7F == 0x7E)
    deq = O.dequant_rows(codes, scale)
    # |error| <= half a code spacing; spacing <= 2^-3 relative (3 mantissa bits), 2^-9 absolute below 2^-6
    err = np.abs(deq - x) / scale[:, None]
    v = np.abs(x) / scale[:, None]
    bound = np.maximum(v * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
    zc, zs = O.quantize_rows_e4m3(np.zeros((2, 8)))
    assert np.all(zc == 0) and np.all(zs == 0)


# ---------------------------------------------------------------------------
# RMSNorm, RoPE
# ---------------------------------------------------------------------------

def test_rms_norm_unit_mean_square():
    rng = np.random.default_rng(3)
    u = rng.normal(0, 5, (10, 64))
    n = O.rms_norm(u, 0.0)
    assert np.allclose(np.mean(n * n, axis=-1), 1.0, atol=1e-14)
    assert np.allclose(n * np.sqrt(np.mean(u * u, axis=-1, keepdims=True)), u)


def test_rope_hand_case_and_frequency():
    # pair (1, 0) at pos 1, p = 0: rotated to (cos 1, sin 1)
    x = np.array([1.0, 0.0])
    assert np.allclose(O.rope(x, 1, 2, 1e4), [math.cos(1), math.sin(1)], atol=1e-15)
    # p = 1 of a 4-wide rope with theta = 100: angle = pos * 100^(-2/4) = pos / 10
    x = np.array([0.0, 0.0, 1.0, 0.0])
    assert np.allclose(O.rope(x, 5, 4, 100.0), [0, 0, math.cos(0.5), math.sin(0.5)], atol=1e-15)


def test_rope_interleaved_pairs_and_untouched_prefix():
    # only the last d_rope channels rotate, and channel 2p+1 is the partner of 2p
    x = np.zeros(8); x[5] = 1.0                   # channel 5 = odd member of the pair (4, 5)
    y = O.rope(x, 3, 4, 1e4)                      # rope channels 4..7; pair (4,5) is p = 0
    assert np.allclose(y[:4], 0)
    assert np.allclose(y[4:6], [-math.sin(3), math.cos(3)], atol=1e-15)
    assert np.allclose(y[6:], 0)


def test_rope_relative_position_property():
    # <R_a x, R_b y> depends only on b - a: the defining property of rotary embeddings
    rng = np.random.default_rng(4)
    x, y = rng.normal(size=16), rng.normal(size=16)
    d1 = O.rope(x, 7, 16, 1e4) @ O.rope(y, 19, 16, 1e4)
    d2 = O.rope(x, 100, 16, 1e4) @ O.rope(y, 112, 16, 1e4)
    assert abs(d1 - d2) < 1e-12
    assert np.allclose(O.rope(O.rope(x, 37, 16, 1e4), -37, 16, 1e4), x)
    assert np.allclose(np.linalg.norm(O.rope(x, 37, 16, 1e4)), np.linalg.norm(x))


# ---------------------------------------------------------------------------
# Compressor
# ---------------------------------------------------------------------------

def _h1_streams():
    # m = 2, c = 2; tokens 0..3 (blocks 0 and 1)
    Ca = np.array([[4, 2], [8, -2], [1, 1], [3, 1]], float)
    Za = np.array([[0, 0], [math.log(3), 0], [0, 0], [0, 0]], float)
    Cb = np.array([[0, 1], [4, 1], [0, 0], [0, 0]], float)
    Zb = np.zeros((4, 2))
    return Ca, Za, Cb, Zb


def test_compressor_hand_case_h1():
    Ca, Za, Cb, Zb = _h1_streams()
    zero = np.zeros((2, 2))
    u = O.compressor_entries(Ca, Za, zero, 2, Cb, Zb, zero)
    # entry 0: b-slots padded (-inf, 0) -> softmax over (0, ln3) per channel 0: 1/4, 3/4
    assert np.allclose(u[0], [7.0, 0.0])
    # entry 1: all logits 0 -> mean of Ca[2:4] and Cb[0:2] = ((1+3+0+4)/4, (1+1+1+1)/4)
    assert np.allclose(u[1], [2.0, 1.0])
    z = O.rms_norm(u, 0.0)
    assert np.allclose(z[0], [math.sqrt(2), 0.0])
    assert np.allclose(z[1], [1.264911064, 0.632455532])
    # with B^b = -inf the b-stream vanishes (HCA collapse): mean of Ca[2:4] = (2, 1)
    ninf = np.full((2, 2), -np.inf)
    u2 = O.compressor_entries(Ca, Za, zero, 2, Cb, Zb, ninf)
    assert np.allclose(u2[1], [2.0, 1.0])


def test_compressor_hca_is_csa_collapsed():
    # HCA is CSA with the streams collapsed and block -1 removed: B^b = -inf gives the single stream
    rng = np.random.default_rng(5)
    T, c, m = 24, 6, 4
    Ca, Za, Cb, Zb = (rng.normal(size=(T, c)) for _ in range(4))
    Ba = rng.normal(size=(m, c))
    single = O.compressor_entries(Ca, Za, Ba, m)
    collapsed = O.compressor_entries(Ca, Za, Ba, m, Cb, Zb, np.full((m, c), -np.inf))
    assert np.allclose(single, collapsed, atol=1e-14)


def test_compressor_first_entry_padding():
    # i = 0 has no previous block: Z^b = -inf, C^b = 0, so entry 0 is the a-stream pool alone
    rng = np.random.default_rng(6)
    T, c, m = 8, 5, 4
    Ca, Za, Cb, Zb = (rng.normal(size=(T, c)) for _ in range(4))
    Ba, Bb = rng.normal(size=(m, c)), rng.normal(size=(m, c))
    csa = O.compressor_entries(Ca, Za, Ba, m, Cb, Zb, Bb)
    single = O.compressor_entries(Ca[:m], Za[:m], Ba, m)
    assert np.allclose(csa[0], single[0], atol=1e-14)
    # and entry 1 does see block 0's b-stream
    assert not np.allclose(csa[1], O.compressor_entries(Ca[m:], Za[m:], Ba, m)[0])


def test_compressor_ratio_one_is_plain_norm():
    # a single slot has softmax weight 1, so m = 1 without overlap is RoPE(RMSNorm(C))
    rng = np.random.default_rng(7)
    d, c, T = 12, 8, 5
    hidden = rng.normal(size=(1, T, d))
    W = rng.normal(size=(d, 2 * c))
    out = O.csa_compress(hidden, W, np.zeros((1, 1, c)), overlap=False, m=1, c=c, d_rope=4,
                         rope_theta=1e4, rms_eps=1e-6, p0=3)
    C = hidden[0] @ W[:, :c]
    for i in range(T):
        n = C[i] / math.sqrt(np.mean(C[i] ** 2) + 1e-6)
        assert np.allclose(out[0, i], O.rope(n, 3 + i, 4, 1e4), atol=1e-13)


def test_compressor_uniform_gate_is_mean_pool():
    rng = np.random.default_rng(8)
    T, c, m = 12, 4, 4
    Ca, Cb = rng.normal(size=(T, c)), rng.normal(size=(T, c))
    Z = np.zeros((T, c)); B0 = np.zeros((m, c))
    u = O.compressor_entries(Ca, Z, B0, m, Cb, Z, B0)
    for i in range(1, T // m):
        mean = (Ca[m * i:m * i + m].sum(0) + Cb[m * (i - 1):m * i].sum(0)) / (2 * m)
        assert np.allclose(u[i], mean, atol=1e-14)


def test_compressor_one_hot_gate_selects_slot():
    # a +1e4 bias on b-slot r of every channel selects token m*(i-1)+r of the b-stream exactly
    rng = np.random.default_rng(9)
    T, c, m, r = 16, 3, 4, 2
    Ca, Za, Cb, Zb = (rng.normal(size=(T, c)) for _ in range(4))
    Ba = np.zeros((m, c)); Bb = np.zeros((m, c)); Bb[r] = 1e4
    u = O.compressor_entries(Ca, Za, Ba, m, Cb, Zb, Bb)
    for i in range(1, T // m):
        assert np.allclose(u[i], Cb[m * (i - 1) + r], atol=1e-12)


def test_compressor_projection_column_order():
    # W = (C^a | Z^a | C^b | Z^b): give token 5's Z^a a huge logit and every Z^b a hugely
    # negative one; entry 1 (tokens 4..7) must then be RoPE(Norm(C^a of token 5)).
    rng = np.random.default_rng(10)
    m, c, T = 4, 6, 8
    d = T
    hidden = np.eye(T)[None]                                  # token t projects to row t of W
    W = rng.normal(size=(d, 4 * c))
    W[:, c:2 * c] = 0.0; W[5, c:2 * c] = 1e4                  # Z^a
    W[:, 3 * c:4 * c] = -1e4                                  # Z^b
    out = O.csa_compress(hidden, W, np.zeros((2, m, c)), overlap=True, m=m, c=c, d_rope=2,
                         rope_theta=1e4, rms_eps=0.0, p0=0)
    expect = O.rope(O.rms_norm(W[5, :c], 0.0), 4, 2, 1e4)
    assert np.allclose(out[0, 1], expect, atol=1e-10)


def test_compressor_chunking_with_previous_block():
    # compressing tokens m..3m-1 with the m tokens before them as hidden_prev reproduces
    # entries 1 and 2 of compressing all 3m tokens from position 0 (offsets and RoPE positions)
    rng = np.random.default_rng(11)
    m, c, d = 4, 8, 10
    hidden = rng.normal(size=(2, 3 * m, d))
    W = rng.normal(size=(d, 4 * c)) * 0.5
    bias = rng.normal(size=(2, m, c))
    kw = dict(overlap=True, m=m, c=c, d_rope=4, rope_theta=1e4, rms_eps=1e-6)
    full = O.csa_compress(hidden, W, bias, p0=0, **kw)
    part = O.csa_compress(hidden[:, m:], W, bias, p0=m, hidden_prev=hidden[:, :m], **kw)
    assert np.allclose(full[:, 1:], part, atol=1e-12)


# ---------------------------------------------------------------------------
# Visibility
# ---------------------------------------------------------------------------

def test_visibility_examples_from_pages():
    rows = [list(map(int, ln.split())) for ln in open(os.path.join(GOLDEN, "visibility_examples.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for m, t, j, vis in rows:
        assert int(j < O.visible_entries(t, m, 10 ** 9)) == vis, (m, t, j)
    assert O.visible_entries(1023, 4, 256) == 256           # tiny config: the last history token
    assert O.visible_entries(131071, 4, 32768) == 32768     # 128K context, m = 4
    assert O.visible_entries(1048575, 128, 8192) == 8192    # 1M context, m = 128


# ---------------------------------------------------------------------------
# Index scores
# ---------------------------------------------------------------------------

def test_index_score_hand_case_h2():
    q = np.array([[[[1.0, 2.0], [-1.0, 1.0]]]])             # [B=1, S=1, H=2, d=2]
    w = np.array([[[0.5, 2.0]]])
    K = np.array([[[3.0, -1.0], [1.0, 1.0]]])                # two entries
    I = O.index_scores(q, w, K, np.array([[7]]), 4)        # t = 7: both entries visible
    assert np.allclose(I[0, 0], [0.5, 1.5])
    # t = 6: only entry 0 is visible (entry 1 ends at token 7)
    I = O.index_scores(q, w, K, np.array([[6]]), 4)
    assert I[0, 0, 0] == 0.5 and I[0, 0, 1] == -np.inf


def test_index_score_properties():
    rng = np.random.default_rng(12)
    q = rng.normal(size=(2, 3, 4, 8)); w = rng.normal(size=(2, 3, 4))
    K = rng.normal(size=(2, 20, 8)); pos = np.array([[70, 71, 79], [3, 40, 100]])
    I = O.index_scores(q, w, K, pos, 4)
    # positive homogeneity in q (ReLU commutes with positive scaling)
    assert np.allclose(O.index_scores(2.5 * q, w, K, pos, 4), np.where(np.isinf(I), I, 2.5 * I))
    # additivity over heads
    parts = sum(np.where(np.isinf(I), 0, O.index_scores(q[:, :, h:h + 1], w[:, :, h:h + 1], K, pos, 4))
                for h in range(4))
    assert np.allclose(np.where(np.isinf(I), 0, I), parts)
    # heads whose dot products are all negative contribute nothing
    assert np.all(O.index_scores(np.abs(q), w, -np.abs(K), pos, 4)[np.isfinite(I)] == 0.0)
    # visibility mask
    for b in range(2):
        for s in range(3):
            nv = min(20, (pos[b, s] + 1) // 4)
            assert np.all(np.isfinite(I[b, s, :nv])) and np.all(I[b, s, nv:] == -np.inf)


# ---------------------------------------------------------------------------
# Top-k
# ---------------------------------------------------------------------------

def test_topk_hand_case_h3():
    s = np.array([0.5, 1.5, 1.5, 0.2]); s[3] = -np.inf      # n_vis = 3
    assert list(O.topk_indices(s, 4)) == [0, 1, 2, -1]
    assert list(O.topk_indices(np.array([2.0, 1.0, 2.0]), 1)) == [0]


def _brute_topk(row, k):
    """Exhaustive search: the unique subset of size min(k, n) in which no unselected
    candidate is better (higher score, or equal score and lower index) than a selected one."""
    cand = [j for j in range(len(row)) if row[j] > -np.inf]
    kk = min(k, len(cand))
    better = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)
    found = [set(sub) for sub in itertools.combinations(cand, kk)
             if not any(better(u, s) for u in cand if u not in sub for s in sub)]
    assert len(found) == 1
    return sorted(found[0]) + [-1] * (k - kk)


def test_topk_exhaustive_small_rows_with_ties():
    rng = np.random.default_rng(13)
    for _ in range(300):
        n = int(rng.integers(1, 9))
        row = rng.integers(0, 4, n).astype(float)           # many ties
        row[rng.random(n) < 0.2] = -np.inf
        k = int(rng.integers(1, 10))
        assert list(O.topk_indices(row, k)) == _brute_topk(row, k)


def test_topk_rank_property_random_rows():
    # every selected entry has fewer than k strictly better candidates; every unselected
    # candidate has at least k of them
    rng = np.random.default_rng(14)
    for _ in range(40):
        n = int(rng.integers(1, 300)); k = int(rng.integers(1, 64))
        row = np.round(rng.normal(size=n), 2)
        row[rng.random(n) < 0.1] = -np.inf
        sel = O.topk_indices(row, k)
        chosen = set(int(j) for j in sel if j >= 0)
        cand = [j for j in range(n) if row[j] > -np.inf]
        assert len(chosen) == min(k, len(cand))
        assert list(sel[:len(chosen)]) == sorted(chosen) and all(sel[len(chosen):] == -1)
        for j in cand:
            nb = sum(1 for u in cand if row[u] > row[j] or (row[u] == row[j] and u < j))
            assert (nb < k) == (j in chosen)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def test_attention_hand_case_h4():
    q = np.array([[math.sqrt(2), 0.0]])                      # H = 1, c = 2, scale = 1/sqrt(2)
    rows = np.array([[0.0, 2.0], [math.log(3), 0.0]])
    o, lse = O._joint_softmax(q, rows, np.array([0.0]), 1 / math.sqrt(2))
    # logits (0, ln 3), sink 0 -> weights (1, 3) / 5
    assert np.allclose(o[0], [3 * math.log(3) / 5, 2 / 5]) and abs(lse[0] - math.log(5)) < 1e-14
    o, _ = O._joint_softmax(q, rows, np.array([-np.inf]), 1 / math.sqrt(2))
    assert np.allclose(o[0], [3 * math.log(3) / 4, 2 / 4])
    o, _ = O._joint_softmax(q, rows, np.array([1e4]), 1 / math.sqrt(2))
    assert np.allclose(o[0], [0.0, 0.0], atol=1e-300)       # sink-only limit: output -> 0


def _rand_layer(rng, B=2, S=3, H=4, c=16, n_c=40, Ls=20, t0=150):
    q = rng.normal(size=(B, S, H, c)); kv = rng.normal(size=(B, n_c, c))
    swa = rng.normal(size=(B, Ls, c)); sink = rng.normal(size=H)
    pos = np.tile(np.arange(t0 - S + 1, t0 + 1), (B, 1))
    return q, kv, swa, sink, pos


def test_attention_without_sink_is_textbook_softmax_attention():
    # sink = -inf reduces to softmax(q K^T * scale) V with K = V: check against the library
    rng = np.random.default_rng(15)
    q, kv, swa, sink, pos = _rand_layer(rng)
    idx = np.stack([np.stack([rng.permutation(40)[:9] for _ in range(3)]) for _ in range(2)])
    scale = 0.3
    o, lse = O.sparse_attention(q, kv, idx, swa, np.full(4, -np.inf), scale, pos, W=8)
    for b in range(2):
        for s in range(3):
            t = pos[b, s]
            win = [r for r in range(20) if t - 7 <= pos[b, -1] - 19 + r <= t]
            rows = torch.from_numpy(np.concatenate([swa[b, win], kv[b, idx[b, s]]]))
            qq = torch.from_numpy(q[b, s])[:, None, :]                       # [H, 1, c]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qq, rows[None].expand(4, -1, -1), rows[None].expand(4, -1, -1), scale=scale)
            assert np.allclose(o[b, s], ref[:, 0].numpy(), atol=1e-12)
            lref = torch.logsumexp(scale * (torch.from_numpy(q[b, s]) @ rows.T), dim=1)
            assert np.allclose(lse[b, s], lref.numpy(), atol=1e-12)


def test_sparse_with_all_visible_selected_equals_dense():
    # top-k >= visible entries: CSA attention over the selection equals dense (HCA) attention
    rng = np.random.default_rng(16)
    q, kv, swa, sink, pos = _rand_layer(rng, t0=100)
    m = 4
    nv = O.visible_entries(pos, m, 40)
    I = rng.normal(size=(2, 3, 40))
    I[np.arange(40)[None, None, :] >= nv[..., None]] = -np.inf
    idx = O.topk_indices(I, 64)                                 # k exceeds every n_vis
    o1, l1 = O.sparse_attention(q, kv, idx, swa, sink, 0.25, pos, W=8)
    o2, l2 = O.dense_attention(q, kv, pos, m, swa, sink, 0.25, W=8)
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


def test_attention_permutation_invariant_in_indices():
    rng = np.random.default_rng(17)
    q, kv, swa, sink, pos = _rand_layer(rng)
    idx = np.array([rng.permutation(40)[:12] for _ in range(6)]).reshape(2, 3, 12)
    idx[0, 1, 5] = -1
    o1, _ = O.sparse_attention(q, kv, idx, swa, sink, 0.2, pos, W=16)
    o2, _ = O.sparse_attention(q, kv, idx[..., ::-1], swa, sink, 0.2, pos, W=16)
    assert np.allclose(o1, o2, atol=1e-14)


def test_attention_lse_merge_identity():
    # attention over A ∪ B = LSE-weighted merge of the parts (the o = (1-R) o_S + R o_notS split)
    rng = np.random.default_rng(18)
    H, c = 4, 16
    q = rng.normal(size=(H, c)); rows = rng.normal(size=(30, c)); sink = rng.normal(size=H)
    o, lse = O._joint_softmax(q, rows, sink, 0.25)
    oa, la = O._joint_softmax(q, rows[:11], sink, 0.25)            # part A carries the sink
    ob, lb = O._joint_softmax(q, rows[11:], np.full(H, -np.inf), 0.25)
    lm = np.logaddexp(la, lb)
    om = (np.exp(la - lm)[:, None] * oa + np.exp(lb - lm)[:, None] * ob)
    assert np.allclose(o, om, atol=1e-14) and np.allclose(lse, lm, atol=1e-14)


def test_attention_selection_error_bound():
    # ||o - o_S|| <= 2 V R(S), V = max row norm, R(S) = softmax mass outside S (sink = -inf)
    rng = np.random.default_rng(19)
    H, c = 3, 8
    q = rng.normal(size=(H, c)) * 2; rows = rng.normal(size=(50, c))
    ninf = np.full(H, -np.inf)
    o, _ = O._joint_softmax(q, rows, ninf, 1.0)
    V = np.linalg.norm(rows, axis=1).max()
    for keep in (5, 20, 45):
        sel = rng.permutation(50)[:keep]
        oS, _ = O._joint_softmax(q, rows[sel], ninf, 1.0)
        p = np.exp(q @ rows.T - (q @ rows.T).max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
        R = 1 - p[:, sel].sum(1)
        assert np.all(np.linalg.norm(o - oS, axis=1) <= 2 * V * R + 1e-12)


def test_sliding_window_boundaries():
    # a row one position older than the window must not count; the oldest row inside must
    rng = np.random.default_rng(20)
    H, c, W, Ls = 2, 8, 16, 40
    q = rng.normal(size=(1, 1, H, c)) * 0.01
    swa = rng.normal(size=(1, Ls, c)) * 0.01
    t = 500
    pos = np.array([[t]])                   # the last swa row holds position t
    outside = Ls - 1 - W                    # position t - W
    inside = Ls - W                         # position t - W + 1
    big = np.zeros(c); big[0] = 1.0
    q[..., 0] = 1e3
    s1 = swa.copy(); s1[0, outside] = big
    o1, _ = O.sparse_attention(q, np.zeros((1, 1, c)), np.full((1, 1, 1), -1), s1,
                               np.full(H, -np.inf), 1.0, pos, W)
    assert np.all(o1[0, 0, :, 0] < 0.1)
    s2 = swa.copy(); s2[0, inside] = big
    o2, _ = O.sparse_attention(q, np.zeros((1, 1, c)), np.full((1, 1, 1), -1), s2,
                               np.full(H, -np.inf), 1.0, pos, W)
    assert np.allclose(o2[0, 0, :, 0], 1.0, atol=1e-6)


def test_attention_empty_row_set_is_zero():
    o, lse = O._joint_softmax(np.ones((2, 4)), np.zeros((0, 4)), np.array([0.3, -np.inf]), 1.0)
    assert np.all(o == 0) and lse[0] == 0.3 and lse[1] == -np.inf
