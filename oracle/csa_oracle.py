"""Plain, slow CPU oracle of the CSA / HCA attention layer (DeepSeek-V4).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
directory.  The product path (the ``compressed_sparse_kv_amd`` package and its
HIP library) never does, and this module imports nothing from it.

Every quantity is computed in float64 from exactly decoded inputs (bfloat16 and
OCP e4m3fn codes decode bit-exactly).  Library primitives used as single steps:
``numpy.matmul`` (a dot product / matrix product), ``numpy.exp``, ``numpy.lexsort``.
Nothing is blocked, fused or reordered beyond what the formulas state.

Sources (web pages; cited by title and section, never by line):
  [HCA-CSA]  zdszero.github.io, "hca_csa"
  [KV-COMP]  jerry609.github.io, "DeepSeek-V4 的 KV 压缩：从删 token 误解到预算检索"
  [V4-CSA2]  yuyanqi.com, "DeepSeek-V4 CSA/HCA 与 DeepSeek-V4.1 CSA2：从模型原理到推理基础设施"
  [ATTN-CMP] blog.javazero.top, "DeepSeek 注意力结构对比：MHA、GQA、MLA、DSA、CSA、HCA、CSA2"

Readings taken where the pages are silent or ambiguous (each is restated in the
design notes of the repository):
  * the attention sink enters the softmax denominator unscaled, as exp(s_h);
  * the softmax scale is 1/sqrt(c) with no YaRN factor;
  * the sliding window holds positions t-W+1 .. t (the current token included);
  * RoPE rotates interleaved pairs (2p, 2p+1) of the last d_rope channels by
    pos * theta**(-2p/d_rope); a compressed entry i takes position m*i (its own
    block's first token);
  * the compressor's RMSNorm has unit gain and eps = 1e-6 unless given;
  * top-k ties go to the lower entry index; the selection is returned in
    ascending index order and padded with -1;
  * FP8 is OCP e4m3fn; per-row scale = amax/448; round-to-nearest-even.

Parity status: every function below is pinned by tests in ``tests/test_oracle_*``
(hand-computed cases, closed forms, invariants, brute force, library routines).
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exact: bf16 is the top half of an fp32."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn code bytes -> float64, exact.

    Layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
    field 0 encodes subnormals m/8 * 2**-6; S.1111.111 is NaN; there is no
    infinity, so the largest finite magnitude is 1.110b * 2**8 = 448.
    """
    c = codes.astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    mag = np.where(exp == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * np.exp2(exp - 7.0))
    out = sign * mag
    return np.where((exp == 15) & (c & 0x7 == 7), np.nan, out)


def _e4m3_finite_table() -> tuple[np.ndarray, np.ndarray]:
    codes = np.arange(0x7F, dtype=np.int64)          # 0x00 .. 0x7E: all finite non-negative codes
    return codes, e4m3fn_to_f64(codes)


def f64_to_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Round real values to the nearest e4m3fn code, ties to the even code.

    Done by brute force over the 127 finite non-negative codes (no bit tricks),
    then the sign is attached.  Magnitudes beyond the largest finite value
    saturate to 448; NaN maps to 0x7F.  Zero keeps its sign bit.
    """
    x = np.asarray(x, dtype=np.float64)
    codes, vals = _e4m3_finite_table()
    mag = np.minimum(np.abs(x), E4M3_MAX)
    d = np.abs(mag[..., None] - vals)                    # distance to every code value
    best = d.min(axis=-1, keepdims=True)
    tied = d == best
    # among the (at most two) nearest codes prefer the one whose mantissa LSB is 0
    even = tied & (codes % 2 == 0)
    pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(tied, axis=-1))
    out = codes[pick]
    out = np.where(np.signbit(x), out | 0x80, out)
    out = np.where(np.isnan(x), 0x7F, out)
    return out.astype(np.uint8)


def quantize_rows_e4m3(x: np.ndarray, precision=np.float32) -> tuple[np.ndarray, np.ndarray]:
    """Per-row FP8 quantisation: scale = amax/448, code = RNE(x / scale).

    ``precision`` is the floating type in which amax, the scale and x/scale are
    formed before rounding to a code (the rounding decision is taken in the
    same precision as the kernel's, fp32).  A row that is all zero gets scale 0
    and all-zero codes.
    """
    xp = np.asarray(x).astype(precision)
    amax = np.max(np.abs(xp), axis=-1)
    scale = (amax / precision(E4M3_MAX)).astype(precision)
    safe = np.where(scale > 0, scale, precision(1))
    v = (xp / safe[..., None]).astype(precision)
    codes = f64_to_e4m3fn(v.astype(np.float64))
    codes = np.where(scale[..., None] > 0, codes, np.uint8(0)).astype(np.uint8)
    return codes, scale.astype(np.float32)


def dequant_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """FP8 codes with a per-row scale -> float64 values (decode, then multiply)."""
    return e4m3fn_to_f64(codes) * np.asarray(scale, dtype=np.float64)[..., None]


# ---------------------------------------------------------------------------
# Shared elementwise pieces: RMSNorm and RoPE
# ---------------------------------------------------------------------------

def rms_norm(u: np.ndarray, eps: float) -> np.ndarray:
    """Norm(u) = u / sqrt(mean(u^2) + eps) over the channel axis, unit gain."""
    u = np.asarray(u, dtype=np.float64)
    return u / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)


def rope(x: np.ndarray, pos, d_rope: int, theta: float) -> np.ndarray:
    """Rotary embedding on the last ``d_rope`` channels of x at position(s) ``pos``.

    Pair p = (x[c-d_rope+2p], x[c-d_rope+2p+1]) is rotated by the angle
    pos * theta**(-2p/d_rope).  ``pos`` broadcasts against x's leading axes.
    The compressed entry's position is its block's first token
    ([ATTN-CMP] section "CSA（DeepSeek-V4）": RMSNorm + RoPE at the block-first
    position).
    """
    x = np.array(x, dtype=np.float64, copy=True)
    if d_rope == 0:
        return x
    c = x.shape[-1]
    pos = np.asarray(pos, dtype=np.float64)[..., None]              # [..., 1]
    p = np.arange(d_rope // 2, dtype=np.float64)
    ang = pos * theta ** (-2.0 * p / d_rope)                        # [..., d_rope/2]
    cs, sn = np.cos(ang), np.sin(ang)
    x0 = x[..., c - d_rope + 0::2].copy()
    x1 = x[..., c - d_rope + 1::2].copy()
    x[..., c - d_rope + 0::2] = x0 * cs - x1 * sn
    x[..., c - d_rope + 1::2] = x0 * sn + x1 * cs
    return x


# ---------------------------------------------------------------------------
# Stage 1: the block compressor
# ---------------------------------------------------------------------------

def compressor_entries(Ca, Za, Ba, m: int, Cb=None, Zb=None, Bb=None,
                       Cb_prev=None, Zb_prev=None):
    """Pooled, un-normalised entries u_i (before Norm and RoPE) of one sequence.

    [HCA-CSA] sections "CSA 的重叠窗口" (overlapping window) and
    "HCA：同一个算子，关掉重叠" (single stream); [KV-COMP] section 9.2 (learned
    gated pooling: per-channel softmax over the block of W_gate h + ape).

    Ca, Za: [T, c] a-stream contents and gate logits of the T tokens (T % m == 0).
    Ba:     [m, c] position bias of the a-slots.
    Single stream (HCA) when Cb is None: entry i pools rows m*i .. m*i+m-1 with
    logits Za + Ba.  With overlap (CSA), entry i additionally pools the b-stream of
    block i-1 (rows m*(i-1) .. m*i-1, logits Zb + Bb); for i == 0 that block is
    Cb_prev/Zb_prev (the m tokens before the chunk) or, when those are None,
    padding with logit -inf and content 0.
    The softmax runs, independently for every channel, over all 2m (or m) slots.
    """
    Ca = np.asarray(Ca, np.float64); Za = np.asarray(Za, np.float64)
    T, c = Ca.shape
    assert T % m == 0
    n = T // m
    out = np.zeros((n, c), dtype=np.float64)
    for i in range(n):
        logits = [Za[m * i:m * i + m] + Ba]          # a-slots of block i
        values = [Ca[m * i:m * i + m]]
        if Cb is not None:                           # b-slots of block i-1
            if i > 0:
                zb = Zb[m * (i - 1):m * i]
                cb = Cb[m * (i - 1):m * i]
            elif Cb_prev is not None:
                zb, cb = Zb_prev, Cb_prev
            else:
                zb = np.full((m, c), -np.inf)
                cb = np.zeros((m, c))
            logits.append(np.asarray(zb, np.float64) + Bb)
            values.append(np.asarray(cb, np.float64))
        L = np.concatenate(logits, axis=0)           # [2m or m, c]
        V = np.concatenate(values, axis=0)
        Lmax = L.max(axis=0, keepdims=True)
        E = np.exp(L - Lmax)
        S = E / E.sum(axis=0, keepdims=True)         # per-channel softmax over slots
        out[i] = (S * V).sum(axis=0)                 # sum of S ⊙ C
    return out


def csa_compress(hidden, W, bias, *, overlap: bool, m: int, c: int, d_rope: int,
                 rope_theta: float, rms_eps: float, p0: int, hidden_prev=None):
    """Compressed entries C^Comp for each sequence of a chunk.

    hidden:      [B, T, d] real values of the chunk's tokens, positions p0 .. p0+T-1
    hidden_prev: [B, m, d] the m tokens before p0 (their b-stream feeds entry p0/m), or None
    W:           [d, 4c] = (C^a | Z^a | C^b | Z^b) with overlap, [d, 2c] = (C | Z) without
    bias:        [2, m, c] = (B^a, B^b) with overlap, [1, m, c] without
    Returns [B, T/m, c] float64: RoPE(Norm(u_i)) at position p0 + m*i.
    ([HCA-CSA] "CSA 的重叠窗口": C_i = RoPE(Norm(sum S^a⊙C^a + sum S^b⊙C^b)).)
    """
    hidden = np.asarray(hidden, np.float64)
    W = np.asarray(W, np.float64)
    bias = np.asarray(bias, np.float64)
    B, T, d = hidden.shape
    n = T // m
    out = np.zeros((B, n, c))
    for b in range(B):
        proj = hidden[b] @ W                                   # the projection W h_t
        if overlap:
            Ca, Za, Cb, Zb = (proj[:, k * c:(k + 1) * c] for k in range(4))
            Cb_prev = Zb_prev = None
            if hidden_prev is not None:
                pp = np.asarray(hidden_prev[b], np.float64) @ W
                Cb_prev, Zb_prev = pp[:, 2 * c:3 * c], pp[:, 3 * c:4 * c]
            u = compressor_entries(Ca, Za, bias[0], m, Cb, Zb, bias[1], Cb_prev, Zb_prev)
        else:
            Ca, Za = proj[:, :c], proj[:, c:2 * c]
            u = compressor_entries(Ca, Za, bias[0], m)
        pos = p0 + m * np.arange(n)
        out[b] = rope(rms_norm(u, rms_eps), pos, d_rope, rope_theta)
    return out


# ---------------------------------------------------------------------------
# Causal block visibility
# ---------------------------------------------------------------------------

def visible_entries(t, m: int, n_c: int):
    """Number of compressed entries a query at position t may read.

    [KV-COMP] section 9.8: entry j covers tokens up to e_j = m*j + m - 1 and is
    visible iff t >= e_j, i.e. j < floor((t+1)/m); capped by the entries stored.
    """
    t = np.asarray(t, dtype=np.int64)
    return np.minimum(n_c, (t + 1) // m)


# ---------------------------------------------------------------------------
# Stage 2: lightning-indexer scores
# ---------------------------------------------------------------------------

def index_scores(qI, w, KI, q_pos, m: int):
    """I[b,s,j] = sum_h w[b,s,h] * ReLU(qI[b,s,h] . KI[b,j]) for visible j, else -inf.

    [HCA-CSA] section "CSA：轻压缩 + 稀疏选择" (indexer equations: no softmax, no
    1/sqrt(d) scale); [KV-COMP] section 9.4.
    qI: [B, S, H_I, d_I], w: [B, S, H_I], KI: [B, N_c, d_I] (real values), q_pos: [B, S].
    """
    qI = np.asarray(qI, np.float64); w = np.asarray(w, np.float64)
    KI = np.asarray(KI, np.float64)
    B, S, H, d = qI.shape
    n_c = KI.shape[1]
    out = np.full((B, S, n_c), -np.inf)
    for b in range(B):
        dots = np.matmul(qI[b], KI[b].T)                       # [S, H, N_c]: q . K per head
        val = np.einsum("sh,shj->sj", w[b], np.maximum(dots, 0.0))
        nv = visible_entries(np.asarray(q_pos)[b], m, n_c)
        for s in range(S):
            out[b, s, :nv[s]] = val[s, :nv[s]]
    return out


# ---------------------------------------------------------------------------
# Stage 3: top-k selection
# ---------------------------------------------------------------------------

def topk_indices(scores, k: int) -> np.ndarray:
    """Per row: the min(k, n_cand) largest candidate scores, as ascending indices, -1 padded.

    Candidates are the entries whose score is not -inf (invisible entries carry
    -inf, [KV-COMP] section 9.8); ties go to the lower index.  Implemented as a
    full stable sort by (score descending, index ascending).
    """
    scores = np.asarray(scores)
    lead = scores.shape[:-1]
    n = scores.shape[-1]
    flat = scores.reshape(-1, n)
    out = np.full((flat.shape[0], k), -1, dtype=np.int32)
    j = np.arange(n)
    for r in range(flat.shape[0]):
        row = flat[r].astype(np.float64)
        cand = j[row > -np.inf]
        order = np.lexsort((cand, -row[cand]))                 # primary: score desc; then index asc
        take = np.sort(cand[order[:k]])
        out[r, :take.size] = take
    return out.reshape(*lead, k)


# ---------------------------------------------------------------------------
# Stage 4: joint-softmax attention over [SWA || compressed || sink]
# ---------------------------------------------------------------------------

def _joint_softmax(q, rows, sink, scale):
    """All heads of one query: logits l[h,e] = scale * (q_h . kv_e); softmax over [l_h ; s_h]
    with the sink only in the denominator; output o_h = sum_e p[h,e] kv_e (K = V).
    q: [H, c], rows: [E, c], sink: [H].  Returns (o [H, c], lse [H]).

    [HCA-CSA] section "设计：近处看原文，远处看摘要" (o = softmax([q K^swa || q K^comp || s]) ·
    [V^swa || V^comp || 0]); the sink contributes exp(s) to the denominator only.
    """
    H, c = q.shape
    logits = scale * (q @ rows.T)                                   # [H, E]
    M = np.maximum(sink, logits.max(axis=1) if rows.shape[0] else -np.inf)   # [H]
    o = np.zeros((H, c)); lse = np.full(H, -np.inf)
    live = M > -np.inf                       # a head with no rows and a -inf sink stays 0
    Ml = M[live]
    e = np.exp(logits[live] - Ml[:, None])                          # [h, E]
    den = np.exp(sink[live] - Ml) + e.sum(axis=1)
    o[live] = (e @ rows) / den[:, None]
    lse[live] = Ml + np.log(den)
    return o, lse


def swa_rows_for_query(t: int, t_last: int, Ls: int, W: int) -> np.ndarray:
    """Indices r of the SWA tensor rows a query at position t reads.

    Row r holds position t_last - Ls + 1 + r; the window covers positions
    t-W+1 .. t ([HCA-CSA]: the latest window_size = 128 tokens, raw).
    """
    pos = t_last - Ls + 1 + np.arange(Ls)
    return np.nonzero((pos >= t - W + 1) & (pos <= t) & (pos >= 0))[0]


def sparse_attention(q, kv_comp, idx, swa, sink, scale, q_pos, W: int):
    """CSA core attention.  q: [B,S,H,c]; kv_comp: [B,N_c,c]; idx: [B,S,k] (-1 = none);
    swa: [B,Ls,c] raw KV of positions t_last-Ls+1 .. t_last where t_last = q_pos[b,-1];
    sink: [H].  Remote set = {kv_comp[j] : j in idx, j != -1} ([KV-COMP] sections 9.5-9.6).
    Returns (o [B,S,H,c], lse [B,S,H]).
    """
    q = np.asarray(q, np.float64); kv_comp = np.asarray(kv_comp, np.float64)
    swa = np.asarray(swa, np.float64); sink = np.asarray(sink, np.float64)
    B, S, H, c = q.shape
    Ls = swa.shape[1]
    o = np.zeros((B, S, H, c)); lse = np.zeros((B, S, H))
    for b in range(B):
        t_last = int(q_pos[b][-1])
        for s in range(S):
            t = int(q_pos[b][s])
            sel = [int(j) for j in idx[b, s] if j != -1]
            rows = np.concatenate([swa[b, swa_rows_for_query(t, t_last, Ls, W)],
                                   kv_comp[b, sel]], axis=0)
            o[b, s], lse[b, s] = _joint_softmax(q[b, s], rows, sink, scale)
    return o, lse


def dense_attention(q, kv_comp, q_pos, m: int, swa, sink, scale, W: int):
    """HCA core attention: remote set = every entry visible at t, j < min(N_c, (t+1)/m)
    ([HCA-CSA] section "HCA：重压缩 + 全量"; [KV-COMP] section 9.5, c128a branch)."""
    q = np.asarray(q, np.float64)
    B, S = q.shape[:2]
    n_c = np.asarray(kv_comp).shape[1]
    nv = visible_entries(np.asarray(q_pos), m, n_c)
    kmax = int(np.max(nv)) if nv.size else 0
    idx = np.full((B, S, max(kmax, 1)), -1, dtype=np.int64)
    for b in range(B):
        for s in range(S):
            idx[b, s, :nv[b, s]] = np.arange(nv[b, s])
    return sparse_attention(q, kv_comp, idx, swa, sink, scale, q_pos, W)


# ---------------------------------------------------------------------------
# Decode-time compressor: the (C, Z) ring and the block-boundary emission
# ---------------------------------------------------------------------------

def decode_compress(hidden, W, bias, *, overlap: bool, m: int, c: int, d_rope: int, rope_theta: float,
                    rms_eps: float, p0: int, hidden_prev=None, online: bool = False):
    """Token-by-token compressor of one sequence, as a decode loop runs it.

    [HCA-CSA] section "KV cache：成品与原料" (a ring of FP32 (C, Z) rows of the last 2m
    tokens for CSA, m for HCA; a compressed entry is produced only when a token completes
    its block) and section "在 SGLang 里的落点" (the CSA emission reads 2m ring slots: the
    current block's and the previous block's); [KV-COMP] section 9.3 (state until the
    block boundary, then one pooled entry written to the cache).  The HCA "online"
    variant keeps, per channel, only a running (max, sum, weighted sum) over the block.

    hidden: [T, d] real values of the tokens at positions p0 .. p0+T-1 (p0 % m == 0);
    hidden_prev: [m, d] the m tokens before p0 (with overlap their b-stream feeds the entry
    of block p0/m), or None: no earlier block (entry 0's b-slots are -inf / 0 padding).
    W, bias as csa_compress.  Returns {entry index i: float64 [c]} for every block that a
    token of `hidden` completes, in the order emitted.

    The pooling below is written for the ring (slot = position mod ring size) and for the
    running (max, sum, acc) triple; it shares no step with compressor_entries beyond the
    Norm and RoPE helpers.
    """
    hidden = np.asarray(hidden, np.float64)
    W = np.asarray(W, np.float64)
    bias = np.asarray(bias, np.float64)
    assert p0 % m == 0
    n_slots = 2 * m if overlap else m
    ring = {}                                    # slot -> projection row of the token stored there
    run = None                                   # online HCA: (mx, sm, acc) per channel
    out = {}

    def push(t, h):
        nonlocal run
        proj = h @ W                                            # this token's C and Z streams
        ring[t % n_slots] = (t, proj)
        if online:
            r = t % m
            z = proj[c:2 * c] + bias[0][r]
            if r == 0:                                          # first token of a block
                run = (z.copy(), np.ones(c), proj[:c].copy())
            else:
                mx, sm, acc = run
                mn = np.maximum(mx, z)
                a_old, a_new = np.exp(mx - mn), np.exp(z - mn)
                run = (mn, sm * a_old + a_new, acc * a_old + a_new * proj[:c])

    if hidden_prev is not None:
        for r in range(m):
            push(p0 - m + r, np.asarray(hidden_prev[r], np.float64))
    for s in range(hidden.shape[0]):
        t = p0 + s
        push(t, hidden[s])
        if (t + 1) % m != 0:
            continue
        i = t // m                                              # the block this token completes
        if online:
            mx, sm, acc = run
            u = acc / sm
        else:
            logits, values = [], []
            for r in range(m):                                  # a-slots: block i
                tt, proj = ring[(m * i + r) % n_slots]
                assert tt == m * i + r
                if overlap:
                    logits.append(proj[c:2 * c] + bias[0][r]); values.append(proj[:c])
                else:
                    logits.append(proj[c:2 * c] + bias[0][r]); values.append(proj[:c])
            if overlap:                                         # b-slots: block i-1, if there is one
                for r in range(m):
                    pos_b = m * (i - 1) + r
                    if pos_b < 0:
                        logits.append(np.full(c, -np.inf)); values.append(np.zeros(c))
                        continue
                    tt, proj = ring[pos_b % n_slots]
                    assert tt == pos_b, "the ring lacks the previous block"
                    logits.append(proj[3 * c:4 * c] + bias[1][r]); values.append(proj[2 * c:3 * c])
            L = np.stack(logits); V = np.stack(values)
            e = np.exp(L - L.max(axis=0))
            u = (e * V).sum(axis=0) / e.sum(axis=0)
        out[i] = rope(rms_norm(u[None], rms_eps), m * i, d_rope, rope_theta)[0]
    return out


# ---------------------------------------------------------------------------
# Inverse RoPE on the attention output
# ---------------------------------------------------------------------------

def inverse_rope(o, pos, d_rope: int, theta: float):
    """The attention output rotated back by the query's own position: RoPE at -t on its
    last d_rope channels, so that a row rotated at position p contributes a rotation by
    p - t ([V4-CSA2] section 12.1 "Partial RoPE 与 inverse RoPE"; [ATTN-CMP] section
    "CSA（DeepSeek-V4）": the last 64 output dimensions are rotated back by RoPE(-t))."""
    return rope(o, -np.asarray(pos, dtype=np.float64), d_rope, theta)


# ---------------------------------------------------------------------------
# CSA2 compressor: single stream, no position bias, indexer K projected from the main KV
# ---------------------------------------------------------------------------

def csa2_compress(hidden, W_kv, W_gate, W_k, *, m: int, d_rope: int, theta_kv: float, theta_k: float,
                  rms_eps: float, p0: int):
    """CSA2 main KV entries and indexer keys of each sequence of a chunk.

    [V4-CSA2] sections 6.1 and 7.2 (one KV projection and one gate, each entry pooling only
    its own m-token block, no position bias inside the compressor: per channel, a softmax
    over the block's gate values weights the block's KV values), 7.5 and 15.1 (ratio 1:
    no gate, the entry is the normalised projection), 6.2 (indexer K is a projection of the
    main KV latent, not a second compressor) and 7.4 (the entry's RoPE position is its
    block's first token); [ATTN-CMP] section on CSA2 (the latent before RoPE feeds the
    indexer-K projection wk, then k_norm and RoPE with the indexer's own theta).

    hidden [B, T, d] at positions p0 .. p0+T-1 (T % m == 0, p0 % m == 0); W_kv, W_gate [d, c]
    (W_gate None when m == 1); W_k [c, d_I].  Returns (kv [B, T/m, c], kI [B, T/m, d_I]),
    both float64:
        latent_i = RMSNorm(sum_r softmax_r(Z_r) * C_r)  over the block's tokens r,
        kv_i     = RoPE_{theta_kv}(latent_i, p0 + m*i),
        kI_i     = RoPE_{theta_k}(RMSNorm(latent_i . W_k), p0 + m*i).
    """
    hidden = np.asarray(hidden, np.float64)
    W_kv = np.asarray(W_kv, np.float64)
    W_k = np.asarray(W_k, np.float64)
    B, T, d = hidden.shape
    assert T % m == 0 and p0 % m == 0
    n = T // m
    c = W_kv.shape[1]
    kv = np.zeros((B, n, c))
    kI = np.zeros((B, n, W_k.shape[1]))
    for b in range(B):
        C = hidden[b] @ W_kv
        Z = None if W_gate is None else hidden[b] @ np.asarray(W_gate, np.float64)
        for i in range(n):
            if m == 1 and Z is None:
                pooled = C[i]
            else:
                z = Z[m * i:m * i + m]                               # [m, c]
                e = np.exp(z - z.max(axis=0))
                pooled = (e * C[m * i:m * i + m]).sum(axis=0) / e.sum(axis=0)
            latent = rms_norm(pooled[None], rms_eps)[0]
            pos = p0 + m * i
            kv[b, i] = rope(latent[None], pos, d_rope, theta_kv)[0]
            kI[b, i] = rope(rms_norm((latent @ W_k)[None], rms_eps), pos, d_rope, theta_k)[0]
    return kv, kI


# ---------------------------------------------------------------------------
# CSA2 hierarchical indexer: block candidates of the Full layer, Reindex over the pool
# ---------------------------------------------------------------------------

def block_scores(scores, block: int):
    """Block score = the largest score among a block's positions ([V4-CSA2] section 11: a
    block of 8 positions scores as its best position); -inf when no position of the block
    is a candidate (all -inf).  scores [..., N] -> [..., ceil(N/block)]."""
    s = np.asarray(scores, np.float64)
    n = s.shape[-1]
    nb = -(-n // block)
    pad = np.full(s.shape[:-1] + (nb * block - n,), -np.inf)
    return np.concatenate([s, pad], axis=-1).reshape(s.shape[:-1] + (nb, block)).max(axis=-1)


def candidate_pool(scores, block: int, n_blocks: int):
    """The Full layer's candidate pool ([V4-CSA2] sections 11 and 11.1): the n_blocks best
    blocks (block score descending, lower block first on ties; blocks with no candidate
    are never chosen) -> the candidate positions of those blocks, ascending, padded with -1
    to n_blocks*block.  Returns (blocks [..., n_blocks] ascending, -1 padded, pool [...,
    n_blocks*block])."""
    s = np.asarray(scores, np.float64)
    lead, n = s.shape[:-1], s.shape[-1]
    blocks = topk_indices(block_scores(s, block), n_blocks)             # ascending block indices
    flat_s = s.reshape(-1, n)
    flat_b = blocks.reshape(-1, n_blocks)
    pool = np.full((flat_s.shape[0], n_blocks * block), -1, np.int64)
    for r in range(flat_s.shape[0]):
        pos = [int(bk) * block + j for bk in flat_b[r] if bk >= 0 for j in range(block)
               if int(bk) * block + j < n and flat_s[r, int(bk) * block + j] > -np.inf]
        pool[r, :len(pos)] = pos
    return blocks, pool.reshape(lead + (n_blocks * block,))


def pool_scores(qI, w, KI, pool, q_pos, m: int):
    """Reindex scores ([V4-CSA2] sections 11 and 15.2: gather the pool's keys, then score):
    I[b,s,e] = sum_h w[b,s,h] * ReLU(qI[b,s,h] . KI[b, pool[b,s,e]]) for a visible pool
    position, -inf for padding (-1) or positions the query may not see."""
    qI = np.asarray(qI, np.float64); w = np.asarray(w, np.float64); KI = np.asarray(KI, np.float64)
    pool = np.asarray(pool)
    B, S = qI.shape[:2]
    n_c = KI.shape[1]
    out = np.full(pool.shape, -np.inf)
    for b in range(B):
        for s in range(S):
            nv = int(visible_entries(np.asarray(q_pos)[b, s], m, n_c))
            for e, p in enumerate(pool[b, s]):
                if 0 <= p < nv:
                    out[b, s, e] = float(np.dot(w[b, s], np.maximum(qI[b, s] @ KI[b, p], 0.0)))
    return out


def reindex_topk(qI, w, KI, pool, q_pos, m: int, k: int):
    """A Reindex layer's selection: its own top-k over the pool (ties to the lower
    position), returned as positions, ascending, -1 padded."""
    sc = pool_scores(qI, w, KI, pool, q_pos, m)
    sel = topk_indices(sc, k)                                          # indices into the pool
    pool = np.asarray(pool)
    return np.where(sel >= 0, np.take_along_axis(pool, np.maximum(sel, 0), axis=-1), -1)


# ---------------------------------------------------------------------------
# Low-precision cache formats: FP4 E2M1 with E8M0 (per 32) or E4M3 (per 16) scales,
# FP8 entries with bf16 RoPE channels, bf16 index scores
# ---------------------------------------------------------------------------

E2M1_MAX = 6.0


def e2m1_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP E2M1 (FP4) codes 0..15 -> values: 1 sign bit, 2 exponent bits (bias 1), 1
    mantissa bit; exponent field 0 is subnormal (0 or 0.5).  Magnitudes 0, 0.5, 1, 1.5, 2,
    3, 4, 6; no infinity or NaN."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e, mt = (c >> 1) & 0x3, (c & 0x1).astype(np.float64)
    mag = np.where(e == 0, mt * 0.5, (1.0 + mt * 0.5) * np.exp2(e - 1.0))
    return sign * mag


def f64_to_e2m1(x: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code (ties to the code with an even mantissa bit), saturating at 6,
    by brute force over the 8 non-negative codes; zero keeps its sign."""
    x = np.asarray(x, np.float64)
    codes = np.arange(8)
    vals = e2m1_to_f64(codes)
    mag = np.minimum(np.abs(x), E2M1_MAX)
    d = np.abs(mag[..., None] - vals)
    tied = d == d.min(axis=-1, keepdims=True)
    even = tied & (codes % 2 == 0)
    pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(tied, axis=-1))
    return (codes[pick] | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def e8m0_to_f64(e: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes -> 2^(e - 127) (255 = NaN)."""
    e = np.asarray(e).astype(np.float64)
    return np.where(e == 255, np.nan, np.exp2(e - 127.0))


def quantize_mxfp4(x: np.ndarray, block: int = 32):
    """MXFP4 quantisation of rows ([V4-CSA2] section 16.2: E2M1 values, one E8M0 scale per
    32; the conversion follows the OCP microscaling format definition): per block, the
    shared exponent is floor(log2(amax)) - 2 (2 = the largest E2M1 exponent), clamped to
    the E8M0 range, and every value becomes the nearest E2M1 code of x / 2^exponent
    (saturating).  An all-zero block gets the smallest scale and zero codes.  Returns
    (codes [..., n] one code per value, scales [..., n/block] E8M0 bytes)."""
    x = np.asarray(x, np.float64)
    lead, n = x.shape[:-1], x.shape[-1]
    xb = x.reshape(lead + (n // block, block))
    amax = np.abs(xb).max(axis=-1)
    with np.errstate(divide="ignore"):
        ex = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2.0, -127.0)
    ex = np.clip(ex, -127.0, 127.0)
    codes = f64_to_e2m1(xb / np.exp2(ex)[..., None]).reshape(lead + (n,))
    return codes, (ex + 127.0).astype(np.uint8)


def dequant_mxfp4(codes, scales, block: int = 32):
    v = e2m1_to_f64(codes)
    n = v.shape[-1]
    s = e8m0_to_f64(scales)
    return (v.reshape(v.shape[:-1] + (n // block, block)) * s[..., None]).reshape(v.shape)


def quantize_fp4_e4m3(x: np.ndarray, block: int = 16):
    """FP4 main-KV quantisation ([V4-CSA2] section 16.1; [ATTN-CMP] section on CSA2: E2M1
    values with one E4M3 scale per 16 channels): per block the scale is amax/6 (the largest
    E2M1 magnitude) rounded to the nearest E4M3 code, and every value becomes the nearest
    E2M1 code of x / scale (saturating).  A block whose scale rounds to 0 gets zero codes.
    Returns (codes [..., n], scales [..., n/block] E4M3 bytes)."""
    x = np.asarray(x, np.float64)
    lead, n = x.shape[:-1], x.shape[-1]
    xb = x.reshape(lead + (n // block, block))
    sc = f64_to_e4m3fn(np.abs(xb).max(axis=-1) / E2M1_MAX)
    s = e4m3fn_to_f64(sc)
    safe = np.where(s > 0, s, 1.0)
    codes = np.where(s[..., None] > 0, f64_to_e2m1(xb / safe[..., None]), 0).astype(np.uint8)
    return codes.reshape(lead + (n,)), sc


def dequant_fp4_e4m3(codes, scales, block: int = 16):
    v = e2m1_to_f64(codes)
    n = v.shape[-1]
    s = e4m3fn_to_f64(scales)
    return (v.reshape(v.shape[:-1] + (n // block, block)) * s[..., None]).reshape(v.shape)


def quantize_fp8_rope_split(x: np.ndarray, d_rope: int):
    """The split entry ([ATTN-CMP] section "CSA（DeepSeek-V4）": the c - d_rope channels
    without RoPE in FP8, the d_rope RoPE channels in bf16): the FP8 part is quantised with
    one power-of-two scale per entry, 2^ceil(log2(amax/448)) (the smallest that avoids
    saturation), so that code * scale is exact in bf16; the RoPE part is rounded to bf16
    (RNE).  Returns (codes [..., c - d_rope] e4m3, exponent [...] int, rope bf16 bit
    patterns [..., d_rope])."""
    x = np.asarray(x, np.float64)
    c = x.shape[-1]
    main, rp = x[..., :c - d_rope], x[..., c - d_rope:]
    amax = np.abs(main).max(axis=-1)
    with np.errstate(divide="ignore"):
        ex = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / E4M3_MAX)), -127.0)
    codes = f64_to_e4m3fn(main / np.exp2(ex)[..., None])
    # RoPE channels: the nearest bf16 (8 significant bits, ties to even), from the real value
    mant, e2 = np.frexp(rp)
    rq = np.ldexp(np.rint(mant * 256.0), e2 - 8)
    rope_bits = (rq.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return codes, ex.astype(np.int64), rope_bits


def dequant_fp8_rope_split(codes, ex, rope_bits):
    return np.concatenate([e4m3fn_to_f64(codes) * np.exp2(np.asarray(ex, np.float64))[..., None],
                           bf16_bits_to_f64(rope_bits)], axis=-1)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """An index score as the pages cast it ([KV-COMP] section 7: scores quantised from FP32
    to BF16 before the top-k): the value as fp32 (nearest), then the nearest bf16 (ties to
    even), back in float64; -inf stays -inf."""
    x = np.asarray(x, np.float64)
    fin = np.isfinite(x)
    r32 = np.where(fin, x, 0.0).astype(np.float32)
    u = r32.view(np.uint32).astype(np.uint64)
    b = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    return np.where(fin, b.view(np.float32).astype(np.float64), x)
