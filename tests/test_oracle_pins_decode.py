"""Pins of the oracle's decode-time compressor, inverse RoPE and CSA2 compressor (CPU only).

The decode compressor is pinned to the prefill compressor (itself pinned by hand cases
and invariants in test_oracle_pins.py), to the hand case H1 run token by token, and to the
emission rule of the pages (an entry only when a token completes its block); the online
HCA variant to the ring.  Inverse RoPE is pinned to a hand rotation, to RoPE itself, and to
the relative-position property it exists for.  The CSA2 compressor is pinned to the
single-stream compressor with zero bias, to the ratio-1 closed form and a hand case, and its
indexer key to the projection of the main latent recovered by inverse RoPE.
"""

import math

import numpy as np

from oracle import csa_oracle as O


def _run_decode(hidden, W, bias, **kw):
    return O.decode_compress(hidden, W, bias, **kw)


def test_decode_compressor_hand_case_h1():
    # the H1 streams of test_oracle_pins (m = 2, c = 2) as the projections of 4 one-hot tokens
    Ca = np.array([[4, 2], [8, -2], [1, 1], [3, 1]], float)
    Za = np.array([[0, 0], [math.log(3), 0], [0, 0], [0, 0]], float)
    Cb = np.array([[0, 1], [4, 1], [0, 0], [0, 0]], float)
    Zb = np.zeros((4, 2))
    W = np.concatenate([Ca, Za, Cb, Zb], axis=1)             # token t projects to row t
    out = _run_decode(np.eye(4), W, np.zeros((2, 2, 2)), overlap=True, m=2, c=2, d_rope=0, rope_theta=1e4,
                      rms_eps=0.0, p0=0)
    assert list(out) == [0, 1]                                 # emitted at t = 1 and t = 3, in order
    assert np.allclose(out[0], [math.sqrt(2), 0.0])
    assert np.allclose(out[1], [1.264911064, 0.632455532])


def test_decode_compressor_equals_prefill_csa():
    rng = np.random.default_rng(21)
    m, c, d, T = 4, 8, 12, 40
    hidden = rng.normal(size=(T, d))
    W = rng.normal(size=(d, 4 * c)) * 0.7
    bias = rng.normal(size=(2, m, c))
    kw = dict(overlap=True, m=m, c=c, d_rope=4, rope_theta=1e4, rms_eps=1e-6)
    ref = O.csa_compress(hidden[None], W, bias, p0=0, **kw)[0]
    out = _run_decode(hidden, W, bias, p0=0, **kw)
    assert sorted(out) == list(range(T // m))
    for i, v in out.items():
        assert np.allclose(v, ref[i], atol=1e-12), i


def test_decode_compressor_after_a_prefill_chunk():
    # a decode loop that starts at p0 > 0 with the previous block's tokens pushed first
    # (no entry emitted for them) continues the chunked prefill exactly
    rng = np.random.default_rng(22)
    m, c, d = 4, 6, 10
    hidden = rng.normal(size=(5 * m, d))
    W = rng.normal(size=(d, 4 * c)) * 0.5
    bias = rng.normal(size=(2, m, c))
    kw = dict(overlap=True, m=m, c=c, d_rope=2, rope_theta=1e4, rms_eps=1e-6)
    full = O.csa_compress(hidden[None], W, bias, p0=0, **kw)[0]
    p0 = 2 * m
    out = _run_decode(hidden[p0:], W, bias, p0=p0, hidden_prev=hidden[p0 - m:p0], **kw)
    assert sorted(out) == [2, 3, 4]
    for i, v in out.items():
        assert np.allclose(v, full[i], atol=1e-12), i


def test_decode_compressor_emits_only_complete_blocks():
    rng = np.random.default_rng(23)
    m, c, d = 4, 4, 6
    W = rng.normal(size=(d, 4 * c))
    bias = np.zeros((2, m, c))
    kw = dict(overlap=True, m=m, c=c, d_rope=0, rope_theta=1e4, rms_eps=1e-6, p0=0)
    assert sorted(_run_decode(rng.normal(size=(10, d)), W, bias, **kw)) == [0, 1]     # tokens 8, 9: no entry yet
    assert _run_decode(rng.normal(size=(3, d)), W, bias, **kw) == {}                   # t < m - 1: nothing


def test_decode_compressor_hca_ring_and_online():
    rng = np.random.default_rng(24)
    m, c, d, T = 8, 6, 10, 32
    hidden = rng.normal(size=(T, d))
    W = rng.normal(size=(d, 2 * c)) * 3.0                      # large gate logits: the running max matters
    bias = rng.normal(size=(1, m, c)) * 4.0
    kw = dict(overlap=False, m=m, c=c, d_rope=4, rope_theta=1e4, rms_eps=1e-6, p0=0)
    ref = O.csa_compress(hidden[None], W, bias, **kw)[0]
    ring = _run_decode(hidden, W, bias, **kw)
    online = _run_decode(hidden, W, bias, online=True, **kw)
    assert sorted(ring) == sorted(online) == list(range(T // m))
    for i in range(T // m):
        assert np.allclose(ring[i], ref[i], atol=1e-12)
        assert np.allclose(online[i], ref[i], atol=1e-12)


def test_inverse_rope_hand_case_and_round_trip():
    # (cos 1, sin 1) at position 1 rotates back to (1, 0)
    assert np.allclose(O.inverse_rope(np.array([math.cos(1), math.sin(1)]), 1, 2, 1e4), [1.0, 0.0], atol=1e-15)
    rng = np.random.default_rng(25)
    x = rng.normal(size=(3, 16))
    pos = np.array([5, 1000, 131071])
    assert np.allclose(O.inverse_rope(O.rope(x, pos, 8, 1e4), pos, 8, 1e4), x, atol=1e-9)
    assert np.allclose(O.inverse_rope(x, pos, 8, 1e4)[:, :8], x[:, :8])        # the prefix is untouched


def test_inverse_rope_makes_the_output_relative():
    # rows rotated at their positions p_e, the query rotated at t, output rotated back by t:
    # moving every position by the same offset leaves the result unchanged
    rng = np.random.default_rng(26)
    c, dr, H, n = 16, 8, 2, 6
    base = rng.normal(size=(n, c))
    qb = rng.normal(size=(H, c))
    sink = rng.normal(size=H)
    zeros_swa = np.zeros((1, 1, c))

    def out_at(shift):
        p = np.arange(n) * 4 + 100 + shift
        t = 140 + shift
        kv = O.rope(base, p, dr, 1e4)[None]
        q = O.rope(qb, t, dr, 1e4)[None, None]
        idx = np.arange(n)[None, None]
        o, _ = O.sparse_attention(q, kv, idx, zeros_swa, sink, 0.3, np.array([[t]]), 1)
        return O.inverse_rope(o[0, 0], t, dr, 1e4)

    assert np.allclose(out_at(0), out_at(977), atol=1e-10)
    assert np.allclose(out_at(0), out_at(-90), atol=1e-10)


# ---------------------------------------------------------------------------
# CSA2 compressor
# ---------------------------------------------------------------------------

def test_csa2_main_is_the_single_stream_compressor_without_bias():
    # the CSA2 main latent is the HCA-style single stream with B = 0
    rng = np.random.default_rng(30)
    m, c, d, T, dI = 4, 8, 12, 24, 4
    hidden = rng.normal(size=(2, T, d))
    Wkv, Wg, Wk = rng.normal(size=(d, c)), rng.normal(size=(d, c)), rng.normal(size=(c, dI))
    kv, _ = O.csa2_compress(hidden, Wkv, Wg, Wk, m=m, d_rope=4, theta_kv=1e4, theta_k=1.6e5, rms_eps=1e-6, p0=8)
    ref = O.csa_compress(hidden, np.concatenate([Wkv, Wg], axis=1), np.zeros((1, m, c)), overlap=False, m=m, c=c,
                         d_rope=4, rope_theta=1e4, rms_eps=1e-6, p0=8)
    assert np.allclose(kv, ref, atol=1e-12)


def test_csa2_ratio_one_and_hand_case():
    rng = np.random.default_rng(31)
    d, c, dI, T = 6, 4, 2, 5
    hidden = rng.normal(size=(1, T, d))
    Wkv, Wk = rng.normal(size=(d, c)), rng.normal(size=(c, dI))
    kv, kI = O.csa2_compress(hidden, Wkv, None, Wk, m=1, d_rope=2, theta_kv=1e4, theta_k=1e4, rms_eps=0.0, p0=3)
    for i in range(T):
        C = hidden[0, i] @ Wkv
        lat = C / math.sqrt(np.mean(C * C))
        assert np.allclose(kv[0, i], O.rope(lat, 3 + i, 2, 1e4), atol=1e-12)
    # hand case, m = 2, c = 2: gates (0, ln 3) on channel 0 -> weights 1/4, 3/4; equal on channel 1
    hidden = np.eye(2)[None]                                  # token r projects to row r
    Wkv = np.array([[4.0, 2.0], [8.0, -2.0]])
    Wg = np.array([[0.0, 0.0], [math.log(3), 0.0]])
    Wk = np.array([[1.0, 0.0], [0.0, 1.0]])                   # identity: K^I = RoPE(Norm(latent))
    kv, kI = O.csa2_compress(hidden, Wkv, Wg, Wk, m=2, d_rope=0, theta_kv=1e4, theta_k=1e4, rms_eps=0.0, p0=0)
    # pooled = (0.25*4 + 0.75*8, 0.5*2 - 0.5*2) = (7, 0): normalised (sqrt 2, 0)
    assert np.allclose(kv[0, 0], [math.sqrt(2), 0.0])
    assert np.allclose(kI[0, 0], [math.sqrt(2), 0.0])


def test_csa2_indexer_key_is_projected_from_the_pre_rope_latent():
    # K^I from the latent before RoPE: undo the main RoPE of kv, project, normalise, rotate
    rng = np.random.default_rng(32)
    m, c, d, T, dI = 2, 8, 10, 12, 6
    hidden = rng.normal(size=(1, T, d))
    Wkv, Wg, Wk = rng.normal(size=(d, c)), rng.normal(size=(d, c)), rng.normal(size=(c, dI))
    kv, kI = O.csa2_compress(hidden, Wkv, Wg, Wk, m=m, d_rope=4, theta_kv=1e4, theta_k=1.6e5, rms_eps=1e-6, p0=100)
    pos = 100 + m * np.arange(T // m)
    latent = O.inverse_rope(kv[0], pos, 4, 1e4)
    expect = O.rope(O.rms_norm(latent @ Wk, 1e-6), pos, 4, 1.6e5)
    assert np.allclose(kI[0], expect, atol=1e-12)
    # and not from the rotated one (the positions are large enough for the two to differ)
    wrong = O.rope(O.rms_norm(kv[0] @ Wk, 1e-6), pos, 4, 1.6e5)
    assert not np.allclose(kI[0], wrong, atol=1e-3)
