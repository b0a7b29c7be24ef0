"""Decode-time compressor (csa_compress_decode) against the oracle's token-by-token
compressor, through the C ABI: one call per decode step, every emitted entry checked
(bf16 entries within one bf16 step + 1e-5, FP8 rows by the FP8 rule, fp32 at 1e-5), the
16-entry blocked FP8 layout against csa_index_keys_b16 of the row-major result, the HCA ring
and online states, priming the ring after a prefill chunk, and the skipped cases."""

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from synthetic import inputs as I
from tests.parity import (TOL_F32, assert_bf16_within_one_step, assert_close, assert_fp8_rows, bf16_f64, dev,
                          dev_bf16, host_bits)

pytestmark = pytest.mark.gpu


def _steps(lib, a, kw, starts, T, Nc_max, out_dtype, layout=0, online=False, prime=None):
    """Runs T decode steps of B sequences; sequence b's token s sits at position starts[b] + s.
    prime: [B, m, d] tokens pushed (emit = 0) before the first step, at the m positions before."""
    B = a["hidden_bf16"].shape[0]
    m, c = kw["m"], kw["c"]
    state = torch.empty(lib.compress_state_size(B, m, c, kw["overlap"], online), dtype=torch.uint8, device="cuda")
    if layout == lib.CSA_LAYOUT_B16:
        cache = torch.zeros(lib.index_keys_b16_size(B, Nc_max), dtype=torch.uint8, device="cuda")
    elif out_dtype == "fp8":
        cache = torch.zeros(B, Nc_max, c, dtype=torch.uint8, device="cuda")
    else:
        cache = torch.zeros(B, Nc_max, c, dtype=torch.bfloat16, device="cuda")
    scale = torch.zeros(B, Nc_max, device="cuda") if out_dtype == "fp8" else None
    W = dev_bf16(np.ascontiguousarray(a["W_bf16"].T))
    bias = dev(a["bias"])
    common = dict(overlap=kw["overlap"], m=m, c=c, d_rope=kw["d_rope"], rope_theta=kw["rope_theta"],
                  rms_eps=kw["rms_eps"], online=online, cache_scale=scale, layout=layout, Nc_max=Nc_max)
    starts = np.asarray(starts, np.int64)
    if prime is not None:
        for r in range(m):
            lib.csa_compress_decode(dev_bf16(np.ascontiguousarray(prime[:, r])), W, bias, dev(starts - m + r), state,
                                    cache, emit=False, **common)
    for s in range(T):
        lib.csa_compress_decode(dev_bf16(np.ascontiguousarray(a["hidden_bf16"][:, s])), W, bias, dev(starts + s),
                                state, cache, **common)
    torch.cuda.synchronize()
    return cache, scale


def _oracle(a, kw, b, start, online=False, prime=None):
    return O.decode_compress(bf16_f64(a["hidden_bf16"][b]), bf16_f64(a["W_bf16"]), a["bias"], p0=start,
                             hidden_prev=None if prime is None else bf16_f64(prime[b]), online=online, **kw)


@pytest.mark.parametrize("c,T,starts", [(512, 24, [0, 8, 40]), (128, 20, [0, 4, 12])])
def test_decode_compress_csa_bf16(lib, c, T, starts):
    m, d, B = 4, 256, 3
    a = I.compressor_inputs(300 + c, B, T, d, m, c, True, 0.05, False)
    kw = dict(overlap=True, m=m, c=c, d_rope=64, rope_theta=1e4, rms_eps=1e-6)
    # each sequence starts at a block start; sequences that do not start at 0 have their
    # previous block primed (emit = 0): the same seeded tokens for all, positions differ
    prev = I.compressor_inputs(400 + c, B, m, d, m, c, True, 0.05, False)["hidden_bf16"]
    Nc_max = 40
    cache, _ = _steps(lib, a, kw, starts, T, Nc_max, "bf16", prime=prev)
    got = host_bits(cache)
    for b in range(B):
        ref = _oracle(a, kw, b, starts[b], prime=prev if starts[b] > 0 else None)
        assert sorted(ref) == list(range(starts[b] // m, (starts[b] + T) // m))
        for i, v in ref.items():
            assert_bf16_within_one_step(got[b, i], v, f"decode entry {i} of sequence {b}")
        # rows no step emitted stay untouched
        untouched = [i for i in range(Nc_max) if i not in ref]
        assert np.all(got[b, untouched] == 0)


def test_decode_compress_indexer_fp8_rows_and_blocks(lib):
    m, d, B, c, T = 4, 256, 2, 128, 40
    a = I.compressor_inputs(500, B, T, d, m, c, True, 0.05, False)
    kw = dict(overlap=True, m=m, c=c, d_rope=64, rope_theta=1e4, rms_eps=1e-6)
    Nc_max = 37                                     # ragged last block of 16
    rows, sc = _steps(lib, a, kw, [0, 0], T, Nc_max, "fp8")
    blocks, sc16 = _steps(lib, a, kw, [0, 0], T, Nc_max, "fp8", layout=lib.CSA_LAYOUT_B16)
    n = T // m
    codes, scales = rows.cpu().numpy(), sc.cpu().numpy()
    for b in range(B):
        ref = _oracle(a, kw, b, 0)
        v = np.stack([ref[i] for i in range(n)])[None]
        assert_fp8_rows(codes[b:b + 1, :n], scales[b:b + 1, :n], v, f"decode indexer K, sequence {b}")
    # the blocked layout holds the same codes: compare with the library's copy of the rows
    want = lib.csa_index_keys_b16(rows, torch.empty(lib.index_keys_b16_size(B, Nc_max), dtype=torch.uint8,
                                                    device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(blocks, want), "blocked decode output differs from the blocked copy of its rows"
    assert torch.equal(sc16, sc), "row scales differ between the layouts"


@pytest.mark.parametrize("online", [False, True])
def test_decode_compress_hca(lib, online):
    m, d, B, c, T = 128, 256, 2, 512, 256
    a = I.compressor_inputs(600, B, T, d, m, c, False, 0.05, False)
    a["bias"] = (a["bias"] * 40.0).astype(np.float32)      # gates far apart: the running max matters
    kw = dict(overlap=False, m=m, c=c, d_rope=64, rope_theta=1e4, rms_eps=1e-6)
    cache, _ = _steps(lib, a, kw, [0, 0], T, 4, "bf16", online=online)
    got = host_bits(cache)
    for b in range(B):
        ref = _oracle(a, kw, b, 0, online=online)
        assert sorted(ref) == [0, 1]
        for i, v in ref.items():
            assert_bf16_within_one_step(got[b, i], v, f"HCA decode entry {i} ({'online' if online else 'ring'})")


def test_decode_compress_fp32_tiny(lib):
    sh = I.TINY
    a = I.tiny_inputs()
    h = a["hidden"][0]                                       # [1024, 256] fp32
    kw = dict(overlap=True, m=sh.m, c=sh.c, d_rope=sh.d_rope, rope_theta=sh.rope_theta, rms_eps=1e-6)
    T = 64
    state = torch.empty(lib.compress_state_size(1, sh.m, sh.c, True), dtype=torch.uint8, device="cuda")
    cache = torch.zeros(1, T // sh.m, sh.c, device="cuda")
    W, bias = dev(np.ascontiguousarray(a["W_comp"].T)), dev(a["B_comp"])
    for s in range(T):
        lib.csa_compress_decode(dev(h[s:s + 1]), W, bias, dev(np.array([s], np.int64)), state, cache, **kw)
    torch.cuda.synchronize()
    ref = O.decode_compress(h[:T], a["W_comp"], a["B_comp"], p0=0, **kw)
    prefill = O.csa_compress(h[None, :T], a["W_comp"], a["B_comp"], p0=0, **kw)[0]
    got = cache.cpu().numpy()[0]
    assert_close(got, np.stack([ref[i] for i in range(T // sh.m)]), TOL_F32, "fp32 decode compressor")
    assert_close(got, prefill, TOL_F32, "fp32 decode compressor vs the prefill definition")


def test_decode_compress_skips(lib):
    # pos < 0: nothing happens to that sequence; an entry index >= Nc_max: not written
    m, d, B, c = 4, 256, 2, 128
    a = I.compressor_inputs(700, B, 8, d, m, c, True, 0.05, False)
    kw = dict(overlap=True, m=m, c=c, d_rope=64, rope_theta=1e4, rms_eps=1e-6)
    state = torch.empty(lib.compress_state_size(B, m, c, True), dtype=torch.uint8, device="cuda")
    cache = torch.zeros(B, 1, c, dtype=torch.bfloat16, device="cuda")
    W, bias = dev_bf16(np.ascontiguousarray(a["W_bf16"].T)), dev(a["bias"])
    for s in range(8):
        pos = np.array([-1, s], np.int64)                    # sequence 0 inactive; sequence 1 emits entries 0, 1
        lib.csa_compress_decode(dev_bf16(np.ascontiguousarray(a["hidden_bf16"][:, s])), W, bias, dev(pos), state,
                                cache, Nc_max=1, **kw)
    torch.cuda.synchronize()
    got = host_bits(cache)
    assert np.all(got[0] == 0), "an inactive sequence was written"
    ref = _oracle(a, kw, 1, 0)
    assert_bf16_within_one_step(got[1, 0], ref[0], "entry 0 of sequence 1")


def test_decode_compress_many_sequences_f32(lib):
    """20 sequences (two token tiles of the fused step, the second partial) at different
    block starts, one of them inactive (position -1): every emitted fp32 entry at 1e-5, the
    inactive sequence untouched."""
    m, d, B, c, T = 4, 256, 20, 128, 12
    a = I.compressor_inputs(800, B, T, d, m, c, True, 0.05, False)
    kw = dict(overlap=True, m=m, c=c, d_rope=64, rope_theta=1e4, rms_eps=1e-6)
    prev = I.compressor_inputs(801, B, m, d, m, c, True, 0.05, False)["hidden_bf16"]
    starts = np.array([4 * (b % 5) for b in range(B)], np.int64)
    Nc_max = 8
    state = torch.empty(lib.compress_state_size(B, m, c, True), dtype=torch.uint8, device="cuda")
    cache = torch.zeros(B, Nc_max, c, device="cuda")
    W, bias = dev_bf16(np.ascontiguousarray(a["W_bf16"].T)), dev(a["bias"])
    live = np.arange(B) != 7
    for r in range(m):
        pos = np.where(live, starts - m + r, -1)
        lib.csa_compress_decode(dev_bf16(np.ascontiguousarray(prev[:, r])), W, bias, dev(pos), state, cache,
                                emit=False, **kw)
    for s in range(T):
        pos = np.where(live, starts + s, -1)
        lib.csa_compress_decode(dev_bf16(np.ascontiguousarray(a["hidden_bf16"][:, s])), W, bias, dev(pos), state,
                                cache, **kw)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    assert np.all(got[7] == 0), "the inactive sequence was written"
    for b in np.flatnonzero(live):
        ref = _oracle(a, kw, b, starts[b], prime=prev if starts[b] > 0 else None)
        for i, v in ref.items():
            assert_close(got[b, i], v, TOL_F32, f"decode entry {i} of sequence {b}")
        untouched = [i for i in range(Nc_max) if i not in ref]
        assert np.all(got[b, untouched] == 0)


@pytest.mark.parametrize("B,d", [(33, 5120), (3, 1024)])
def test_decode_compress_many_equals_single_calls(lib, B, d):
    """A CSA layer's main (c = 512, bf16 rows) and indexer (c = 128, FP8 in 16-entry blocks)
    compressors through one csa_compress_decode_many call per token, against one
    csa_compress_decode per compressor: caches, scales and ring states bit-identical after
    every token.  Sequences sit at different phases of their blocks (boundary and
    non-boundary steps in the same call), one is skipped (pos -1), and the ring is primed
    with emit = 0 first; B = 33 spans two token tiles of the projection."""
    m, c, dI, Nc = 4, 512, 128, 64
    a = I.decode_layer_inputs(700 + B, B, d, m, c, dI)
    Wm, Bm = dev_bf16(a["W_main_t_bf16"]), dev(a["B_main"])
    Wi, Bi = dev_bf16(a["W_idx_t_bf16"]), dev(a["B_idx"])
    kw = dict(overlap=True, m=m, d_rope=64, rope_theta=1e4, rms_eps=1e-6)

    def buffers():
        z = lambda n: torch.zeros(n, dtype=torch.uint8, device="cuda")
        return {"kv": torch.zeros(B, Nc, c, dtype=torch.bfloat16, device="cuda"),
                "k16": z(lib.index_keys_b16_size(B, Nc)), "ks": torch.zeros(B, Nc, device="cuda"),
                "st_m": z(lib.compress_state_size(B, m, c, True)), "st_i": z(lib.compress_state_size(B, m, dI, True))}

    one, many = buffers(), buffers()
    tokens = [a["prime_bf16"][:, r] for r in range(2 * m - 1)] + [a["hidden_bf16"]] + \
        [a["prime_bf16"][:, r] for r in range(2 * m - 1)]
    base = np.int64(4 * 40 - (2 * m - 1))
    for r, hid in enumerate(tokens):
        h = dev_bf16(np.ascontiguousarray(hid))
        pos_h = base + r + (np.arange(B, dtype=np.int64) % 3)
        pos_h[B // 2] = -1
        pos = dev(pos_h)
        emit = r >= 2 * m - 1
        lib.csa_compress_decode(h, Wm, Bm, pos, one["st_m"], one["kv"], c=c, emit=emit, **kw)
        lib.csa_compress_decode(h, Wi, Bi, pos, one["st_i"], one["k16"], c=dI, cache_scale=one["ks"],
                                layout=lib.CSA_LAYOUT_B16, Nc_max=Nc, emit=emit, **kw)
        lib.csa_compress_decode_many(h, pos, [
            dict(w_proj=Wm, bias=Bm, state=many["st_m"], cache=many["kv"], c=c, **kw),
            dict(w_proj=Wi, bias=Bi, state=many["st_i"], cache=many["k16"], c=dI, cache_scale=many["ks"],
                 layout=lib.CSA_LAYOUT_B16, Nc_max=Nc, **kw)], emit=emit)
        torch.cuda.synchronize()
        for name in one:
            assert torch.equal(one[name], many[name]), f"token {r}: {name} differs between the two paths"
    assert int((many["ks"] > 0).sum()) > 0, "no entry was emitted"


@pytest.mark.parametrize("bf16_in", [True, False])
def test_decode_compress_many_mixed_compressors(lib, bf16_in):
    """Two unlike compressors in one csa_compress_decode_many call: a CSA ring (overlap,
    m = 4, c = 64, bf16 rows) and an HCA online state (m = 8, c = 32, fp32 rows, no RoPE
    part), over bf16 inputs (one projection launch) or fp32 inputs (one compressor after
    the other): bit-identical to one csa_compress_decode per compressor after every token,
    over 20 tokens (boundaries of both block sizes)."""
    rng = np.random.default_rng(4242 + int(bf16_in))
    B, d, Nc = 5, 256, 8
    specs = [dict(overlap=True, online=False, m=4, c=64, d_rope=16, out=torch.bfloat16),
             dict(overlap=False, online=True, m=8, c=32, d_rope=0, out=torch.float32)]

    def to_dev(x):
        if bf16_in:
            return dev_bf16(I.to_bf16_bits(x))
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()

    weights = []
    for sp in specs:
        ns = 4 if sp["overlap"] else 2
        W = to_dev(rng.normal(0.0, 0.05, (ns * sp["c"], d)))
        bias = dev(rng.normal(0.0, 0.05, (ns // 2, sp["m"], sp["c"])).astype(np.float32))
        weights.append((W, bias))

    def buffers():
        out = []
        for sp in specs:
            st = torch.zeros(lib.compress_state_size(B, sp["m"], sp["c"], sp["overlap"], sp["online"]),
                             dtype=torch.uint8, device="cuda")
            out.append((st, torch.zeros(B, Nc, sp["c"], dtype=sp["out"], device="cuda")))
        return out

    one, many = buffers(), buffers()
    kw = lambda sp: dict(overlap=sp["overlap"], online=sp["online"], m=sp["m"], c=sp["c"], d_rope=sp["d_rope"],
                         rope_theta=1e4, rms_eps=1e-6)
    for r in range(20):
        h = to_dev(rng.normal(0.0, 1.0, (B, d)))
        pos = dev((8 + r + np.arange(B) % 3).astype(np.int64))
        for i, sp in enumerate(specs):
            lib.csa_compress_decode(h, weights[i][0], weights[i][1], pos, one[i][0], one[i][1], **kw(sp))
        lib.csa_compress_decode_many(h, pos, [dict(w_proj=weights[i][0], bias=weights[i][1], state=many[i][0],
                                                   cache=many[i][1], **kw(sp)) for i, sp in enumerate(specs)])
        torch.cuda.synchronize()
        for i in range(len(specs)):
            assert torch.equal(one[i][0], many[i][0]), f"token {r}: state of compressor {i} differs"
            assert torch.equal(one[i][1], many[i][1]), f"token {r}: cache of compressor {i} differs"
    assert bool((many[0][1] != 0).any()) and bool((many[1][1] != 0).any()), "no entries emitted"


def test_decode_compress_many_graph_replay(lib):
    """Both compressors' decode step (csa_compress_decode_many, bf16, a block boundary) captured
    in a HIP graph: from the same primed state, every replay writes the eager call's entries
    and state, with eager calls between the replays."""
    B, d, m, c, dI, Nc = 4, 512, 4, 64, 32, 16
    a = I.decode_layer_inputs(99, B, d, m, c, dI)
    Wm, Bm = dev_bf16(a["W_main_t_bf16"]), dev(a["B_main"])
    Wi, Bi = dev_bf16(a["W_idx_t_bf16"]), dev(a["B_idx"])
    kw = dict(overlap=True, m=m, d_rope=16, rope_theta=1e4, rms_eps=1e-6)
    st_m = torch.zeros(lib.compress_state_size(B, m, c, True), dtype=torch.uint8, device="cuda")
    st_i = torch.zeros(lib.compress_state_size(B, m, dI, True), dtype=torch.uint8, device="cuda")
    kv = torch.zeros(B, Nc, c, dtype=torch.bfloat16, device="cuda")
    kk = torch.zeros(B, Nc, dI, dtype=torch.uint8, device="cuda")
    ks = torch.zeros(B, Nc, device="cuda")
    comps = lib.decode_compressors(B, [dict(w_proj=Wm, bias=Bm, state=st_m, cache=kv, c=c, **kw),
                                       dict(w_proj=Wi, bias=Bi, state=st_i, cache=kk, c=dI, cache_scale=ks,
                                            out_dtype=lib.CSA_FP8_E4M3, **kw)])
    ws = torch.empty(lib.compress_decode_many_workspace_size(B, d, lib.CSA_BF16, comps), dtype=torch.uint8,
                     device="cuda")
    t = 4 * 10 + 3                                   # completes block 10
    for r in range(2 * m - 1):
        lib.csa_compress_decode_many(dev_bf16(np.ascontiguousarray(a["prime_bf16"][:, r])),
                                     dev(np.full(B, t - (2 * m - 1) + r, np.int64)), comps, emit=False, ws=ws)
    torch.cuda.synchronize()
    primed = (st_m.clone(), st_i.clone())
    h, pos = dev_bf16(a["hidden_bf16"]), dev(np.full(B, t, np.int64))

    def reset():
        st_m.copy_(primed[0]); st_i.copy_(primed[1])
        kv.zero_(); kk.zero_(); ks.zero_()

    def step():
        lib.csa_compress_decode_many(h, pos, comps, ws=ws)

    reset()
    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (st_m, st_i, kv, kk, ks)]
    assert bool((ks > 0).any()), "no entry emitted"
    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y, name in zip((st_m, st_i, kv, kk, ks), ref, ("main state", "indexer state", "KV entries",
                                                                  "key codes", "key scales")):
            assert torch.equal(x, y), f"{name} differ on replay {r}"
        reset()
        step()                                       # eager work between the replays
        torch.cuda.synchronize()
