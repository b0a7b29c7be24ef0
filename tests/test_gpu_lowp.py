"""Low-precision cache rows through the C ABI against the oracle: index scores over MXFP4
queries and keys (E2M1 + E8M0 per 32) on the scaled MFMA, their bf16 cast before the
top-k, and the measured precision of the FP8 form of the same unit (the reason the exact
FP8 path contracts on bf16 MFMA after an exact conversion)."""

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
