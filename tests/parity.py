"""Comparison rules between the HIP path and the oracle (test infrastructure).

* fp32 outputs: max |gpu - oracle| <= 1e-5;  bf16 attention outputs: <= 2e-3, except
  where no bf16 number lies within 2e-3 of the exact value (|o| >= 1, where half a
  rounding step is >= 3.9e-3): there half a bf16 step (x (1 + 2^-10)) plus 1e-5 for the
  kernel's fp32 value before its rounding.
* bf16 compressed KV: within one bf16 spacing of the oracle's value (its rounding
  step, taken at the oracle's magnitude).
* FP8 codes: the row scale within 1e-5 relative; every code is the e4m3 rounding (ties
  to even, saturating) of some value within 1e-5 of the oracle's value, divided by the
  kernel's row scale: the kernel quantises its fp32 value, which carries the 1e-5 fp32
  tolerance, so only values that close to a rounding midpoint may take the other code.
* top-k: identical index sets except among entries whose oracle score is within
  1e-5 relative of the oracle's k-th score (ties the two precisions may order
  differently); same count, ascending order and -1 padding.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import csa_oracle as O

TOL_F32 = 1e-5
TOL_BF16_ATTN = 2e-3


# ---- device transfer (plumbing) ----------------------------------------------------------

def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """bfloat16 device tensor -> uint16 bit patterns on the host."""
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return O.bf16_bits_to_f64(bits)


# ---- rules -----------------------------------------------------------------------------

def bf16_output_tolerance(ref):
    """max(2e-3, half a bf16 step at the oracle's value x (1 + 2^-10) + 1e-5).

    A correctly rounded bf16 output lies within half a step of the exact value; the
    kernel rounds its own fp32 value, whose error before rounding (P carried as a bf16
    hi + lo pair, about 2^-18 of the weighted row sum, fp32 accumulation) stays below
    1e-5 at these magnitudes.  Below |o| = 1 the bound is the flat 2e-3."""
    ref = np.asarray(ref, np.float64)
    return np.maximum(TOL_BF16_ATTN, 0.5 * bf16_spacing(ref) * (1.0 + 2.0 ** -10) + TOL_F32)


def assert_bf16_output(gpu, ref, what=""):
    """bf16 outputs: |gpu - oracle| <= bf16_output_tolerance(oracle)."""
    ref = np.asarray(ref, np.float64)
    tol = bf16_output_tolerance(ref)
    err = np.abs(np.asarray(gpu, np.float64) - ref)
    if np.any(err > tol):
        i = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError(f"{what}: error {err[i]:.3e} > {tol[i]:.1e} at {i}: gpu {gpu[i]!r} oracle {ref[i]!r}")
    return float(err.max())


def assert_close(gpu, ref, tol, what=""):
    gpu = np.asarray(gpu, np.float64); ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    both_inf = np.isinf(gpu) & np.isinf(ref) & (np.sign(gpu) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(gpu - ref))
    err = np.where(np.isnan(err), np.inf, err)
    worst = float(err.max()) if err.size else 0.0
    if worst > tol:
        i = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{what}: max abs error {worst:.3e} > {tol:.1e} at {i}: gpu {gpu[i]!r} oracle {ref[i]!r}")
    return worst


def bf16_spacing(x: np.ndarray) -> np.ndarray:
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_bf16_within_one_step(gpu_bits: np.ndarray, ref: np.ndarray, what=""):
    """|gpu - oracle| <= one bf16 step at the oracle's value + the fp32 allowance 1e-5.

    The kernel rounds its own fp32 result to bf16; that result differs from the oracle's
    by fp32 rounding noise, which near zero can exceed a (tiny) bf16 step."""
    g = bf16_f64(gpu_bits)
    err = np.abs(g - ref)
    lim = bf16_spacing(ref) + TOL_F32
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err / lim), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} values beyond one bf16 step + 1e-5; worst at {i}: "
                             f"gpu {g[i]!r} oracle {ref[i]!r}")
    return float((err / lim).max())


def e4m3_step(v: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 2.0 ** (e - 3)


def assert_fp8_rows(codes_g: np.ndarray, scale_g: np.ndarray, ref: np.ndarray, what="", tol=TOL_F32):
    codes_o, scale_o = O.quantize_rows_e4m3(ref)
    rel = np.abs(scale_g.astype(np.float64) - scale_o) / np.maximum(scale_o, 1e-30)
    assert rel.max() <= 1e-5, f"{what}: scale mismatch {rel.max():.2e}"
    s = scale_g.astype(np.float64)[..., None]
    live = s > 0
    safe = np.where(live, s, 1.0)
    # rounding is monotone: the codes of values within tol of ref lie between these two
    lo = O.e4m3fn_to_f64(O.f64_to_e4m3fn((ref - tol) / safe))
    hi = O.e4m3fn_to_f64(O.f64_to_e4m3fn((ref + tol) / safe))
    dec = O.e4m3fn_to_f64(codes_g)
    ok = np.where(live, (dec >= lo) & (dec <= hi), dec == 0)
    assert ok.all(), (f"{what}: {int((~ok).sum())} codes are not the rounding of a value within {tol} "
                      f"of the oracle's")
    return int((codes_g != codes_o).sum())


def assert_topk_equal(idx_g: np.ndarray, idx_o: np.ndarray, scores_o: np.ndarray, k: int, what="",
                      rel=1e-5, exact=False):
    idx_g = np.asarray(idx_g).reshape(-1, k)
    idx_o = np.asarray(idx_o).reshape(-1, k)
    sc = np.asarray(scores_o, np.float64).reshape(idx_o.shape[0], -1)
    for r in range(idx_o.shape[0]):
        g, o = idx_g[r], idx_o[r]
        ng, no = int((g >= 0).sum()), int((o >= 0).sum())
        assert ng == no, f"{what} row {r}: {ng} selected vs {no}"
        assert np.all(g[ng:] == -1) and np.all(np.diff(g[:ng]) > 0), f"{what} row {r}: not ascending / padded"
        if exact:
            assert np.array_equal(g, o), f"{what} row {r}: index sets differ"
            continue
        sg, so = set(g[:ng].tolist()), set(o[:no].tolist())
        if sg == so:
            continue
        kth = sc[r, o[:no]].min()
        for j in sg ^ so:
            assert abs(sc[r, j] - kth) <= rel * abs(kth), \
                f"{what} row {r}: entry {j} (score {sc[r, j]}) differs, k-th score {kth}"


# ---------------------------------------------------------------------------------------
# Low-precision entries written by the GPU from its own fp32 rows: the scales and codes must
# be the oracle's quantisation of the oracle's rows, except where the oracle's value lies
# so close to a rounding boundary that the fp32 rows may fall on the other side.
# ---------------------------------------------------------------------------------------

E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
NEAR = 1e-4                                   # relative distance to a boundary that may flip


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, np.uint8)
    return np.stack([b & 0xF, b >> 4], axis=-1).reshape(b.shape[:-1] + (2 * b.shape[-1],))


def _near_e2m1_mid(v):
    a = np.abs(v)[..., None]
    return (np.abs(a - E2M1_MIDS) <= NEAR * np.maximum(a, 0.25)).any(axis=-1)


def _near_e4m3_mid(v):
    a = np.abs(np.asarray(v, np.float64))
    step = e4m3_step(a)
    frac = a / step
    return np.abs(frac - (np.floor(frac) + 0.5)) * step <= NEAR * np.maximum(a, 2.0 ** -9)


def _check_codes(codes_g, codes_o, near, what):
    diff = codes_g != codes_o
    bad = diff & ~near
    assert not bad.any(), f"{what}: {int(bad.sum())} codes differ away from a rounding boundary"
    return int(diff.sum())


def assert_mxfp4_rows(codes_g, scales_g, ref, what=""):
    """codes_g [..., n/2] packed E2M1, scales_g [..., n/32] E8M0 bytes, ref [..., n] oracle rows."""
    ref = np.asarray(ref, np.float64)
    n = ref.shape[-1]
    _, sc_o = O.quantize_mxfp4(ref)
    amax = np.abs(ref.reshape(ref.shape[:-1] + (n // 32, 32))).max(axis=-1)
    frac = np.log2(np.maximum(amax, 1e-300))
    near_pow2 = np.abs(frac - np.rint(frac)) <= NEAR
    bad = (scales_g != sc_o) & ~near_pow2
    assert not bad.any(), f"{what}: {int(bad.sum())} MX block exponents differ"
    v = ref / np.repeat(O.e8m0_to_f64(scales_g), 32, axis=-1)
    return _check_codes(unpack_nibbles(codes_g), O.f64_to_e2m1(v), _near_e2m1_mid(v), what)


def assert_packed_fp4_rows(rows_g, ref, what=""):
    """rows_g [..., 288] packed main-KV rows (E2M1 + E4M3 per 16), ref [..., 512]."""
    ref = np.asarray(ref, np.float64)
    codes_g, sc_g = unpack_nibbles(rows_g[..., :256]), rows_g[..., 256:288]
    _, sc_o = O.quantize_fp4_e4m3(ref)
    amax6 = np.abs(ref.reshape(ref.shape[:-1] + (32, 16))).max(axis=-1) / O.E2M1_MAX
    bad = (sc_g != sc_o) & ~_near_e4m3_mid(amax6)
    assert not bad.any(), f"{what}: {int(bad.sum())} E4M3 block scales differ"
    s = np.repeat(O.e4m3fn_to_f64(sc_g), 16, axis=-1)
    v = ref / np.where(s > 0, s, 1.0)
    codes_o = np.where(s > 0, O.f64_to_e2m1(v), 0)
    return _check_codes(codes_g, codes_o, _near_e2m1_mid(v) & (s > 0), what)


def assert_packed_fp8_rope_rows(rows_g, ref, what=""):
    """rows_g [..., 584] packed rows (e4m3 * 2^e over 448 channels, bf16 RoPE channels)."""
    ref = np.asarray(ref, np.float64)
    _, ex_o, _ = O.quantize_fp8_rope_split(ref, 64)
    ex_g = rows_g[..., 576].astype(np.int64) - 127
    amax = np.abs(ref[..., :448]).max(axis=-1) / O.E4M3_MAX
    frac = np.log2(np.maximum(amax, 1e-300))
    near_pow2 = np.abs(frac - np.rint(frac)) <= NEAR
    bad = (ex_g != ex_o) & ~near_pow2
    assert not bad.any(), f"{what}: {int(bad.sum())} row exponents differ"
    assert not rows_g[..., 577:].any(), f"{what}: padding bytes not zero"
    v = ref[..., :448] / np.exp2(ex_g.astype(np.float64))[..., None]
    n_diff = _check_codes(rows_g[..., :448], O.f64_to_e4m3fn(v), _near_e4m3_mid(v), what)
    assert_bf16_within_one_step(np.ascontiguousarray(rows_g[..., 448:576]).view("<u2"), ref[..., 448:],
                                what + " (RoPE channels)")
    return n_diff
