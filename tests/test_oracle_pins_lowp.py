"""Pins of the oracle's low-precision formats (CPU only): the E2M1 and E8M0 tables of the OCP
microscaling formats, round-to-nearest-even ties, the MX shared-exponent rule and its
saturation bound, the E4M3-scaled FP4 blocks, the FP8 + bf16 split entry (exact round
trip of values on its grid, no saturation) and the bf16 cast of scores (ties, and torch's
own bfloat16 cast of the same fp32 values)."""

import math

import numpy as np
import torch

from oracle import csa_oracle as O


def test_e2m1_table_and_ties():
    assert np.array_equal(O.e2m1_to_f64(np.arange(8)), [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    assert np.array_equal(O.e2m1_to_f64(np.arange(8, 16)), -np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6]))
    # ties go to the even mantissa bit; beyond 6 saturates; the sign is kept
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -0.75, -5.0])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, -1.0, -4.0])
    assert np.array_equal(O.e2m1_to_f64(O.f64_to_e2m1(x)), want)
    # every code round-trips
    assert np.array_equal(O.f64_to_e2m1(O.e2m1_to_f64(np.arange(16)))[1:], np.arange(1, 16))


def test_e8m0_scale_bytes():
    assert np.array_equal(O.e8m0_to_f64(np.array([127, 128, 126, 0, 254])),
                          [1.0, 2.0, 0.5, 2.0 ** -127, 2.0 ** 127])
    assert math.isnan(O.e8m0_to_f64(np.array([255]))[0])


def test_mxfp4_shared_exponent_and_error_bound():
    # block amax 6 -> exponent floor(log2 6) - 2 = 0: values on the E2M1 grid stay exact
    x = np.zeros(32); x[:8] = [6, 3, 0.5, -1.5, 4, 2, 1, -6]
    codes, sc = O.quantize_mxfp4(x[None])
    assert sc[0, 0] == 127 and np.array_equal(O.dequant_mxfp4(codes, sc)[0], x)
    # amax in [2^e, 2^(e+1)) -> scale 2^(e-2); x / scale < 8, so saturation costs at most
    # 2 * scale and everything else at most half a grid step (scale * 1 at the top binade)
    rng = np.random.default_rng(50)
    x = rng.normal(size=(200, 128)) * np.exp2(rng.integers(-8, 8, size=(200, 1)))
    codes, sc = O.quantize_mxfp4(x)
    s = O.e8m0_to_f64(sc)
    amax = np.abs(x.reshape(200, 4, 32)).max(axis=-1)
    assert np.all(s == np.exp2(np.floor(np.log2(amax)) - 2))
    err = np.abs(O.dequant_mxfp4(codes, sc) - x).reshape(200, 4, 32)
    assert np.all(err <= 2 * s[..., None] + 1e-300)
    inside = np.abs(x.reshape(200, 4, 32)) <= 6 * s[..., None]
    assert np.all(err[inside] <= (np.abs(x.reshape(200, 4, 32)) / 4 + 0.25 * s[..., None])[inside])
    # an all-zero block
    codes, sc = O.quantize_mxfp4(np.zeros((1, 32)))
    assert np.all(codes == 0) and np.all(O.dequant_mxfp4(codes, sc) == 0)


def test_fp4_e4m3_blocks():
    # amax 3 -> scale 3/6 = 0.5 (an exact E4M3 value): values on the grid round-trip
    x = np.zeros(16); x[:6] = [3.0, -1.5, 0.25, 2.0, -0.5, 1.0]
    codes, sc = O.quantize_fp4_e4m3(x[None])
    assert O.e4m3fn_to_f64(sc)[0, 0] == 0.5
    assert np.array_equal(O.dequant_fp4_e4m3(codes, sc)[0], x)
    # random rows: the scale is the E4M3 rounding of amax / 6 and no value exceeds its block's
    # reach by more than the E4M3 rounding of the scale allows
    rng = np.random.default_rng(51)
    x = rng.normal(size=(100, 512))
    codes, sc = O.quantize_fp4_e4m3(x)
    assert np.array_equal(sc, O.f64_to_e4m3fn(np.abs(x.reshape(100, 32, 16)).max(axis=-1) / 6))
    rel = np.abs(O.dequant_fp4_e4m3(codes, sc) - x).max() / np.abs(x).max()
    assert rel < 0.2
    # 288 bytes per 512-channel entry: 256 of codes, 32 of scales
    assert codes.shape[-1] // 2 + sc.shape[-1] == 288


def test_fp8_rope_split_entry():
    rng = np.random.default_rng(52)
    x = rng.normal(size=(50, 512))
    codes, ex, rope = O.quantize_fp8_rope_split(x, 64)
    # power-of-two scale: the smallest with no saturation
    amax = np.abs(x[:, :448]).max(axis=-1)
    assert np.all(amax / np.exp2(ex) <= 448) and np.all(amax / np.exp2(ex - 1) > 448)
    y = O.dequant_fp8_rope_split(codes, ex, rope)
    assert np.array_equal(y[:, 448:], O.bf16_bits_to_f64(rope))
    assert np.abs(y[:, 448:] - x[:, 448:]).max() <= np.abs(x[:, 448:]).max() * 2 ** -8
    # values already on the grid come back exactly, and the dequantised values are bf16 numbers
    back = O.quantize_fp8_rope_split(y, 64)
    assert np.array_equal(O.dequant_fp8_rope_split(*back), y)
    assert np.array_equal(O.round_bf16(y), y)
    # 576 bytes of payload per entry: 448 codes + 64 bf16 channels
    assert codes.shape[-1] + 2 * rope.shape[-1] == 576


def test_bf16_cast_of_scores():
    one = 1.0
    assert O.round_bf16(np.array([one + 2 ** -8]))[0] == 1.0                      # tie -> even
    assert O.round_bf16(np.array([one + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6         # tie -> even
    assert O.round_bf16(np.array([-np.inf]))[0] == -np.inf
    rng = np.random.default_rng(53)
    x = rng.normal(size=10000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), ref)


def test_lowp_row_checks_accept_the_oracle_rows_and_catch_layout_mistakes():
    # the GPU-side row checks (tests/parity.py) applied to the oracle's own quantisation laid
    # out as the library documents, and to the same rows with a plausible layout mistake
    import pytest
    from tests.parity import assert_mxfp4_rows, assert_packed_fp4_rows, assert_packed_fp8_rope_rows
    rng = np.random.default_rng(77)
    x = rng.standard_normal((3, 512))
    x /= np.sqrt(np.mean(x * x, axis=-1, keepdims=True))

    def nib(c):
        return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)

    c4, s4 = O.quantize_fp4_e4m3(x)
    rows = np.concatenate([nib(c4), s4], axis=-1)
    assert assert_packed_fp4_rows(rows, x) == 0
    swapped = np.concatenate([(c4[..., 1::2] | (c4[..., 0::2] << 4)).astype(np.uint8), s4], axis=-1)
    with pytest.raises(AssertionError):
        assert_packed_fp4_rows(swapped, x)                    # nibble order
    cm, sm = O.quantize_mxfp4(x[:, :128])
    assert assert_mxfp4_rows(nib(cm), sm, x[:, :128]) == 0
    with pytest.raises(AssertionError):
        assert_mxfp4_rows(nib(cm), sm + 1, x[:, :128])        # exponent off by one
    c8, ex, rb = O.quantize_fp8_rope_split(x, 64)
    tail = np.zeros((3, 8), np.uint8)
    tail[:, 0] = ex + 127
    r8 = np.concatenate([c8, rb.astype("<u2").view(np.uint8), tail], axis=-1)
    assert assert_packed_fp8_rope_rows(r8, x) == 0
    bad = r8.copy()
    bad[:, 448:576] = np.roll(bad[:, 448:576], 2, axis=-1)    # RoPE channels shifted by one
    with pytest.raises(AssertionError):
        assert_packed_fp8_rope_rows(bad, x)


def test_fp8_row_check_accepts_the_oracle_rows_and_catches_mistakes():
    # the GPU-side FP8 row check (tests/parity.py) on the oracle's own quantisation, on values
    # moved by less than the fp32 tolerance, and on rows with a plausible mistake
    import pytest
    from tests.parity import assert_fp8_rows
    rng = np.random.default_rng(78)
    x = rng.standard_normal((4, 128))
    codes, sc = O.quantize_rows_e4m3(x)
    assert assert_fp8_rows(codes, sc, x) == 0
    # a value 5e-6 past a rounding midpoint may take either code
    v = x / sc[:, None].astype(np.float64)
    mid = np.array([1.0625, -2.125])                       # midpoints between e4m3 codes
    y = x.copy()
    y[0, :2] = mid * sc[0]
    y[0, :2] += np.sign(mid) * 5e-6
    c2, s2 = O.quantize_rows_e4m3(y)
    flipped = c2.copy()
    flipped[0, :2] = O.f64_to_e4m3fn(np.array([1.0, -2.0]))   # the other side of the midpoint
    assert assert_fp8_rows(flipped, s2, y) == 2
    bad = codes.copy()                                    # the row maximum (448) one code lower
    j = int(np.argmax(np.abs(v[1])))
    bad[1, j] = O.f64_to_e4m3fn(np.array([v[1, j] * 416.0 / 448.0]))[0]
    with pytest.raises(AssertionError):
        assert_fp8_rows(bad, sc, x)
    with pytest.raises(AssertionError):                   # two channels swapped
        sw = codes.copy()
        sw[2, [3, 40]] = sw[2, [40, 3]]
        if sw[2, 3] == codes[2, 3]:
            sw[2, 3] ^= 0x08
        assert_fp8_rows(sw, sc, x)
