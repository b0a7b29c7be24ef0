"""CSA2 (DeepSeek-V4.1) rows through the C ABI against the oracle: the compressor (single
stream, no bias, ratio 1, indexer key from the main latent)."""

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from synthetic import inputs as I
from tests.parity import (TOL_F32, assert_bf16_within_one_step, assert_close, assert_fp8_rows, bf16_f64, dev,
                          dev_bf16, host_bits)

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
