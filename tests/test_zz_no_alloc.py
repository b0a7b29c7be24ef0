"""csa_sparse_attn_noalloc (the entry point that allocates nothing: its split partials live
in the library's fixed scratch array) against csa_sparse_attn on the same inputs: identical
outputs on two calls in a row, the second smaller than the first, for the bf16 and the fp32
kernels; a call that needs more than the scratch holds is refused before any launch."""

import math

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from synthetic import inputs as I
from tests.parity import TOL_F32, assert_bf16_output, assert_close, bf16_f64, dev, dev_bf16, host_bits

pytestmark = pytest.mark.gpu


def _bf16_case(lib, seed, B, S, Nc, k, W, n_valid):
    Ls = S + W - 1
    a = I.attention_inputs(seed, B, S, Nc, Ls)
    idx = I.random_selection(seed, B, S, Nc, k, n_valid)
    q, kv, swa, sink = dev_bf16(a["q_bf16"]), dev_bf16(a["kv_comp_bf16"]), dev_bf16(a["swa_bf16"]), dev(a["sink"])
    di = dev(idx)
    out_ref = torch.empty(B, S, 64, 512, dtype=torch.bfloat16, device="cuda")
    lse_ref = torch.empty(B, S, 64, device="cuda")
    lib.csa_sparse_attn(q, kv, di, swa, sink, W=W, out=out_ref, lse=lse_ref)
    out = torch.full_like(out_ref, 3.0)
    lse = torch.full_like(lse_ref, 3.0)
    lib.csa_sparse_attn_noalloc(q, kv, di, swa, sink, W=W, out=out, lse=lse)
    torch.cuda.synchronize()
    return a, idx, out_ref, lse_ref, out, lse


def test_noalloc_matches_workspace_entry_point(lib):
    assert lib.sparse_attn_noalloc_max_bytes() == 32 << 20
    # first call: the V4-Flash decode shape (32 queries, 4 splits each: 16.8 MB of partials)
    big = _bf16_case(lib, 61, B=32, S=1, Nc=4000, k=512, W=128, n_valid=512)
    need = lib.attn_workspace_size(32, 1, 64, 512, 128 + 512, lib.CSA_BF16)
    assert 0 < need <= lib.sparse_attn_noalloc_max_bytes()
    # second call, smaller: 3 queries with padded selections (fewer, shorter partials)
    small = _bf16_case(lib, 62, B=3, S=1, Nc=2000, k=256, W=128, n_valid=np.array([[256], [100], [0]]))
    for name, (a, idx, out_ref, lse_ref, out, lse) in (("first", big), ("second", small)):
        assert torch.equal(out, out_ref), f"{name} call: output differs from csa_sparse_attn"
        assert torch.equal(lse, lse_ref), f"{name} call: lse differs from csa_sparse_attn"
    # the second (last) call against the oracle as well
    a, idx, _, _, out, lse = small
    q_pos = np.full((3, 1), 10 ** 6, np.int64)
    o_ref, l_ref = O.sparse_attention(bf16_f64(a["q_bf16"]), bf16_f64(a["kv_comp_bf16"]), idx, bf16_f64(a["swa_bf16"]),
                                      a["sink"], 1 / math.sqrt(512), q_pos, 128)
    assert_bf16_output(bf16_f64(host_bits(out)), o_ref, "noalloc attention vs oracle")
    assert_close(lse.cpu().numpy(), l_ref, TOL_F32, "noalloc lse vs oracle")


def test_noalloc_fp32_kernel(lib):
    # the fp32 path keeps its one partial per (query, head) in the scratch too
    sh = I.TINY
    rng = np.random.default_rng(63)
    for B, Nc, k in ((4, 256, 32), (2, 100, 16)):
        q = rng.standard_normal((B, 1, 8, 64)).astype(np.float32)
        kv = rng.standard_normal((B, Nc, 64)).astype(np.float32)
        swa = rng.standard_normal((B, 128, 64)).astype(np.float32)
        sink = rng.standard_normal(8).astype(np.float32)
        idx = np.sort(np.stack([rng.choice(Nc, k, replace=False) for _ in range(B)]), axis=1)[:, None].astype(np.int32)
        out_ref = torch.empty(B, 1, 8, 64, device="cuda")
        out = torch.full_like(out_ref, 3.0)
        lib.csa_sparse_attn(dev(q), dev(kv), dev(idx), dev(swa), dev(sink), W=sh.W, out=out_ref)
        lib.csa_sparse_attn_noalloc(dev(q), dev(kv), dev(idx), dev(swa), dev(sink), W=sh.W, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref), f"fp32 noalloc output differs (B={B})"


def test_noalloc_refuses_more_than_the_scratch(lib):
    # 64 queries x 2048 selected rows: 4 splits of 64 heads x 514 fp32 each = 33.7 MB > 32 MiB
    B, k, W = 64, 2048, 128
    assert lib.attn_workspace_size(B, 1, 64, 512, W + k, lib.CSA_BF16) > lib.sparse_attn_noalloc_max_bytes()
    q = torch.zeros(B, 1, 64, 512, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(B, 4096, 512, dtype=torch.bfloat16, device="cuda")
    swa = torch.zeros(B, W, 512, dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(B, 1, k, dtype=torch.int32, device="cuda")
    out = torch.zeros(B, 1, 64, 512, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.CSAError) as e:
        lib.csa_sparse_attn_noalloc(q, kv, idx, swa, torch.zeros(64, device="cuda"), W=W, out=out)
    assert e.value.status == 5
