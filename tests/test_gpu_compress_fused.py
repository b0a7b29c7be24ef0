"""The bf16 overlapping compressor with m = 4 runs its projection and pooling in one kernel
(the b-stream products taken from the token rows 4 earlier, so each lane holds a whole
2m-slot softmax); these cases cover both tile shapes it picks (256 and 64 tokens per tile),
chunks that end inside a tile, the first tile's halo rows from hidden_prev or padding, a
single entry, several sequences, fp32 output against the oracle at 1e-5, and the 16-entry
blocked key layout written straight from the compressor ([HCA-CSA] sections
"压缩算子：逐通道 softmax 的软池化" and "CSA 的重叠窗口"; [KV-COMP] section 9.3 for the cache
written per block)."""

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from synthetic import inputs as I
from tests.parity import TOL_F32, assert_close, assert_fp8_rows, bf16_f64, dev, dev_bf16

pytestmark = pytest.mark.gpu

KW = dict(overlap=True, m=4, d_rope=64, rope_theta=1e4, rms_eps=1e-6)


def _case(seed, B, T, d, c, with_prev):
    a = I.compressor_inputs(seed, B, T, d, 4, c, True, 0.05, with_prev)
    hp = a.get("hidden_prev_bf16")
    p0 = 4096 if with_prev else 0
    ref = O.csa_compress(bf16_f64(a["hidden_bf16"]), bf16_f64(a["W_bf16"]), a["bias"],
                         hidden_prev=None if hp is None else bf16_f64(hp), c=c, p0=p0, **KW)
    args = (dev_bf16(a["hidden_bf16"]), None if hp is None else dev_bf16(hp),
            dev_bf16(np.ascontiguousarray(a["W_bf16"].T)), dev(a["bias"]))
    return args, ref, p0


# (B, T, c, prev): tiles of 64 tokens unless B * ceil(T/256) * c/64 >= 192
@pytest.mark.parametrize("B,T,c,with_prev", [
    (1, 4, 128, False),          # one entry, padding b-slots
    (2, 200, 512, True),         # 64-token tiles, the last one 8 tokens long
    (3, 1000, 128, True),        # three sequences, ragged
    (2, 3000, 512, True),        # 256-token tiles (2 x 12 x 8 = 192), the last one 184 tokens long
    (1, 6144, 512, False),       # 256-token tiles, no previous block
])
def test_fused_compressor_f32(lib, B, T, c, with_prev):
    d = 256
    args, ref, p0 = _case(900 + T + c, B, T, d, c, with_prev)
    out = torch.full((B, T // 4, c), float("nan"), device="cuda")
    lib.csa_compress(*args, c=c, p0=p0, out=out, **KW)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, TOL_F32, f"fused compressor B={B} T={T} c={c}")


def test_fused_compressor_fp8_rows(lib):
    B, T, d, c = 2, 520, 256, 128
    args, ref, p0 = _case(931, B, T, d, c, True)
    out = torch.empty(B, T // 4, c, dtype=torch.uint8, device="cuda")
    sc = torch.empty(B, T // 4, device="cuda")
    lib.csa_compress(*args, c=c, p0=p0, out=out, out_scale=sc, **KW)
    torch.cuda.synchronize()
    assert_fp8_rows(out.cpu().numpy(), sc.cpu().numpy(), ref, "fused compressor, FP8 rows")


def test_blocked_keys_equal_the_relayout_of_the_rows(lib):
    """layout B16 from the compressor = csa_index_keys_b16 of its row-major codes, bit for
    bit (a chunk at p0 = 0 filling a cache of T/m entries, the last block partial)."""
    B, T, d, c = 2, 200, 256, 128
    n = T // 4
    args, _, _ = _case(941, B, T, d, c, False)
    rows = torch.empty(B, n, c, dtype=torch.uint8, device="cuda")
    rsc = torch.empty(B, n, device="cuda")
    lib.csa_compress(*args, c=c, p0=0, out=rows, out_scale=rsc, **KW)
    blocks = torch.zeros(lib.index_keys_b16_size(B, n), dtype=torch.uint8, device="cuda")
    bsc = torch.zeros(B, n, device="cuda")
    lib.csa_compress(*args, c=c, p0=0, out=blocks, out_scale=bsc, layout=lib.CSA_LAYOUT_B16, Nc_max=n, **KW)
    want = lib.csa_index_keys_b16(rows, torch.empty(lib.index_keys_b16_size(B, n), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(blocks, want), "blocked keys differ from csa_index_keys_b16 of the rows"
    assert torch.equal(bsc, rsc), "row scales differ"


def test_blocked_keys_at_a_cache_offset(lib):
    """A chunk at p0 > 0 lands at cache entries p0/m .. p0/m + T/m - 1 of each sequence's
    blocked cache; every other byte and scale keeps its previous value."""
    B, T, d, c = 2, 96, 256, 128
    n, e0 = T // 4, 4096 // 4 + 0
    Nc_max = e0 + n + 5
    args, ref, p0 = _case(951, B, T, d, c, True)
    rows = torch.empty(B, n, c, dtype=torch.uint8, device="cuda")
    rsc = torch.empty(B, n, device="cuda")
    lib.csa_compress(*args, c=c, p0=p0, out=rows, out_scale=rsc, **KW)
    nbytes = lib.index_keys_b16_size(B, Nc_max)
    blocks = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    bsc = torch.full((B, Nc_max), -1.0, device="cuda")
    lib.csa_compress(*args, c=c, p0=p0, out=blocks, out_scale=bsc, layout=lib.CSA_LAYOUT_B16, Nc_max=Nc_max, **KW)
    torch.cuda.synchronize()
    nblk = -(-Nc_max // 16)
    want = np.full(nbytes, 0xA5, np.uint8)
    r = rows.cpu().numpy()
    for b in range(B):
        for i in range(n):
            e = e0 + i
            for pc in range(4):
                o = (b * nblk + e // 16) * 2048 + pc * 512 + (e % 16) * 32
                want[o:o + 32] = r[b, i, 32 * pc:32 * pc + 32]
    assert np.array_equal(blocks.cpu().numpy(), want)
    s = bsc.cpu().numpy()
    assert np.array_equal(s[:, e0:e0 + n], rsc.cpu().numpy())
    assert np.all(s[:, :e0] == -1.0) and np.all(s[:, e0 + n:] == -1.0)
    assert_fp8_rows(r, rsc.cpu().numpy(), ref, "rows of the offset chunk")
