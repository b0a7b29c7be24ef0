"""Seeded synthetic inputs for the CSA / HCA hot path.

This module is shared by the tests (which feed both the oracle and the HIP
library) and by ``bench.py``.  It holds no arithmetic of the method itself: only
random draws, row rescaling to a target root-mean-square, and the library's own
dtype casts (torch CPU casts to bfloat16 and to float8_e4m3fn).

Storage conventions of the returned numpy arrays:
  * bfloat16 tensors are ``np.uint16`` bit patterns (``bf16`` in the name map);
  * FP8 tensors are ``np.uint8`` OCP e4m3fn codes plus an ``np.float32`` per-row
    scale, scale = amax/448 of the row before the cast;
  * fp32 tensors are ``np.float32``; positions are ``np.int64``.

Distributions (the recipe the design notes restate):
  * hidden states: N(0, 1);  projection weights and position biases: N(0, sigma);
  * "normalised" rows (compressed KV, SWA KV, indexer K): Gaussian rows rescaled to
    unit root-mean-square, i.e. uniform on the sphere of radius sqrt(c).  A rotary
    embedding maps that distribution onto itself, so no rotation is drawn;
  * main query: unit root-mean-square rows per head (a per-head RMSNorm then a
    rotation);  indexer query: N(0, 1) (its per-row FP8 scale absorbs the magnitude);
    indexer head weights: N(0, 1) / sqrt(d_I * H_I);
  * attention sink: N(0, 1).
Every tensor has its own child stream of ``SeedSequence(seed)``, drawn in the
order the generator lists them.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

E4M3_MAX = 448.0


# ---------------------------------------------------------------------------
# dtype helpers (library casts)
# ---------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (round to nearest even, by torch) as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_fp8_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Rows of float32 -> (e4m3fn codes, per-row scale amax/448) using torch's cast."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1)).astype(np.float32)
    v = torch.from_numpy(x / safe[..., None])
    codes = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _streams(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def gaussian(rng, shape, sigma=1.0) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        out *= np.float32(sigma)
    return out


def unit_rms_rows(rng, shape) -> np.ndarray:
    """Gaussian rows rescaled to unit root-mean-square (uniform on the sqrt(c) sphere)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    ms = np.mean(np.square(x, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
    x /= np.sqrt(ms)
    return x


_CHUNK_ROWS = 8192


def _chunked(rng, lead: int, fn, outs):
    """Fills row slabs of `outs` (arrays with `lead` rows) with fn(child_rng, r0, r1).

    Slab i always draws from child stream i (seeded from `rng`), so the result does not
    depend on how many threads run the slabs."""
    import concurrent.futures as cf
    import os
    nch = (lead + _CHUNK_ROWS - 1) // _CHUNK_ROWS
    seeds = rng.integers(0, 2 ** 63 - 1, size=nch)

    def work(i):
        r0, r1 = i * _CHUNK_ROWS, min(lead, (i + 1) * _CHUNK_ROWS)
        res = fn(np.random.default_rng(int(seeds[i])), r1 - r0)
        for o, v in zip(outs, res):
            o[r0:r1] = v

    with cf.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(work, range(nch)))


def unit_rms_rows_bf16(rng, shape) -> np.ndarray:
    """Unit-RMS Gaussian rows produced slab by slab straight to bf16 bits."""
    lead = int(np.prod(shape[:-1]))
    c = shape[-1]
    out = np.empty((lead, c), dtype=np.uint16)
    _chunked(rng, lead, lambda r, n: (to_bf16_bits(unit_rms_rows(r, (n, c))),), (out,))
    return out.reshape(shape)


def unit_rms_rows_fp8(rng, shape) -> tuple[np.ndarray, np.ndarray]:
    """Unit-RMS Gaussian rows as e4m3 codes with their per-row scale, slab by slab."""
    lead = int(np.prod(shape[:-1]))
    c = shape[-1]
    codes = np.empty((lead, c), dtype=np.uint8)
    scale = np.empty((lead,), dtype=np.float32)
    _chunked(rng, lead, lambda r, n: to_fp8_rows(unit_rms_rows(r, (n, c))), (codes, scale))
    return codes.reshape(shape), scale.reshape(shape[:-1])


# ---------------------------------------------------------------------------
# Workload definitions
# ---------------------------------------------------------------------------

@dataclass
class DecodeShape:
    """One CSA (m = 4) or HCA (m = 128) decode step: one query per sequence."""
    name: str
    B: int
    n_c: int
    m: int
    t: int                     # absolute position of the query
    k: int = 0                 # top-k (CSA only)
    H: int = 64
    c: int = 512
    H_I: int = 64
    d_I: int = 128
    W: int = 128
    seed: int = 1


FLASH_DECODE = DecodeShape("v4flash_csa_decode_b32_ctx128k", B=32, n_c=32768, m=4, t=131071,
                           k=512, seed=1)
PRO_DECODE = DecodeShape("v4pro_csa_decode_b4_ctx1m", B=4, n_c=262144, m=4, t=1048575,
                         k=1024, seed=2)
HCA_DECODE = DecodeShape("hca_dense_decode_b64_ctx1m", B=64, n_c=8192, m=128, t=1048575,
                         seed=3)


@dataclass
class DecodeInputs:
    shape: DecodeShape
    arrays: dict = field(default_factory=dict)


def decode_inputs(sh: DecodeShape, seed: int | None = None, with_indexer: bool = True) -> DecodeInputs:
    """Inputs of one decode step (per sequence b: history of n_c entries, one query at sh.t).

    Draw order: kv_comp, swa, q, sink, then (CSA) k_I, q_I, w.
    """
    seed = sh.seed if seed is None else seed
    rs = _streams(seed, 7)
    a = {}
    a["kv_comp_bf16"] = unit_rms_rows_bf16(rs[0], (sh.B, sh.n_c, sh.c))
    a["swa_bf16"] = to_bf16_bits(unit_rms_rows(rs[1], (sh.B, sh.W, sh.c)))
    a["q_bf16"] = to_bf16_bits(unit_rms_rows(rs[2], (sh.B, 1, sh.H, sh.c)))
    a["sink"] = gaussian(rs[3], (sh.H,))
    a["q_pos"] = np.full((sh.B, 1), sh.t, dtype=np.int64)
    if with_indexer:
        a["kI_fp8"], a["kI_scale"] = unit_rms_rows_fp8(rs[4], (sh.B, sh.n_c, sh.d_I))
        a["qI_fp8"], a["qI_scale"] = to_fp8_rows(gaussian(rs[5], (sh.B, 1, sh.H_I, sh.d_I)))
        a["w"] = gaussian(rs[6], (sh.B, 1, sh.H_I), sigma=1.0 / np.sqrt(sh.d_I * sh.H_I))
    return DecodeInputs(sh, a)


@dataclass
class PrefillShape:
    """A CSA prefill chunk of S new tokens appended to a context of `ctx` tokens."""
    name: str = "csa_prefill_chunk8192_ctx128k"
    ctx: int = 131072
    S: int = 8192
    d: int = 5120
    m: int = 4
    c: int = 512
    d_I: int = 128
    H: int = 64
    H_I: int = 64
    k: int = 512
    W: int = 128
    d_rope: int = 64
    rope_theta: float = 1e4
    sigma_w: float = 0.02
    seed: int = 4


PREFILL = PrefillShape()


def prefill_inputs(sh: PrefillShape = PREFILL, seed: int | None = None) -> dict:
    """Inputs of one prefill chunk.  The context's compressed entries (ctx/m of them) are
    given precompressed; the chunk's hidden states (plus the m tokens before it, whose
    b-stream feeds the chunk's first entry) go through the compressor.

    Draw order: hidden (m+S rows), W_main, B_main, W_idx, B_idx, kv_ctx, kI_ctx, q,
    qI, w, swa, sink.
    """
    seed = sh.seed if seed is None else seed
    rs = _streams(seed, 12)
    n_ctx = sh.ctx // sh.m
    a = {}
    hid = gaussian(rs[0], (1, sh.m + sh.S, sh.d))
    a["hidden_bf16"] = to_bf16_bits(hid[:, sh.m:])
    a["hidden_prev_bf16"] = to_bf16_bits(hid[:, :sh.m])
    del hid
    a["W_main_bf16"] = to_bf16_bits(gaussian(rs[1], (sh.d, 4 * sh.c), sh.sigma_w))
    a["B_main"] = gaussian(rs[2], (2, sh.m, sh.c), sh.sigma_w)
    a["W_idx_bf16"] = to_bf16_bits(gaussian(rs[3], (sh.d, 4 * sh.d_I), sh.sigma_w))
    a["B_idx"] = gaussian(rs[4], (2, sh.m, sh.d_I), sh.sigma_w)
    a["kv_ctx_bf16"] = unit_rms_rows_bf16(rs[5], (1, n_ctx, sh.c))
    a["kI_ctx_fp8"], a["kI_ctx_scale"] = unit_rms_rows_fp8(rs[6], (1, n_ctx, sh.d_I))
    a["q_bf16"] = unit_rms_rows_bf16(rs[7], (1, sh.S, sh.H, sh.c))
    a["qI_fp8"], a["qI_scale"] = to_fp8_rows(gaussian(rs[8], (1, sh.S, sh.H_I, sh.d_I)))
    a["w"] = gaussian(rs[9], (1, sh.S, sh.H_I), sigma=1.0 / np.sqrt(sh.d_I * sh.H_I))
    a["swa_bf16"] = unit_rms_rows_bf16(rs[10], (1, sh.S + sh.W - 1, sh.c))
    a["sink"] = gaussian(rs[11], (sh.H,))
    a["q_pos"] = (sh.ctx + np.arange(sh.S, dtype=np.int64))[None]
    return a


@dataclass
class TinyShape:
    """The fp32 tiny layer: N = 1024 history tokens, d = 256, m = 4 with overlap,
    c = 64 (last 16 rope), indexer 4 x 32 with its own compressor, top-k 32, H = 8."""
    N: int = 1024
    d: int = 256
    m: int = 4
    c: int = 64
    d_rope: int = 16
    H: int = 8
    H_I: int = 4
    d_I: int = 32
    k: int = 32
    W: int = 128
    rope_theta: float = 1e4
    sigma_w: float = 0.05
    seed: int = 0


TINY = TinyShape()


def tiny_inputs(sh: TinyShape = TINY, seed: int | None = None) -> dict:
    """Draw order: hidden, W_comp, B_comp, W_icomp, B_icomp, q, qI, w, swa, sink."""
    seed = sh.seed if seed is None else seed
    rs = _streams(seed, 10)
    a = {}
    a["hidden"] = gaussian(rs[0], (1, sh.N, sh.d))
    a["W_comp"] = gaussian(rs[1], (sh.d, 4 * sh.c), sh.sigma_w)
    a["B_comp"] = gaussian(rs[2], (2, sh.m, sh.c), sh.sigma_w)
    a["W_icomp"] = gaussian(rs[3], (sh.d, 4 * sh.d_I), sh.sigma_w)
    a["B_icomp"] = gaussian(rs[4], (2, sh.m, sh.d_I), sh.sigma_w)
    a["q"] = unit_rms_rows(rs[5], (1, 1, sh.H, sh.c))
    # an indexer query is a projection of a hidden state with N(0, sigma_w) weights
    a["qI"] = gaussian(rs[6], (1, 1, sh.H_I, sh.d_I), sigma=sh.sigma_w * np.sqrt(sh.d))
    a["w"] = gaussian(rs[7], (1, 1, sh.H_I), sigma=sh.sigma_w * np.sqrt(sh.d) / np.sqrt(sh.d_I * sh.H_I))
    a["swa"] = unit_rms_rows(rs[8], (1, sh.W, sh.c))
    a["sink"] = gaussian(rs[9], (sh.H,))
    a["q_pos"] = np.array([[sh.N - 1]], dtype=np.int64)
    return a


# ---------------------------------------------------------------------------
# Score rows for the top-k stage on its own
# ---------------------------------------------------------------------------

def score_rows(seed: int, rows: int, n: int, kind: str = "gauss", n_vis=None) -> np.ndarray:
    """fp32 score rows with -inf beyond n_vis[r] (the invisible entries).

    kind: "gauss" (continuous), "ties" (few distinct values), "const" (all equal),
    "mixed" (Gaussian with a block of exact duplicates of one value),
    "narrow" (uniform in [1, 1.25): every score shares its sign, exponent and top two
    mantissa bits).
    """
    rng = _streams(seed, 1)[0]
    if kind == "gauss":
        s = rng.standard_normal((rows, n), dtype=np.float32)
    elif kind == "ties":
        s = rng.integers(0, 7, (rows, n)).astype(np.float32) * np.float32(0.25)
    elif kind == "const":
        s = np.full((rows, n), 0.5, np.float32)
    elif kind == "mixed":
        s = rng.standard_normal((rows, n), dtype=np.float32)
        dup = rng.random((rows, n)) < 0.05
        s[dup] = np.float32(1.25)
        s[rng.random((rows, n)) < 0.01] = -0.0
        s[rng.random((rows, n)) < 0.01] = 0.0
    elif kind == "narrow":
        s = (1.0 + 0.25 * rng.random((rows, n), dtype=np.float32)).astype(np.float32)
        s = np.minimum(s, np.float32(np.nextafter(np.float32(1.25), np.float32(0))))
    else:
        raise ValueError(kind)
    if n_vis is not None:
        nv = np.broadcast_to(np.asarray(n_vis), (rows,))
        s[np.arange(n)[None, :] >= nv[:, None]] = -np.inf
    return s


# ---------------------------------------------------------------------------
# Small stage-level workloads for the parity tests
# ---------------------------------------------------------------------------

def indexer_inputs(seed: int, B: int, S: int, Nc: int, H_I: int = 64, d_I: int = 128) -> dict:
    """FP8 indexer inputs: K rows unit-RMS, q Gaussian, w = N(0,1)/sqrt(d_I*H_I)."""
    rs = _streams(seed, 3)
    a = {}
    a["kI_fp8"], a["kI_scale"] = unit_rms_rows_fp8(rs[0], (B, Nc, d_I))
    a["qI_fp8"], a["qI_scale"] = to_fp8_rows(gaussian(rs[1], (B, S, H_I, d_I)))
    a["w"] = gaussian(rs[2], (B, S, H_I), sigma=1.0 / np.sqrt(d_I * H_I))
    return a


def attention_inputs(seed: int, B: int, S: int, Nc: int, Ls: int, H: int = 64, c: int = 512) -> dict:
    """bf16 attention inputs: unit-RMS KV and window rows, unit-RMS queries, N(0,1) sink."""
    rs = _streams(seed, 4)
    return {
        "kv_comp_bf16": unit_rms_rows_bf16(rs[0], (B, Nc, c)),
        "swa_bf16": to_bf16_bits(unit_rms_rows(rs[1], (B, Ls, c))),
        "q_bf16": to_bf16_bits(unit_rms_rows(rs[2], (B, S, H, c))),
        "sink": gaussian(rs[3], (H,)),
    }


def random_selection(seed: int, B: int, S: int, Nc: int, k: int, n_valid) -> np.ndarray:
    """idx [B,S,k] int32: n_valid[b,s] distinct entries in ascending order, then -1."""
    rng = _streams(seed, 1)[0]
    idx = np.full((B, S, k), -1, np.int32)
    nv = np.broadcast_to(np.asarray(n_valid), (B, S))
    for b in range(B):
        for s in range(S):
            n = int(min(nv[b, s], k, Nc))
            idx[b, s, :n] = np.sort(rng.choice(Nc, size=n, replace=False))
    return idx


def compressor_inputs(seed: int, B: int, T: int, d: int, m: int, c: int, overlap: bool, sigma_w: float,
                      with_prev: bool) -> dict:
    """hidden N(0,1) bf16 (plus the m previous tokens), W [d, S*c] and bias N(0, sigma_w)."""
    rs = _streams(seed, 4)
    ns = 4 if overlap else 2
    a = {"hidden_bf16": to_bf16_bits(gaussian(rs[0], (B, T, d)))}
    if with_prev:
        a["hidden_prev_bf16"] = to_bf16_bits(gaussian(rs[1], (B, m, d)))
    a["W_bf16"] = to_bf16_bits(gaussian(rs[2], (d, ns * c), sigma_w))
    a["bias"] = gaussian(rs[3], (ns // 2, m, c), sigma_w)
    return a


def decode_layer_inputs(seed: int, B: int, d: int, m: int, c: int, d_I: int, sigma_w: float = 0.02) -> dict:
    """The compressor side of one CSA decode step: the new token's hidden state per sequence
    (N(0,1) bf16), the 2m - 1 tokens before it (to fill the (C, Z) ring before the first
    step), and the main / indexer compressor weights and biases (N(0, sigma_w); W in the
    "out x in" layout the library takes, bf16)."""
    rs = _streams(seed, 6)
    return {
        "hidden_bf16": to_bf16_bits(gaussian(rs[0], (B, d))),
        "prime_bf16": to_bf16_bits(gaussian(rs[1], (B, 2 * m - 1, d))),
        "W_main_t_bf16": to_bf16_bits(gaussian(rs[2], (4 * c, d), sigma_w)),
        "B_main": gaussian(rs[3], (2, m, c), sigma_w),
        "W_idx_t_bf16": to_bf16_bits(gaussian(rs[4], (4 * d_I, d), sigma_w)),
        "B_idx": gaussian(rs[5], (2, m, d_I), sigma_w),
    }


def csa2_inputs(seed: int, B: int, T: int, d: int, m: int, c: int, d_I: int, sigma_w: float = 0.05,
                bf16: bool = True) -> dict:
    """CSA2 compressor inputs: hidden N(0,1), W_kv and W_gate [d, c] (no gate for m = 1) and
    W_k [c, d_I], all N(0, sigma_w) with W_k scaled by sqrt(d / c) (it reads the unit-RMS
    latent, not the hidden state); bf16 bit patterns, or fp32 with bf16=False."""
    rs = _streams(seed, 4)
    cast = to_bf16_bits if bf16 else (lambda x: np.ascontiguousarray(x, np.float32))
    a = {"hidden": cast(gaussian(rs[0], (B, T, d))),
         "W_kv": cast(gaussian(rs[1], (d, c), sigma_w)),
         "W_gate": cast(gaussian(rs[2], (d, c), sigma_w)) if m > 1 else None,
         "W_k": cast(gaussian(rs[3], (c, d_I), sigma_w * np.sqrt(d / c)))}
    return a
