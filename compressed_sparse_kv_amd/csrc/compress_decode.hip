// Decode-time compressor step (one new token per sequence).
//
// [HCA-CSA] section "KV cache：成品与原料": the compressor keeps an FP32 ring of the (C, Z)
// projections of the last 2m tokens (CSA: the current block and the previous one, whose
// b-stream the next entry pools) or m tokens (HCA); a compressed entry is produced only by
// the token that completes its block, and section "在 SGLang 里的落点": that step reads the
// 2m slots (this block's a-stream and the previous block's b-stream).  The HCA "online"
// state keeps only a running (max, sum, weighted sum) per channel.  [KV-COMP] section 9.3:
// state until the boundary, then one pooled entry written to the cache.
//
// Two kernels per call:
//   1. proj_token_bf16 / proj_token_f32: P[b, :] = W . h_b for the B new tokens (fp32, in
//      the workspace).  bf16: v_mfma_f32_16x16x32_bf16, a workgroup per (64 output columns,
//      512-wide K slice, 32 tokens): the slice of the tokens' hidden vectors is staged once
//      in LDS and shared by the 4 waves, each wave holding its 16 W rows of the slice in
//      registers; partial sums per slice in the workspace.  The weights are read once per
//      call and spread over many workgroups: decode projection is bound by that stream.
//      (A single pass with full-K dot products per workgroup, the pooling in its epilogue,
//      measured slower: every workgroup then pulls all the tokens' hidden vectors, 320 KB
//      for 32 tokens, and a compute unit streams only about 20 GB/s of such loads.)
//   2. compress_step: one workgroup per sequence, one thread per channel pair.  The K
//      slices are summed (fixed order, loaded in groups); the token's streams go into ring
//      slot t mod 2m (or m), or update the online triple;
//      when (t + 1) % m == 0 entry i = t / m is pooled (per-channel softmax over the slots,
//      weighted sum; the other slots are loaded before the slices), RMS-normalised, rotated
//      (RoPE at position m*i, angle formed in double) and written as fp32 / bf16 / e4m3
//      (+ row scale amax/448), row-major or, for the indexer keys, straight into the
//      16-entry blocked layout the decode scoring pass reads.
#include <algorithm>

#include "common.hpp"
#include "entry_store.hpp"

namespace csa {

constexpr int kPjK = 128;                   // K block: 4 MFMA steps of 32
constexpr int kPjSlice = 512;               // K per workgroup (4 blocks); one partial sum per slice
constexpr int kPjWaves = 4;
constexpr int kPjCols = 16 * kPjWaves;      // output columns per workgroup, 16 per wave
constexpr int kPjTok = 32;                  // tokens per workgroup (2 MFMA tiles)
constexpr int kPjStride = 2 * kPjSlice + 16;   // LDS bytes per token row (8 rows in 8 bank groups)

// Partial projection over K slice blockIdx.y: Pk[slice][b][n] for the up to 32 tokens of
// blockIdx.z and the 64 columns of column block xb; W [N, d] bf16 ("out x in").  The slice
// of the tokens' hidden vectors is read once into LDS (hs) and shared by the 4 waves; each
// wave holds its 16 W rows of the slice in registers (A operand: rows = output columns,
// B operand: the tokens), so a lane ends with 4 consecutive columns of one token.
__device__ __forceinline__ void proj_token_body(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W,
                                                int B, int d, int N, float* __restrict__ Pk, int xb, uint8_t* hs) {
  const int tid = threadIdx.x, l = static_cast<int>(lane_id()), wave = tid >> 6, g = l >> 4;
  const int n0 = xb * kPjCols + 16 * wave;
  const int slice = blockIdx.y, k0 = slice * kPjSlice;
  const int b0 = blockIdx.z * kPjTok;
  const int nblk = min(kPjSlice, d - k0) / kPjK;        // blocks of this slice (d % 128 == 0)
  // this wave's W rows: 4 blocks x 4 MFMA steps, 16 bytes per lane each (issued first)
  const uint16_t* wrow = W + static_cast<size_t>(min(n0 + (l & 15), N - 1)) * d + k0 + 8 * g;
  v8s wa[kPjSlice / kPjK][4];
#pragma unroll
  for (int jb = 0; jb < kPjSlice / kPjK; ++jb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      wa[jb][ks] = jb < nblk ? *reinterpret_cast<const v8s*>(wrow + jb * kPjK + 32 * ks) : v8s{};
  // the tokens' slice: 32 rows x 64 pieces of 16 bytes, 8 per thread
#pragma unroll
  for (int i = 0; i < kPjTok * 64 / (kPjWaves * 64); ++i) {
    const int q = tid + kPjWaves * 64 * i, tok = q >> 6, piece = q & 63;
    if (8 * piece < nblk * kPjK) {
      const uint4 v = *reinterpret_cast<const uint4*>(hidden + static_cast<size_t>(min(b0 + tok, B - 1)) * d + k0 +
                                                      8 * piece);
      *reinterpret_cast<uint4*>(&hs[tok * kPjStride + 16 * piece]) = v;
    }
  }
  __syncthreads();
  v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int jb = 0; jb < kPjSlice / kPjK; ++jb)
    if (jb < nblk)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const v8s hb = *reinterpret_cast<const v8s*>(&hs[(16 * tt + (l & 15)) * kPjStride +
                                                           2 * (jb * kPjK + 32 * ks + 8 * g)]);
          acc[tt] = mfma_bf16_16x16x32(wa[jb][ks], hb, acc[tt]);
        }
  // lane l: columns n0 + 4g .. +3 of token b0 + 16*tt + (l & 15)
  float* P = Pk + static_cast<size_t>(slice) * B * N;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int b = b0 + 16 * tt + (l & 15), n = n0 + 4 * g;
    if (b < B && n < N) *reinterpret_cast<v4f*>(P + static_cast<size_t>(b) * N + n) = acc[tt];
  }
}

// The projections of up to two compressors that read the same tokens (a CSA layer's main
// and indexer compressors), in one launch: column blocks [0, xb1) are job 0's, the rest
// job 1's.
struct ProjJobs {
  const uint16_t* W0;
  const uint16_t* W1;
  float* P0;
  float* P1;
  int N0, N1, xb1;
};

__global__ __launch_bounds__(kPjWaves * 64) void proj_token_bf16(const uint16_t* __restrict__ hidden, ProjJobs j,
                                                                 int B, int d) {
  __shared__ __attribute__((aligned(16))) uint8_t hs[kPjTok * kPjStride];
  const int xb = static_cast<int>(blockIdx.x);
  if (xb < j.xb1) proj_token_body(hidden, j.W0, B, d, j.N0, j.P0, xb, hs);
  else proj_token_body(hidden, j.W1, B, d, j.N1, j.P1, xb - j.xb1, hs);
}

// fp32 inputs (small shapes): one thread per (token, column).
__global__ __launch_bounds__(256) void proj_token_f32(const float* __restrict__ hidden, const float* __restrict__ W,
                                                      int B, int d, int N, float* __restrict__ P) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (n >= N) return;
  const float* h = hidden + static_cast<size_t>(b) * d;
  const float* w = W + static_cast<size_t>(n) * d;
  float acc = 0.0f;
  for (int k = 0; k < d; ++k) acc = fmaf(h[k], w[k], acc);
  P[static_cast<size_t>(b) * N + n] = acc;
}

struct StepArgs {
  const float* P;            // [n_slices, B, ns*c] partial projections of this call's tokens
  int n_slices;
  int B;
  const float* bias;         // [ns/2, m, c]
  const int64_t* pos;        // [B]
  float* state;              // ring [B, nslot, ns*c] or online [B, 3, c]
  int overlap, online, emit;
  int m, c, d_rope;
  double rope_r;             // theta^(-2/d_rope)
  float rms_eps;
  int out_dtype, out_layout, Nc_max;
  void* cache;
  float* cache_scale;
};

constexpr int kStepMaxSlots = 8;            // ring slots held in registers by the pooling (2m <= 8)
constexpr int kStepSliceGroup = 8;          // K-slice partials loaded together (16: no faster)

// Entry i of sequence b from its pooled pair (u0, u1) of thread p = threadIdx.x: RMSNorm over
// the c channels, RoPE at position m*i, the store (every thread of the workgroup calls it).
__device__ void emit_entry(const StepArgs& a, int b, int64_t i, float u0, float u1, bool live, float* red) {
  const int c = a.c, m = a.m;
  const int p = threadIdx.x;
  float u[2] = {u0, u1};
  // RMSNorm over the c channels
  float ss = live ? u[0] * u[0] + u[1] * u[1] : 0.f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
  if (lane_id() == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(c) + a.rms_eps);
  float x0 = u[0] * inv, x1 = u[1] * inv;
  const int pr = p - (c - a.d_rope) / 2;                // RoPE pair index
  if (live && pr >= 0) {
    float cs, sn;
    rope_cos_sin(m * i, pr, a.rope_r, cs, sn);
    const float y0 = fmaf(x0, cs, -x1 * sn), y1 = fmaf(x0, sn, x1 * cs);
    x0 = y0;
    x1 = y1;
  }
  const bool store = i < a.Nc_max;
  const size_t row = static_cast<size_t>(b) * a.Nc_max + static_cast<size_t>(i);
  if (a.out_dtype == CSA_F32) {
    if (live && store) reinterpret_cast<float2*>(static_cast<float*>(a.cache) + row * c)[p] = make_float2(x0, x1);
  } else if (a.out_dtype == CSA_BF16) {
    if (live && store) {
      const uint32_t v = static_cast<uint32_t>(f32_to_bf16(x0)) | (static_cast<uint32_t>(f32_to_bf16(x1)) << 16);
      reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.cache) + row * c)[p] = v;
    }
  } else if (a.out_dtype != CSA_FP8_E4M3) {
    store_entry_lowp(a.out_dtype, a.cache, reinterpret_cast<uint8_t*>(a.cache_scale), row, c, p, live && store, x0,
                     x1, red);
  } else {
    float am = live ? fmaxf(fabsf(x0), fabsf(x1)) : 0.f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, kWave));
    __syncthreads();
    if (lane_id() == 0) red[threadIdx.x >> 6] = am;
    __syncthreads();
    float amax = 0.f;
    for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) amax = fmaxf(amax, red[w]);
    const float scale = amax / 448.0f;
    if (live && store) {
      uint8_t c0 = 0, c1 = 0;
      if (scale > 0.f) {
        c0 = f32_to_e4m3(x0 / scale);
        c1 = f32_to_e4m3(x1 / scale);
      }
      uint8_t* dst;
      if (a.out_layout == CSA_LAYOUT_B16) {
        // block i/16 of the sequence, piece (2p)/32, entry i%16, byte (2p)%32
        const size_t nblk = static_cast<size_t>(cdiv(a.Nc_max, 16));
        dst = static_cast<uint8_t*>(a.cache) + (static_cast<size_t>(b) * nblk + static_cast<size_t>(i / 16)) * (16 * 128) +
              ((2 * p) >> 5) * 512 + static_cast<int>(i % 16) * 32 + ((2 * p) & 31);
      } else {
        dst = static_cast<uint8_t*>(a.cache) + row * c + 2 * p;
      }
      dst[0] = c0;
      dst[1] = c1;
    }
    if (threadIdx.x == 0 && store) a.cache_scale[row] = scale;
  }
}

// The 2m-slot softmax of a CSA entry from the ring in registers: ra = the ring half of this
// block (its a-streams; slot m - 1 is the token itself, in tok), rb = the previous block's
// half (its b-streams, pooled when bslots); slots in order a then b.
template <int kH>
__device__ __forceinline__ void pool_csa_ring(const float2 (&ra)[kH][4], const float2 (&rb)[kH][4],
                                              const float2 (&bza)[kH], const float2 (&bzb)[kH], const float2 (&tok)[4],
                                              int m, bool bslots, float (&u)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float za[kH], va[kH], zb[kH], vb[kH];
#pragma unroll
    for (int jr = 0; jr < kH; ++jr) {
      const float2 z2 = jr == m - 1 ? tok[1] : ra[jr][1], v2 = jr == m - 1 ? tok[0] : ra[jr][0];
      za[jr] = (h ? z2.y : z2.x) + (h ? bza[jr].y : bza[jr].x);
      va[jr] = h ? v2.y : v2.x;
      zb[jr] = (h ? rb[jr][3].y : rb[jr][3].x) + (h ? bzb[jr].y : bzb[jr].x);
      vb[jr] = h ? rb[jr][2].y : rb[jr][2].x;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int jr = 0; jr < kH; ++jr)
      if (jr < m) mx = fmaxf(mx, za[jr]);
    if (bslots)
#pragma unroll
      for (int jr = 0; jr < kH; ++jr)
        if (jr < m) mx = fmaxf(mx, zb[jr]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int jr = 0; jr < kH; ++jr)
      if (jr < m) {
        const float e = expf(za[jr] - mx);
        den += e;
        num = fmaf(e, va[jr], num);
      }
    if (bslots)
#pragma unroll
      for (int jr = 0; jr < kH; ++jr)
        if (jr < m) {
          const float e = expf(zb[jr] - mx);
          den += e;
          num = fmaf(e, vb[jr], num);
        }
    u[h] = num / den;
  }
}

__device__ __forceinline__ void compress_step_body(const StepArgs& a, int b, float* red) {
  const int c = a.c, m = a.m;
  const int ns = a.overlap ? 4 : 2;
  const int N = ns * c;
  const int nslot = a.overlap ? 2 * m : m;
  const int p = threadIdx.x;                            // channel pair (2p, 2p+1)
  const bool live = p < c / 2;
  const int64_t t = a.pos[b];
  // Everything that does not depend on the token's position is loaded before the position
  // is used, so one memory latency covers the position, the K-slice partials, the biases
  // and, for the CSA ring (overlap, m <= 4), the whole ring: at a block boundary the entry
  // pools every slot but the token's own (this block in one half of the ring, the previous
  // block in the other; which half follows from t mod 2m).
  const bool csa_ring = !a.online && a.overlap && m <= kStepMaxSlots / 2;
  constexpr int kH = kStepMaxSlots / 2;
  float2 rs0[kH][4], rs1[kH][4];                        // ring halves: [slot][stream]
  float2 bza[kH], bzb[kH];                              // logit biases of the a- and b-slots
  if (csa_ring && a.emit && live) {
    const float* ring = a.state + static_cast<size_t>(b) * nslot * N;
#pragma unroll
    for (int jr = 0; jr < kH; ++jr)
      if (jr < m)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          rs0[jr][st] = *reinterpret_cast<const float2*>(ring + static_cast<size_t>(jr) * N + st * c + 2 * p);
          rs1[jr][st] = *reinterpret_cast<const float2*>(ring + static_cast<size_t>(m + jr) * N + st * c + 2 * p);
        }
#pragma unroll
    for (int jr = 0; jr < kH; ++jr)
      if (jr < m) {
        bza[jr] = *reinterpret_cast<const float2*>(a.bias + jr * c + 2 * p);
        bzb[jr] = *reinterpret_cast<const float2*>(a.bias + (m + jr) * c + 2 * p);
      }
  }
  // this token's streams for the pair: the sum of the K slices (fixed order)
  float2 tok[4] = {make_float2(0.f, 0.f), make_float2(0.f, 0.f), make_float2(0.f, 0.f), make_float2(0.f, 0.f)};
  if (live) {
    // slices in groups of kStepSliceGroup with all their loads issued together (a loop over
    // single slices would wait for each one in turn); summed in slice order
    for (int s0 = 0; s0 < a.n_slices; s0 += kStepSliceGroup) {
      float2 v[kStepSliceGroup][4];
#pragma unroll
      for (int k = 0; k < kStepSliceGroup; ++k) {
        const float* Pb = a.P + (static_cast<size_t>(min(s0 + k, a.n_slices - 1)) * a.B + b) * N;
#pragma unroll
        for (int s = 0; s < 4; ++s) v[k][s] = s < ns ? *reinterpret_cast<const float2*>(Pb + s * c + 2 * p) : float2{};
      }
#pragma unroll
      for (int k = 0; k < kStepSliceGroup; ++k)
        if (s0 + k < a.n_slices)
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            tok[s].x += v[k][s].x;
            tok[s].y += v[k][s].y;
          }
    }
  }
  if (t < 0) return;
  const int r = static_cast<int>(t % m);                // slot of the token within its block
  const bool boundary = a.emit && r == m - 1;
  // The HCA ring (no overlap, m <= 8) at a boundary: the block's other slots and the biases,
  // loaded before this token's slot is written (never the same slot).
  const bool reg_pool = !a.online && (m <= kStepMaxSlots / 2 || (!a.overlap && m <= kStepMaxSlots));
  const int64_t i_e = t / m;
  float2 zc[kStepMaxSlots][2];                          // [slot][logit, value]
  if (!a.online && !a.overlap && boundary && live && reg_pool) {
    const float* ring = a.state + static_cast<size_t>(b) * nslot * N;
#pragma unroll
    for (int j = 0; j < kStepMaxSlots; ++j) {
      if (j < m) {
        const float2 bz = *reinterpret_cast<const float2*>(a.bias + j * c + 2 * p);
        if (j == m - 1) {
          zc[j][0] = bz;                                  // this token's logit is added below
          zc[j][1] = make_float2(0.f, 0.f);
        } else {
          const float* sl = ring + static_cast<size_t>((m * i_e + j) % nslot) * N;
          const float2 zz = *reinterpret_cast<const float2*>(sl + c + 2 * p);
          zc[j][0] = make_float2(zz.x + bz.x, zz.y + bz.y);
          zc[j][1] = *reinterpret_cast<const float2*>(sl + 2 * p);
        }
      }
    }
  }
  float u[2] = {0.f, 0.f};
  if (a.online) {
    float* st = a.state + static_cast<size_t>(b) * 3 * c;
    if (live) {
      const float2 bz = *reinterpret_cast<const float2*>(a.bias + r * c + 2 * p);
      const float z[2] = {tok[1].x + bz.x, tok[1].y + bz.y}, cv[2] = {tok[0].x, tok[0].y};
      float2 mo = make_float2(0.f, 0.f), so = mo, ao = mo;
      if (r != 0) {
        mo = *reinterpret_cast<const float2*>(st + 2 * p);
        so = *reinterpret_cast<const float2*>(st + c + 2 * p);
        ao = *reinterpret_cast<const float2*>(st + 2 * c + 2 * p);
      }
      const float mov[2] = {mo.x, mo.y}, sov[2] = {so.x, so.y}, aov[2] = {ao.x, ao.y};
      float mx[2], sm[2], acc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (r == 0) {
          mx[h] = z[h]; sm[h] = 1.0f; acc[h] = cv[h];
        } else {
          mx[h] = fmaxf(mov[h], z[h]);
          const float e_old = expf(mov[h] - mx[h]), e_new = expf(z[h] - mx[h]);
          sm[h] = sov[h] * e_old + e_new;
          acc[h] = fmaf(e_new, cv[h], aov[h] * e_old);
        }
        u[h] = acc[h] / sm[h];
      }
      *reinterpret_cast<float2*>(st + 2 * p) = make_float2(mx[0], mx[1]);
      *reinterpret_cast<float2*>(st + c + 2 * p) = make_float2(sm[0], sm[1]);
      *reinterpret_cast<float2*>(st + 2 * c + 2 * p) = make_float2(acc[0], acc[1]);
    }
  } else {
    float* ring = a.state + static_cast<size_t>(b) * nslot * N;
    const int my_slot = static_cast<int>(t % nslot);
    if (live) {
      float* slot = ring + static_cast<size_t>(my_slot) * N;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (s < ns) *reinterpret_cast<float2*>(slot + s * c + 2 * p) = tok[s];
    }
    if (boundary && live) {
      const int64_t i = t / m;
      const bool bslots = a.overlap && i > 0;
      // slots of block i (a-stream: C at stream 0, Z at stream 1) and, with overlap, of
      // block i-1 (b-stream: C at stream 2, Z at stream 3); this thread wrote every slot of
      // its channels, in this call or an earlier one.  Loaded first, then pooled.
      const int nsl = bslots ? 2 * m : m;
      if (csa_ring) {
        // this block's slots are the upper ring half when t mod 2m >= m (the same for the
        // whole workgroup: a branch, so that each arm reads its halves at fixed indices)
        if ((t % nslot) >= m) pool_csa_ring(rs1, rs0, bza, bzb, tok, m, bslots, u);
        else pool_csa_ring(rs0, rs1, bza, bzb, tok, m, bslots, u);
      } else if (reg_pool) {
        // the token's own slot (slot m - 1) joins the slots loaded at the start
#pragma unroll
        for (int j = 0; j < kStepMaxSlots; ++j)
          if (j == m - 1) {
            zc[j][0] = make_float2(tok[1].x + zc[j][0].x, tok[1].y + zc[j][0].y);
            zc[j][1] = tok[0];
          }
        float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
        for (int j = 0; j < kStepMaxSlots; ++j)
          if (j < nsl) { mx0 = fmaxf(mx0, zc[j][0].x); mx1 = fmaxf(mx1, zc[j][0].y); }
        float d0 = 0.f, d1 = 0.f, n0 = 0.f, n1 = 0.f;
#pragma unroll
        for (int j = 0; j < kStepMaxSlots; ++j)
          if (j < nsl) {
            const float e0 = expf(zc[j][0].x - mx0), e1 = expf(zc[j][0].y - mx1);
            d0 += e0; d1 += e1;
            n0 = fmaf(e0, zc[j][1].x, n0);
            n1 = fmaf(e1, zc[j][1].y, n1);
          }
        u[0] = n0 / d0;
        u[1] = n1 / d1;
      } else {
        // long blocks (HCA ring, m > 8): two passes over the slots in memory
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ch = 2 * p + h;
          float mx = -INFINITY;
          for (int j = 0; j < nsl; ++j) {
            const bool bs = j >= m;
            const int jr = bs ? j - m : j;
            const float* s = ring + static_cast<size_t>(((bs ? m * (i - 1) : m * i) + jr) % nslot) * N;
            mx = fmaxf(mx, s[(bs ? 3 : 1) * c + ch] + a.bias[((bs ? m : 0) + jr) * c + ch]);
          }
          float den = 0.f, num = 0.f;
          for (int j = 0; j < nsl; ++j) {
            const bool bs = j >= m;
            const int jr = bs ? j - m : j;
            const float* s = ring + static_cast<size_t>(((bs ? m * (i - 1) : m * i) + jr) % nslot) * N;
            const float e = expf(s[(bs ? 3 : 1) * c + ch] + a.bias[((bs ? m : 0) + jr) * c + ch] - mx);
            den += e;
            num = fmaf(e, s[(bs ? 2 : 0) * c + ch], num);
          }
          u[h] = num / den;
        }
      }
    }
  }
  if (!boundary) return;                                // uniform over the workgroup
  emit_entry(a, b, t / m, u[0], u[1], live, red);
}

// One workgroup per (compressor, sequence): workgroups [0, B0) run job 0, the rest job 1
// (a CSA layer's two compressors in one launch; threads beyond a job's c/2 only join its
// reductions).
struct StepJobs {
  StepArgs a0, a1;
  int B0;
};

__global__ __launch_bounds__(512) void compress_step(StepJobs j) {
  __shared__ float red[8];
  const int wg = static_cast<int>(blockIdx.x);
  if (wg < j.B0) compress_step_body(j.a0, wg, red);
  else compress_step_body(j.a1, wg - j.B0, red);
}

size_t compress_state_bytes(int B, int m, int c, int overlap, int online) {
  if (online) return static_cast<size_t>(B) * 3 * c * sizeof(float);
  const size_t nslot = overlap ? 2 * static_cast<size_t>(m) : static_cast<size_t>(m);
  return static_cast<size_t>(B) * nslot * (overlap ? 4 : 2) * c * sizeof(float);
}

// K slices of the bf16 projection (each summed by the step kernel); 1 for fp32 inputs.
static int proj_slices(int d, int in_dtype) { return in_dtype == CSA_BF16 ? cdiv(d, kPjSlice) : 1; }

size_t compress_decode_workspace_bytes(int B, int d, int c, int overlap, int in_dtype) {
  return static_cast<size_t>(proj_slices(d, in_dtype)) * B * (overlap ? 4 : 2) * c * sizeof(float);
}

using DecodeComp = csa_decode_compressor;

// One compressor's step arguments.
static StepArgs step_args(const DecodeComp& k, const float* P, int n_slices, int B, const int64_t* pos, int emit) {
  return StepArgs{P, n_slices, B, k.bias, pos, k.state, k.overlap, k.online, emit, k.m, k.c, k.d_rope,
                  rope_ratio(k.rope_theta, k.d_rope), k.rms_eps, k.out_dtype, k.out_layout, k.Nc_max, k.cache,
                  k.cache_scale};
}

// Compressor i's partial projections start at the 256-aligned end of those before it; the
// last one's size is exact (one compressor needs what csa_compress_decode_workspace_size says).
size_t compress_decode_many_workspace_bytes(int B, int d, int in_dtype, int n, const DecodeComp* comps) {
  size_t total = 0;
  for (int i = 0; i < n; ++i) {
    const size_t sz = compress_decode_workspace_bytes(B, d, comps[i].c, comps[i].overlap, in_dtype);
    total += i + 1 < n ? (sz + 255) / 256 * 256 : sz;
  }
  return total;
}

// n = 1 or 2 compressors over the same B tokens: bf16 inputs take one projection launch and
// one step launch for all of them; fp32 inputs run the compressors one after the other.
int launch_compress_decode_many(const void* hidden, int in_dtype, int B, int d, const int64_t* pos, int emit, int n,
                                const DecodeComp* comps, void* ws, hipStream_t st) {
  const int n_slices = proj_slices(d, in_dtype);
  float* P[2] = {nullptr, nullptr};
  int N[2] = {0, 0}, threads = kWave;
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    P[i] = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + off);
    off += (compress_decode_workspace_bytes(B, d, comps[i].c, comps[i].overlap, in_dtype) + 255) / 256 * 256;
    N[i] = (comps[i].overlap ? 4 : 2) * comps[i].c;
    threads = std::max(threads, cdiv(comps[i].c / 2, kWave) * kWave);
  }
  if (in_dtype != CSA_BF16) {
    for (int i = 0; i < n; ++i) {
      hipLaunchKernelGGL(proj_token_f32, dim3(cdiv(N[i], 256), B), dim3(256), 0, st, static_cast<const float*>(hidden),
                         static_cast<const float*>(comps[i].w_proj), B, d, N[i], P[i]);
      CSA_LAUNCH_CHECK();
      const StepArgs a = step_args(comps[i], P[i], n_slices, B, pos, emit);
      hipLaunchKernelGGL(compress_step, dim3(B), dim3(std::max(kWave, cdiv(comps[i].c / 2, kWave) * kWave)), 0, st,
                         StepJobs{a, a, B});
      CSA_LAUNCH_CHECK();
    }
    return CSA_OK;
  }
  const int xb0 = cdiv(N[0], kPjCols), xb_all = xb0 + (n > 1 ? cdiv(N[1], kPjCols) : 0);
  const ProjJobs pj{static_cast<const uint16_t*>(comps[0].w_proj),
                    static_cast<const uint16_t*>(comps[n > 1 ? 1 : 0].w_proj), P[0], P[n > 1 ? 1 : 0], N[0],
                    N[n > 1 ? 1 : 0], xb0};
  hipLaunchKernelGGL(proj_token_bf16, dim3(xb_all, n_slices, cdiv(B, kPjTok)), dim3(kPjWaves * 64), 0, st,
                     static_cast<const uint16_t*>(hidden), pj, B, d);
  CSA_LAUNCH_CHECK();
  const StepArgs a0 = step_args(comps[0], P[0], n_slices, B, pos, emit);
  const StepArgs a1 = n > 1 ? step_args(comps[1], P[1], n_slices, B, pos, emit) : a0;
  hipLaunchKernelGGL(compress_step, dim3(n * B), dim3(threads), 0, st, StepJobs{a0, a1, B});
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

}  // namespace csa
