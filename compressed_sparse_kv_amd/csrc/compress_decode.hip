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
//      the workspace).  bf16: v_mfma_f32_16x16x32_bf16 with M = the tokens (16 per tile),
//      N = 16 output columns per workgroup, K = d split over the 4 waves of the workgroup;
//      each lane streams 64 contiguous bytes of its W row per 128-wide K block (the same
//      permutation of the K slots on both operands, so the pairing is exact).  The weights
//      are read once per call: decode projection is bound by that stream.
//   2. compress_step: one workgroup per sequence, one thread per channel pair.  The
//      token's streams go into ring slot t mod 2m (or m), or update the online triple;
//      when (t + 1) % m == 0 entry i = t / m is pooled (per-channel softmax over the slots,
//      weighted sum), RMS-normalised, rotated (RoPE at position m*i, angle in double) and
//      written as fp32 / bf16 / e4m3 (+ row scale amax/448), row-major or, for the indexer
//      keys, straight into the 16-entry blocked layout the decode scoring pass reads.
#include <algorithm>

#include "common.hpp"

namespace csa {

constexpr int kPjK = 128;                   // K block: 4 MFMA steps of 32
constexpr int kPjWaves = 4;
constexpr int kPjMaxTiles = 8;              // token tiles of 16 per launch row (128 tokens)

// P[b, n0 + (l & 15)] for the tokens b of tile group blockIdx.y; W [N, d] bf16 ("out x in").
__global__ __launch_bounds__(kPjWaves * 64) void proj_token_bf16(const uint16_t* __restrict__ hidden,
                                                                 const uint16_t* __restrict__ W, int B, int d, int N,
                                                                 float* __restrict__ P) {
  __shared__ v4f red[kPjWaves - 1][kPjMaxTiles][64];
  const int l = static_cast<int>(lane_id());
  const int wave = threadIdx.x >> 6;
  const int g = l >> 4;
  const int n0 = blockIdx.x * 16;
  const int b0 = blockIdx.y * 16 * kPjMaxTiles;
  const int ntiles = min(kPjMaxTiles, cdiv(B - b0, 16));
  const int nblk = d / kPjK;
  const uint16_t* wrow = W + static_cast<size_t>(min(n0 + (l & 15), N - 1)) * d + 32 * g;
  v4f acc[kPjMaxTiles];
#pragma unroll
  for (int mt = 0; mt < kPjMaxTiles; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
  // hidden rows of this lane in every tile (clamped to the last token; extra rows unused)
  const uint16_t* hrow[kPjMaxTiles];
#pragma unroll
  for (int mt = 0; mt < kPjMaxTiles; ++mt)
    hrow[mt] = hidden + static_cast<size_t>(min(b0 + 16 * mt + (l & 15), B - 1)) * d + 32 * g;
  for (int j = wave; j < nblk; j += kPjWaves) {
    const size_t k0 = static_cast<size_t>(j) * kPjK;
    v8s wb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) wb[ks] = *reinterpret_cast<const v8s*>(wrow + k0 + 8 * ks);
#pragma unroll
    for (int mt = 0; mt < kPjMaxTiles; ++mt) {
      if (mt < ntiles) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const v8s ha = *reinterpret_cast<const v8s*>(hrow[mt] + k0 + 8 * ks);
          acc[mt] = mfma_bf16_16x16x32(ha, wb[ks], acc[mt]);
        }
      }
    }
  }
  // sum the waves' partial products (fixed order) and store: lane l holds tokens
  // 16*mt + 4*g + i of column n0 + (l & 15)
  if (wave > 0) {
#pragma unroll
    for (int mt = 0; mt < kPjMaxTiles; ++mt)
      if (mt < ntiles) red[wave - 1][mt][l] = acc[mt];
  }
  __syncthreads();
  if (wave != 0) return;
  const int n = n0 + (l & 15);
#pragma unroll
  for (int mt = 0; mt < kPjMaxTiles; ++mt) {
    if (mt >= ntiles) continue;
    v4f s = acc[mt];
#pragma unroll
    for (int w = 0; w < kPjWaves - 1; ++w) {
      const v4f x = red[w][mt][l];
      s[0] += x[0]; s[1] += x[1]; s[2] += x[2]; s[3] += x[3];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = b0 + 16 * mt + 4 * g + i;
      if (b < B && n < N) P[static_cast<size_t>(b) * N + n] = s[i];
    }
  }
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
  const float* P;            // [B, ns*c] this call's projections
  const float* bias;         // [ns/2, m, c]
  const int64_t* pos;        // [B]
  float* state;              // ring [B, nslot, ns*c] or online [B, 3, c]
  int overlap, online, emit;
  int m, c, d_rope;
  float rope_theta, rms_eps;
  int out_dtype, out_layout, Nc_max;
  void* cache;
  float* cache_scale;
};

__global__ __launch_bounds__(512) void compress_step(StepArgs a) {
  __shared__ float red[8];
  const int b = blockIdx.x;
  const int64_t t = a.pos[b];
  if (t < 0) return;
  const int c = a.c, m = a.m;
  const int ns = a.overlap ? 4 : 2;
  const int N = ns * c;
  const int nslot = a.overlap ? 2 * m : m;
  const int p = threadIdx.x;                            // channel pair (2p, 2p+1)
  const bool live = p < c / 2;
  const float* Pb = a.P + static_cast<size_t>(b) * N;
  const int r = static_cast<int>(t % m);                // slot of the token within its block
  const bool boundary = a.emit && r == m - 1;
  float u[2] = {0.f, 0.f};
  if (a.online) {
    float* st = a.state + static_cast<size_t>(b) * 3 * c;
    if (live) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ch = 2 * p + h;
        const float z = Pb[c + ch] + a.bias[r * c + ch], cv = Pb[ch];
        float mx, sm, acc;
        if (r == 0) {
          mx = z; sm = 1.0f; acc = cv;
        } else {
          const float mo = st[ch], so = st[c + ch], ao = st[2 * c + ch];
          mx = fmaxf(mo, z);
          const float e_old = expf(mo - mx), e_new = expf(z - mx);
          sm = so * e_old + e_new;
          acc = fmaf(e_new, cv, ao * e_old);
        }
        st[ch] = mx; st[c + ch] = sm; st[2 * c + ch] = acc;
        u[h] = acc / sm;
      }
    }
  } else {
    float* ring = a.state + static_cast<size_t>(b) * nslot * N;
    float* slot = ring + static_cast<size_t>(t % nslot) * N;
    if (live)
      for (int s = 0; s < ns; ++s) {
        slot[s * c + 2 * p] = Pb[s * c + 2 * p];
        slot[s * c + 2 * p + 1] = Pb[s * c + 2 * p + 1];
      }
    if (boundary && live) {
      const int64_t i = t / m;
      const bool bslots = a.overlap && i > 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ch = 2 * p + h;
        // this thread wrote every slot of its channels (in this and earlier calls)
        float mx = -INFINITY;
        for (int j = 0; j < m; ++j) {
          const float* s = ring + static_cast<size_t>((m * i + j) % nslot) * N;
          mx = fmaxf(mx, s[c + ch] + a.bias[j * c + ch]);
        }
        if (bslots)
          for (int j = 0; j < m; ++j) {
            const float* s = ring + static_cast<size_t>((m * (i - 1) + j) % nslot) * N;
            mx = fmaxf(mx, s[3 * c + ch] + a.bias[(m + j) * c + ch]);
          }
        float den = 0.f, num = 0.f;
        for (int j = 0; j < m; ++j) {
          const float* s = ring + static_cast<size_t>((m * i + j) % nslot) * N;
          const float e = expf(s[c + ch] + a.bias[j * c + ch] - mx);
          den += e;
          num = fmaf(e, s[ch], num);
        }
        if (bslots)
          for (int j = 0; j < m; ++j) {
            const float* s = ring + static_cast<size_t>((m * (i - 1) + j) % nslot) * N;
            const float e = expf(s[3 * c + ch] + a.bias[(m + j) * c + ch] - mx);
            den += e;
            num = fmaf(e, s[2 * c + ch], num);
          }
        u[h] = num / den;
      }
    }
  }
  if (!boundary) return;                                // uniform over the workgroup
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
  const int64_t i = t / m;
  const int pr = p - (c - a.d_rope) / 2;                // RoPE pair index
  if (live && pr >= 0) {
    const double ang = static_cast<double>(m * i) * pow(static_cast<double>(a.rope_theta), -2.0 * pr / a.d_rope);
    const double cs = cos(ang), sn = sin(ang);
    const double y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
    x0 = static_cast<float>(y0);
    x1 = static_cast<float>(y1);
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

size_t compress_state_bytes(int B, int m, int c, int overlap, int online) {
  if (online) return static_cast<size_t>(B) * 3 * c * sizeof(float);
  const size_t nslot = overlap ? 2 * static_cast<size_t>(m) : static_cast<size_t>(m);
  return static_cast<size_t>(B) * nslot * (overlap ? 4 : 2) * c * sizeof(float);
}

size_t compress_decode_workspace_bytes(int B, int c, int overlap) {
  return static_cast<size_t>(B) * (overlap ? 4 : 2) * c * sizeof(float);
}

int launch_compress_decode(const void* hidden, int in_dtype, const void* w_proj, const float* bias, int overlap,
                           int online, int B, int d, int m, int c, int d_rope, float rope_theta, float rms_eps,
                           const int64_t* pos, int emit, float* state, void* cache, float* cache_scale,
                           int out_dtype, int out_layout, int Nc_max, void* ws, hipStream_t st) {
  const int N = (overlap ? 4 : 2) * c;
  float* P = static_cast<float*>(ws);
  if (in_dtype == CSA_BF16) {
    const dim3 grid(cdiv(N, 16), cdiv(B, 16 * kPjMaxTiles));
    hipLaunchKernelGGL(proj_token_bf16, grid, dim3(kPjWaves * 64), 0, st, static_cast<const uint16_t*>(hidden),
                       static_cast<const uint16_t*>(w_proj), B, d, N, P);
  } else {
    hipLaunchKernelGGL(proj_token_f32, dim3(cdiv(N, 256), B), dim3(256), 0, st, static_cast<const float*>(hidden),
                       static_cast<const float*>(w_proj), B, d, N, P);
  }
  CSA_LAUNCH_CHECK();
  StepArgs a{P, bias, pos, state, overlap, online, emit, m, c, d_rope, rope_theta, rms_eps, out_dtype, out_layout,
             Nc_max, cache, cache_scale};
  const int threads = std::max(kWave, cdiv(c / 2, kWave) * kWave);
  hipLaunchKernelGGL(compress_step, dim3(B), dim3(threads), 0, st, a);
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

}  // namespace csa
