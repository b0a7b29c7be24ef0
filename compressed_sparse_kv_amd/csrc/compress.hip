// Block compressor (stage 1).
//
// [HCA-CSA] sections "压缩算子：逐通道 softmax 的软池化" (per-token C and Z from one linear
// map, position bias B, per-channel softmax over the block's slots, weighted sum, then
// RMSNorm and RoPE), "CSA 的重叠窗口" (entry i pools the a-stream of block i and the
// b-stream of block i-1: 2m slots, stride m; for i = 0 the b-slots are -inf / 0 padding)
// and "HCA：同一个算子，关掉重叠" (one stream, m slots).  [ATTN-CMP] section "CSA（DeepSeek-V4）":
// RoPE at the block's first position.
//
// Two kernels:
//   1. projection GEMM  P[r, :] = hidden_row(r) . w_proj^T  (fp32 result in the workspace;
//      bf16 inputs on MFMA v_mfma_f32_16x16x32_bf16, fp32 inputs on VALU), rows ordered
//      per sequence as [previous block (m rows, when given) | chunk (T rows)];
//   2. pooling: one workgroup per entry, one thread per channel pair (2p, 2p+1) so the
//      RoPE pair is thread-local; softmax per channel, block-wide RMS, RoPE with the
//      angle formed in double (positions reach 2^20 and beyond; rope_cos_sin), output
//      in fp32 / bf16 / e4m3 with the row scale amax/448.
#include <algorithm>

#include "common.hpp"
#include "entry_store.hpp"

namespace csa {

// ---------------------------------------------------------------------------------------
// bf16 MFMA GEMM, C[M,N] fp32 = A[M,K] . B[N,K]^T, K % 64 == 0.
// 128x128 tile, 4 waves in 2x2, each wave 64x64 (4x4 MFMA tiles), K step 64 via LDS
// (row stride 144 B).  A rows are gathered from (hidden_prev, hidden) per sequence.
// ---------------------------------------------------------------------------------------
constexpr int kGT = 128;
constexpr int kGK = 64;
constexpr int kGStride = kGK * 2 + 16;     // bytes per LDS row

struct GemmA {
  const uint16_t* hidden;
  const uint16_t* prev;      // may be null
  int T, m, d, rows_pb;      // rows per sequence in the projection buffer
};

__device__ __forceinline__ const uint16_t* a_row_bf16(const GemmA& A, int r) {
  const int bi = r / A.rows_pb, rr = r % A.rows_pb;
  if (A.prev) {
    if (rr < A.m) return A.prev + (static_cast<size_t>(bi) * A.m + rr) * A.d;
    return A.hidden + (static_cast<size_t>(bi) * A.T + rr - A.m) * A.d;
  }
  return A.hidden + (static_cast<size_t>(bi) * A.T + rr) * A.d;
}

__global__ __launch_bounds__(256) void proj_gemm_bf16(GemmA A, const uint16_t* __restrict__ Bw, int M, int N,
                                                      float* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) uint8_t la[2][kGT * kGStride];
  __shared__ __attribute__((aligned(16))) uint8_t lb[2][kGT * kGStride];
  const int tid = threadIdx.x, wave = tid >> 6, l = static_cast<int>(lane_id()), g = l >> 4;
  const int m0 = blockIdx.y * kGT, n0 = blockIdx.x * kGT;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int K = A.d;

  // loader: 128 rows x 128 bytes per operand = 16 KiB = 256 threads x 4 x 16 B
  // thread t moves row (t / 8) + 32*i, 16-byte piece t % 8
  const int lr = tid >> 3, lp = tid & 7;
  const uint16_t* arow[4];
  const uint16_t* brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    arow[i] = a_row_bf16(A, min(m0 + lr + 32 * i, M - 1));
    brow[i] = Bw + static_cast<size_t>(min(n0 + lr + 32 * i, N - 1)) * K;
  }
  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define CSA_GEMM_GLOAD(k0)                                                    \
  do {                                                                        \
    ra0 = *reinterpret_cast<const uint4*>(arow[0] + (k0) + 8 * lp);           \
    ra1 = *reinterpret_cast<const uint4*>(arow[1] + (k0) + 8 * lp);           \
    ra2 = *reinterpret_cast<const uint4*>(arow[2] + (k0) + 8 * lp);           \
    ra3 = *reinterpret_cast<const uint4*>(arow[3] + (k0) + 8 * lp);           \
    rb0 = *reinterpret_cast<const uint4*>(brow[0] + (k0) + 8 * lp);           \
    rb1 = *reinterpret_cast<const uint4*>(brow[1] + (k0) + 8 * lp);           \
    rb2 = *reinterpret_cast<const uint4*>(brow[2] + (k0) + 8 * lp);           \
    rb3 = *reinterpret_cast<const uint4*>(brow[3] + (k0) + 8 * lp);           \
  } while (0)
#define CSA_GEMM_SWRITE(buf)                                                                  \
  do {                                                                                        \
    *reinterpret_cast<uint4*>(&la[buf][(lr + 0) * kGStride + 16 * lp]) = ra0;                 \
    *reinterpret_cast<uint4*>(&la[buf][(lr + 32) * kGStride + 16 * lp]) = ra1;                \
    *reinterpret_cast<uint4*>(&la[buf][(lr + 64) * kGStride + 16 * lp]) = ra2;                \
    *reinterpret_cast<uint4*>(&la[buf][(lr + 96) * kGStride + 16 * lp]) = ra3;                \
    *reinterpret_cast<uint4*>(&lb[buf][(lr + 0) * kGStride + 16 * lp]) = rb0;                 \
    *reinterpret_cast<uint4*>(&lb[buf][(lr + 32) * kGStride + 16 * lp]) = rb1;                \
    *reinterpret_cast<uint4*>(&lb[buf][(lr + 64) * kGStride + 16 * lp]) = rb2;                \
    *reinterpret_cast<uint4*>(&lb[buf][(lr + 96) * kGStride + 16 * lp]) = rb3;                \
  } while (0)

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nk = K / kGK;
  CSA_GEMM_GLOAD(0);
  CSA_GEMM_SWRITE(0);
  __syncthreads();
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) CSA_GEMM_GLOAD((kt + 1) * kGK);
#pragma unroll
    for (int ks = 0; ks < kGK / 32; ++ks) {
      v8s af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const v8s*>(&la[buf][(wm + 16 * i + (l & 15)) * kGStride + 64 * ks + 16 * g]);
        bf[i] = *reinterpret_cast<const v8s*>(&lb[buf][(wn + 16 * i + (l & 15)) * kGStride + 64 * ks + 16 * g]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16_16x16x32(af[i], bf[j], acc[i][j]);
    }
    if (more) CSA_GEMM_SWRITE(buf ^ 1);
    __syncthreads();
  }
#undef CSA_GEMM_GLOAD
#undef CSA_GEMM_SWRITE
  // D tile (i, j): lane l holds rows 4*g + r, column l%16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn + 16 * j + (l & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm + 16 * i + 4 * g + r;
        if (row < M && col < N) C[static_cast<size_t>(row) * N + col] = acc[i][j][r];
      }
    }
}

// fp32 GEMM for small shapes: 16x16 output tile per 256 threads, K staged in 16-wide slabs.
__global__ __launch_bounds__(256) void proj_gemm_f32(const float* __restrict__ hidden, const float* __restrict__ prev,
                                                     int T, int m, int d, int rows_pb, const float* __restrict__ Bw,
                                                     int M, int N, float* __restrict__ C) {
  __shared__ float sa[16][17], sb[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int row = blockIdx.y * 16 + ty, col = blockIdx.x * 16 + tx;
  const int ra = min(blockIdx.y * 16 + tx, M - 1);     // loader roles
  const int bi = ra / rows_pb, rr = ra % rows_pb;
  const float* arow = prev ? (rr < m ? prev + (static_cast<size_t>(bi) * m + rr) * d
                                     : hidden + (static_cast<size_t>(bi) * T + rr - m) * d)
                           : hidden + (static_cast<size_t>(bi) * T + rr) * d;
  const float* brow = Bw + static_cast<size_t>(min(blockIdx.x * 16 + tx, N - 1)) * d;
  float acc = 0.0f;
  for (int k0 = 0; k0 < d; k0 += 16) {
    sa[tx][ty] = k0 + ty < d ? arow[k0 + ty] : 0.0f;
    sb[tx][ty] = k0 + ty < d ? brow[k0 + ty] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(sa[ty][kk], sb[tx][kk], acc);
    __syncthreads();
  }
  if (row < M && col < N) C[static_cast<size_t>(row) * N + col] = acc;
}

// ---------------------------------------------------------------------------------------
// Pooling + RMSNorm + RoPE (+ quantisation).  Grid (T/m, B); block = c/2 threads rounded
// up to whole waves (64 .. 512), one channel pair per thread.
// ---------------------------------------------------------------------------------------
struct PoolArgs {
  const float* P;            // projection [B*rows_pb, ns*c]
  const float* bias;         // [ns/2, m, c]
  int overlap, has_prev;
  int T, m, c, d_rope, rows_pb;
  double rope_r;             // theta^(-2/d_rope)
  float rms_eps;
  int64_t p0;
  int out_dtype;
  void* out;
  float* out_scale;
};

__global__ __launch_bounds__(512) void compress_pool(PoolArgs a) {
  __shared__ float red[8];
  const int i = blockIdx.x, b = blockIdx.y;
  const int ns = a.overlap ? 4 : 2;
  const int N = ns * a.c;
  const int off = a.has_prev ? a.m : 0;              // buffer row of chunk token 0
  const float* Pb = a.P + static_cast<size_t>(b) * a.rows_pb * N;
  const int npairs = a.c / 2;
  const int pidx = threadIdx.x;                        // channel pair handled by this thread
  const bool live = pidx < npairs;
  float u[2] = {0.f, 0.f};
  if (live) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = 2 * pidx + h;
      // slots: a-stream of block i, then (overlap) b-stream of block i-1
      float mx = -INFINITY;
      for (int j = 0; j < a.m; ++j) {
        const size_t r = static_cast<size_t>(off + a.m * i + j) * N;
        mx = fmaxf(mx, Pb[r + a.c + ch] + a.bias[j * a.c + ch]);
      }
      const bool bslots = a.overlap && (i > 0 || a.has_prev);
      if (bslots) {
        for (int j = 0; j < a.m; ++j) {
          const size_t r = static_cast<size_t>(off + a.m * (i - 1) + j) * N;
          mx = fmaxf(mx, Pb[r + 3 * a.c + ch] + a.bias[(a.m + j) * a.c + ch]);
        }
      }
      float den = 0.f, num = 0.f;
      for (int j = 0; j < a.m; ++j) {
        const size_t r = static_cast<size_t>(off + a.m * i + j) * N;
        const float e = expf(Pb[r + a.c + ch] + a.bias[j * a.c + ch] - mx);
        den += e;
        num = fmaf(e, Pb[r + ch], num);
      }
      if (bslots) {
        for (int j = 0; j < a.m; ++j) {
          const size_t r = static_cast<size_t>(off + a.m * (i - 1) + j) * N;
          const float e = expf(Pb[r + 3 * a.c + ch] + a.bias[(a.m + j) * a.c + ch] - mx);
          den += e;
          num = fmaf(e, Pb[r + 2 * a.c + ch], num);
        }
      }
      u[h] = num / den;
    }
  }
  // RMSNorm over the c channels
  float ss = u[0] * u[0] + u[1] * u[1];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
  if (lane_id() == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(a.c) + a.rms_eps);
  float x0 = u[0] * inv, x1 = u[1] * inv;
  // RoPE on the last d_rope channels, pair p = pidx - (c - d_rope)/2, position p0 + m*i
  const int p = pidx - (a.c - a.d_rope) / 2;
  if (live && p >= 0) {
    float cs, sn;
    rope_cos_sin(a.p0 + static_cast<int64_t>(a.m) * i, p, a.rope_r, cs, sn);
    const float y0 = fmaf(x0, cs, -x1 * sn), y1 = fmaf(x0, sn, x1 * cs);
    x0 = y0;
    x1 = y1;
  }
  const size_t orow = static_cast<size_t>(b) * (a.T / a.m) + i;
  if (a.out_dtype == CSA_F32) {
    if (live) reinterpret_cast<float2*>(static_cast<float*>(a.out) + orow * a.c)[pidx] = make_float2(x0, x1);
  } else if (a.out_dtype == CSA_BF16) {
    if (live) {
      const uint32_t v = static_cast<uint32_t>(f32_to_bf16(x0)) | (static_cast<uint32_t>(f32_to_bf16(x1)) << 16);
      reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + orow * a.c)[pidx] = v;
    }
  } else if (a.out_dtype != CSA_FP8_E4M3) {
    store_entry_lowp(a.out_dtype, a.out, reinterpret_cast<uint8_t*>(a.out_scale), orow, a.c, pidx, live, x0, x1, red);
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
    if (live) {
      uint8_t c0 = 0, c1 = 0;
      if (scale > 0.f) {
        c0 = f32_to_e4m3(x0 / scale);
        c1 = f32_to_e4m3(x1 / scale);
      }
      uint8_t* o8 = static_cast<uint8_t*>(a.out) + orow * a.c;
      o8[2 * pidx] = c0;
      o8[2 * pidx + 1] = c1;
    }
    if (threadIdx.x == 0) a.out_scale[orow] = scale;
  }
}

size_t compress_workspace_bytes(int B, int T, int m, int c, int overlap, int has_prev) {
  const size_t rows = static_cast<size_t>(B) * (T + (has_prev ? m : 0));
  return rows * (overlap ? 4 : 2) * static_cast<size_t>(c) * sizeof(float);
}

// P[B*rows_pb, N] = rows of (hidden_prev | hidden) . w^T: the projection GEMM alone (also
// used by the CSA2 compressor).
int launch_proj_gemm(const void* hidden, const void* hidden_prev, int in_dtype, const void* w, int B, int T, int m,
                     int d, int N, float* P, hipStream_t st) {
  const int has_prev = hidden_prev != nullptr;
  const int rows_pb = T + (has_prev ? m : 0);
  const int M = B * rows_pb;
  if (in_dtype == CSA_BF16) {
    GemmA A{static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(hidden_prev), T, m, d, rows_pb};
    dim3 grid(cdiv(N, kGT), cdiv(M, kGT));
    hipLaunchKernelGGL(proj_gemm_bf16, grid, dim3(256), 0, st, A, static_cast<const uint16_t*>(w), M, N, P);
  } else {
    dim3 grid(cdiv(N, 16), cdiv(M, 16));
    hipLaunchKernelGGL(proj_gemm_f32, grid, dim3(256), 0, st, static_cast<const float*>(hidden),
                       static_cast<const float*>(hidden_prev), T, m, d, rows_pb, static_cast<const float*>(w), M, N, P);
  }
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

int launch_compress(const void* hidden, const void* hidden_prev, int in_dtype, const void* w_proj, const float* bias,
                    int overlap, int B, int T, int d, int m, int c, int d_rope, float rope_theta, float rms_eps,
                    int64_t p0, void* out, float* out_scale, int out_dtype, void* ws, hipStream_t st) {
  const int has_prev = hidden_prev != nullptr;
  const int rows_pb = T + (has_prev ? m : 0);
  const int N = (overlap ? 4 : 2) * c;
  float* P = static_cast<float*>(ws);
  const int rc = launch_proj_gemm(hidden, hidden_prev, in_dtype, w_proj, B, T, m, d, N, P, st);
  if (rc != CSA_OK) return rc;
  PoolArgs pa{P, bias, overlap, has_prev, T, m, c, d_rope, rows_pb, rope_ratio(rope_theta, d_rope), rms_eps, p0,
              out_dtype, out, out_scale};
  const int threads = std::max(kWave, cdiv(c / 2, kWave) * kWave);
  hipLaunchKernelGGL(compress_pool, dim3(T / m, B), dim3(threads), 0, st, pa);
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

}  // namespace csa
