// CSA2 compressor (DeepSeek-V4.1): one stream, no position bias, indexer key from the main KV.
//
// [V4-CSA2] sections 6.1 and 7.2 (one KV projection and one gate; entry i pools only its
// own m-token block: per channel a softmax over the block's gate values weights the block's
// KV values; no block-slot bias), 7.5 and 15.1 (ratio 1: no gate, the entry is the
// normalised projection), 6.2 (the indexer key is a projection of the main KV latent, not
// a second compressor) and 7.4 (RoPE at the block's first token); [ATTN-CMP] section on
// CSA2 (the latent before RoPE feeds wk, then k_norm and RoPE with the indexer's theta).
//
// Kernels: the projection GEMM of the prefill compressor (P = hidden . [W_kv | W_gate]^T,
// fp32 in the workspace), then csa2_pool with one workgroup per entry: thread p pools the
// channel pair (2p, 2p+1) over the block, the block-wide RMS gives the latent, which stays
// in LDS; the main entry is the latent rotated on its last d_rope channels; thread j then
// forms indexer channel j as the dot product of the latent with row j of W_k (d_I x c,
// read from L2), the block-wide RMS over d_I normalises it, and thread q rotates and
// stores the indexer pair (2q, 2q+1).
#include <algorithm>

#include "common.hpp"
#include "entry_store.hpp"

namespace csa {

int launch_proj_gemm(const void* hidden, const void* hidden_prev, int in_dtype, const void* w, int B, int T, int m,
                     int d, int N, float* P, hipStream_t st);

struct Csa2Args {
  const float* P;            // [B*T, ng*c]: C (and Z when ng == 2) of every token
  const void* w_k;           // [d_I, c], in_dtype
  int in_dtype;
  int T, m, c, dI, ng, d_rope;
  double r_kv, r_k;          // theta^(-2/d_rope) of the main KV and of the indexer key
  float rms_eps;
  int64_t p0;
  void* kv;                  // [B, T/m, c]
  float* kv_scale;
  int kv_dtype;
  void* kI;                  // [B, T/m, d_I]
  float* kI_scale;
  int kI_dtype;
};

// Block-wide sum over the threads of the workgroup (every thread gets it).
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  __syncthreads();
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) t += red[w];
  return t;
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  __syncthreads();
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) t = fmaxf(t, red[w]);
  return t;
}

// Stores the channel pair (2p, 2p+1) of row `row` (n channels) in dtype; FP8 and the
// low-precision types need reductions (every thread of the workgroup calls this, live or not).
__device__ __forceinline__ void store_pair(void* out, float* out_scale, int dtype, size_t row, int n, int p, bool live,
                                           float x0, float x1, float* red) {
  if (dtype == CSA_F32) {
    if (live) reinterpret_cast<float2*>(static_cast<float*>(out) + row * n)[p] = make_float2(x0, x1);
  } else if (dtype == CSA_BF16) {
    if (live) {
      const uint32_t v = static_cast<uint32_t>(f32_to_bf16(x0)) | (static_cast<uint32_t>(f32_to_bf16(x1)) << 16);
      reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + row * n)[p] = v;
    }
  } else if (dtype != CSA_FP8_E4M3) {
    store_entry_lowp(dtype, out, reinterpret_cast<uint8_t*>(out_scale), row, n, p, live, x0, x1, red);
  } else {
    const float amax = block_max(live ? fmaxf(fabsf(x0), fabsf(x1)) : 0.f, red);
    const float scale = amax / 448.0f;
    if (live) {
      uint8_t c0 = 0, c1 = 0;
      if (scale > 0.f) {
        c0 = f32_to_e4m3(x0 / scale);
        c1 = f32_to_e4m3(x1 / scale);
      }
      uint8_t* o8 = static_cast<uint8_t*>(out) + row * n;
      o8[2 * p] = c0;
      o8[2 * p + 1] = c1;
    }
    if (threadIdx.x == 0) out_scale[row] = scale;
  }
}

__global__ __launch_bounds__(512) void csa2_pool(Csa2Args a) {
  __shared__ float lat[1024];
  __shared__ float kk[256];
  __shared__ float red[8];
  const int i = blockIdx.x, b = blockIdx.y;
  const int c = a.c, m = a.m, N = a.ng * c;
  const int p = threadIdx.x;
  const bool live = p < c / 2;
  const float* Pb = a.P + (static_cast<size_t>(b) * a.T + static_cast<size_t>(m) * i) * N;
  // ---- pooled pair of the main latent
  float u0 = 0.f, u1 = 0.f;
  if (live) {
    if (a.ng == 1) {                                       // ratio 1, no gate
      const float2 v = *reinterpret_cast<const float2*>(Pb + 2 * p);
      u0 = v.x;
      u1 = v.y;
    } else {
      float mx0 = -INFINITY, mx1 = -INFINITY;
      for (int r = 0; r < m; ++r) {
        const float2 z = *reinterpret_cast<const float2*>(Pb + static_cast<size_t>(r) * N + c + 2 * p);
        mx0 = fmaxf(mx0, z.x);
        mx1 = fmaxf(mx1, z.y);
      }
      float d0 = 0.f, d1 = 0.f, n0 = 0.f, n1 = 0.f;
      for (int r = 0; r < m; ++r) {
        const float2 z = *reinterpret_cast<const float2*>(Pb + static_cast<size_t>(r) * N + c + 2 * p);
        const float2 v = *reinterpret_cast<const float2*>(Pb + static_cast<size_t>(r) * N + 2 * p);
        const float e0 = expf(z.x - mx0), e1 = expf(z.y - mx1);
        d0 += e0; d1 += e1;
        n0 = fmaf(e0, v.x, n0);
        n1 = fmaf(e1, v.y, n1);
      }
      u0 = n0 / d0;
      u1 = n1 / d1;
    }
  }
  const float inv = 1.0f / sqrtf(block_sum(u0 * u0 + u1 * u1, red) / static_cast<float>(c) + a.rms_eps);
  float x0 = u0 * inv, x1 = u1 * inv;
  if (live) {
    lat[2 * p] = x0;
    lat[2 * p + 1] = x1;
  }
  const int64_t pos = a.p0 + static_cast<int64_t>(m) * i;
  const int pr = p - (c - a.d_rope) / 2;
  if (live && pr >= 0) {
    float cs, sn;
    rope_cos_sin(pos, pr, a.r_kv, cs, sn);
    const float y0 = fmaf(x0, cs, -x1 * sn), y1 = fmaf(x0, sn, x1 * cs);
    x0 = y0;
    x1 = y1;
  }
  const size_t row = static_cast<size_t>(b) * (a.T / m) + i;
  store_pair(a.kv, a.kv_scale, a.kv_dtype, row, c, p, live, x0, x1, red);
  __syncthreads();                                         // the latent is in LDS
  // ---- indexer key: latent . W_k^T, then k_norm over d_I
  const int j = threadIdx.x;
  float kj = 0.f;
  if (j < a.dI) {
    if (a.in_dtype == CSA_BF16) {
      const uint16_t* wr = static_cast<const uint16_t*>(a.w_k) + static_cast<size_t>(j) * c;
      for (int ch = 0; ch < c; ch += 8) {
        const uint4 w8 = *reinterpret_cast<const uint4*>(wr + ch);
        const uint32_t ws[4] = {w8.x, w8.y, w8.z, w8.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          kj = fmaf(lat[ch + 2 * q], __uint_as_float(ws[q] << 16), kj);
          kj = fmaf(lat[ch + 2 * q + 1], __uint_as_float(ws[q] & 0xffff0000u), kj);
        }
      }
    } else {
      const float* wr = static_cast<const float*>(a.w_k) + static_cast<size_t>(j) * c;
      for (int ch = 0; ch < c; ++ch) kj = fmaf(lat[ch], wr[ch], kj);
    }
  }
  const float kinv = 1.0f / sqrtf(block_sum(kj * kj, red) / static_cast<float>(a.dI) + a.rms_eps);
  if (j < a.dI) kk[j] = kj * kinv;
  __syncthreads();
  const bool klive = p < a.dI / 2;
  float k0 = klive ? kk[2 * p] : 0.f, k1 = klive ? kk[2 * p + 1] : 0.f;
  const int pk = p - (a.dI - a.d_rope) / 2;
  if (klive && pk >= 0) {
    float cs, sn;
    rope_cos_sin(pos, pk, a.r_k, cs, sn);
    const float y0 = fmaf(k0, cs, -k1 * sn), y1 = fmaf(k0, sn, k1 * cs);
    k0 = y0;
    k1 = y1;
  }
  store_pair(a.kI, a.kI_scale, a.kI_dtype, row, a.dI, p, klive, k0, k1, red);
}

size_t csa2_workspace_bytes(int B, int T, int m, int c) {
  return static_cast<size_t>(B) * T * (m > 1 ? 2 : 1) * c * sizeof(float);
}

int launch_csa2_compress(const void* hidden, int in_dtype, const void* w_proj, const void* w_k, int B, int T, int d,
                         int m, int c, int dI, int d_rope, float theta_kv, float theta_k, float rms_eps, int64_t p0,
                         void* kv, float* kv_scale, int kv_dtype, void* kI, float* kI_scale, int kI_dtype, void* ws,
                         hipStream_t st) {
  const int ng = m > 1 ? 2 : 1;
  float* P = static_cast<float*>(ws);
  const int rc = launch_proj_gemm(hidden, nullptr, in_dtype, w_proj, B, T, m, d, ng * c, P, st);
  if (rc != CSA_OK) return rc;
  Csa2Args a{P, w_k, in_dtype, T, m, c, dI, ng, d_rope, rope_ratio(theta_kv, d_rope), rope_ratio(theta_k, d_rope),
             rms_eps, p0, kv, kv_scale, kv_dtype, kI, kI_scale, kI_dtype};
  const int threads = std::max(kWave, cdiv(std::max(c / 2, dI), kWave) * kWave);
  hipLaunchKernelGGL(csa2_pool, dim3(T / m, B), dim3(threads), 0, st, a);
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

}  // namespace csa
