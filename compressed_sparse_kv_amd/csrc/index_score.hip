// Lightning-indexer scores (stage 2).
//
//   scores[b,s,j] = sum_h w[b,s,h] * ReLU(qI[b,s,h] . KI[b,j])   for j < n_vis(b,s), else -inf
//   n_vis = min(Nc, (q_pos + 1) / m)
// [HCA-CSA] section "CSA：轻压缩 + 稀疏选择" (indexer equations); [KV-COMP] sections 9.4
// (score = sum over heads of w * ReLU(q . z)) and 9.8 (entry j visible once t >= m*j+m-1).
//
// FP8 path.  With q = dec(q8)*sq and K = dec(k8)*sk and non-negative scales,
//   w * ReLU(sq*sk*dot) = sk * (w*sq) * ReLU(dot),   dot = dec(q8) . dec(k8),
// so the MFMA contracts the raw codes (exact products, fp32 accumulation), each head's
// partial is weighted by w' = w*sq after the ReLU, and the row scale sk multiplies once.
//
// MFMA mapping (v_mfma_f32_16x16x128_f8f6f4): M = 16 heads, N = 16 entries, K = d_I = 128
// in one instruction.  Output lane l of a 16x16 tile holds heads 4*(l/16)+i of entry l%16;
// a lane therefore weights-and-sums 16 heads of the 64 locally, and three cross-lane
// exchanges finish the head sum for 4 entry blocks at once (a reduce-scatter that leaves
// lane l holding entry e0+l of a 64-entry group, so stores are coalesced).
#include "common.hpp"

namespace csa {

constexpr int kIH = 64;    // indexer heads handled by the FP8 kernels
constexpr int kID = 128;   // indexer head dim handled by the FP8 kernels

// p[nb] = partial head-sum of entry (lane&15) of block nb over this lane's heads.
// Returns, in lane l, the full sum for entry 16*(l>>4) + (l&15) = l of the 4 blocks.
__device__ __forceinline__ float reduce_scatter4(const float p[4]) {
  const int g = static_cast<int>(lane_id()) >> 4;
  const bool lo = g < 2;
  const float s0 = lo ? p[2] : p[0], s1 = lo ? p[3] : p[1];
  const float k0 = lo ? p[0] : p[2], k1 = lo ? p[1] : p[3];
  const float q0 = k0 + wave_xor(s0, 32);
  const float q1 = k1 + wave_xor(s1, 32);
  const bool odd = g & 1;
  const float send = odd ? q0 : q1, keep = odd ? q1 : q0;
  return keep + wave_xor(send, 16);
}

// Weighted ReLU head-sum of one 16-entry block against the 4 head blocks of one query.
__device__ __forceinline__ float head_sum(const v8i a[4], const v8i& bk, const float wv[16]) {
  float acc = 0.0f;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    v4f d = {0.f, 0.f, 0.f, 0.f};
    d = mfma_fp8_16x16x128(a[hb], bk, d);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(wv[hb * 4 + i], fmaxf(d[i], 0.0f), acc);
  }
  return acc;
}

// Loads the A operand (64 heads x 128 codes of one query) and its head weights w*sq.
__device__ __forceinline__ void load_query(const uint8_t* __restrict__ q8, const float* __restrict__ qs,
                                           const float* __restrict__ w, size_t row, v8i a[4],
                                           float wv[16]) {
  const int l = static_cast<int>(lane_id());
  const uint8_t* qr = q8 + row * (kIH * kID);
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
    a[hb] = *reinterpret_cast<const v8i*>(qr + (16 * hb + (l & 15)) * kID + 32 * (l >> 4));
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * hb + 4 * (l >> 4) + i;
      wv[hb * 4 + i] = w[row * kIH + h] * qs[row * kIH + h];
    }
}

// ------------------------------------------------------------------------------------
// Decode: few queries per sequence.  Each wave streams 64-entry groups of its sequence's
// K straight from HBM into MFMA operand registers (one 128-byte row = one cache line,
// read by 4 lanes x 32 bytes); the next group's loads are in flight while the current
// group is multiplied.  Grid: (ceil(Nc / kDecEntWG), B*S).
// ------------------------------------------------------------------------------------
constexpr int kDecGroups = 4;                         // 64-entry groups per wave
constexpr int kDecEntWG = 4 * 64 * kDecGroups;        // entries per workgroup

__global__ __launch_bounds__(256) void index_score_fp8_decode(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, const int64_t* __restrict__ q_pos,
    int S, int Nc, int m, float* __restrict__ scores) {
  const size_t row = blockIdx.y;
  const int b = static_cast<int>(row / S);
  const int l = static_cast<int>(lane_id());
  const int wave = threadIdx.x >> 6;
  const int64_t t = q_pos[row];
  const int nvis = static_cast<int>(min(static_cast<int64_t>(Nc), (t + 1) / m));

  v8i a[4];
  float wv[16];
  load_query(q8, qs, w, row, a, wv);

  const uint8_t* kb = k8 + static_cast<size_t>(b) * Nc * kID;
  const float* ksb = ks + static_cast<size_t>(b) * Nc;
  float* out = scores + row * Nc;

  // group gi of this wave covers entries e0 = base + 64*(gi*4 + wave) .. +63
  const int base = blockIdx.x * kDecEntWG;
  auto load_group = [&](int e0, v8i bk[4]) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int e = min(e0 + 16 * nb + (l & 15), Nc - 1);
      bk[nb] = *reinterpret_cast<const v8i*>(kb + static_cast<size_t>(e) * kID + 32 * (l >> 4));
    }
  };

  v8i cur[4], nxt[4];
  int e0 = base + 64 * wave;
  if (e0 < Nc && e0 < nvis) load_group(e0, cur);
#pragma unroll 1
  for (int gi = 0; gi < kDecGroups; ++gi) {
    e0 = base + 64 * (gi * 4 + wave);
    if (e0 >= Nc) break;
    const int e1 = e0 + 256;
    const bool more = gi + 1 < kDecGroups && e1 < Nc && e1 < nvis;
    if (more) load_group(e1, nxt);
    const int e = e0 + l;
    if (e0 < nvis) {
      float p[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) p[nb] = head_sum(a, cur[nb], wv);
      const float v = reduce_scatter4(p);
      if (e < Nc) out[e] = e < nvis ? v * ksb[e] : -INFINITY;
    } else if (e < Nc) {
      out[e] = -INFINITY;
    }
    if (more) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) cur[nb] = nxt[nb];
    }
  }
}

// ------------------------------------------------------------------------------------
// Prefill: many queries per sequence.  A workgroup owns kPfQ queries (2 per wave, A
// operands resident in registers) and walks the entry axis in tiles of kPfTile entries
// staged in LDS (row stride 144 B: the 16 rows one MFMA operand read touches fall in
// distinct banks).  Tiles beyond every query's visible range are written as -inf
// without touching K.  Grid: (ceil(S / kPfQ), B).
// ------------------------------------------------------------------------------------
constexpr int kPfQW = 2;                 // queries per wave
constexpr int kPfQ = 4 * kPfQW;          // queries per workgroup
constexpr int kPfTile = 64;              // entries per LDS tile
constexpr int kPfStride = kID + 16;      // LDS row stride in bytes

__global__ __launch_bounds__(256) void index_score_fp8_prefill(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, const int64_t* __restrict__ q_pos,
    int S, int Nc, int m, float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kPfTile * kPfStride];
  const int b = blockIdx.y;
  const int s0 = blockIdx.x * kPfQ;
  const int l = static_cast<int>(lane_id());
  const int wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;

  // this wave's queries (clamped duplicates of the last one are computed, never stored)
  v8i a[kPfQW][4];
  float wv[kPfQW][16];
  int nvis[kPfQW];
  int qrow[kPfQW];
  bool qlive[kPfQW];
#pragma unroll
  for (int j = 0; j < kPfQW; ++j) {
    const int s = s0 + wave * kPfQW + j;
    qlive[j] = s < S;
    const size_t row = static_cast<size_t>(b) * S + min(s, S - 1);
    qrow[j] = static_cast<int>(row);
    load_query(q8, qs, w, row, a[j], wv[j]);
    const int64_t t = q_pos[row];
    nvis[j] = static_cast<int>(min(static_cast<int64_t>(Nc), (t + 1) / m));
  }
  // the workgroup's visible bound (max over its queries) decides which tiles are computed
  int wg_vis = 0;
  for (int s = s0; s < min(S, s0 + kPfQ); ++s) {
    const int64_t t = q_pos[static_cast<size_t>(b) * S + s];
    wg_vis = max(wg_vis, static_cast<int>(min(static_cast<int64_t>(Nc), (t + 1) / m)));
  }

  const uint8_t* kb = k8 + static_cast<size_t>(b) * Nc * kID;
  const float* ksb = ks + static_cast<size_t>(b) * Nc;
  const int ntiles_vis = cdiv(wg_vis, kPfTile);
  const int ntiles = cdiv(Nc, kPfTile);

  // cooperative tile load: thread t copies 32 bytes of entry t/4
  const int le = tid >> 2, lb = 32 * (tid & 3);
  auto gload = [&](int ti, uint4& x0, uint4& x1) {
    const int e = min(ti * kPfTile + le, Nc - 1);
    const uint4* src = reinterpret_cast<const uint4*>(kb + static_cast<size_t>(e) * kID + lb);
    x0 = src[0];
    x1 = src[1];
  };
  auto swrite = [&](int buf, const uint4& x0, const uint4& x1) {
    uint4* dst = reinterpret_cast<uint4*>(&tile[buf][le * kPfStride + lb]);
    dst[0] = x0;
    dst[1] = x1;
  };

  uint4 x0, x1;
  if (ntiles_vis > 0) {
    gload(0, x0, x1);
    swrite(0, x0, x1);
  }
  __syncthreads();
#pragma unroll 1
  for (int ti = 0; ti < ntiles_vis; ++ti) {
    const int buf = ti & 1;
    const bool more = ti + 1 < ntiles_vis;
    if (more) gload(ti + 1, x0, x1);
    const int e0 = ti * kPfTile;
    v8i bk[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      bk[nb] = *reinterpret_cast<const v8i*>(&tile[buf][(16 * nb + (l & 15)) * kPfStride + 32 * (l >> 4)]);
    const int e = e0 + l;
    const float sk = e < Nc ? ksb[e] : 0.0f;
#pragma unroll
    for (int j = 0; j < kPfQW; ++j) {
      float p[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) p[nb] = head_sum(a[j], bk[nb], wv[j]);
      const float v = reduce_scatter4(p);
      if (qlive[j] && e < Nc) scores[static_cast<size_t>(qrow[j]) * Nc + e] = e < nvis[j] ? v * sk : -INFINITY;
    }
    if (more) swrite(buf ^ 1, x0, x1);
    __syncthreads();
  }
  // tiles no query of this workgroup can see
  for (int ti = ntiles_vis; ti < ntiles; ++ti) {
    const int e = ti * kPfTile + l;
#pragma unroll
    for (int j = 0; j < kPfQW; ++j)
      if (qlive[j] && e < Nc) scores[static_cast<size_t>(qrow[j]) * Nc + e] = -INFINITY;
  }
}

// ------------------------------------------------------------------------------------
// fp32 path (small shapes): one thread per (query, entry), heads and dims looped.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void index_score_f32(
    const float* __restrict__ q, const float* __restrict__ w, const float* __restrict__ k,
    const int64_t* __restrict__ q_pos, int S, int H, int D, int Nc, int m, float* __restrict__ scores) {
  extern __shared__ float qsh[];                 // H*D query values + H weights
  const size_t row = blockIdx.y;
  const int b = static_cast<int>(row / S);
  for (int i = threadIdx.x; i < H * D; i += blockDim.x) qsh[i] = q[row * H * D + i];
  for (int i = threadIdx.x; i < H; i += blockDim.x) qsh[H * D + i] = w[row * H + i];
  __syncthreads();
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= Nc) return;
  const int64_t t = q_pos[row];
  const int nvis = static_cast<int>(min(static_cast<int64_t>(Nc), (t + 1) / m));
  float out = -INFINITY;
  if (e < nvis) {
    const float* kr = k + (static_cast<size_t>(b) * Nc + e) * D;
    float acc = 0.0f;
    for (int h = 0; h < H; ++h) {
      float dot = 0.0f;
      for (int d = 0; d < D; ++d) dot = fmaf(qsh[h * D + d], kr[d], dot);
      acc = fmaf(qsh[H * D + h], fmaxf(dot, 0.0f), acc);
    }
    out = acc;
  }
  scores[row * Nc + e] = out;
}

int launch_index_score(const void* q, const float* q_scale, const float* w, const void* k,
                       const float* k_scale, int dtype, const int64_t* q_pos, int B, int S,
                       int H_I, int d_I, int Nc, int m, float* scores, hipStream_t st) {
  if (dtype == CSA_FP8_E4M3) {
    if (S <= 4) {
      dim3 grid(cdiv(Nc, kDecEntWG), B * S);
      hipLaunchKernelGGL(index_score_fp8_decode, grid, dim3(256), 0, st,
                         static_cast<const uint8_t*>(q), q_scale, w, static_cast<const uint8_t*>(k),
                         k_scale, q_pos, S, Nc, m, scores);
    } else {
      dim3 grid(cdiv(S, kPfQ), B);
      hipLaunchKernelGGL(index_score_fp8_prefill, grid, dim3(256), 0, st,
                         static_cast<const uint8_t*>(q), q_scale, w, static_cast<const uint8_t*>(k),
                         k_scale, q_pos, S, Nc, m, scores);
    }
  } else {
    dim3 grid(cdiv(Nc, 256), B * S);
    const size_t shm = sizeof(float) * (static_cast<size_t>(H_I) * d_I + H_I);
    hipLaunchKernelGGL(index_score_f32, grid, dim3(256), shm, st, static_cast<const float*>(q), w,
                       static_cast<const float*>(k), q_pos, S, H_I, d_I, Nc, m, scores);
  }
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

}  // namespace csa
