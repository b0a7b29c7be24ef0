// Core attention (stage 4): shared-KV MQA over [SWA window || compressed entries || sink].
//
// For query (b,s) and head h over its row set E (window rows, then remote rows):
//   l_e = scale * (q_h . kv_e);  M = max(sink_h, max_e l_e)
//   o_h = sum_e exp(l_e - M) kv_e / (exp(sink_h - M) + sum_e exp(l_e - M)),  lse = M + log(den)
// [HCA-CSA] section "设计：近处看原文，远处看摘要" (one softmax over the three segments;
// the sink only in the denominator; K = V, one KV head for all query heads);
// [KV-COMP] sections 9.5-9.6 (window indices concatenated with the remote indices; the
// kernel gathers only the rows the indices name).  CSA: remote rows = kv_comp[idx];
// HCA ("HCA：重压缩 + 全量"): remote rows = every visible entry.
//
// bf16 kernel (H = 64 heads, c = 512).  A workgroup (4 waves, 16 heads each) owns one
// query and a contiguous range of row chunks, so every gathered KV row is read from HBM
// once for all 64 heads.  Per chunk of kRows rows:
//   1. the rows are staged in LDS, row stride 1072 B (rows shift by 12 banks: the 16
//      rows of a 16-byte operand read and the 4 rows of a transposed read never share
//      a bank);
//   2. S^T = KV_chunk . Q^T on MFMA (A = rows from LDS, B = the wave's Q in registers);
//      the output layout of S^T (lane: head l%16, rows 4*(l/16)+i) is exactly the
//      A-operand layout P needs below, so P never leaves registers;
//   3. online softmax in the log2 domain (running max and sum per head);
//   4. O += P . V on MFMA with V read from the same LDS rows (K = V) through the LDS
//      transpose read ds_read_b64_tr_b16: in each 16-lane group, output lane i' slot j'
//      receives input lane 4j'+i'/4 slot i'%4, so lanes 4j'..4j'+3 reading 16 columns of
//      row R(j') hand every lane its column of 4 rows.  P enters as a bf16 hi + lo pair
//      (two MFMAs on one V operand) so it keeps ~16 bits.
// Several workgroups may split one query's rows; they write (m, l, O) partials and
// attn_merge combines them with the sink (LSE merge).
#include <algorithm>

#include "common.hpp"

namespace csa {

constexpr int kAH = 64;
constexpr int kAC = 512;
constexpr int kRows = 32;
constexpr int kMaxSplitSlots = 4096;              // selected entries staged per workgroup
constexpr int kRowStride = kAC * 2 + 48;          // bytes
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* idx;
  const int64_t* q_pos;
  const uint16_t* swa;
  const float* sink;
  float scale_log2;          // scale * log2(e)
  int S, Nc, k, Ls, W, m;
  int nsplit, chunks_per_split;
  uint16_t* out;
  float* lse;
  float* part_o;             // [B*S, nsplit, H, c] fp32, unnormalised
  float* part_ml;            // [B*S, nsplit, H, 2]: running max (log2 units), sum
};

// Window rows of query s: [w_lo, w_hi] of the sequence's swa tensor.
__device__ __forceinline__ void window_rows(int s, int S, int Ls, int W, int& w_lo, int& n_swa) {
  const int w_hi = s + Ls - S;
  w_lo = max(0, w_hi - W + 1);
  n_swa = w_hi - w_lo + 1;
}

template <bool kDense>
__global__ __launch_bounds__(256) void attn_bf16(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t rows_lds[kRows * kRowStride];
  __shared__ int valid_lds[kRows];
  __shared__ int sel_lds[kMaxSplitSlots];
  const int qi = blockIdx.y;
  const int split = blockIdx.x;
  const int b = qi / a.S, s = qi % a.S;
  const int wave = threadIdx.x >> 6;
  const int l = static_cast<int>(lane_id());
  const int g = l >> 4;

  int w_lo, n_swa;
  window_rows(s, a.S, a.Ls, a.W, w_lo, n_swa);
  const int n_rem = kDense ? static_cast<int>(min(static_cast<int64_t>(a.Nc), (a.q_pos[qi] + 1) / a.m)) : a.k;
  const int n_slots = n_swa + n_rem;
  const int n_chunks = cdiv(n_slots, kRows);
  const int ch0 = split * a.chunks_per_split;
  const int ch1 = min(n_chunks, ch0 + a.chunks_per_split);

  const uint16_t* kvb = a.kv + static_cast<size_t>(b) * a.Nc * kAC;
  const uint16_t* swab = a.swa + static_cast<size_t>(b) * a.Ls * kAC;
  // CSA: this split's selected entries, staged once in LDS so the row loads of a chunk
  // can be issued back to back (no index load between them)
  const int slot0 = ch0 * kRows;
  if (!kDense) {
    const int32_t* idxq = a.idx + static_cast<size_t>(qi) * a.k;
    const int r0 = max(0, slot0 - n_swa);
    const int r1 = min(a.k, ch1 * kRows - n_swa);
    for (int r = r0 + static_cast<int>(threadIdx.x); r < r1; r += 256) sel_lds[r - r0] = idxq[r];
    __syncthreads();
  }
  // slot -> row pointer, nullptr for padding / an absent (-1) index
  auto slot_row = [&](int slot) -> const uint16_t* {
    if (slot >= n_slots) return nullptr;
    if (slot < n_swa) return swab + static_cast<size_t>(w_lo + slot) * kAC;
    const int r = slot - n_swa;
    const int j = kDense ? r : sel_lds[r - max(0, slot0 - n_swa)];
    if (j < 0 || j >= a.Nc) return nullptr;
    return kvb + static_cast<size_t>(j) * kAC;
  };

  // staging: round r moves chunk row 4*r + wave, 16 bytes per lane
  uint4 stage[kRows / 4];
  int stage_ok[kRows / 4];
  auto gload = [&](int ch) {
#pragma unroll
    for (int r = 0; r < kRows / 4; ++r) {
      const uint16_t* p = slot_row(ch * kRows + 4 * r + wave);
      stage_ok[r] = p != nullptr;
      stage[r] = p ? reinterpret_cast<const uint4*>(p)[l] : make_uint4(0, 0, 0, 0);
    }
  };
  auto swrite = [&]() {
#pragma unroll
    for (int r = 0; r < kRows / 4; ++r) {
      const int row = 4 * r + wave;
      *reinterpret_cast<uint4*>(&rows_lds[row * kRowStride + 16 * l]) = stage[r];
      if (l == 0) valid_lds[row] = stage_ok[r];
    }
  };

  // Q of this wave's 16 heads as the B operand of S^T = KV . Q^T: lane l holds head
  // 16*wave + l%16, channels 32*ks + 8*g .. +7
  v8s qb[kAC / 32];
  {
    const uint16_t* qh = a.q + (static_cast<size_t>(qi) * kAH + 16 * wave + (l & 15)) * kAC;
#pragma unroll
    for (int ks = 0; ks < kAC / 32; ++ks) qb[ks] = *reinterpret_cast<const v8s*>(qh + 32 * ks + 8 * g);
  }

  v4f o[kAC / 16];
#pragma unroll
  for (int t = 0; t < kAC / 16; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // per head l%16 (log2 units)
  float l_run = 0.0f;        // this lane's share of the per-head sum

  if (ch0 < ch1) {
    gload(ch0);
    swrite();
  }
  __syncthreads();
#pragma unroll 1
  for (int ch = ch0; ch < ch1; ++ch) {
    const bool more = ch + 1 < ch1;
    if (more) gload(ch + 1);

    // ---- S^T for 32 rows x 16 heads
    v4f st[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < kAC / 32; ++ks) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const v8s av = *reinterpret_cast<const v8s*>(&rows_lds[(16 * rb + (l & 15)) * kRowStride + 64 * ks + 16 * g]);
        st[rb] = mfma_bf16_16x16x32(av, qb[ks], st[rb]);
      }
    }
    // ---- online softmax; slot j <-> chunk row rho(j) = 16*(j/4) + 4*g + j%4
    float sv[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 16 * (j >> 2) + 4 * g + (j & 3);
      sv[j] = valid_lds[row] ? st[j >> 2][j & 3] * a.scale_log2 : -INFINITY;
      cmax = fmaxf(cmax, sv[j]);
    }
    cmax = fmaxf(cmax, wave_xor(cmax, 16));
    cmax = fmaxf(cmax, wave_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = exp2f(m_run - m_use);          // 0 when m_run = -inf
    // P = P_hi + P_lo, both bf16: the two products with V keep P to ~16 bits, so the
    // weights carry no bf16 rounding into the output (only its final rounding remains)
    float psum = 0.0f;
    v8s pa, pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = exp2f(sv[j] - m_use);
      psum += p;
      const uint16_t hi = f32_to_bf16(p);
      pa[j] = static_cast<short>(hi);
      pb[j] = static_cast<short>(f32_to_bf16(p - bf16_to_f32(hi)));
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // rescale O rows (heads 4*g+i) when any head's max moved
    if (__ballot(alpha != 1.0f)) {
      float ah[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ah[i] = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
      for (int t = 0; t < kAC / 16; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[t][i] *= ah[i];
    }
    // ---- O += P . V; lane (g, i) reads row 4g + i/4 (and 16 + ...) at columns 4*(i%4) ..
    const uint8_t* vt = rows_lds + (4 * g + ((l & 15) >> 2)) * kRowStride + 8 * (l & 3);
#pragma unroll
    for (int t = 0; t < kAC / 16; ++t) {
      const v4s v0 = lds_read_tr16(vt + 32 * t);
      const v4s v1 = lds_read_tr16(vt + 32 * t + 16 * kRowStride);
      const v8s vb = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      o[t] = mfma_bf16_16x16x32(pa, vb, o[t]);
      o[t] = mfma_bf16_16x16x32(pb, vb, o[t]);
    }
    __syncthreads();
    if (more) swrite();
    __syncthreads();
  }

  // ---- finish: per-head totals
  float l_tot = l_run + wave_xor(l_run, 16);
  l_tot += wave_xor(l_tot, 32);
  const int head_l = 16 * wave + (l & 15);            // head whose statistics this lane holds
  if (a.nsplit == 1) {
    const float sink2 = a.sink[head_l] * kLog2e;
    const float M = fmaxf(m_run, sink2);
    float f, lse2;
    if (M == -INFINITY) {
      f = 0.0f;
      lse2 = -INFINITY;
    } else {
      const float em = m_run == -INFINITY ? 0.0f : exp2f(m_run - M);
      const float den = l_tot * em + exp2f(sink2 - M);
      f = den > 0.0f ? em / den : 0.0f;
      lse2 = M + log2f(den);
    }
    if (a.lse && g == 0) a.lse[static_cast<size_t>(qi) * kAH + head_l] = lse2 * kLn2;
    float fh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fh[i] = __shfl(f, 4 * g + i, kWave);
    uint16_t* ob = a.out + static_cast<size_t>(qi) * kAH * kAC;
#pragma unroll
    for (int t = 0; t < kAC / 16; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ob[(16 * wave + 4 * g + i) * kAC + 16 * t + (l & 15)] = f32_to_bf16(o[t][i] * fh[i]);
  } else {
    const size_t pbase = static_cast<size_t>(qi) * a.nsplit + split;
    if (g == 0) {
      a.part_ml[(pbase * kAH + head_l) * 2 + 0] = m_run;
      a.part_ml[(pbase * kAH + head_l) * 2 + 1] = l_tot;
    }
    float* po = a.part_o + pbase * kAH * kAC;
#pragma unroll
    for (int t = 0; t < kAC / 16; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) po[(16 * wave + 4 * g + i) * kAC + 16 * t + (l & 15)] = o[t][i];
  }
}

// Combines the split partials with the sink.  One wave per (query, head); lane l owns
// columns 8l .. 8l+7 (c = 512) or a strided share of them, loads of every split in flight
// together.  Grid: ceil(B*S*H / 4) blocks of 256 threads.
template <typename OutT>
__global__ __launch_bounds__(256) void attn_merge(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                  const float* __restrict__ sink, int nsplit, int H, int c, int nqh,
                                                  OutT* __restrict__ out, float* __restrict__ lse) {
  const int qh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (qh >= nqh) return;
  const int lane = threadIdx.x & 63;
  const size_t qi = qh / H;
  const int h = qh % H;
  const float sink2 = sink[h] * kLog2e;
  float M = sink2;
  for (int i = 0; i < nsplit; ++i) M = fmaxf(M, part_ml[((qi * nsplit + i) * H + h) * 2]);
  float den = M == -INFINITY ? 0.0f : exp2f(sink2 - M);
  for (int i = 0; i < nsplit; ++i) {
    const float mi = part_ml[((qi * nsplit + i) * H + h) * 2];
    if (mi != -INFINITY) den += part_ml[((qi * nsplit + i) * H + h) * 2 + 1] * exp2f(mi - M);
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  for (int c0 = 8 * lane; c0 < c; c0 += 512) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < nsplit; ++i) {
      const float mi = part_ml[((qi * nsplit + i) * H + h) * 2];
      const float wgt = mi == -INFINITY ? 0.0f : exp2f(mi - M);
      const float* src = part_o + ((qi * nsplit + i) * H + h) * c + c0;
      if (c0 + 8 <= c) {
        const float4 x0 = reinterpret_cast<const float4*>(src)[0];
        const float4 x1 = reinterpret_cast<const float4*>(src)[1];
        acc[0] = fmaf(wgt, x0.x, acc[0]); acc[1] = fmaf(wgt, x0.y, acc[1]);
        acc[2] = fmaf(wgt, x0.z, acc[2]); acc[3] = fmaf(wgt, x0.w, acc[3]);
        acc[4] = fmaf(wgt, x1.x, acc[4]); acc[5] = fmaf(wgt, x1.y, acc[5]);
        acc[6] = fmaf(wgt, x1.z, acc[6]); acc[7] = fmaf(wgt, x1.w, acc[7]);
      } else {
        for (int j = 0; j < 8 && c0 + j < c; ++j) acc[j] = fmaf(wgt, src[j], acc[j]);
      }
    }
    OutT* dst = out + (qi * H + h) * c + c0;
    for (int j = 0; j < 8 && c0 + j < c; ++j) {
      if constexpr (sizeof(OutT) == 2) dst[j] = f32_to_bf16(acc[j] * inv);
      else dst[j] = acc[j] * inv;
    }
  }
  if (lse && lane == 0) lse[qi * H + h] = (M == -INFINITY || den <= 0.0f) ? -INFINITY : (M + log2f(den)) * kLn2;
}

// ------------------------------------------------------------------------------------
// fp32 path (small shapes): one workgroup per (query, head); 256 slots per step, each
// thread one slot's logit, then each thread accumulates channels.  Writes partials in
// the same format as the bf16 kernel so attn_merge finishes it.
// ------------------------------------------------------------------------------------
template <bool kDense>
__global__ __launch_bounds__(256) void attn_f32(const float* __restrict__ q, const float* __restrict__ kv,
                                                const int32_t* __restrict__ idx, const int64_t* __restrict__ q_pos,
                                                const float* __restrict__ swa, float scale_log2, int S, int H,
                                                int c, int Nc, int k, int Ls, int W, int m,
                                                float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ float qv[1024];
  __shared__ float pl[256];
  __shared__ const float* rp[256];
  __shared__ float red[4];
  const int qi = blockIdx.y, h = blockIdx.x;
  const int b = qi / S, s = qi % S;
  int w_lo, n_swa;
  window_rows(s, S, Ls, W, w_lo, n_swa);
  const int n_rem = kDense ? static_cast<int>(min(static_cast<int64_t>(Nc), (q_pos[qi] + 1) / m)) : k;
  const int n_slots = n_swa + n_rem;
  for (int i = threadIdx.x; i < c; i += 256) qv[i] = q[(static_cast<size_t>(qi) * H + h) * c + i];
  float m_run = -INFINITY, l_run = 0.0f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};       // channels threadIdx.x + 256*i
  __syncthreads();
  for (int base = 0; base < n_slots; base += 256) {
    const int slot = base + threadIdx.x;
    const float* p = nullptr;
    if (slot < n_slots) {
      if (slot < n_swa) {
        p = swa + (static_cast<size_t>(b) * Ls + w_lo + slot) * c;
      } else {
        const int r = slot - n_swa;
        const int j = kDense ? r : idx[static_cast<size_t>(qi) * k + r];
        if (j >= 0 && j < Nc) p = kv + (static_cast<size_t>(b) * Nc + j) * c;
      }
    }
    float lg = -INFINITY;
    if (p) {
      float d = 0.0f;
      for (int i = 0; i < c; ++i) d = fmaf(qv[i], p[i], d);
      lg = d * scale_log2;
    }
    rp[threadIdx.x] = p;
    // block max
    float mx = lg;
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = exp2f(m_run - m_use);
    const float pv = exp2f(lg - m_use);
    pl[threadIdx.x] = pv;
    __syncthreads();
    float ps = 0.0f;
    for (int i = 0; i < 256; ++i) ps += pl[i];
    l_run = l_run * alpha + ps;
    m_run = m_new;
    for (int ci = 0; ci < 4; ++ci) {
      const int col = threadIdx.x + 256 * ci;
      if (col >= c) break;
      float x = acc[ci] * alpha;
      for (int i = 0; i < 256; ++i)
        if (rp[i]) x = fmaf(pl[i], rp[i][col], x);
      acc[ci] = x;
    }
    __syncthreads();
  }
  const size_t pbase = static_cast<size_t>(qi);      // one split
  for (int ci = 0; ci < 4; ++ci) {
    const int col = threadIdx.x + 256 * ci;
    if (col < c) part_o[(pbase * H + h) * c + col] = acc[ci];
  }
  if (threadIdx.x == 0) {
    part_ml[(pbase * H + h) * 2] = m_run;
    part_ml[(pbase * H + h) * 2 + 1] = l_run;
  }
}

// Splits of one query's rows over workgroups (bf16 kernel).  Enough workgroups to cover
// the 256 compute units, but every split keeps >= 128 rows: a split's partial result
// (64 x 512 fp32 = 128 KiB) must stay small next to the rows it reads (1 KiB each).
int attn_nsplit(int nq, int max_rows) {
  const int by_fill = cdiv(256, nq);
  const int by_rows = max_rows / 128;
  const int by_lds = cdiv(max_rows, kMaxSplitSlots);  // a split's selection fits its LDS table
  return std::max(by_lds, std::max(1, std::min(by_fill, by_rows)));
}

size_t attn_workspace_bytes(int B, int S, int H, int c, int max_rows, int dtype) {
  const size_t nq = static_cast<size_t>(B) * S;
  const int ns = dtype == CSA_F32 ? 1 : attn_nsplit(static_cast<int>(nq), max_rows);
  if (dtype != CSA_F32 && ns == 1) return 0;
  return nq * ns * H * (static_cast<size_t>(c) + 2) * sizeof(float);
}

int launch_attention(bool dense, const void* q, const void* kv, const int32_t* idx, const int64_t* q_pos, int m,
                     const void* swa, const float* sink, int dtype, float scale, int B, int S, int H, int c, int Nc,
                     int k, int Ls, int W, void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t st) {
  const int nq = B * S;
  const int max_rows = std::min(W, Ls) + (dense ? Nc : k);
  if (ws_bytes < attn_workspace_bytes(B, S, H, c, max_rows, dtype)) return CSA_ERR_WORKSPACE;
  const float scale_log2 = scale * kLog2e;
  if (dtype == CSA_BF16) {
    const int ns = attn_nsplit(nq, max_rows);
    AttnArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.kv = static_cast<const uint16_t*>(kv);
    a.idx = idx;
    a.q_pos = q_pos;
    a.swa = static_cast<const uint16_t*>(swa);
    a.sink = sink;
    a.scale_log2 = scale_log2;
    a.S = S; a.Nc = Nc; a.k = k; a.Ls = Ls; a.W = W; a.m = m;
    a.nsplit = ns;
    a.chunks_per_split = cdiv(cdiv(max_rows, kRows), ns);   // <= kMaxSplitSlots / kRows by attn_nsplit
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    float* wsf = static_cast<float*>(ws);
    a.part_o = wsf;
    a.part_ml = wsf ? wsf + static_cast<size_t>(nq) * ns * H * c : nullptr;
    dim3 grid(ns, nq);
    if (dense) hipLaunchKernelGGL(attn_bf16<true>, grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(attn_bf16<false>, grid, dim3(256), 0, st, a);
    CSA_LAUNCH_CHECK();
    if (ns > 1) {
      hipLaunchKernelGGL(attn_merge<uint16_t>, dim3(cdiv(nq * H, 4)), dim3(256), 0, st, a.part_o, a.part_ml, sink,
                         ns, H, c, nq * H, static_cast<uint16_t*>(out), lse);
      CSA_LAUNCH_CHECK();
    }
    return CSA_OK;
  }
  float* wsf = static_cast<float*>(ws);
  float* part_o = wsf;
  float* part_ml = wsf + static_cast<size_t>(nq) * H * c;
  dim3 grid(H, nq);
  if (dense)
    hipLaunchKernelGGL(attn_f32<true>, grid, dim3(256), 0, st, static_cast<const float*>(q),
                       static_cast<const float*>(kv), idx, q_pos, static_cast<const float*>(swa), scale_log2, S, H, c,
                       Nc, k, Ls, W, m, part_o, part_ml);
  else
    hipLaunchKernelGGL(attn_f32<false>, grid, dim3(256), 0, st, static_cast<const float*>(q),
                       static_cast<const float*>(kv), idx, q_pos, static_cast<const float*>(swa), scale_log2, S, H, c,
                       Nc, k, Ls, W, m, part_o, part_ml);
  CSA_LAUNCH_CHECK();
  hipLaunchKernelGGL(attn_merge<float>, dim3(cdiv(nq * H, 4)), dim3(256), 0, st, part_o, part_ml, sink, 1, H, c,
                     nq * H, static_cast<float*>(out), lse);
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

}  // namespace csa
