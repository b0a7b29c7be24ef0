// Constants, argument block, window rule and workgroup numbering of the bf16 attention
// kernel (attention.hip).
#pragma once

#include "common.hpp"

namespace csa {

constexpr int kAH = 64;                             // query heads
constexpr int kAC = 512;                            // channels of a KV row
constexpr int kHG = 16;                             // heads per MFMA tile (one head group)
constexpr int kNHG = kAH / kHG;
constexpr int kRows = 32;                           // rows per chunk
constexpr int kRowStride = kAC * 2 + 32;            // bytes
constexpr int kChunkBytes = kRows * kRowStride;
constexpr int kMaxSplitChunks = 72;                 // chunks of row addresses tabled per workgroup
constexpr float kLazy = 8.0f;                       // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Workgroup barrier without a memory fence: the row loads still in flight (later chunks)
// are not waited for; LDS writes of this wave are waited for explicitly.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xc07f);               // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* idx;
  const int64_t* q_pos;
  const uint16_t* swa;
  const float* sink;
  float scale_log2;          // scale * log2(e)
  int nq, S, Nc, k, Ls, W, m;
  int nsplit, chunks_per_split;
  uint16_t* out;
  float* lse;
  float* part_o;             // [B*S, nsplit, H, c] fp32, unnormalised
  float* part_ml;            // [B*S, nsplit, H, 2]: reference max (log2 units), sum
  const uint2* cand;         // (key, entry) pairs of the segment top-k sets, n_cand per row
  int n_cand;
  size_t cand_stride;        // pairs from one row of cand to the next
  int32_t* idx_out;          // [B*S, k] the selection made from cand, or null
  int rope_d;                // > 0: rotate the output's last rope_d channels back by the query position
  double rope_r;             // theta^(-2/rope_d)
};

// cos / sin of the inverse-RoPE angle of channel `col` (pair p of the last d_rope of c
// channels): the rotation by -t * theta^(-2p/d_rope) uses cos(a) and sin(a) of
// a = t * r^p (rope_cos_sin; r = theta^(-2/d_rope) from the host).
__device__ __forceinline__ void rope_cs_sn(int col, int c, int d_rope, double r, int64_t t, float& cs, float& sn) {
  rope_cos_sin(t, (col - (c - d_rope)) >> 1, r, cs, sn);
}

// x' = x cos + y sin (even channel), y' = y cos - x sin (odd channel); `partner` is the
// other member of the pair.
__device__ __forceinline__ float rope_back(float v, float partner, int col, float cs, float sn) {
  return (col & 1) ? fmaf(-partner, sn, v * cs) : fmaf(partner, sn, v * cs);
}

// The value held by the lane whose index differs in bit 0 (DPP quad permutation 1,0,3,2).
__device__ __forceinline__ float pair_lane(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// Window rows of query s: rows w_lo .. w_lo + n_swa - 1 of the sequence's swa tensor,
// whose last row holds the last query's position t_last.  Rows of negative positions
// (r < Ls - 1 - t_last: the sequence is shorter than the tensor) are left out.
__device__ __forceinline__ void window_rows(int s, int S, int Ls, int W, int64_t t_last, int& w_lo, int& n_swa) {
  const int w_hi = s + Ls - S;
  const int64_t first = static_cast<int64_t>(Ls) - 1 - t_last;
  w_lo = max(0, w_hi - W + 1);
  if (first > w_lo) w_lo = first > w_hi + 1 ? w_hi + 1 : static_cast<int>(first);
  n_swa = w_hi - w_lo + 1;
}

// Position of the last query of sequence b, or "every row is a real position" without q_pos.
__device__ __forceinline__ int64_t last_position(const int64_t* q_pos, int b, int S) {
  return q_pos ? q_pos[static_cast<size_t>(b) * S + S - 1] : static_cast<int64_t>(1) << 62;
}

// Workgroup -> (query, unit) with units_per_query units: consecutive workgroup ids go
// round-robin over the 8 XCDs, so all units of one query land on the same XCD (and share
// its L2 for the rows they read).  Returns false for padding workgroups.
__device__ __forceinline__ bool attn_unit(int nq, int units, int& qi, int& u) {
  const int xcd = blockIdx.x & 7, t8 = blockIdx.x >> 3;
  u = t8 % units;
  qi = (t8 / units) * 8 + xcd;
  return qi < nq;
}

}  // namespace csa
