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

// Where the remote rows of a query come from.
constexpr int kSrcIdx = 0;     // idx[q][0..k): selected entries, -1 = none
constexpr int kSrcDense = 1;   // every visible entry (HCA)
constexpr int kSrcCand = 2;    // the k best of the query's segment candidates, selected in the kernel
constexpr int kSrcCand2 = 3;   // the same from up to twice as many candidates
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Workgroup barrier without a memory fence: the row loads still in flight (later chunks)
// are not waited for; LDS writes of this wave are waited for explicitly.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xc07f);               // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// Formats of the compressed KV rows (the window rows are always bf16).
constexpr int kFmtBf16 = 0;                         // 512 bf16 channels, 1024 bytes
constexpr int kFmtFp4 = 1;                          // 512 E2M1 codes (256 B) + 32 E4M3 scales per 16: 288 bytes
constexpr int kFmtFp8Rope = 2;                      // 448 e4m3 codes + 64 bf16 + E8M0 exponent + pad: 584 bytes
constexpr int kFp8RopeCodes = 448;
__host__ __device__ constexpr inline int kv_row_bytes(int fmt) {
  return fmt == kFmtFp4 ? 288 : fmt == kFmtFp8Rope ? 584 : kAC * 2;
}

// Lane l's share of a compressed row (channels 8l .. 8l+7) is loaded raw and decoded only
// when it is written to LDS, so that the loads of later chunks stay in flight meanwhile.
// FP4: two codes per byte, the even channel in the low nibble, the E4M3 scale of channels
// 16i .. 16i+15 in byte 256 + i.  FP8 + RoPE: channels below 448 are e4m3 codes times
// 2^(e - 127) with e = byte 576, the last 64 channels bf16 at byte 448.
template <int kFmt>
__device__ __forceinline__ v4u load_row8(uint64_t row, int l) {
  typedef const __attribute__((address_space(1))) uint8_t g8;
  typedef const __attribute__((address_space(1))) uint32_t g32;
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  typedef const __attribute__((address_space(1))) u2 g64;
  g8* r = reinterpret_cast<g8*>(row);
  v4u v = {0u, 0u, 0u, 0u};
  if constexpr (kFmt == kFmtFp4) {
    v[0] = *reinterpret_cast<g32*>(r + 4 * l);              // codes of channels 8l .. 8l+7
    v[1] = r[256 + (l >> 1)];                               // their block's scale
  } else {
    if (8 * l < kFp8RopeCodes) {
      const u2 c = *reinterpret_cast<g64*>(r + 8 * l);
      v[0] = c[0];
      v[1] = c[1];
      v[2] = r[kFp8RopeCodes + 128];
    } else {                                                // 8-byte aligned: two 8-byte loads
      g64* b = reinterpret_cast<g64*>(r + kFp8RopeCodes + 2 * (8 * l - kFp8RopeCodes));
      const u2 lo = b[0], hi = b[1];
      v = v4u{lo[0], lo[1], hi[0], hi[1]};
    }
  }
  return v;
}

// The 8 bf16 values of a raw share from load_row8, exactly: an E2M1 value times an E4M3
// scale has at most 6 significant bits, an e4m3 value times a power of two at most 4, so
// both products are bf16 numbers and dropping the low half of the fp32 word is exact.
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

template <int kFmt>
__device__ __forceinline__ v4u decode_row8(v4u v, int l) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  v4u out;
  if constexpr (kFmt == kFmtFp4) {
    const uint32_t codes = v[0];
    const float s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[1], 1.0f, false)[0];
    v2f f;
    f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0); out[0] = pack_bf16_exact(f[0] * s, f[1] * s);
    f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1); out[1] = pack_bf16_exact(f[0] * s, f[1] * s);
    f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2); out[2] = pack_bf16_exact(f[0] * s, f[1] * s);
    f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3); out[3] = pack_bf16_exact(f[0] * s, f[1] * s);
  } else {
    if (8 * l < kFp8RopeCodes) {
      const float s = ldexpf(1.0f, static_cast<int>(v[2]) - 127);
      v2f f;
      f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[0], 1.0f, false); out[0] = pack_bf16_exact(f[0] * s, f[1] * s);
      f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[0], 1.0f, true); out[1] = pack_bf16_exact(f[0] * s, f[1] * s);
      f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[1], 1.0f, false); out[2] = pack_bf16_exact(f[0] * s, f[1] * s);
      f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[1], 1.0f, true); out[3] = pack_bf16_exact(f[0] * s, f[1] * s);
    } else {
      out = v;
    }
  }
  return out;
}

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kv;
  int kv_fmt;                // kFmt* of the compressed rows
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

// One wave's KT tiles from the merged numerators acc, denominators den and reference
// maxima M (log2 units) of the lane's 4 heads: division, inverse RoPE, bf16 cast; the wave
// holding tile 0 writes the lse of its heads.
template <int KT>
__device__ __forceinline__ void merge_store(const float (&acc)[KT][4], const float (&den)[4], const float (&M)[4],
                                            size_t qi, int h0, int ct0, int l, uint16_t* __restrict__ out,
                                            float* __restrict__ lse, const int64_t* __restrict__ q_pos, int rope_d,
                                            double rope_r) {
  uint16_t* dst = out + (qi * kAH + h0) * kAC + 16 * ct0 + (l & 15);
  const int64_t tq = rope_d > 0 ? q_pos[qi] : 0;
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = den[i] > 0.0f ? acc[t][i] / den[i] : 0.0f;
    // inverse RoPE of the output (lane pairs hold channel pairs)
    if (rope_d > 0 && 16 * (ct0 + t) + 16 > kAC - rope_d) {
      const int col = 16 * (ct0 + t) + (l & 15);
      float cs = 1.0f, sn = 0.0f;
      if (col >= kAC - rope_d) rope_cs_sn(col, kAC, rope_d, rope_r, tq, cs, sn);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = rope_back(v[i], pair_lane(v[i]), col, cs, sn);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i * kAC + 16 * t] = f32_to_bf16(v[i]);
  }
  if (lse && ct0 == 0 && (l & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lse[qi * kAH + h0 + i] = (M[i] == -INFINITY || den[i] <= 0.0f) ? -INFINITY : (M[i] + log2f(den[i])) * kLn2;
  }
}

}  // namespace csa
