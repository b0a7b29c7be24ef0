// Lightning-indexer scores over microscaled (MX) caches: E2M1 (FP4) or E4M3 (FP8) values
// with one E8M0 power-of-two scale per 32 values, for the query and the keys.
//
// [V4-CSA2] sections 16.2 (indexer keys of 128 FP4 values + 4 E8M0 scales = 68 bytes) and
// 11.2 (the indexer scans run on the 128-dimensional FP4 keys); [ATTN-CMP] section on CSA2
// (indexer query in FP4; K FP4 with E8M0 per 32); [KV-COMP] section 7 (index scores cast
// from FP32 to BF16 before the top-k: score_bf16).  The score is the one of
// csa_index_score: I = sum_h w_h * ReLU(q_h . K) over the dequantised values.
//
// The contraction runs on v_mfma_scale_f32_16x16x128_f8f6f4: M = 16 heads, N = 16 entries,
// K = 128 = the whole head dimension in one instruction; lane l supplies row l % 16 of both
// operands (32 values: one block for FP4, halves of two blocks for FP8, see load_codes) and
// the E8M0 scale byte of block l / 16, so each block's products are scaled by 2^(eq + ek)
// inside the matrix unit.  FP4
// products (multiples of 1/4 up to 36) sum over a block of 32 to a multiple of 1/4 below
// 2^11: such block sums are exact in the unit, and the scaled sums accumulate in fp32.
// (FP8 products are not exact there: the FP8 form is kept for measuring that difference.)
// Epilogue as in index_score.hip: ReLU and head weights per lane, a cross-lane
// reduce-scatter leaves lane l with entry e0 + l of each 64-entry group.
#include "common.hpp"
#include "index_common.hpp"
#include "select.hpp"

namespace csa {

template <bool kFp4>
__device__ __forceinline__ v4f mfma_mx(const v8i& a, int sa, const v8i& b, int sb, const v4f& c) {
  constexpr int kFmt = kFp4 ? 4 : 0;                 // operand format: 4 = E2M1, 0 = E4M3
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kFmt, kFmt, 0, sa, 0, sb);
}

// Decode / few queries: grid (ceil(Nc / entries per workgroup), B*S); each wave streams
// 64-entry groups of its row's keys, two groups in flight; kTopk as in
// index_score_fp8_decode (segment top-k pairs, 4096-entry segments).
template <bool kFp4, bool kTopk>
__global__ __launch_bounds__(dec_waves<kTopk>() * 64) void index_score_mx(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ ks, const int64_t* __restrict__ q_pos, int S, int Nc,
    int m, int score_bf16, float* __restrict__ scores, int ktop, uint2* __restrict__ cand, size_t cand_stride) {
  constexpr int kWaves = dec_waves<kTopk>();
  constexpr int kThreads = kWaves * 64;
  constexpr int kEntWG = dec_entries<kTopk>();
  constexpr int kRowB = kFp4 ? kID / 2 : kID;        // code bytes of a 128-value row
  constexpr int kRing = 3;
  const size_t row = blockIdx.y;
  const int b = static_cast<int>(row / S);
  const int l = static_cast<int>(lane_id());
  const int g = l >> 4;
  const int wave = threadIdx.x >> 6;
  const int64_t t = q_pos[row];
  const int nvis = static_cast<int>(min(static_cast<int64_t>(Nc), (t + 1) / m));
  const uint8_t* kb = k + static_cast<size_t>(b) * Nc * kRowB;
  const uint8_t* ksb = ks + static_cast<size_t>(b) * Nc * (kID / 32);
  float* out = scores ? scores + row * Nc : nullptr;

  // Lane l's operand bytes of a row, placed so that the scale the unit applies to them is
  // the scale of their own block (lane group g passes block g's scale byte).  FP4: the unit
  // scales a group's 16 bytes (32 values) by the group's own scale, so group g takes row
  // bytes 16g .. 16g+15 (block g).  FP8 (measured on gfx950): bytes 0..15 of group g are
  // scaled by group g/2's scale and bytes 16..31 by group 2+g/2's, so group g takes row
  // bytes 16g .. 16g+15 (half g%2 of block g/2) and 64+16g .. 64+16g+15 (half g%2 of block
  // 2+g/2).  Both operands use the same placement, so the products pair the same values.
  auto load_codes = [&](const uint8_t* rowp) -> v8i {
    v8i v = {0, 0, 0, 0, 0, 0, 0, 0};
    const uint4 x = *reinterpret_cast<const uint4*>(rowp + 16 * g);
    v[0] = static_cast<int>(x.x); v[1] = static_cast<int>(x.y); v[2] = static_cast<int>(x.z); v[3] = static_cast<int>(x.w);
    if constexpr (!kFp4) {
      const uint4 y = *reinterpret_cast<const uint4*>(rowp + 64 + 16 * g);
      v[4] = static_cast<int>(y.x); v[5] = static_cast<int>(y.y); v[6] = static_cast<int>(y.z); v[7] = static_cast<int>(y.w);
    }
    return v;
  };
  // A operands: the query's 64 heads in 4 head blocks; lane: head 16*hb + l%16, block g
  v8i a[4];
  int sa[4];
  float wv[16];
  {
    const uint8_t* qr = q + row * (kIH * kRowB);
    const uint8_t* qsr = qs + row * (kIH * (kID / 32));
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int h = 16 * hb + (l & 15);
      a[hb] = load_codes(qr + h * kRowB);
      sa[hb] = qsr[h * (kID / 32) + g];
    }
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[hb * 4 + i] = w[row * kIH + 16 * hb + 4 * g + i];
  }
  const int base = blockIdx.x * kEntWG;
  auto group_e0 = [&](int gi) { return base + 64 * (gi * kWaves + wave); };
  v8i ring[kRing][4];
  int sring[kRing][4];
#define CSA_MX_LOAD(gi_)                                                                  \
  do {                                                                                    \
    _Pragma("unroll") for (int nb = 0; nb < 4; ++nb) {                                    \
      const int e_ = min(group_e0(gi_) + 16 * nb + (l & 15), Nc - 1);                     \
      ring[(gi_) % kRing][nb] = load_codes(kb + static_cast<size_t>(e_) * kRowB);         \
      sring[(gi_) % kRing][nb] = ksb[static_cast<size_t>(e_) * (kID / 32) + g];           \
    }                                                                                     \
  } while (0)
  CSA_MX_LOAD(0);
  CSA_MX_LOAD(1);
  __shared__ uint32_t kst[kTopk ? kEntWG : 1];
#pragma unroll
  for (int gi = 0; gi < kDecGroups; ++gi) {
    if (gi + kRing - 1 < kDecGroups) CSA_MX_LOAD(gi + kRing - 1);
    const int e = group_e0(gi) + l;
    float p[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      float s4[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        const v4f d = mfma_mx<kFp4>(a[hb], sa[hb], ring[gi % kRing][nb], sring[gi % kRing][nb],
                                    v4f{0.f, 0.f, 0.f, 0.f});
        s4[hb] = wv[hb * 4] * relu(d[0]);
#pragma unroll
        for (int i = 1; i < 4; ++i) s4[hb] = fmaf(wv[hb * 4 + i], relu(d[i]), s4[hb]);
      }
      p[nb] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
    float v = reduce_scatter4(p);
    if (score_bf16) v = __uint_as_float(static_cast<uint32_t>(f32_to_bf16(v)) << 16);
    const bool vis = e < nvis;
    if (out && e < Nc) out[e] = vis ? v : -INFINITY;
    if (kTopk) kst[64 * (gi * kWaves + wave) + l] = vis ? score_key(v) : 0u;
  }
#undef CSA_MX_LOAD
  if constexpr (kTopk) {
    __shared__ TkShared sh;
    __syncthreads();
    uint32_t key[1][8];
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) key[0][s2] = kst[8 * threadIdx.x + s2];
    uint64_t taken;
    int obase[1];
    static_assert(kThreads * 8 == kEntWG, "8 keys per thread");
    const int kk = select_regs<kThreads, 8, 1>(sh, key, ktop, taken, obase);
    uint2* dst = cand + row * cand_stride + blockIdx.x * static_cast<size_t>(ktop);
    int o = obase[0];
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
      if ((taken >> s2) & 1ull) dst[o++] = make_uint2(key[0][s2], static_cast<uint32_t>(base + 8 * threadIdx.x + s2));
    for (int pp = kk + static_cast<int>(threadIdx.x); pp < ktop; pp += kThreads) dst[pp] = make_uint2(0u, 0u);
  }
}

int index_topk_segments(int Nc);
size_t topk_merge_pairs_per_row(int G, int k);

int launch_index_mx(const void* q, const void* q_scale, const float* w, const void* k, const void* k_scale, int fp4,
                    const int64_t* q_pos, int B, int S, int Nc, int m, int score_bf16, float* scores, int ktop,
                    uint2* cand, hipStream_t st) {
  const uint8_t *q8 = static_cast<const uint8_t*>(q), *qs8 = static_cast<const uint8_t*>(q_scale);
  const uint8_t *k8 = static_cast<const uint8_t*>(k), *ks8 = static_cast<const uint8_t*>(k_scale);
  if (cand != nullptr) {
    const int G = index_topk_segments(Nc);
    const size_t stride = topk_merge_pairs_per_row(G, ktop);
    const dim3 grid(G, B * S), block(dec_waves<true>() * 64);
    if (fp4)
      hipLaunchKernelGGL((index_score_mx<true, true>), grid, block, 0, st, q8, qs8, w, k8, ks8, q_pos, S, Nc, m,
                         score_bf16, scores, ktop, cand, stride);
    else
      hipLaunchKernelGGL((index_score_mx<false, true>), grid, block, 0, st, q8, qs8, w, k8, ks8, q_pos, S, Nc, m,
                         score_bf16, scores, ktop, cand, stride);
  } else {
    const dim3 grid(cdiv(Nc, dec_entries<false>()), B * S), block(dec_waves<false>() * 64);
    if (fp4)
      hipLaunchKernelGGL((index_score_mx<true, false>), grid, block, 0, st, q8, qs8, w, k8, ks8, q_pos, S, Nc, m,
                         score_bf16, scores, 0, nullptr, size_t{0});
    else
      hipLaunchKernelGGL((index_score_mx<false, false>), grid, block, 0, st, q8, qs8, w, k8, ks8, q_pos, S, Nc, m,
                         score_bf16, scores, 0, nullptr, size_t{0});
  }
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

}  // namespace csa
