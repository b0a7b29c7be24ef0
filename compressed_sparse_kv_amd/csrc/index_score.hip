// Lightning-indexer scores (stage 2).
//
//   scores[b,s,j] = sum_h w[b,s,h] * ReLU(qI[b,s,h] . KI[b,j])   for j < n_vis(b,s), else -inf
//   n_vis = min(Nc, (q_pos + 1) / m)
// [HCA-CSA] section "CSA：轻压缩 + 稀疏选择" (indexer equations); [KV-COMP] sections 9.4
// (score = sum over heads of w * ReLU(q . z)) and 9.8 (entry j visible once t >= m*j+m-1).
//
// FP8 inputs.  With q = dec(q8)*sq and K = dec(k8)*sk and non-negative scales,
//   w * ReLU(sq*sk*dot) = sk * (w*sq) * ReLU(dot),   dot = dec(q8) . dec(k8),
// so the matrix unit contracts the decoded codes, each head's partial is weighted by
// w' = w*sq after the ReLU, and the row scale sk multiplies once.
//
// Precision.  The e4m3 codes stay the storage format (128 B + 4 B per entry) but the
// contraction runs on bf16 MFMA (v_mfma_f32_16x16x32_bf16): e4m3 -> bf16 is exact
// (v_cvt_scalef32_pk_bf16_fp8, scale 1), bf16 x bf16 products are exact in fp32 and the
// bf16 unit accumulates at fp32 precision.  The gfx950 FP8 MFMA forms keep only about
// 12 bits below the largest product of each 32-element block, about 1e-4 relative on
// these dot products, which would not meet the 1e-5 bound on the fp32 scores.
//
// MFMA mapping: M = 16 heads, N = 16 entries, K = d_I = 128 in four 32-wide steps.
// Lane l owns bytes 32*(l/16) .. +31 of its head's / entry's row and feeds them to the
// four steps 8 at a time (the same k-slots on both operands, so the pairing is exact).
// Output lane l of a 16x16 tile holds heads 4*(l/16)+i of entry l%16; a lane weights and
// sums 16 heads of the 64 locally, and three cross-lane exchanges finish the head sum for
// 4 entry blocks at once (a reduce-scatter leaving lane l with entry e0+l of a 64-entry
// group, so stores are coalesced).
#include "common.hpp"
#include "index_common.hpp"
#include "select.hpp"

namespace csa {

// 32 e4m3 codes (8 dwords) -> 32 bf16 (4 MFMA operands of 8 values each), exactly.
__device__ __forceinline__ void e4m3x32_to_bf16(const v8i& c, v8s out[4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<unsigned>(c[2 * ks]), 1.0f, false);
    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<unsigned>(c[2 * ks]), 1.0f, true);
    const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<unsigned>(c[2 * ks + 1]), 1.0f, false);
    const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<unsigned>(c[2 * ks + 1]), 1.0f, true);
    typedef int v4i __attribute__((ext_vector_type(4)));
    v4i w;
    w[0] = __builtin_bit_cast(int, p0);
    w[1] = __builtin_bit_cast(int, p1);
    w[2] = __builtin_bit_cast(int, p2);
    w[3] = __builtin_bit_cast(int, p3);
    out[ks] = __builtin_bit_cast(v8s, w);
  }
}

// Weighted ReLU head-sum of one 16-entry block against the 4 head blocks of one query.
// Each head block is a chain of 4 MFMAs followed by its 16 VALU epilogue operations; the
// epilogue of block hb overlaps the MFMA chain of block hb+1 (MFMA and VALU co-issue),
// and each head block sums into its own accumulator.
__device__ __forceinline__ float head_sum1(const v8s a[4][4], const v8s b[4], const float wv[16]) {
  float s[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) d = mfma_bf16_16x16x32(a[hb][ks], b[ks], d);
    s[hb] = wv[hb * 4] * relu(d[0]);
#pragma unroll
    for (int i = 1; i < 4; ++i) s[hb] = fmaf(wv[hb * 4 + i], relu(d[i]), s[hb]);
  }
  return (s[0] + s[1]) + (s[2] + s[3]);
}

// A operand (64 heads x 128 codes of one query, as bf16) and its head weights w*sq.
__device__ __forceinline__ void load_query(const uint8_t* __restrict__ q8, const float* __restrict__ qs,
                                           const float* __restrict__ w, size_t row, v8s a[4][4],
                                           float wv[16]) {
  const int l = static_cast<int>(lane_id());
  const uint8_t* qr = q8 + row * (kIH * kID);
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
    e4m3x32_to_bf16(*reinterpret_cast<const v8i*>(qr + (16 * hb + (l & 15)) * kID + 32 * (l >> 4)), a[hb]);
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
// K straight from HBM into registers (one 128-byte row = one cache line, read by 4 lanes
// x 32 bytes), converts them and multiplies; the keys (and row scales) of the next two
// groups are in flight while a group is multiplied.  The unrolled group loop has no
// branches (loads clamped to the last entry, results past the visible range masked), so
// the compiler schedules one group's epilogue against the next group's MFMAs; entries
// past a query's visible range cost compute but never memory outside K.
// Grid: (ceil(Nc / kDecEntWG), B*S).
//
// kTopk: the workgroup also selects the top-k of its kDecEntWG scores (select_regs over
// the scores' order-preserving keys, [KV-COMP] section 9.4) and writes them as (key,
// entry) pairs in entry order to cand + row * cand_stride + blockIdx.x * k (key 0 = empty
// slot); the union of these local selections holds the row's top-k, which topk_merge
// finishes (rows are cand_stride pairs apart: room for the merge's first level when there
// are many segments).  Scores are then written only when `scores` is not null.
// ------------------------------------------------------------------------------------
// kB16: the keys are stored in blocks of 16 entries (index_keys_b16 below), so that each
// quarter-wave's load is 512 contiguous bytes already in the MFMA layout; one group is
// then kept in flight instead of two.
// kBmax: the maxima of the row's scores over blocks of 8 entries (-inf where a block has
// no visible entry) also go to bmax [row][ceil(Nc/8)] (the Full layer of the hierarchical
// indexer, [V4-CSA2] section 11); 8 consecutive lanes hold a block's scores.
// kPool: the entries scanned are a candidate pool of 8 * n_blk positions, pool entry e
// being position 8 * blk[row][e / 8] + e % 8 (blk = -1: no position); keys are gathered
// from the row-major cache by position (gather, then score: a Reindex layer, [V4-CSA2]
// sections 11 and 15.2).  Scores are written in pool order; candidate pairs carry the
// position.
template <bool kTopk, bool kB16 = false, bool kPool = false, bool kBmax = false>
__global__ __launch_bounds__(dec_waves<kTopk>() * 64) void index_score_fp8_decode(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, const int64_t* __restrict__ q_pos,
    int S, int Nc, int m, float* __restrict__ scores, int ktop, uint2* __restrict__ cand, size_t cand_stride,
    float* __restrict__ bmax = nullptr, const int32_t* __restrict__ pool_blk = nullptr, int n_blk = 0) {
  static_assert(!(kPool && kB16), "pool positions are gathered from the row-major cache");
  constexpr int kDecWaves = dec_waves<kTopk>();
  constexpr int kDecThreads = kDecWaves * 64;
  constexpr int kDecEntWG = dec_entries<kTopk>();
  const size_t row = blockIdx.y;
  const int b = static_cast<int>(row / S);
  const int l = static_cast<int>(lane_id());
  const int wave = threadIdx.x >> 6;
  const int64_t t = q_pos[row];
  const int nvis = static_cast<int>(min(static_cast<int64_t>(Nc), (t + 1) / m));
  const int n_ent = kPool ? 8 * n_blk : Nc;          // entries of the row scanned

  const uint8_t* kb = k8 + static_cast<size_t>(b) * (kB16 ? cdiv(Nc, 16) * 16 : Nc) * kID;
  const float* ksb = ks + static_cast<size_t>(b) * Nc;
  float* out = scores ? scores + row * n_ent : nullptr;
  const int32_t* pb = kPool ? pool_blk + row * n_blk : nullptr;
  // position of (pool) entry e, e < n_ent; -1 when the pool has no position there
  auto pos_of = [&](int e) -> int {
    if constexpr (kPool) {
      const int bk = pb[e >> 3];
      return bk >= 0 ? 8 * bk + (e & 7) : -1;
    } else {
      return e;
    }
  };
  // the cache row a load of entry e reads (clamped: never outside the cache)
  auto load_row = [&](int e) -> int { return min(max(pos_of(min(e, n_ent - 1)), 0), Nc - 1); };

  // group gi of this wave covers entries base + 64*(gi*kDecWaves + wave) .. +63; the keys of
  // the next two groups are in flight while a group is multiplied
  const int base = blockIdx.x * kDecEntWG;
  auto group_e0 = [&](int gi) { return base + 64 * (gi * kDecWaves + wave); };
  constexpr int kRingD = kB16 ? 2 : 3;       // groups held: the one multiplied + those in flight
  v8i ring[kRingD][4];
  float sring[kRingD];       // row scale of entry e0 + l, fetched with the group's keys
  // lane l's 32 bytes of entry e: bytes 32*(l/16) .. +31 of its row
  auto key_off = [&](int e) -> size_t {
    return kB16 ? static_cast<size_t>(e >> 4) * (16 * kID) + (l >> 4) * (16 * 32) + (e & 15) * 32
                : static_cast<size_t>(e) * kID + 32 * (l >> 4);
  };
#define CSA_DEC_LOAD(gi_)                                                                           \
  do {                                                                                              \
    _Pragma("unroll") for (int nb = 0; nb < 4; ++nb) {                                              \
      const int e_ = load_row(group_e0(gi_) + 16 * nb + (l & 15));                                  \
      ring[(gi_) % kRingD][nb] = *reinterpret_cast<const v8i*>(kb + key_off(e_));                   \
    }                                                                                               \
    sring[(gi_) % kRingD] = ksb[load_row(group_e0(gi_) + l)];                                       \
  } while (0)
  // The query (64 x 128 codes, 8 KiB), its head weights and scales are read once per
  // workgroup, ahead of the keys, and shared through LDS: loads complete in order, so a
  // query each wave read behind its first key groups would wait for all of them, and
  // every wave reading the whole query multiplies the start burst by the waves.
  constexpr int kQv = kIH * kID / 16 / kDecThreads;   // 16-byte pieces per thread
  __shared__ v4u qlds[kIH * kID / 16];
  __shared__ float wlds[2 * kIH];                    // w, then qs
  v4u qv[kQv];
  float wq = 0.0f;
  {
    const v4u* qsrc = reinterpret_cast<const v4u*>(q8 + row * (kIH * kID));
#pragma unroll
    for (int i = 0; i < kQv; ++i) qv[i] = qsrc[threadIdx.x + i * kDecThreads];
    if (threadIdx.x < 2 * kIH) wq = threadIdx.x < kIH ? w[row * kIH + threadIdx.x] : qs[row * kIH + threadIdx.x - kIH];
  }
  CSA_DEC_LOAD(0);
  if constexpr (kRingD == 3) CSA_DEC_LOAD(1);
  __builtin_amdgcn_sched_barrier(0);      // every load above the query's staging
#pragma unroll
  for (int i = 0; i < kQv; ++i) qlds[threadIdx.x + i * kDecThreads] = qv[i];
  if (threadIdx.x < 2 * kIH) wlds[threadIdx.x] = wq;
  __builtin_amdgcn_s_waitcnt(0xc07f);     // lgkmcnt(0): this wave's LDS writes done; key loads stay in flight
  __builtin_amdgcn_s_barrier();

  // A operand: lane l, head block hb: head 16*hb + l%16, codes 32*(l/16) .. +31
  v8s a[4][4];
  float wv[16];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int p = ((16 * hb + (l & 15)) * kID + 32 * (l >> 4)) / 16;
    const v4u lo = qlds[p], hi = qlds[p + 1];
    e4m3x32_to_bf16(v8i{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]), static_cast<int>(lo[3]),
                        static_cast<int>(hi[0]), static_cast<int>(hi[1]), static_cast<int>(hi[2]), static_cast<int>(hi[3])},
                    a[hb]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * hb + 4 * (l >> 4) + i;
      wv[hb * 4 + i] = wlds[h] * wlds[kIH + h];
    }
  }

  __shared__ uint32_t kst[kTopk ? kDecEntWG : 1];       // keys of the workgroup's entries
  // the selection's step 1 (candidate count, key range), kept per lane during the scoring
  uint32_t sel_min1 = 0xffffffffu, sel_max = 0u;
  int sel_cnt = 0;
#pragma unroll
  for (int gi = 0; gi < kDecGroups; ++gi) {
    const int e0 = group_e0(gi);
    if (gi + kRingD - 1 < kDecGroups) CSA_DEC_LOAD(gi + kRingD - 1);
    const int e = e0 + l;
    float p[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      v8s bk[4];
      e4m3x32_to_bf16(ring[gi % kRingD][nb], bk);
      p[nb] = head_sum1(a, bk, wv);
    }
    const float v = reduce_scatter4(p) * sring[gi % kRingD];
    bool vis;
    if constexpr (kPool) {
      const int pe = e < n_ent ? pos_of(e) : -1;
      vis = pe >= 0 && pe < nvis;
    } else {
      vis = e < nvis;
    }
    if (out && e < n_ent) out[e] = vis ? v : -INFINITY;
    const uint32_t key = vis ? score_key(v) : 0u;
    if (kTopk) {
      kst[64 * (gi * kDecWaves + wave) + l] = key;
      sel_cnt += key != 0u ? 1 : 0;
      sel_max = max(sel_max, key);
      sel_min1 = min(sel_min1, key - 1u);
    }
    if constexpr (kBmax) {
      float bm = vis ? v : -INFINITY;
      bm = fmaxf(bm, __shfl_xor(bm, 1, kWave));
      bm = fmaxf(bm, __shfl_xor(bm, 2, kWave));
      bm = fmaxf(bm, __shfl_xor(bm, 4, kWave));
      if ((l & 7) == 0 && e < Nc) bmax[row * static_cast<size_t>(cdiv(Nc, 8)) + (e >> 3)] = bm;
    }
  }
#undef CSA_DEC_LOAD
  if (kTopk) {
    __shared__ TkShared sh;
    sel_clear<kDecThreads, kDecEntWG>(sh);
    sel_wave_range(sh, wave, l, sel_min1, sel_max, sel_cnt);
    __syncthreads();
    uint32_t key[1][8];
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) key[0][s2] = kst[8 * threadIdx.x + s2];
    uint64_t taken;
    int obase[1];
    static_assert(kDecThreads * 8 == kDecEntWG, "8 keys per thread");
    const int kk = select_regs<kDecThreads, 8, 1, true>(sh, key, ktop, taken, obase);
    uint2* dst = cand + row * cand_stride + blockIdx.x * static_cast<size_t>(ktop);
    int o = obase[0];
    // the entries 8*tid .. 8*tid+7 of the segment: one block of 8 (positions from the pool)
    int e8 = base + 8 * static_cast<int>(threadIdx.x);
    if constexpr (kPool) {
      if (taken != 0ull) e8 = 8 * pb[min(e8, n_ent - 1) >> 3];
    }
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
      if ((taken >> s2) & 1ull) dst[o++] = make_uint2(key[0][s2], static_cast<uint32_t>(e8 + s2));
    for (int p = kk + static_cast<int>(threadIdx.x); p < ktop; p += kDecThreads) dst[p] = make_uint2(0u, 0u);
  }
}

// ------------------------------------------------------------------------------------
// Prefill: many queries per sequence.  A workgroup of 8 waves owns kPfQ = 8 queries (one
// per wave, A operands resident in registers) and walks the entry axis in tiles of
// kPfTile entries: each tile is read once from memory as e4m3, converted to bf16 once by
// the loading threads, and staged in LDS (row stride 272 B: the 16 rows one operand read
// touches fall in distinct banks).  Tiles beyond every query's visible range are written
// as -inf without touching K.  Grid: (ceil(S / kPfQ), B).
// ------------------------------------------------------------------------------------
constexpr int kPfWaves = 8;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfQ = kPfWaves;            // one query per wave
constexpr int kPfSub = 1;                // 64-entry parts per LDS tile (2: one barrier per 128 entries, measured slower: 4 more VGPRs spill)
constexpr int kPfTile = 64 * kPfSub;      // entries per LDS tile
constexpr int kPfStride = 2 * kID + 16;   // LDS row stride in bytes (bf16 rows)

__global__ __launch_bounds__(kPfThreads, 4) void index_score_fp8_prefill(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, const int64_t* __restrict__ q_pos,
    int S, int Nc, int m, float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kPfTile * kPfStride];
  const int b = blockIdx.y;
  const int s0 = blockIdx.x * kPfQ;
  const int l = static_cast<int>(lane_id());
  const int wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const int g = l >> 4;

  // this wave's query (a clamped duplicate of the last one is computed, never stored)
  const int s = s0 + wave;
  const bool qlive = s < S;
  const size_t qrow = static_cast<size_t>(b) * S + min(s, S - 1);
  v8s a[4][4];
  float wv[16];
  load_query(q8, qs, w, qrow, a, wv);
  const int nvis = static_cast<int>(min(static_cast<int64_t>(Nc), (q_pos[qrow] + 1) / m));
  // the workgroup's visible bound (max over its queries) decides which tiles are computed
  int wg_vis = 0;
  for (int j = s0; j < min(S, s0 + kPfQ); ++j) {
    const int64_t t = q_pos[static_cast<size_t>(b) * S + j];
    wg_vis = max(wg_vis, static_cast<int>(min(static_cast<int64_t>(Nc), (t + 1) / m)));
  }

  const uint8_t* kb = k8 + static_cast<size_t>(b) * Nc * kID;
  const float* ksb = ks + static_cast<size_t>(b) * Nc;
  float* out = scores + qrow * Nc;
  const int ntiles_vis = cdiv(wg_vis, kPfTile);

  // cooperative tile load: thread t converts codes 16*(t%8) .. +15 of entry t/8 of each
  // 64-entry part of the tile
  const int le = tid >> 3, lb = 16 * (tid & 7);
  uint4 raw[kPfSub];
  auto gload = [&](int ti) {
#pragma unroll
    for (int j = 0; j < kPfSub; ++j) {
      const int e = min(ti * kPfTile + 64 * j + le, Nc - 1);
      raw[j] = *reinterpret_cast<const uint4*>(kb + static_cast<size_t>(e) * kID + lb);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kPfSub; ++j) {
      const unsigned wd[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
      unsigned cv[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cv[2 * q] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[q], 1.0f, false));
        cv[2 * q + 1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[q], 1.0f, true));
      }
      uint4* dst = reinterpret_cast<uint4*>(&tile[buf][(64 * j + le) * kPfStride + 2 * lb]);
      dst[0] = make_uint4(cv[0], cv[1], cv[2], cv[3]);
      dst[1] = make_uint4(cv[4], cv[5], cv[6], cv[7]);
    }
  };

  if (ntiles_vis > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();
#pragma unroll 1
  for (int ti = 0; ti < ntiles_vis; ++ti) {
    const int buf = ti & 1;
    const bool more = ti + 1 < ntiles_vis;
    // the row scales of this tile, used after its MFMAs (their latency hides behind them)
    float sk[kPfSub];
#pragma unroll
    for (int j = 0; j < kPfSub; ++j) sk[j] = ksb[min(ti * kPfTile + 64 * j + l, Nc - 1)];
    if (more) gload(ti + 1);
#pragma unroll
    for (int j = 0; j < kPfSub; ++j) {
      const int e = ti * kPfTile + 64 * j + l;
      float p[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        v8s bk[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
          bk[k4] = *reinterpret_cast<const v8s*>(&tile[buf][(64 * j + 16 * nb + (l & 15)) * kPfStride + 64 * g + 16 * k4]);
        p[nb] = head_sum1(a, bk, wv);
      }
      const float v = reduce_scatter4(p);
      if (qlive && e < Nc) out[e] = e < nvis ? v * sk[j] : -INFINITY;
    }
    if (more) swrite(buf ^ 1);
    __syncthreads();
  }
  // tiles no query of this workgroup can see
  if (qlive)
    for (int e = ntiles_vis * kPfTile + l; e < Nc; e += 64) out[e] = -INFINITY;
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
      dim3 grid(cdiv(Nc, dec_entries<false>()), B * S);
      hipLaunchKernelGGL(index_score_fp8_decode<false>, grid, dim3(dec_waves<false>() * 64), 0, st,
                         static_cast<const uint8_t*>(q), q_scale, w, static_cast<const uint8_t*>(k),
                         k_scale, q_pos, S, Nc, m, scores, 0, nullptr, size_t{0}, nullptr, nullptr, 0);
    } else {
      dim3 grid(cdiv(S, kPfQ), B);
      hipLaunchKernelGGL(index_score_fp8_prefill, grid, dim3(kPfThreads), 0, st,
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

// Scores and per-segment top-k in one pass (decode shapes, FP8, H_I = 64, d_I = 128), then
// the per-row merge: idx = the k largest of each row, as csa_topk would return.
int launch_topk_merge(uint2* cand, int rows, int G, int k, int32_t* idx, hipStream_t st);
int topk_merge_supported(int G, int k);
size_t topk_merge_pairs_per_row(int G, int k);

int index_topk_segments(int Nc) { return cdiv(Nc, dec_entries<true>()); }

bool index_topk_fused_ok(int S, int Nc, int k) {
  return S <= 4 && k <= dec_entries<true>() && topk_merge_supported(index_topk_segments(Nc), k);
}

// Scores (optional) and every segment's top-k as (key, entry) pairs in cand[rows][G][k];
// b16: the keys in 16-entry blocks; bmax (optional): the block-of-8 maxima of the scores.
int launch_index_segments(const void* q, const float* q_scale, const float* w, const void* k, const float* k_scale,
                          const int64_t* q_pos, int B, int S, int Nc, int m, int ktop, float* scores, uint2* cand,
                          hipStream_t st, bool b16, float* bmax) {
  dim3 grid(index_topk_segments(Nc), B * S);
  const size_t stride = topk_merge_pairs_per_row(index_topk_segments(Nc), ktop);
  const uint8_t* q8 = static_cast<const uint8_t*>(q);
  const uint8_t* k8 = static_cast<const uint8_t*>(k);
  const dim3 block(dec_waves<true>() * 64);
  if (b16 && bmax)
    hipLaunchKernelGGL((index_score_fp8_decode<true, true, false, true>), grid, block, 0, st, q8, q_scale, w, k8,
                       k_scale, q_pos, S, Nc, m, scores, ktop, cand, stride, bmax, nullptr, 0);
  else if (bmax)
    hipLaunchKernelGGL((index_score_fp8_decode<true, false, false, true>), grid, block, 0, st, q8, q_scale, w, k8,
                       k_scale, q_pos, S, Nc, m, scores, ktop, cand, stride, bmax, nullptr, 0);
  else if (b16)
    hipLaunchKernelGGL((index_score_fp8_decode<true, true>), grid, block, 0, st, q8, q_scale, w, k8, k_scale, q_pos,
                       S, Nc, m, scores, ktop, cand, stride, nullptr, nullptr, 0);
  else
    hipLaunchKernelGGL((index_score_fp8_decode<true, false>), grid, block, 0, st, q8, q_scale, w, k8, k_scale, q_pos,
                       S, Nc, m, scores, ktop, cand, stride, nullptr, nullptr, 0);
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

// Reindex over a candidate pool of 8 * n_blk positions (blocks [rows][n_blk] of 8
// positions, -1 = none): scores of the pool (optional, pool order) and each 4096-entry
// segment's top-k as (key, position) pairs, as launch_index_segments writes them for a row
// of 8 * n_blk entries.
int launch_index_pool(const void* q, const float* q_scale, const float* w, const void* k, const float* k_scale,
                      const int64_t* q_pos, const int32_t* blocks, int n_blk, int B, int S, int Nc, int m, int ktop,
                      float* scores, uint2* cand, hipStream_t st) {
  const int P = 8 * n_blk;
  dim3 grid(index_topk_segments(P), B * S);
  const size_t stride = topk_merge_pairs_per_row(index_topk_segments(P), ktop);
  hipLaunchKernelGGL((index_score_fp8_decode<true, false, true, false>), grid, dim3(dec_waves<true>() * 64), 0, st,
                     static_cast<const uint8_t*>(q), q_scale, w, static_cast<const uint8_t*>(k), k_scale, q_pos, S,
                     Nc, m, scores, ktop, cand, stride, nullptr, blocks, n_blk);
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

// Keys in 16-entry blocks: block j of a sequence holds entries 16j .. 16j+15 as four
// 512-byte pieces; piece p holds bytes 32p .. 32p+31 of each of the 16 entries (32 bytes
// per entry, entry order).  Entries past Nc in the last block are zero.  One workgroup of
// 64 threads per block: thread t copies piece t/16 of entry t%16.
__global__ __launch_bounds__(64) void index_keys_b16(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                     int Nc) {
  const int nblk = static_cast<int>(gridDim.x), blk = static_cast<int>(blockIdx.x), b = static_cast<int>(blockIdx.y);
  const int t = static_cast<int>(threadIdx.x), e = 16 * blk + (t & 15), pc = t >> 4;
  const uint4* s = reinterpret_cast<const uint4*>(src + (static_cast<size_t>(b) * Nc + min(e, Nc - 1)) * kID + 32 * pc);
  uint4 lo = s[0], hi = s[1];
  if (e >= Nc) lo = hi = make_uint4(0u, 0u, 0u, 0u);
  uint4* d = reinterpret_cast<uint4*>(dst + (static_cast<size_t>(b) * nblk + blk) * (16 * kID) + pc * 512 + (t & 15) * 32);
  d[0] = lo;
  d[1] = hi;
}

size_t index_keys_b16_bytes(int B, int Nc) { return static_cast<size_t>(B) * cdiv(Nc, 16) * 16 * kID; }

int launch_index_keys_b16(const void* src, void* dst, int B, int Nc, hipStream_t st) {
  hipLaunchKernelGGL(index_keys_b16, dim3(cdiv(Nc, 16), B), dim3(64), 0, st, static_cast<const uint8_t*>(src),
                     static_cast<uint8_t*>(dst), Nc);
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

int launch_index_topk(const void* q, const float* q_scale, const float* w, const void* k, const float* k_scale,
                      const int64_t* q_pos, int B, int S, int Nc, int m, int ktop, float* scores, int32_t* idx,
                      void* ws, hipStream_t st) {
  uint2* cand = static_cast<uint2*>(ws);
  const int rc = launch_index_segments(q, q_scale, w, k, k_scale, q_pos, B, S, Nc, m, ktop, scores, cand, st, false,
                                       nullptr);
  if (rc != CSA_OK) return rc;
  return launch_topk_merge(cand, B * S, index_topk_segments(Nc), ktop, idx, st);
}

}  // namespace csa
