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
// bf16 kernel (H = 64 heads, c = 512).  A workgroup owns one query, some groups of 16
// heads and a contiguous range of 32-row chunks of its row set; its 8 waves are (head
// group, channel part) pairs.  Two shapes: channel quarters (2 head groups per workgroup,
// two workgroups per query: more workgroups for few queries) and channel halves (all 4
// head groups in one workgroup, so each row read from memory serves all 64 heads: for
// many queries or long row sets).  Per chunk:
//   1. the 32 rows sit in one of three LDS slots; each wave loads 4 of them (16 bytes per
//      lane per row) into one of two register sets four chunks ahead of the chunk being
//      finished and writes a set to its slot two chunks ahead.  (Direct global->LDS
//      loads measured at about half the gather rate of register loads here.)  Row
//      stride 1056 B: rows shift by 8 banks, so the 8 rows that 32 lanes of a
//      transposed read touch never share a bank (measured: 1/5 of the conflict cycles
//      of a 12-bank shift);
//   2. every wave computes its part's share of S^T = KV_chunk . Q^T for its 16 heads on
//      MFMA (A = rows from LDS, B = its Q part in registers); the shares of a head group
//      are summed through LDS (fixed order, so its waves hold the identical S^T).  The
//      shares of chunk c+1 are formed in the same step as chunk c is finished (two
//      exchange buffers), so one barrier per chunk orders everything;
//   3. online softmax in the log2 domain with a lazy reference: the running maximum is
//      only moved (and O rescaled) when a chunk exceeds it by more than 2^8, which leaves
//      the result unchanged (numerator and denominator share the reference);
//   4. O_part += P . V on MFMA with V read from the same LDS rows (K = V) through
//      ds_read_b64_tr_b16: in each 16-lane group, output lane i' slot j' receives input
//      lane 4j'+i'/4 slot i'%4, so lanes 4j'..4j'+3 reading 16 columns of row R(j') hand
//      every lane its column of 4 rows.  The S^T output layout (lane: head l%16, rows
//      4*(l/16)+i and 16+4*(l/16)+i) is the A-operand layout of P under the matching
//      k-slot order, so P never leaves registers.  P enters as a bf16 hi + lo pair (two
//      MFMAs on one V operand) so it keeps ~16 bits.
// The remote rows come from idx (CSA), from every visible entry (HCA), or from a
// selection each workgroup makes itself from the segment top-k candidates of the indexer
// pass (the k best of G*k (key, entry) pairs, with the selection core of select.hpp), so
// that selection and attention are one launch.
// A row set split over several workgroups writes (m, l, O) partials that attn_merge_tiles
// combines with the sink (LSE merge).  (Merging in the last workgroup of a query instead
// measured far slower: its device-scope release writes back the XCD's whole L2.)  Workgroups are numbered so that all workgroups
// of one query land on the same XCD (consecutive workgroup ids go round-robin over the
// 8 XCDs) and share its L2 for the rows they all read.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "attention_common.hpp"
#include "select.hpp"

namespace csa {

constexpr int kRing = 3;                            // chunks resident in LDS
constexpr int kValidSlots = 4;                      // row-mask slots (kRing, padded)

// Workgroup shape: kWaves waves = (head group, channel part) pairs with kParts channel
// parts per head group (4: quarters, 2: halves).
template <int kParts, int kWaves>
struct AttnShape {
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kRowsPerWave = kRows / kWaves;   // rows of a chunk each wave loads
  // chunks of row loads in flight (register sets of kRowsPerWave rows).  (4 measured
  // slower for decode splits of 5 chunks: the loads past a split's end double.)
  static constexpr int kDepth = 2;
  // splits of at most this many chunks may load all of them at once (the quarter-channel
  // shape, whose registers have room for them)
  static constexpr int kAllChunks = kParts == 4 ? 4 : 0;
  static constexpr int kPart = kAC / kParts;            // channels per wave
  static constexpr int kWGHG = kWaves / kParts;         // head groups per workgroup
  static constexpr int kUnits = kNHG / kWGHG;           // workgroups per (query, split)
  // S^T share buffers: two (shares of chunk c+1 formed while chunk c's are read, one
  // barrier per chunk) when they fit next to the ring, else one and a second barrier
  static constexpr int kSxBytes = kWaves * kWave * 8 * 4;
  static constexpr int kSxBufs = kWaves <= 8 ? 2 : 1;
  static constexpr int kLdsFixed = kRing * kChunkBytes + kSxBufs * kSxBytes + kValidSlots * kWaves * 4;
  static constexpr int kLdsMax = kLdsFixed + kMaxSplitChunks * kRows * 8;
  static_assert(kLdsMax <= 160 * 1024, "LDS of one compute unit");
  // candidate selection (8 or 16 keys per thread) and its result sit in the ring before it is used
  static constexpr int kMaxCand = 8 * kThreads;
  static constexpr int kMaxCand2 = 16 * kThreads;
  static_assert(sizeof(TkShared) + 4 * kMaxCand2 <= kRing * kChunkBytes, "selection fits the ring");
  static_assert(kRowsPerWave == 4 || kRowsPerWave == 2, "the row staging moves 4 or 2 rows per wave");
  static_assert(kWGHG >= 1 && kWGHG <= kNHG, "head groups per workgroup");
};
// the 64-head shape (all head groups in one workgroup) once a call has this many queries:
// 8 waves = 4 head groups x channel halves.  (16 waves x channel quarters fits 128 VGPRs
// for 4 waves per SIMD, but the 4-way share exchange, the second barrier and spills made
// HCA decode 1.3x slower.)
constexpr int kWideMinQueries = 64;
constexpr int kWideParts = 2;
constexpr int kWideWaves = 8;

// Source of the rows that are absent (index -1, padding, chunks past a split's end):
// every chunk is the same loads per wave, so the compiler's count of loads in flight is
// the same on every path.  Many zero rows, so that these reads spread over the L2
// channels (all workgroups reading one line serialise on one channel); the low address
// bit marks an absent row in the row table.
constexpr int kZeroRows = 64;
__device__ __attribute__((aligned(1024))) uint16_t g_zero_rows[kZeroRows * kAC];


// ---- merge of split partials (attn_merge_tiles, and the last workgroup of a query in
// attn_bf16).  The partials are in register order: for (query qi, head group hg,
// 16-channel tile ct), lane l holds heads 16*hg + 4*(l/16) + i and channel 16*ct + l%16.

// Merges the nsplit partials of one wave's KT tiles with the sink and stores them (every
// load in flight at once for up to 4 splits, or up to kMergeAllSplits with one tile, else
// one split's at a time).
constexpr int kMergeAllSplits = 16;
template <int KT>
__device__ __forceinline__ void merge_splits(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                             const float* __restrict__ sink, int nsplit, size_t qi, int hg, int ct0,
                                             uint16_t* __restrict__ out, float* __restrict__ lse,
                                             const int64_t* __restrict__ q_pos, int rope_d, double rope_r) {
  constexpr int kTiles = kAC / 16;
  const int l = static_cast<int>(lane_id());
  const int h0 = kHG * hg + 4 * (l >> 4);
  float M[4], den[4], acc[KT][4], sk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sk[i] = sink[h0 + i];
    M[i] = sk[i] * kLog2e;
#pragma unroll
    for (int t = 0; t < KT; ++t) acc[t][i] = 0.0f;
  }
  auto ml_of = [&](int sp, v4f& a, v4f& b) __attribute__((always_inline)) {
    const v4f* p = reinterpret_cast<const v4f*>(part_ml + ((qi * nsplit + sp) * kAH + h0) * 2);
    a = p[0];                                                 // m0 l0 m1 l1
    b = p[1];                                                 // m2 l2 m3 l3
  };
  auto po_of = [&](int sp, int ct) __attribute__((always_inline)) {
    return *reinterpret_cast<const v4f*>(part_o + (((qi * nsplit + sp) * kNHG + hg) * kTiles + ct) * (kWave * 4) +
                                         4 * l);
  };
  if (nsplit <= 4) {
    // every load of the wave in flight at once
    v4f ma[4], mb[4], x[4][KT];
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
      if (sp < nsplit) {
        ml_of(sp, ma[sp], mb[sp]);
#pragma unroll
        for (int t = 0; t < KT; ++t) x[sp][t] = po_of(sp, ct0 + t);
      }
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
      if (sp < nsplit) {
        M[0] = fmaxf(M[0], ma[sp][0]); M[1] = fmaxf(M[1], ma[sp][2]);
        M[2] = fmaxf(M[2], mb[sp][0]); M[3] = fmaxf(M[3], mb[sp][2]);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) den[i] = M[i] == -INFINITY ? 0.0f : exp2f(sk[i] * kLog2e - M[i]);
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
      if (sp < nsplit) {
        const float mi[4] = {ma[sp][0], ma[sp][2], mb[sp][0], mb[sp][2]};
        const float li[4] = {ma[sp][1], ma[sp][3], mb[sp][1], mb[sp][3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float wgt = mi[i] == -INFINITY ? 0.0f : exp2f(mi[i] - M[i]);
          den[i] = fmaf(wgt, li[i], den[i]);
#pragma unroll
          for (int t = 0; t < KT; ++t) acc[t][i] = fmaf(wgt, x[sp][t][i], acc[t][i]);
        }
      }
    merge_store<KT>(acc, den, M, qi, h0, ct0, l, out, lse, q_pos, rope_d, rope_r);
    return;
  }
  if constexpr (KT == 1) {
    if (nsplit <= kMergeAllSplits) {
      // one tile: every split's loads in flight at once (a loop over the splits would
      // wait for each one in turn); the same arithmetic in the same split order
      v4f ma[kMergeAllSplits], mb[kMergeAllSplits], x[kMergeAllSplits];
#pragma unroll
      for (int sp = 0; sp < kMergeAllSplits; ++sp)
        if (sp < nsplit) {
          ml_of(sp, ma[sp], mb[sp]);
          x[sp] = po_of(sp, ct0);
        }
#pragma unroll
      for (int sp = 0; sp < kMergeAllSplits; ++sp)
        if (sp < nsplit) {
          M[0] = fmaxf(M[0], ma[sp][0]); M[1] = fmaxf(M[1], ma[sp][2]);
          M[2] = fmaxf(M[2], mb[sp][0]); M[3] = fmaxf(M[3], mb[sp][2]);
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) den[i] = M[i] == -INFINITY ? 0.0f : exp2f(sk[i] * kLog2e - M[i]);
#pragma unroll
      for (int sp = 0; sp < kMergeAllSplits; ++sp)
        if (sp < nsplit) {
          const float mi[4] = {ma[sp][0], ma[sp][2], mb[sp][0], mb[sp][2]};
          const float li[4] = {ma[sp][1], ma[sp][3], mb[sp][1], mb[sp][3]};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float wgt = mi[i] == -INFINITY ? 0.0f : exp2f(mi[i] - M[i]);
            den[i] = fmaf(wgt, li[i], den[i]);
            acc[0][i] = fmaf(wgt, x[sp][i], acc[0][i]);
          }
        }
      merge_store<KT>(acc, den, M, qi, h0, ct0, l, out, lse, q_pos, rope_d, rope_r);
      return;
    }
  }
  for (int sp = 0; sp < nsplit; ++sp) {
    v4f a, b;
    ml_of(sp, a, b);
    M[0] = fmaxf(M[0], a[0]); M[1] = fmaxf(M[1], a[2]);
    M[2] = fmaxf(M[2], b[0]); M[3] = fmaxf(M[3], b[2]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) den[i] = M[i] == -INFINITY ? 0.0f : exp2f(sk[i] * kLog2e - M[i]);
  for (int sp = 0; sp < nsplit; ++sp) {
    v4f a, b;
    ml_of(sp, a, b);
    v4f x[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) x[t] = po_of(sp, ct0 + t);
    const float mi[4] = {a[0], a[2], b[0], b[2]};
    const float li[4] = {a[1], a[3], b[1], b[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float wgt = mi[i] == -INFINITY ? 0.0f : exp2f(mi[i] - M[i]);
      den[i] = fmaf(wgt, li[i], den[i]);
#pragma unroll
      for (int t = 0; t < KT; ++t) acc[t][i] = fmaf(wgt, x[t][i], acc[t][i]);
    }
  }
  merge_store<KT>(acc, den, M, qi, h0, ct0, l, out, lse, q_pos, rope_d, rope_r);
}

// One wave's result (head group hg, channels kPart*part .. +kPart-1; O unnormalised, its
// reference maximum m_ref in log2 units, l_run this lane's share of the per-head sums):
// with one split the output (sink in the denominator, inverse RoPE, bf16) and the lse,
// else the split's partial in register order for attn_merge_tiles.
template <int kPart>
__device__ __forceinline__ void attn_finish(const AttnArgs& a, const v4f (&o)[kPart / 16], float m_ref, float l_run,
                                            int qi, int split, int hg, int part) {
  const int l = static_cast<int>(lane_id());
  const int g = l >> 4;
  float l_tot = l_run + wave_xor(l_run, 16);
  l_tot += wave_xor(l_tot, 32);
  const int head_l = kHG * hg + (l & 15);             // head whose statistics this lane holds
  const int col0 = kPart * part + (l & 15);
  if (a.nsplit == 1) {
    const float sink2 = a.sink[head_l] * kLog2e;
    const float M = fmaxf(m_ref, sink2);
    float f, lse2;
    if (M == -INFINITY) {
      f = 0.0f;
      lse2 = -INFINITY;
    } else {
      const float em = m_ref == -INFINITY ? 0.0f : exp2f(m_ref - M);
      const float den = l_tot * em + exp2f(sink2 - M);
      f = den > 0.0f ? em / den : 0.0f;
      lse2 = M + log2f(den);
    }
    if (a.lse && part == 0 && g == 0) a.lse[static_cast<size_t>(qi) * kAH + head_l] = lse2 * kLn2;
    float fh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fh[i] = __shfl(f, 4 * g + i, kWave);
    uint16_t* ob = a.out + (static_cast<size_t>(qi) * kAH + kHG * hg) * kAC;
    const int64_t tq = a.rope_d > 0 ? a.q_pos[qi] : 0;
#pragma unroll
    for (int t = 0; t < kPart / 16; ++t) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = o[t][i] * fh[i];
      // inverse RoPE of the output (the tile's 16 columns: lane pairs hold channel pairs)
      if (a.rope_d > 0 && kPart * part + 16 * t + 16 > kAC - a.rope_d) {
        const int col = col0 + 16 * t;
        float cs = 1.0f, sn = 0.0f;
        if (col >= kAC - a.rope_d) rope_cs_sn(col, kAC, a.rope_d, a.rope_r, tq, cs, sn);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = rope_back(v[i], pair_lane(v[i]), col, cs, sn);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) ob[(4 * g + i) * kAC + col0 + 16 * t] = f32_to_bf16(v[i]);
    }
  } else {
    const size_t pbase = static_cast<size_t>(qi) * a.nsplit + split;
    if (part == 0 && g == 0) {
      a.part_ml[(pbase * kAH + head_l) * 2 + 0] = m_ref;
      a.part_ml[(pbase * kAH + head_l) * 2 + 1] = l_tot;
    }
    // the partial in register order: [head group][16-channel tile][lane][4 heads], 16
    // bytes per lane per store
    float* po = a.part_o + ((pbase * kNHG + hg) * (kAC / 16) + kPart / 16 * part) * (kWave * 4) + 4 * l;
#pragma unroll
    for (int t = 0; t < kPart / 16; ++t) *reinterpret_cast<v4f*>(po + t * (kWave * 4)) = o[t];
  }
}

template <int kSrc, int kParts, int kWaves, int kFmt = kFmtBf16, bool kShort = false>
__global__ __launch_bounds__(kWaves * kWave, 1) void attn_bf16(AttnArgs a) {
  constexpr bool kDense = kSrc == kSrcDense;
  constexpr bool kCand = kSrc == kSrcCand || kSrc == kSrcCand2;
  constexpr int kCandChunks = kSrc == kSrcCand2 ? 2 : 1;   // 8 candidates per thread per chunk
  using Sh = AttnShape<kParts, kWaves>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* ring = smem;                                                          // [slot][32 rows]
  float* sx = reinterpret_cast<float*>(smem + kRing * kChunkBytes);              // [buffer][wave][lane][8]
  int* validw = reinterpret_cast<int*>(smem + kRing * kChunkBytes + Sh::kSxBufs * Sh::kSxBytes);  // [slot][wave]
  uint64_t* rowptr = reinterpret_cast<uint64_t*>(validw + kValidSlots * kWaves);  // the split's row addresses

  // ---- workgroup -> (query, head groups, split)
  int qi, u;
  if (!attn_unit(a.nq, Sh::kUnits * a.nsplit, qi, u)) return;
  const int hp = u % Sh::kUnits, split = u / Sh::kUnits;
  const int b = qi / a.S, s = qi % a.S;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int hg = Sh::kWGHG * hp + wave / kParts;      // this wave's head group
  const int part = wave % kParts;                     // this wave's channel part
  const int l = static_cast<int>(lane_id());
  const int g = l >> 4;

  int w_lo, n_swa;
  window_rows(s, a.S, a.Ls, a.W, last_position(a.q_pos, b, a.S), w_lo, n_swa);
  const int n_rem = kDense ? static_cast<int>(min(static_cast<int64_t>(a.Nc), (a.q_pos[qi] + 1) / a.m)) : a.k;
  const int n_slots = n_swa + n_rem;
  const int n_chunks = cdiv(n_slots, kRows);
  const int ch0 = split * a.chunks_per_split;
  const int ch1 = min(n_chunks, ch0 + a.chunks_per_split);

  constexpr int kRowBytes = kv_row_bytes(kFmt);
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(a.kv) + static_cast<size_t>(b) * a.Nc * kRowBytes;
  const uint16_t* swab = a.swa + static_cast<size_t>(b) * a.Ls * kAC;
  const int32_t* idxq = kSrc == kSrcIdx ? a.idx + static_cast<size_t>(qi) * a.k : nullptr;

  // Q part of the 16 heads as the B operand: lane l holds head 16*hg + l%16,
  // channels kPart*part + 32*ks + 8*g .. +7.  These loads complete under the waits of
  // the row table below (one memory latency for both).
  v8s qb[Sh::kPart / 32];
  {
    const uint16_t* qh = a.q + (static_cast<size_t>(qi) * kAH + kHG * hg + (l & 15)) * kAC + Sh::kPart * part;
#pragma unroll
    for (int ks = 0; ks < Sh::kPart / 32; ++ks) qb[ks] = *reinterpret_cast<const v8s*>(qh + 32 * ks + 8 * g);
  }

  // Selection from candidates: the query's n_cand (key, entry) pairs (segment-major, each
  // segment in entry order, key 0 = empty; rows cand_stride pairs apart) -> the k best in
  // entry order, as the top-k stage returns them, in LDS (sel) for the row table; the
  // first workgroup of the query also writes them to idx_out.  Every workgroup of the
  // query selects for itself (the same result); the ring is free until the pipeline starts.
  int32_t* sel = reinterpret_cast<int32_t*>(ring + sizeof(TkShared));
  if constexpr (kCand) {
    constexpr int NU = kCandChunks;
    TkShared& tsh = *reinterpret_cast<TkShared*>(ring);
    const uint2* cq = a.cand + static_cast<size_t>(qi) * a.cand_stride;
    uint32_t key[NU][8], ent[NU][8];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int p0 = 8 * (static_cast<int>(threadIdx.x) + u * Sh::kThreads);
      if ((a.n_cand & 1) == 0 && p0 + 7 < a.n_cand) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 v = reinterpret_cast<const uint4*>(cq + p0)[j];
          key[u][2 * j] = v.x; ent[u][2 * j] = v.y;
          key[u][2 * j + 1] = v.z; ent[u][2 * j + 1] = v.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint2 v = p0 + j < a.n_cand ? cq[p0 + j] : make_uint2(0u, 0u);
          key[u][j] = v.x; ent[u][j] = v.y;
        }
      }
    }
    uint64_t taken;
    int obase[NU];
    const int kk = select_regs<Sh::kThreads, 8, NU>(tsh, key, a.k, taken, obase);
    int32_t* io = a.idx_out && split == 0 && hp == 0 ? a.idx_out + static_cast<size_t>(qi) * a.k : nullptr;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      int o = obase[u];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((taken >> (8 * u + j)) & 1ull) {
          sel[o] = static_cast<int32_t>(ent[u][j]);
          if (io) io[o] = static_cast<int32_t>(ent[u][j]);
          ++o;
        }
    }
    for (int p = kk + static_cast<int>(threadIdx.x); p < a.k; p += Sh::kThreads) {
      sel[p] = -1;
      if (io) io[p] = -1;
    }
    __syncthreads();
  }

  // The address of every row of the split (window row, selected or visible entry, or a
  // zero row with the low bit set for absent ones), computed once by all threads.
  const uint64_t zero_rows = reinterpret_cast<uint64_t>(static_cast<const uint16_t*>(g_zero_rows));
  {
    const int nsl = (ch1 - ch0) * kRows;
    for (int e = static_cast<int>(threadIdx.x); e < nsl; e += Sh::kThreads) {
      const int slot = ch0 * kRows + e;
      uint64_t p = (zero_rows + static_cast<uint64_t>(e % kZeroRows) * (kAC * 2)) | 1u;
      if (slot < n_swa) {
        p = reinterpret_cast<uint64_t>(swab + static_cast<size_t>(w_lo + slot) * kAC);
      } else if (slot < n_slots) {
        const int j = kDense ? slot - n_swa : kCand ? sel[slot - n_swa] : idxq[slot - n_swa];
        // a compressed row of another format carries bit 1 (its address is a multiple of 8)
        if (j >= 0 && j < a.Nc)
          p = reinterpret_cast<uint64_t>(kvb + static_cast<size_t>(j) * kRowBytes) | (kFmt != kFmtBf16 ? 2u : 0u);
      }
      rowptr[e] = p;
    }
    // Q complete before any row load: otherwise the compiler's wait for Q inside the
    // loop becomes a wait for all rows in flight
    __builtin_amdgcn_s_waitcnt(0x0f70);               // vmcnt(0)
    __syncthreads();
  }

  // The wave's 4 (or 2) rows of chunk CH (zero rows for chunks past the split): addresses
  // from the table with 16-byte LDS reads, then one 16-byte load per lane per row,
  // non-temporal, so that the rows streaming through L2 evict less of the split partials
  // the merge reads back (Flash decode call 25.1 -> 24.1 us).
#define CSA_ATT_LOAD1(ST, VM, R, PTR)                                                   \
  do {                                                                                 \
    const uint64_t p_ = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>((PTR) >> 32))) << 32) | \
                        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(PTR)));   \
    (VM) |= static_cast<uint32_t>(~p_ & 1u) << (R);                                    \
    if (kFmt != kFmtBf16 && (p_ & 2u)) {             /* raw share, decoded at the store */ \
      (VM) |= 1u << (8 + (R));                                                         \
      (ST)[R] = load_row8<kFmt>(p_ & ~static_cast<uint64_t>(3), l);                   \
    } else                                                                             \
      (ST)[R] = __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) v4u*>(p_ & ~static_cast<uint64_t>(1)) + l);  \
  } while (0)
#define CSA_ATT_LOAD(CH, ST, VM)                                                        \
  do {                                                                                 \
    uint64_t q_[4];                                                                    \
    if ((CH) < ch1) {                                                                  \
      const uint64_t* t_ = rowptr + ((CH) - ch0) * kRows + Sh::kRowsPerWave * wave;    \
      const ulonglong2 a_ = reinterpret_cast<const ulonglong2*>(t_)[0];                 \
      q_[0] = a_.x; q_[1] = a_.y;                                                      \
      if constexpr (Sh::kRowsPerWave == 4) {                                           \
        const ulonglong2 b_ = reinterpret_cast<const ulonglong2*>(t_)[1];               \
        q_[2] = b_.x; q_[3] = b_.y;                                                    \
      }                                                                                \
    } else {                                                                           \
      const uint64_t z_ = zero_rows | 1u;                                              \
      const int r_ = ((CH) * kRows + Sh::kRowsPerWave * wave) & (kZeroRows - 1);       \
      q_[0] = z_ + static_cast<uint64_t>(r_) * (kAC * 2);                              \
      q_[1] = z_ + static_cast<uint64_t>(r_ + 1) * (kAC * 2);                          \
      q_[2] = z_ + static_cast<uint64_t>(r_ + 2) * (kAC * 2);                          \
      q_[3] = z_ + static_cast<uint64_t>(r_ + 3) * (kAC * 2);                          \
    }                                                                                  \
    (VM) = 0;                                                                          \
    CSA_ATT_LOAD1(ST, VM, 0, q_[0]); CSA_ATT_LOAD1(ST, VM, 1, q_[1]);                  \
    if constexpr (Sh::kRowsPerWave == 4) {                                             \
      CSA_ATT_LOAD1(ST, VM, 2, q_[2]); CSA_ATT_LOAD1(ST, VM, 3, q_[3]);                \
    }                                                                                  \
  } while (0)
#define CSA_ATT_STORE1(BUF, ST, R, VM)                                                  \
  do {                                                                                 \
    if (kFmt != kFmtBf16 && (((VM) >> (8 + (R))) & 1u)) (ST)[R] = decode_row8<kFmt>((ST)[R], l); \
    *reinterpret_cast<v4u*>((BUF) + (Sh::kRowsPerWave * wave + (R)) * kRowStride + 16 * l) = (ST)[R]; \
  } while (0)
#define CSA_ATT_STORE(SLOT, ST, VM)                                                     \
  do {                                                                                 \
    uint8_t* buf_ = ring + (SLOT) * kChunkBytes;                                       \
    CSA_ATT_STORE1(buf_, ST, 0, VM); CSA_ATT_STORE1(buf_, ST, 1, VM);                  \
    if constexpr (Sh::kRowsPerWave == 4) {                                             \
      CSA_ATT_STORE1(buf_, ST, 2, VM); CSA_ATT_STORE1(buf_, ST, 3, VM);                \
    }                                                                                  \
    if (l == 0) validw[(SLOT) * kWaves + wave] = static_cast<int>((VM) & 0xffu);       \
  } while (0)

  v4f o[Sh::kPart / 16];
#pragma unroll
  for (int t = 0; t < Sh::kPart / 16; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;   // per head l%16 (log2 units)
  float l_run = 0.0f;        // this lane's share of the per-head sum

  // This wave's share of S^T (32 rows x 16 heads) over its channel part for the chunk in
  // ring slot SL, written to exchange buffer XB.
  auto s_part = [&](int sl, int xb) __attribute__((always_inline)) {
    const uint8_t* buf = ring + sl * kChunkBytes;
    v4f st[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < Sh::kPart / 32; ++ks) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const v8s av = *reinterpret_cast<const v8s*>(buf + (16 * rb + (l & 15)) * kRowStride + 2 * Sh::kPart * part +
                                                     64 * ks + 16 * g);
        st[rb] = mfma_bf16_16x16x32(av, qb[ks], st[rb]);
      }
    }
    float* w = sx + (xb & (Sh::kSxBufs - 1)) * (Sh::kSxBytes / 4) + (wave * kWave + l) * 8;
    *reinterpret_cast<v4f*>(w) = st[0];
    *reinterpret_cast<v4f*>(w + 4) = st[1];
  };

  // Chunk in ring slot SL whose S^T shares are in exchange buffer XB: online softmax and
  // O_part += P . V; the S^T share of the next chunk (slot SN, buffer XN) is formed
  // between the two, in the same basic block as the exponentials and P . V, so that its
  // MFMAs can overlap them (NEXT false: no next chunk).
  auto softmax_pv = [&](int sl, int xb, int sn, int xn, auto next) __attribute__((always_inline)) {
    const uint8_t* buf = ring + sl * kChunkBytes;
    float sv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sv[j] = 0.0f;
#pragma unroll
    for (int w = 0; w < kParts; ++w) {                // fixed order: identical sums in the group's waves
      const float* src = sx + (xb & (Sh::kSxBufs - 1)) * (Sh::kSxBytes / 4) + ((wave & ~(kParts - 1)) + w) * kWave * 8 +
                         l * 8;
      const v4f x0 = *reinterpret_cast<const v4f*>(src);
      const v4f x1 = *reinterpret_cast<const v4f*>(src + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] += x0[i];
        sv[4 + i] += x1[i];
      }
    }
    // ---- online softmax; slot j <-> chunk row 16*(j/4) + 4*g + j%4
    uint32_t vmask = 0;
#pragma unroll
    for (int w4 = 0; w4 < kWaves / 4; ++w4) {               // the waves' row masks, in row order
      constexpr int R = Sh::kRowsPerWave;
      const int4 v = *reinterpret_cast<const int4*>(validw + sl * kWaves + 4 * w4);
      vmask |= (static_cast<uint32_t>(v.x) << (R * (4 * w4))) | (static_cast<uint32_t>(v.y) << (R * (4 * w4 + 1))) |
               (static_cast<uint32_t>(v.z) << (R * (4 * w4 + 2))) | (static_cast<uint32_t>(v.w) << (R * (4 * w4 + 3)));
    }
    float lmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 16 * (j >> 2) + 4 * g + (j & 3);
      sv[j] = (vmask >> row) & 1u ? sv[j] * a.scale_log2 : -INFINITY;
      lmax = fmaxf(lmax, sv[j]);
    }
    // the reference moves only when some logit exceeds it by more than kLazy; then the
    // per-head maximum over the 4 lane groups is taken
    if (__ballot(lmax > m_ref + kLazy)) {
      float cmax = fmaxf(lmax, wave_xor(lmax, 16));
      cmax = fmaxf(cmax, wave_xor(cmax, 32));
      const bool move = cmax > m_ref + kLazy;
      const float m_new = move ? cmax : m_ref;
      const float alpha = move ? exp2f(m_ref - m_new) : 1.0f;      // 0 when m_ref = -inf
      l_run *= alpha;
      m_ref = m_new;
      float ah[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ah[i] = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
      for (int t = 0; t < Sh::kPart / 16; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[t][i] *= ah[i];
    }
    const float m_use = m_ref == -INFINITY ? 0.0f : m_ref;
    // P = P_hi + P_lo, both bf16: the two products with V keep P to ~16 bits
    float psum = 0.0f;
    v8s pa, pb;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
      typedef float v2f __attribute__((ext_vector_type(2)));
      // v_exp_f32: results below 2^-126 flush to 0, far below the >= 1 of the chunk's top weight
      const v2f p = {__builtin_amdgcn_exp2f(sv[j] - m_use), __builtin_amdgcn_exp2f(sv[j + 1] - m_use)};
      psum += p[0] + p[1];
      const v2bf hi = __builtin_convertvector(p, v2bf);
      const uint32_t hb = __builtin_bit_cast(uint32_t, hi);
      const v2f r = {p[0] - __uint_as_float(hb << 16), p[1] - __uint_as_float(hb & 0xffff0000u)};
      const uint32_t lb = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, v2bf));
      pa[j] = static_cast<short>(hb & 0xffffu);
      pa[j + 1] = static_cast<short>(hb >> 16);
      pb[j] = static_cast<short>(lb & 0xffffu);
      pb[j + 1] = static_cast<short>(lb >> 16);
    }
    l_run += psum;
    if constexpr (decltype(next)::value) {
      if constexpr (Sh::kSxBufs == 1) barrier_lds();     // every wave has read the one share buffer
      s_part(sn, xn);
    }
    // ---- O_part += P . V; lane (g, i) reads row 4g + i/4 (and 16 + ...) at columns 4*(i%4) ..
    const uint8_t* vt = buf + (4 * g + ((l & 15) >> 2)) * kRowStride + 2 * Sh::kPart * part + 8 * (l & 3);
#pragma unroll
    for (int t = 0; t < Sh::kPart / 16; ++t) {
      const v4s v0 = lds_read_tr16(vt + 32 * t);
      const v4s v1 = lds_read_tr16(vt + 32 * t + 16 * kRowStride);
      const v8s vb = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      o[t] = mfma_bf16_16x16x32(pa, vb, o[t]);
      o[t] = mfma_bf16_16x16x32(pb, vb, o[t]);
    }
  };

  // Pipeline over chunks c (ring slot c % 3, exchange buffer c % 2) with kDepth register
  // sets of row loads in flight, kDepth chunks per loop trip (no exit between them, which
  // keeps the compiler's load counts exact; the last ch1 - ch < kDepth chunks are finished
  // after the loop): step c finishes chunk c (its shares were exchanged before the last
  // barrier) and forms the S^T share of chunk c+1, moves chunk c+2 from registers into its
  // slot and starts the loads of chunk c+2+kDepth into the set it freed; one barrier per
  // chunk.  Chunk x lives in set (x - ch0) % kDepth.  Every step issues its loads, also
  // past the split's end (zero rows), so the count of loads in flight is the same on every
  // path and the compiler's waits before a store only cover the set being stored; stores
  // past the end go to a slot no later step reads for a result.
  // kShort (splits of at most kAllChunks chunks, e.g. long-context decode) loads every
  // chunk at once, so the split waits for one memory latency instead of one per kDepth
  // chunks; chunks past the split's end are zero rows, loaded but neither stored nor
  // computed.  All loads are issued before the first store, so the compiler's count of
  // loads in flight is exact on every path.  (A separate instantiation: compiled into the
  // pipelined kernel, this path's registers slowed that kernel down.)
  const int n_loc = ch1 - ch0;
  if constexpr (kShort) {
    static_assert(Sh::kAllChunks > 0, "short splits need the quarter-channel shape");
    constexpr int kA = Sh::kAllChunks;
    v4u sa[kA][4];
    uint32_t va[kA];
#pragma unroll
    for (int i = 0; i < kA; ++i) CSA_ATT_LOAD(ch0 + i, sa[i], va[i]);
    CSA_ATT_STORE(0, sa[0], va[0]);
    barrier_lds();
    s_part(0, 0);
    if (n_loc > 1) CSA_ATT_STORE(1, sa[1], va[1]);
    barrier_lds();
#pragma unroll
    for (int j = 0; j < kA; ++j) {
      if (j < n_loc) {                                  // uniform over the workgroup
        const int s0 = j % kRing, s1 = (j + 1) % kRing, s2 = (j + 2) % kRing;
        if (j + 1 < n_loc) {
          softmax_pv(s0, j & 1, s1, (j + 1) & 1, std::true_type{});
          if (j + 2 < kA && j + 2 < n_loc) CSA_ATT_STORE(s2, sa[j + 2], va[j + 2]);
          barrier_lds();
        } else {
          softmax_pv(s0, j & 1, s0, j & 1, std::false_type{});
        }
      }
    }
  } else {
    constexpr int kDepth = Sh::kDepth;
    v4u st[kDepth][4];
    uint32_t vm[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth; ++i) CSA_ATT_LOAD(ch0 + i, st[i], vm[i]);
    int sl = ch0 % kRing;                               // slot of chunk ch
    const int sl1 = sl == kRing - 1 ? 0 : sl + 1;
    CSA_ATT_STORE(sl, st[0], vm[0]);
    CSA_ATT_LOAD(ch0 + kDepth, st[0], vm[0]);
    barrier_lds();
    s_part(sl, ch0 & 1);
    CSA_ATT_STORE(sl1, st[1], vm[1]);
    CSA_ATT_LOAD(ch0 + kDepth + 1, st[1], vm[1]);
    barrier_lds();
    int ch = ch0;
#pragma unroll 1
    for (; ch + kDepth - 1 < ch1; ch += kDepth) {
#pragma unroll
      for (int i = 0; i < kDepth; ++i) {
        const int c = ch + i;
        const int sn = sl == kRing - 1 ? 0 : sl + 1;     // slot of c + 1
        const int s2 = sn == kRing - 1 ? 0 : sn + 1;     // slot of c + 2
        softmax_pv(sl, c & 1, sn, (c + 1) & 1, std::true_type{});   // past the split's end: S^T unused
        CSA_ATT_STORE(s2, st[(i + 2) % kDepth], vm[(i + 2) % kDepth]);
        CSA_ATT_LOAD(c + 2 + kDepth, st[(i + 2) % kDepth], vm[(i + 2) % kDepth]);
        barrier_lds();
        sl = sn;
      }
    }
    // the last chunks: ch and ch + 1 are in their slots, the later ones in their sets
#pragma unroll
    for (int i = 0; i < kDepth - 1; ++i) {
      const int c = ch + i;
      if (c < ch1) {
        const int sn = sl == kRing - 1 ? 0 : sl + 1;
        const int s2 = sn == kRing - 1 ? 0 : sn + 1;
        if (c + 1 < ch1) {
          softmax_pv(sl, c & 1, sn, (c + 1) & 1, std::true_type{});
          if (c + 2 < ch1) CSA_ATT_STORE(s2, st[(i + 2) % kDepth], vm[(i + 2) % kDepth]);
          barrier_lds();
        } else {
          softmax_pv(sl, c & 1, sl, c & 1, std::false_type{});
        }
        sl = sn;
      }
    }
  }
#undef CSA_ATT_LOAD1
#undef CSA_ATT_LOAD
#undef CSA_ATT_STORE1
#undef CSA_ATT_STORE

  attn_finish<Sh::kPart>(a, o, m_ref, l_run, qi, split, hg, part);
}

// ------------------------------------------------------------------------------------
// Two-set bf16 kernel for 64+ queries whose rows are bf16: the window, then every visible
// entry (HCA, kSrcDense: addresses by arithmetic) or the selected entries (kSrcIdx: a row
// table built once in LDS); 64 heads per workgroup.  The 8 waves form two sets of 4, one
// wave of each set per SIMD; wave w owns head group w % 4 over all 512 channels (its Q
// part 64 VGPRs, its O 128), so S^T needs no exchange between waves.  Set s takes the
// split's chunks of parity s, and every chunk passes two half-phases: S^T + online
// softmax (32 MFMAs, P kept in registers), then O += P . V (64 MFMAs, P as bf16 hi + lo).
// The sets run one half-phase apart, so at every barrier one wave of a SIMD starts the
// S^T of a chunk while the other starts the P . V of the previous one: the matrix unit
// stays fed while the other wave reads LDS or exponentiates.  Rows go straight from
// memory into a 4-slot LDS ring (global_load_lds_dwordx4: one row per wave instruction,
// no staging registers), two chunks ahead; one barrier per half-phase.  At the end set 1
// hands its (m, l, O) to set 0 through the ring and set 0 writes the result as attn_bf16
// does.  [HCA-CSA] "HCA：重压缩 + 全量" (dense attention over all compressed entries with
// the window and the sink); [KV-COMP] sections 9.5-9.6 (the selected rows); the softmax is
// the one of the kernel above.
// ------------------------------------------------------------------------------------
constexpr int kDnSlots = 4;
constexpr int kDnWaves = 8;
constexpr int kDnRowsPerWave = kRows / kDnWaves;

// One 1 KiB row from global memory (row, wave-uniform) into LDS at dst (wave-uniform):
// lane l moves bytes voff = 16 * l .. +15.  Written as an instruction of its own so that
// the compiler, which cannot see that it writes LDS, does not wait for it before every
// LDS read: the code waits for these loads itself (dn_wait_vmcnt, then a barrier) before
// a slot is read, and the ring never reads a slot a load in flight writes.  It has no
// result register.  The compiler does not see the load inside, so the asm provides the
// wait states the load's scalar inputs need: 5 after a VALU instruction wrote the address
// SGPRs (v_readfirstlane of a table entry), which also covers the 1 after M0 is written.
// kStream: the row is read once (nt: streamed past the caches' retention).
template <bool kStream>
__device__ __forceinline__ void dn_dma_row(const void* row, uint8_t* dst, int voff) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst));
  if constexpr (kStream)
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(row), "{m0}"(lds) : "memory");
  else
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(row), "{m0}"(lds) : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void dn_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int kSrc>
__global__ __launch_bounds__(kDnWaves * kWave, 1) void attn_rows_bf16(AttnArgs a) {
  constexpr bool kDense = kSrc == kSrcDense;
  constexpr bool kCand = kSrc == kSrcCand || kSrc == kSrcCand2;
  __shared__ __attribute__((aligned(16))) uint8_t ring[kDnSlots * kChunkBytes];
  // selected rows (kSrcIdx): the split's row addresses (low bit: absent, a zero row) and
  // each chunk's mask of present rows, built once
  __shared__ uint64_t rowtab[kDense ? 1 : kMaxSplitChunks * kRows];
  __shared__ uint32_t rowmask[kDense ? 1 : kMaxSplitChunks];
  int qi, split;
  if (!attn_unit(a.nq, a.nsplit, qi, split)) return;
  const int b = qi / a.S, s = qi % a.S;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int set = wave >> 2, hg = wave & 3;
  const int l = static_cast<int>(lane_id());
  const int g = l >> 4;

  int w_lo, n_swa;
  window_rows(s, a.S, a.Ls, a.W, last_position(a.q_pos, b, a.S), w_lo, n_swa);
  const int n_rem = kDense ? static_cast<int>(min(static_cast<int64_t>(a.Nc), (a.q_pos[qi] + 1) / a.m)) : a.k;
  const int n_slots = n_swa + n_rem;
  const int ch0 = split * a.chunks_per_split;
  const int n = max(0, min(cdiv(n_slots, kRows), ch0 + a.chunks_per_split) - ch0);   // chunks of the split
  const uint16_t* kvb = a.kv + static_cast<size_t>(b) * a.Nc * kAC;
  const uint16_t* swab = a.swa + static_cast<size_t>(b) * a.Ls * kAC;
  if constexpr (!kDense) {
    // Selection from candidates (kSrcCand, kSrcCand2), as attn_bf16 makes it: the query's
    // n_cand (key, entry) pairs -> the k best in entry order, in the ring (free until the
    // rows are loaded); the first split of the query also writes them to idx_out.
    constexpr int kT = kDnWaves * kWave;
    int32_t* sel = reinterpret_cast<int32_t*>(ring + sizeof(TkShared));
    if constexpr (kCand) {
      constexpr int NU = kSrc == kSrcCand2 ? 2 : 1;
      static_assert(sizeof(TkShared) + 4 * 8 * NU * kT <= kDnSlots * kChunkBytes, "selection fits the ring");
      TkShared& tsh = *reinterpret_cast<TkShared*>(ring);
      const uint2* cq = a.cand + static_cast<size_t>(qi) * a.cand_stride;
      uint32_t key[NU][8], ent[NU][8];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int p0 = 8 * (static_cast<int>(threadIdx.x) + u * kT);
        if ((a.n_cand & 1) == 0 && p0 + 7 < a.n_cand) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint4 v = reinterpret_cast<const uint4*>(cq + p0)[j];
            key[u][2 * j] = v.x; ent[u][2 * j] = v.y;
            key[u][2 * j + 1] = v.z; ent[u][2 * j + 1] = v.w;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint2 v = p0 + j < a.n_cand ? cq[p0 + j] : make_uint2(0u, 0u);
            key[u][j] = v.x; ent[u][j] = v.y;
          }
        }
      }
      uint64_t taken;
      int obase[NU];
      const int kk = select_regs<kT, 8, NU>(tsh, key, a.k, taken, obase);
      int32_t* io = a.idx_out && split == 0 ? a.idx_out + static_cast<size_t>(qi) * a.k : nullptr;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        int o = obase[u];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if ((taken >> (8 * u + j)) & 1ull) {
            sel[o] = static_cast<int32_t>(ent[u][j]);
            if (io) io[o] = static_cast<int32_t>(ent[u][j]);
            ++o;
          }
      }
      for (int p = kk + static_cast<int>(threadIdx.x); p < a.k; p += kT) {
        sel[p] = -1;
        if (io) io[p] = -1;
      }
      __syncthreads();
    }
    // row e of the split: a window row, the selected entry (idx or sel; -1 or out of
    // range: absent), or past the row set; each wave's ballot covers two chunks' masks
    const int32_t* idxq = kCand ? sel : a.idx + static_cast<size_t>(qi) * a.k;
    for (int e0 = 0; e0 < n * kRows; e0 += kT) {
      const int e = e0 + static_cast<int>(threadIdx.x);
      const int slot = ch0 * kRows + e;
      uint64_t p = reinterpret_cast<uint64_t>(g_zero_rows + static_cast<size_t>(e & (kZeroRows - 1)) * kAC) | 1u;
      if (e < n * kRows) {
        if (slot < n_swa) {
          p = reinterpret_cast<uint64_t>(swab + static_cast<size_t>(w_lo + slot) * kAC);
        } else if (slot < n_slots) {
          const int j = idxq[slot - n_swa];
          if (j >= 0 && j < a.Nc) p = reinterpret_cast<uint64_t>(kvb + static_cast<size_t>(j) * kAC);
        }
        rowtab[e] = p;
      }
      const uint64_t present = __ballot(e < n * kRows && !(p & 1u));
      if (l == 0 && e < n * kRows) {
        rowmask[e >> 5] = static_cast<uint32_t>(present);
        if ((e >> 5) + 1 < n) rowmask[(e >> 5) + 1] = static_cast<uint32_t>(present >> 32);
      }
    }
    __syncthreads();
  }

  // Q part of head group hg as the B operand: lane l holds head 16*hg + l%16, channels
  // 32*ks + 8*g .. +7 (loaded before the first rows, so the first wait covers both)
  v8s qb[kAC / 32];
  {
    const uint16_t* qh = a.q + (static_cast<size_t>(qi) * kAH + kHG * hg + (l & 15)) * kAC;
#pragma unroll
    for (int ks = 0; ks < kAC / 32; ++ks) qb[ks] = *reinterpret_cast<const v8s*>(qh + 32 * ks + 8 * g);
  }

  // Chunk c of the split (c >= n: zero rows) into ring slot S = c % kDnSlots: this wave's
  // kDnRowsPerWave rows, one instruction each; rows past the row set read zero rows.
  auto issue = [&](int c) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* slot = ring + (c % kDnSlots) * kChunkBytes;
#pragma unroll
    for (int i = 0; i < kDnRowsPerWave; ++i) {
      const int r = kDnRowsPerWave * wave + i;
      const int e = (ch0 + c) * kRows + r;              // slot of the query's row set
      const uint16_t* src;
      if constexpr (kDense) {
        const bool win = c < n && e < n_swa, ent = c < n && e >= n_swa && e < n_slots;
        src = win ? swab + static_cast<size_t>(w_lo + e) * kAC
            : ent ? kvb + static_cast<size_t>(e - n_swa) * kAC
                  : g_zero_rows + static_cast<size_t>(e & (kZeroRows - 1)) * kAC;
      } else {
        const uint64_t v = c < n ? rowtab[c * kRows + r] : reinterpret_cast<uint64_t>(g_zero_rows);
        // the same entry in every lane: a scalar address
        const uint64_t p = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32))) << 32) |
                           static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
        src = reinterpret_cast<const uint16_t*>(p & ~static_cast<uint64_t>(1));
      }
      // HCA's rows are read by one workgroup once; selected entries may serve other queries
      dn_dma_row<kDense>(src, slot + r * kRowStride, 16 * l);
    }
  };

  v4f o[kAC / 16];
#pragma unroll
  for (int t = 0; t < kAC / 16; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;   // per head l%16 (log2 units)
  float l_run = 0.0f;        // this lane's share of the per-head sum
  v8s pa, pb;                // P of the chunk between its two half-phases (bf16 hi, lo)

  // S^T of chunk c (32 rows x 16 heads, all channels) and its online softmax; P -> pa, pb.
  auto step_s = [&](int c) __attribute__((always_inline)) {
    // the S^T chain and the softmax are the latency-bound half: issued ahead of the other
    // set's P . V on the same SIMD (which fills the matrix unit's gaps)
    __builtin_amdgcn_s_setprio(1);
    const uint8_t* buf = ring + (c % kDnSlots) * kChunkBytes;
    v4f st[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < kAC / 32; ++ks)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const v8s av = *reinterpret_cast<const v8s*>(buf + (16 * rb + (l & 15)) * kRowStride + 64 * ks + 16 * g);
        st[rb] = mfma_bf16_16x16x32(av, qb[ks], st[rb]);
      }
    // fragment reads two steps ahead of their MFMAs (bounds the registers they hold)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int k = 0; k < kAC / 16 - 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    // slot j <-> chunk row 16*(j/4) + 4*g + j%4; rows past the row set are masked
    const int e0 = (ch0 + c) * kRows;
    // the chunk's present rows, shifted by this lane's 4g: the remaining bit positions
    // (16 * (j / 4) + j % 4) are constants (no per-lane masks live through the loop)
    uint32_t present = 0;
    if constexpr (!kDense) present = (c < n ? rowmask[c] : 0u) >> (4 * g);
    float sv[8];
    float lmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 16 * (j >> 2) + 4 * g + (j & 3);
      const bool ok = kDense ? c < n && e0 + row < n_slots : ((present >> (16 * (j >> 2) + (j & 3))) & 1u) != 0;
      sv[j] = ok ? st[j >> 2][j & 3] * a.scale_log2 : -INFINITY;
      lmax = fmaxf(lmax, sv[j]);
    }
    if (__ballot(lmax > m_ref + kLazy)) {
      float cmax = fmaxf(lmax, wave_xor(lmax, 16));
      cmax = fmaxf(cmax, wave_xor(cmax, 32));
      const bool move = cmax > m_ref + kLazy;
      const float m_new = move ? cmax : m_ref;
      const float alpha = move ? exp2f(m_ref - m_new) : 1.0f;      // 0 when m_ref = -inf
      l_run *= alpha;
      m_ref = m_new;
      float ah[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ah[i] = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
      for (int t = 0; t < kAC / 16; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[t][i] *= ah[i];
    }
    const float m_use = m_ref == -INFINITY ? 0.0f : m_ref;
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
      typedef float v2f __attribute__((ext_vector_type(2)));
      const v2f p = {__builtin_amdgcn_exp2f(sv[j] - m_use), __builtin_amdgcn_exp2f(sv[j + 1] - m_use)};
      psum += p[0] + p[1];
      const v2bf hi = __builtin_convertvector(p, v2bf);
      const uint32_t hb = __builtin_bit_cast(uint32_t, hi);
      const v2f r = {p[0] - __uint_as_float(hb << 16), p[1] - __uint_as_float(hb & 0xffff0000u)};
      const uint32_t lb = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, v2bf));
      pa[j] = static_cast<short>(hb & 0xffffu);
      pa[j + 1] = static_cast<short>(hb >> 16);
      pb[j] = static_cast<short>(lb & 0xffffu);
      pb[j + 1] = static_cast<short>(lb >> 16);
    }
    l_run += psum;
    // P complete here: otherwise its exponentials sink past the row loads and the barrier
    // into the P . V step, whose V reads then find no registers to run ahead in
    asm volatile("" : : "v"(pa), "v"(pb));
    __builtin_amdgcn_s_setprio(0);
  };

  // O += P . V for chunk c (V rows read transposed from the same LDS rows), tiles in pairs:
  // the P_hi products of both, then their P_lo products, so that no MFMA waits for the
  // result of the one just before it; V reads run four tiles ahead.
  auto step_pv = [&](int c) __attribute__((always_inline)) {
    const uint8_t* vt = ring + (c % kDnSlots) * kChunkBytes + (4 * g + ((l & 15) >> 2)) * kRowStride + 8 * (l & 3);
#pragma unroll
    for (int t = 0; t < kAC / 16; t += 2) {
      v8s vb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const v4s v0 = lds_read_tr16(vt + 32 * (t + j));
        const v4s v1 = lds_read_tr16(vt + 32 * (t + j) + 16 * kRowStride);
        vb[j] = v8s{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      }
      o[t] = mfma_bf16_16x16x32(pa, vb[0], o[t]);
      o[t + 1] = mfma_bf16_16x16x32(pa, vb[1], o[t + 1]);
      o[t] = mfma_bf16_16x16x32(pb, vb[0], o[t]);
      o[t + 1] = mfma_bf16_16x16x32(pb, vb[1], o[t + 1]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int k = 0; k < kAC / 16 - 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  // Half-phase h: set h%2 forms S^T of chunk h, the other set finishes chunk h-1.  Before
  // it: chunk h has landed (this wave's own rows: at most chunk h+1's still in flight; the
  // barrier: every wave's), chunk h-2 is no longer read; after its step each wave issues
  // its rows of chunk h+2 into that slot (no wave reads it again before the next barrier).
  // Each wave runs its two half-phase kinds in one straight loop (set 1 starting one
  // half-phase later); every wave passes the n + 1 barriers and issues the same loads.
  auto top = [&](int h) __attribute__((always_inline)) {
    dn_wait_vmcnt<kDnRowsPerWave>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);                // each step scheduled on its own
  };
  issue(0);
  issue(1);
  // Q and both chunks complete before the loop (the compiler's own count of the Q loads
  // would otherwise put a full wait inside it); so are the scalar loads of arguments only
  // the finish reads (a scalar load in flight, which may return out of order, would make
  // every LDS wait in the loop a wait for all of them)
  {
    const double rope_r = a.rope_r;
    asm volatile("" : : "s"(rope_r));
  }
  dn_wait_vmcnt<0>();
  int h = set;
  if (set == 1) {
    top(0);
    issue(2);
  }
#pragma unroll 1
  while (h <= n) {
    top(h);
    step_s(h);                                          // all rows masked when h = n
    issue(h + 2);
    if (h == n) break;
    top(h + 1);
    step_pv(h);
    issue(h + 3);
    h += 2;
  }

  // set 1 hands (m, l, O) to set 0 through the ring: [head group][tile][lane][4] + (m, l)
  dn_wait_vmcnt<0>();
  __syncthreads();
  static_assert((kAC / 16 * kWave * 4 + 2 * kWave) * 4 <= kChunkBytes, "a head group's (O, m, l) fits one slot");
  float* xo = reinterpret_cast<float*>(ring + hg * kChunkBytes);
  if (set == 1) {
#pragma unroll
    for (int t = 0; t < kAC / 16; ++t) *reinterpret_cast<v4f*>(xo + (t * kWave + l) * 4) = o[t];
    xo[kAC / 16 * kWave * 4 + 2 * l] = m_ref;
    xo[kAC / 16 * kWave * 4 + 2 * l + 1] = l_run;
  }
  __syncthreads();
  if (set == 1) return;
  {
    const float mb = xo[kAC / 16 * kWave * 4 + 2 * l], lb = xo[kAC / 16 * kWave * 4 + 2 * l + 1];
    const float M = fmaxf(m_ref, mb);
    const float ea = m_ref == -INFINITY ? 0.0f : exp2f(m_ref - M);
    const float eb = mb == -INFINITY ? 0.0f : exp2f(mb - M);
    l_run = l_run * ea + lb * eb;
    m_ref = M;
    float ah[4], bh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ah[i] = __shfl(ea, 4 * g + i, kWave);
      bh[i] = __shfl(eb, 4 * g + i, kWave);
    }
#pragma unroll
    for (int t = 0; t < kAC / 16; ++t) {
      const v4f x = *reinterpret_cast<const v4f*>(xo + (t * kWave + l) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[t][i] = o[t][i] * ah[i] + x[i] * bh[i];
    }
  }
  attn_finish<kAC>(a, o, m_ref, l_run, qi, split, hg, 0);
}

// Combines the split partials of the bf16 kernel (register-order layout) with the sink.
// One wave per (query, head group, KT consecutive 16-channel tiles): lane l holds heads
// 16*hg + 4*(l/16) + i and channel 16*ct + l%16 of each tile, as the kernel's waves wrote
// them.  KT = 4 (few splits: every load of the wave in flight at once) or 1.  Blocks of 4
// waves, numbered like the attention's workgroups so that a query's partials are read on
// the XCD whose L2 received them.  Grid: ceil(B*S / 8) * 8 * (128 / KT / 4) blocks.
template <int KT>
__global__ __launch_bounds__(256) void attn_merge_tiles(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_ml,
                                                        const float* __restrict__ sink, int nsplit, int nq,
                                                        uint16_t* __restrict__ out, float* __restrict__ lse,
                                                        const int64_t* __restrict__ q_pos, int rope_d,
                                                        double rope_r) {
  constexpr int kTiles = kAC / 16;
  constexpr int kBlocksPerQuery = kNHG * kTiles / KT / 4;
  constexpr int kMaxFast = KT == 1 ? 8 : 4;             // splits held in registers at once
  int q, ub;
  if (!attn_unit(nq, kBlocksPerQuery, q, ub)) return;
  const size_t qi = q;
  const int unit = 4 * ub + (threadIdx.x >> 6);
  const int ct0 = KT * (unit % (kTiles / KT));
  const int hg = unit / (kTiles / KT);
  const int l = static_cast<int>(lane_id());
  const int h0 = kHG * hg + 4 * (l >> 4);
  float M[4], den[4], acc[KT][4];
  float sk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sk[i] = sink[h0 + i];
    M[i] = sk[i] * kLog2e;
#pragma unroll
    for (int t = 0; t < KT; ++t) acc[t][i] = 0.0f;
  }
  auto po_of = [&](int sp, int ct) __attribute__((always_inline)) {
    return *reinterpret_cast<const v4f*>(part_o + (((qi * nsplit + sp) * kNHG + hg) * kTiles + ct) * (kWave * 4) +
                                         4 * l);
  };
  if (nsplit <= kMaxFast) {
    // every partial load in flight at once; the (m, l) of the block's 16 heads are read
    // once per block into LDS (the 4 waves share the head group)
    __shared__ v4f sml[kMaxFast][kHG / 2];
    v4f ma[kMaxFast], mb[kMaxFast], x[kMaxFast][KT];
#pragma unroll
    for (int sp = 0; sp < kMaxFast; ++sp)
      if (sp < nsplit)
#pragma unroll
        for (int t = 0; t < KT; ++t) x[sp][t] = po_of(sp, ct0 + t);
    if (static_cast<int>(threadIdx.x) < nsplit * (kHG / 2)) {
      const int sp = threadIdx.x / (kHG / 2), j = threadIdx.x % (kHG / 2);
      sml[sp][j] = *reinterpret_cast<const v4f*>(part_ml + ((qi * nsplit + sp) * kAH + kHG * hg) * 2 + 4 * j);
    }
    __syncthreads();
#pragma unroll
    for (int sp = 0; sp < kMaxFast; ++sp)
      if (sp < nsplit) {
        ma[sp] = sml[sp][2 * (l >> 4)];
        mb[sp] = sml[sp][2 * (l >> 4) + 1];
      }
#pragma unroll
    for (int sp = 0; sp < kMaxFast; ++sp)
      if (sp < nsplit) {
        M[0] = fmaxf(M[0], ma[sp][0]); M[1] = fmaxf(M[1], ma[sp][2]);
        M[2] = fmaxf(M[2], mb[sp][0]); M[3] = fmaxf(M[3], mb[sp][2]);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) den[i] = M[i] == -INFINITY ? 0.0f : exp2f(sk[i] * kLog2e - M[i]);
#pragma unroll
    for (int sp = 0; sp < kMaxFast; ++sp)
      if (sp < nsplit) {
        const float mi[4] = {ma[sp][0], ma[sp][2], mb[sp][0], mb[sp][2]};
        const float li[4] = {ma[sp][1], ma[sp][3], mb[sp][1], mb[sp][3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float wgt = mi[i] == -INFINITY ? 0.0f : exp2f(mi[i] - M[i]);
          den[i] = fmaf(wgt, li[i], den[i]);
#pragma unroll
          for (int t = 0; t < KT; ++t) acc[t][i] = fmaf(wgt, x[sp][t][i], acc[t][i]);
        }
      }
    merge_store<KT>(acc, den, M, qi, h0, ct0, l, out, lse, q_pos, rope_d, rope_r);
  } else {
    merge_splits<KT>(part_o, part_ml, sink, nsplit, qi, hg, ct0, out, lse, q_pos, rope_d, rope_r);
  }
}

// Inverse RoPE of 8 consecutive output channels c0 .. c0+7 (c0 even: they hold whole pairs).
__device__ __forceinline__ void rope_back8(float (&v)[8], int c0, int c, int d_rope, double r, int64_t t) {
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const int col = c0 + j;
    if (col >= c - d_rope && col + 1 < c) {
      float cs, sn;
      rope_cs_sn(col, c, d_rope, r, t, cs, sn);
      const float x = v[j], y = v[j + 1];
      v[j] = rope_back(x, y, col, cs, sn);
      v[j + 1] = rope_back(y, x, col + 1, cs, sn);
    }
  }
}

// Combines the split partials with the sink.  One wave per (query, head); lane l owns
// columns 8l .. 8l+7 (c = 512) or a strided share of them, loads of every split in flight
// together.  Grid: ceil(B*S*H / 4) blocks of 256 threads.
template <typename OutT>
__global__ __launch_bounds__(256) void attn_merge(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                  const float* __restrict__ sink, int nsplit, int H, int c, int nqh,
                                                  OutT* __restrict__ out, float* __restrict__ lse,
                                                  const int64_t* __restrict__ q_pos, int rope_d, double rope_r) {
  const int qh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (qh >= nqh) return;
  const int lane = threadIdx.x & 63;
  const size_t qi = qh / H;
  const int h = qh % H;
  const float sink2 = sink[h] * kLog2e;
  if (c == kAC && nsplit <= 8) {
    // every load of the (query, head) in flight at once: lane l owns channels 8l .. 8l+7,
    // lane i < nsplit holds split i's (m, l)
    float4 x[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nsplit) {
        const float4* src = reinterpret_cast<const float4*>(part_o + ((qi * nsplit + i) * H + h) * kAC + 8 * lane);
        x[i][0] = src[0];
        x[i][1] = src[1];
      }
    }
    const float mi = lane < nsplit ? part_ml[((qi * nsplit + lane) * H + h) * 2] : -INFINITY;
    const float li = lane < nsplit ? part_ml[((qi * nsplit + lane) * H + h) * 2 + 1] : 0.0f;
    float M = sink2;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < nsplit) M = fmaxf(M, __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mi), i)));
    const float wl = (M == -INFINITY || mi == -INFINITY) ? 0.0f : exp2f(mi - M);
    float den = M == -INFINITY ? 0.0f : exp2f(sink2 - M);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nsplit) {
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), i));
        den += w * __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, li), i));
        acc[0] = fmaf(w, x[i][0].x, acc[0]); acc[1] = fmaf(w, x[i][0].y, acc[1]);
        acc[2] = fmaf(w, x[i][0].z, acc[2]); acc[3] = fmaf(w, x[i][0].w, acc[3]);
        acc[4] = fmaf(w, x[i][1].x, acc[4]); acc[5] = fmaf(w, x[i][1].y, acc[5]);
        acc[6] = fmaf(w, x[i][1].z, acc[6]); acc[7] = fmaf(w, x[i][1].w, acc[7]);
      }
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    OutT* dst = out + (qi * H + h) * kAC + 8 * lane;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= inv;
    if (rope_d > 0) rope_back8(acc, 8 * lane, kAC, rope_d, rope_r, q_pos[qi]);
    if constexpr (sizeof(OutT) == 2) {
      uint32_t pk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pk[j] = static_cast<uint32_t>(f32_to_bf16(acc[2 * j])) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * j + 1])) << 16);
      *reinterpret_cast<uint4*>(dst) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[j] = acc[j];
    }
    if (lse && lane == 0) lse[qi * H + h] = (M == -INFINITY || den <= 0.0f) ? -INFINITY : (M + log2f(den)) * kLn2;
    return;
  }
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
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= inv;
    if (rope_d > 0) rope_back8(acc, c0, c, rope_d, rope_r, q_pos[qi]);
    for (int j = 0; j < 8 && c0 + j < c; ++j) {
      if constexpr (sizeof(OutT) == 2) dst[j] = f32_to_bf16(acc[j]);
      else dst[j] = acc[j];
    }
  }
  if (lse && lane == 0) lse[qi * H + h] = (M == -INFINITY || den <= 0.0f) ? -INFINITY : (M + log2f(den)) * kLn2;
}

// ------------------------------------------------------------------------------------
// fp32 path (small shapes): one workgroup per (query, head); 256 slots per step, each
// thread one slot's logit, then each thread accumulates channels.  Writes partials in
// [query][head][channel] order, which attn_merge finishes.
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
  window_rows(s, S, Ls, W, last_position(q_pos, b, S), w_lo, n_swa);
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

// The two shapes of the bf16 path: few queries -> 8 waves over 2 head groups x channel
// quarters (two workgroups per query: more workgroups); many queries -> all 64 heads in one
// workgroup (every row read serves 64 heads).
using NarrowShape = AttnShape<4, 8>;
using WideShape = AttnShape<kWideParts, kWideWaves>;
static_assert(WideShape::kUnits == 1, "the dense kernel takes the wide shape's splits: one workgroup per (query, split)");
static bool attn_wide(int nq) { return nq >= kWideMinQueries; }

// Splits of one query's rows over workgroups (bf16 kernel): enough workgroups (units per
// query x splits) to give every compute unit one, but every split keeps >= 4 chunks (128
// rows) per 32 heads it covers: a split's partial result (heads x 512 fp32, 2 KiB per
// head) must stay small next to the rows it reads (1 KiB each).  The row table of a
// split fits in LDS.
int attn_nsplit(int nq, int max_rows) {
  const int units = attn_wide(nq) ? WideShape::kUnits : NarrowShape::kUnits;
  const int min_chunks = attn_wide(nq) ? 8 : 4;
  const int chunks = cdiv(max_rows, kRows);
  const int by_fill = cdiv(256, units * nq);
  const int by_rows = chunks / min_chunks;
  const int by_lds = cdiv(chunks, kMaxSplitChunks);
  return std::max(by_lds, std::max(1, std::min(by_fill, by_rows)));
}

size_t attn_workspace_bytes(int B, int S, int H, int c, int max_rows, int dtype) {
  const size_t nq = static_cast<size_t>(B) * S;
  const int ns = dtype == CSA_F32 ? 1 : attn_nsplit(static_cast<int>(nq), max_rows);
  if (dtype != CSA_F32 && ns == 1) return 0;
  return nq * ns * H * (static_cast<size_t>(c) + 2) * sizeof(float);
}

template <int kParts, int kWaves, int kFmt, bool kShort>
static int launch_attn_bf16_fmt(int src, const AttnArgs& a, hipStream_t st) {
  using Sh = AttnShape<kParts, kWaves>;
  // the dynamic-LDS limit of every source's kernel, raised once per device (any thread may call)
  static std::atomic<uint64_t> raised{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CSA_ERR_HIP;
  const uint64_t bit = uint64_t{1} << (dev & 63);
  if (!(raised.load(std::memory_order_acquire) & bit)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bf16<kSrcIdx, kParts, kWaves, kFmt, kShort>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, Sh::kLdsMax) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bf16<kSrcDense, kParts, kWaves, kFmt, kShort>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, Sh::kLdsMax) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bf16<kSrcCand, kParts, kWaves, kFmt, kShort>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, Sh::kLdsMax) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bf16<kSrcCand2, kParts, kWaves, kFmt, kShort>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, Sh::kLdsMax) != hipSuccess)
      return CSA_ERR_HIP;
    raised.fetch_or(bit, std::memory_order_release);
  }
  const dim3 grid(cdiv(a.nq, 8) * 8 * Sh::kUnits * a.nsplit);
  const int lds = Sh::kLdsFixed + a.chunks_per_split * kRows * 8;
  const dim3 block(Sh::kThreads);
  if (src == kSrcDense) hipLaunchKernelGGL((attn_bf16<kSrcDense, kParts, kWaves, kFmt, kShort>), grid, block, lds, st, a);
  else if (src == kSrcCand) hipLaunchKernelGGL((attn_bf16<kSrcCand, kParts, kWaves, kFmt, kShort>), grid, block, lds, st, a);
  else if (src == kSrcCand2) hipLaunchKernelGGL((attn_bf16<kSrcCand2, kParts, kWaves, kFmt, kShort>), grid, block, lds, st, a);
  else hipLaunchKernelGGL((attn_bf16<kSrcIdx, kParts, kWaves, kFmt, kShort>), grid, block, lds, st, a);
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

template <int kParts, int kWaves, bool kShort>
static int launch_attn_bf16_short(int src, const AttnArgs& a, hipStream_t st) {
  if (a.kv_fmt == kFmtFp4) return launch_attn_bf16_fmt<kParts, kWaves, kFmtFp4, kShort>(src, a, st);
  if (a.kv_fmt == kFmtFp8Rope) return launch_attn_bf16_fmt<kParts, kWaves, kFmtFp8Rope, kShort>(src, a, st);
  return launch_attn_bf16_fmt<kParts, kWaves, kFmtBf16, kShort>(src, a, st);
}

template <int kParts, int kWaves>
static int launch_attn_bf16(int src, const AttnArgs& a, hipStream_t st) {
  if constexpr (AttnShape<kParts, kWaves>::kAllChunks > 0)
    if (a.chunks_per_split <= AttnShape<kParts, kWaves>::kAllChunks)
      return launch_attn_bf16_short<kParts, kWaves, true>(src, a, st);
  return launch_attn_bf16_short<kParts, kWaves, false>(src, a, st);
}

// The bf16 path for row source SRC: splits of the row set, the attention kernel, then the
// merge of split partials.  A carries everything but the split plan and the partials.
static int run_attn_bf16(int src, AttnArgs& a, int max_rows, void* ws, hipStream_t st) {
  const int nq = a.nq;
  const int ns = attn_nsplit(nq, max_rows);
  a.nsplit = ns;
  a.chunks_per_split = cdiv(cdiv(max_rows, kRows), ns);
  float* wsf = static_cast<float*>(ws);
  a.part_o = wsf;
  a.part_ml = wsf ? wsf + static_cast<size_t>(nq) * ns * kAH * kAC : nullptr;
  int rc = CSA_OK;
  if (a.kv_fmt == kFmtBf16 && attn_wide(nq)) {
    // bf16 rows, 64+ queries: the two-set kernel (same splits, one workgroup per (query, split))
    const dim3 grid(cdiv(nq, 8) * 8 * ns), block(kDnWaves * kWave);
    if (src == kSrcDense) hipLaunchKernelGGL(attn_rows_bf16<kSrcDense>, grid, block, 0, st, a);
    else if (src == kSrcCand) hipLaunchKernelGGL(attn_rows_bf16<kSrcCand>, grid, block, 0, st, a);
    else if (src == kSrcCand2) hipLaunchKernelGGL(attn_rows_bf16<kSrcCand2>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(attn_rows_bf16<kSrcIdx>, grid, block, 0, st, a);
    CSA_LAUNCH_CHECK();
  } else {
    rc = attn_wide(nq) ? launch_attn_bf16<kWideParts, kWideWaves>(src, a, st) : launch_attn_bf16<4, 8>(src, a, st);
  }
  if (rc != CSA_OK) return rc;
  if (ns > 1) {
    if (ns <= 4)
      hipLaunchKernelGGL(attn_merge_tiles<4>, dim3(cdiv(nq, 8) * 8 * (kNHG * (kAC / 16) / 16)), dim3(256), 0, st,
                         a.part_o, a.part_ml, a.sink, ns, nq, a.out, a.lse, a.q_pos, a.rope_d, a.rope_r);
    else
      hipLaunchKernelGGL(attn_merge_tiles<1>, dim3(cdiv(nq, 8) * 8 * (kNHG * (kAC / 16) / 4)), dim3(256), 0, st,
                         a.part_o, a.part_ml, a.sink, ns, nq, a.out, a.lse, a.q_pos, a.rope_d, a.rope_r);
    CSA_LAUNCH_CHECK();
  }
  return CSA_OK;
}

static AttnArgs attn_args(const void* q, const void* kv, int kv_fmt, const int64_t* q_pos, int m, const void* swa,
                          const float* sink, float scale, int B, int S, int Nc, int k, int Ls, int W, int rope_d,
                          float rope_theta, void* out, float* lse) {
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(kv);
  a.kv_fmt = kv_fmt;
  a.q_pos = q_pos;
  a.swa = static_cast<const uint16_t*>(swa);
  a.sink = sink;
  a.scale_log2 = scale * kLog2e;
  a.nq = B * S; a.S = S; a.Nc = Nc; a.k = k; a.Ls = Ls; a.W = W; a.m = m;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.rope_d = rope_d;
  a.rope_r = rope_ratio(rope_theta, rope_d);
  return a;
}

// Largest candidate set per row the fused selection takes (16 per thread).
int topk_attention_max_cand() { return std::min(NarrowShape::kMaxCand2, WideShape::kMaxCand2); }

// Top-k selection from candidates fused with the bf16 attention: row r's n_cand (key,
// entry) pairs start at cand + r * cand_stride (the segment pairs, or a first merge
// level's; 8 per thread up to kMaxCand, else 16); idx_out (optional) receives the
// selection.  The caller has checked shapes and the workspace.

int launch_topk_attention(const void* q, const void* kv, int kv_fmt, const uint2* cand, int n_cand, size_t cand_stride,
                          const int64_t* q_pos, const void* swa, const float* sink, float scale, int B, int S, int Nc,
                          int k, int Ls, int W, int rope_d, float rope_theta, void* out, float* lse, int32_t* idx_out,
                          void* ws, size_t ws_bytes, hipStream_t st) {
  const int max_rows = std::min(W, Ls) + k;
  if (ws_bytes < attn_workspace_bytes(B, S, kAH, kAC, max_rows, CSA_BF16)) return CSA_ERR_WORKSPACE;
  if (n_cand > topk_attention_max_cand() || k > n_cand || cand_stride < static_cast<size_t>(n_cand))
    return CSA_ERR_UNSUPPORTED;
  AttnArgs a = attn_args(q, kv, kv_fmt, q_pos, 1, swa, sink, scale, B, S, Nc, k, Ls, W, rope_d, rope_theta, out, lse);
  a.cand = cand;
  a.n_cand = n_cand;
  a.cand_stride = cand_stride;
  a.idx_out = idx_out;
  const bool one = n_cand <= NarrowShape::kMaxCand && n_cand <= WideShape::kMaxCand;
  return run_attn_bf16(one ? kSrcCand : kSrcCand2, a, max_rows, ws, st);
}


int launch_attention(bool dense, const void* q, const void* kv, int kv_fmt, const int32_t* idx, const int64_t* q_pos,
                     int m,
                     const void* swa, const float* sink, int dtype, float scale, int B, int S, int H, int c, int Nc,
                     int k, int Ls, int W, int rope_d, float rope_theta, void* out, float* lse, void* ws,
                     size_t ws_bytes, hipStream_t st) {
  const int nq = B * S;
  const int max_rows = std::min(W, Ls) + (dense ? Nc : k);
  if (ws_bytes < attn_workspace_bytes(B, S, H, c, max_rows, dtype)) return CSA_ERR_WORKSPACE;
  const float scale_log2 = scale * kLog2e;
  if (dtype == CSA_BF16) {
    AttnArgs a = attn_args(q, kv, kv_fmt, q_pos, m, swa, sink, scale, B, S, Nc, k, Ls, W, rope_d, rope_theta, out,
                           lse);
    a.idx = idx;
    return run_attn_bf16(dense ? kSrcDense : kSrcIdx, a, max_rows, ws, st);
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
                     nq * H, static_cast<float*>(out), lse, q_pos, rope_d, rope_ratio(rope_theta, rope_d));
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}


// ------------------------------------------------------------------------------------
// Fixed scratch for callers that cannot allocate (csa_sparse_attn_noalloc): the split
// partials live in this file-scope device array instead of a caller workspace.  Each GPU
// the library runs on holds its own copy, at its own device address, until the process
// ends.  In host code `scratch` names a host-side stand-in, never the device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is handed to kernels.
// ------------------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t{32} << 20;
__device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

size_t attn_scratch_bytes() { return kScratchBytes; }

// Device address of this device's scratch array (looked up on the first call per device).
int attn_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return CSA_ERR_HIP;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return CSA_OK;
}

}  // namespace csa
