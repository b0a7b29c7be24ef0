// Top-k selection (stage 3).
//
// Per row of Nc fp32 scores: the indices of the min(k, n_cand) largest candidate scores
// (candidates: not -inf, not NaN), ties to the lower index, ascending, padded with -1.
// [KV-COMP] sections 9.4 (S_t = TopK_k of the indexer scores) and 9.8 (invisible entries
// are -inf before the selection and -1 after it).
//
// Scores become order-preserving 32-bit keys (score_key); the order used throughout is
// (key descending, position ascending), a total order, and positions are laid out in
// ascending index order, so "the kk first elements in this order" is exactly the
// required selection.  One workgroup of 1024 threads selects over a set of up to
// kTkMaxChunks * 4096 keys held in registers (4 consecutive positions per thread and
// 4096-position chunk):
//   1. candidate count and min/max of the candidate values (block reduction);
//   2. histogram over 2048 equal-width bins of [min, max]  (bin = trunc((x-min)*scale),
//      monotone in x because every rounding step is);
//   3. the bin b holding the kk-th element; elements in higher bins are taken, elements
//      in b go to an LDS candidate list;
//   4. the candidates are ranked against each other in the total order, which finds the
//      pivot: the kk-th element (T, posT);
//   5. an element is taken iff it precedes or equals the pivot, and an ordered compaction
//      (per-wave counts, one scan) writes the taken indices in position order.
// When equal-width bins cannot separate the values (all equal, infinities, or more
// than kTkCandCap elements in bin b), steps 2-4 become an exact radix select over the
// three key digits (11, 11, 10 bits) followed by a tie rank among keys equal to T.
//
// Schedules:
//   * one workgroup per row when the row fits one workgroup's registers;
//   * G segments per row: one workgroup per segment writes its local top-k as (key,
//     index) pairs in index order, then one workgroup per row selects the global top-k
//     among the G*k pairs.  The union of the local top-k sets holds the global top-k
//     (same total order), so the result is identical.
#include <algorithm>
#include <cmath>

#include "common.hpp"

namespace csa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkChunk = 4 * kTkThreads;       // positions per register chunk
constexpr int kTkMaxChunks = 9;                // 36864 keys per workgroup
constexpr int kTkMaxSet = kTkMaxChunks * kTkChunk;
constexpr int kTkBins = 1024;                  // equal-width bins of the fast path
constexpr int kTkPB = kTkBins / kWave;
constexpr int kTkHistWords = 2048 + 4 * 64;    // largest padded histogram (11-bit digit)
constexpr int kTkCandCap = 1024;

// radix digits, most significant first: bits 31..21, 20..10, 9..0
__host__ __device__ constexpr inline int digit_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__host__ __device__ constexpr inline int digit_bins(int pass) { return pass < 2 ? 2048 : 1024; }

struct alignas(16) TkShared {
  uint32_t hist[kTkHistWords];
  uint32_t ckey[kTkCandCap];
  int32_t cpos[kTkCandCap];
  int cell_nz[kTkMaxChunks * kTkWaves];   // candidates per (chunk, wave)
  int cell[kTkMaxChunks * kTkWaves];      // taken elements per (chunk, wave) above bin b / > T
  int cell_eq[kTkMaxChunks * kTkWaves];   // exact path: keys equal to T per (chunk, wave)
  uint32_t red_lo[kTkWaves], red_hi[kTkWaves];   // smallest and largest candidate key per wave
  int ncand, posT;
  uint32_t T;
};

// Wave64 inclusive prefix sum by DPP: row shifts 1, 2, 4, 8 scan each 16-lane row, then
// row broadcasts of lanes 15 and 31 carry the row totals forward.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

// Wave64 maximum (the same DPP pattern; 0 is the identity).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  const int x = static_cast<int>(v);
  int m = x;
  m = static_cast<int>(max(static_cast<uint32_t>(m), static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, m, 0x111, 0xf, 0xf, false))));
  m = static_cast<int>(max(static_cast<uint32_t>(m), static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, m, 0x112, 0xf, 0xf, false))));
  m = static_cast<int>(max(static_cast<uint32_t>(m), static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, m, 0x114, 0xf, 0xf, false))));
  m = static_cast<int>(max(static_cast<uint32_t>(m), static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, m, 0x118, 0xf, 0xf, false))));
  m = static_cast<int>(max(static_cast<uint32_t>(m), static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, m, 0x142, 0xa, 0xf, false))));
  m = static_cast<int>(max(static_cast<uint32_t>(m), static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, m, 0x143, 0xc, 0xf, false))));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(m, 63));
}

__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6); }

// Candidate value of a non-zero key (inverse of score_key).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Histograms have 64 * PB bins stored with 4 padding words after every PB bins, so
// that 64 lanes reading PB consecutive bins each hit distinct LDS banks.
template <int PB>
__device__ __forceinline__ int hist_slot(int bin) { return bin + 4 * (bin / PB); }

// Threshold search run by every wave on its own over the complete histogram (no
// barrier): with 1 <= remain <= total, returns the bin b with
// (#keys in bins > b) < remain <= (#keys in bins >= b) and sets above = #keys in bins > b.
template <int PB>
__device__ __forceinline__ int wave_threshold_bin(const uint32_t* hist, int remain, int& above) {
  constexpr int nbins = kWave * PB;
  const int l = static_cast<int>(lane_id());
  // lane l sums group l counted from the top: bins nbins - PB*(l+1) .. nbins - 1 - PB*l
  const uint32_t* g = hist + hist_slot<PB>(nbins - PB * (l + 1));
  int sum = 0;
#pragma unroll
  for (int i = 0; i < PB; i += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(g + i);
    sum += static_cast<int>(v.x + v.y + v.z + v.w);
  }
  const int incl = wave_incl_scan(sum);
  const int L = __ffsll(static_cast<long long>(__ballot(incl >= remain))) - 1;
  const int before = __builtin_amdgcn_readlane(incl - sum, L);
  // inside group L, lane j < PB takes the j-th bin from the top
  const int c = l < PB ? static_cast<int>(hist[hist_slot<PB>(nbins - 1 - (PB * L + l))]) : 0;
  const int incl2 = wave_incl_scan(c);
  const int J = __ffsll(static_cast<long long>(__ballot(l < PB && before + incl2 >= remain))) - 1;
  above = before + __builtin_amdgcn_readlane(incl2 - c, J);
  return nbins - 1 - (PB * L + J);
}

// (chunk, wave) cell of a position, and the first position of a cell
__device__ __forceinline__ int cell_of(int pos) { return (pos >> 12) * kTkWaves + ((pos & (kTkChunk - 1)) >> 8); }

// Exclusive prefix sums over the cells (chunk, wave) order, computed by every wave:
// returns the sum over the cells before cell (u, w) for each chunk u.
template <int NU>
__device__ __forceinline__ void cells_before(const int* cells, int w, int (&out)[NU]) {
  constexpr int kCells = NU * kTkWaves;
  constexpr int kJ = (kCells + kWave - 1) / kWave;
  const int l = static_cast<int>(lane_id());
  int cexcl[kJ], cbase[kJ];
  int run = 0;
#pragma unroll
  for (int j = 0; j < kJ; ++j) {        // cell 64*j + lane in register j
    const int c = kWave * j + l;
    const int v = c < kCells ? cells[c] : 0;
    const int incl = wave_incl_scan(v);
    cexcl[j] = incl - v;
    cbase[j] = run;
    run += __builtin_amdgcn_readlane(incl, 63);
  }
#pragma unroll
  for (int u = 0; u < NU; ++u)          // cell u*16 + w: register u/4, lane 16*(u%4) + w
    out[u] = cbase[u >> 2] + __builtin_amdgcn_readlane(cexcl[u >> 2], 16 * (u & 3) + w);
}

// Selection over the keys of one set held in registers: key[u][s] is the key of position
// 4096*u + 4*threadIdx.x + s (0 = not a candidate).  Returns kk = min(k, #candidates);
// sets bit 4u+s of `taken` for the taken elements and obase[u] to the output slot of
// this thread's first taken element of chunk u (taken elements fill slots 0..kk-1 in
// position order).
template <int NU>
__device__ int select_regs(TkShared& sh, const uint32_t (&key)[NU][4], int k, uint64_t& taken, int (&obase)[NU]) {
  const int tid = threadIdx.x, w = wave_index();
  const int l = static_cast<int>(lane_id());
  // ---- 1. candidates per cell and the key range
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t kv = key[u][s];
      cnt += __popcll(__ballot(kv != 0u));
      if (kv != 0u) {
        kmin = min(kmin, kv);
        kmax = max(kmax, kv);
      }
    }
    if (l == 0) sh.cell_nz[u * kTkWaves + w] = cnt;
  }
  for (int i = tid; i < kTkHistWords; i += kTkThreads) sh.hist[i] = 0;
  if (tid == 0) sh.ncand = 0;
  kmax = wave_max_u32(kmax);
  kmin = ~wave_max_u32(~kmin);
  if (l == 0) { sh.red_lo[w] = kmin; sh.red_hi[w] = kmax; }
  __syncthreads();                                                    // barrier 1
  int total = 0;
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int i = 0; i < kTkWaves; ++i) {
    kmin = min(kmin, sh.red_lo[i]);
    kmax = max(kmax, sh.red_hi[i]);
  }
#pragma unroll
  for (int i = 0; i < NU * kTkWaves; ++i) total += sh.cell_nz[i];
  const int kk = __builtin_amdgcn_readfirstlane(min(k, total));
  taken = 0;
#pragma unroll
  for (int u = 0; u < NU; ++u) obase[u] = 0;
  if (kk == 0) return 0;

  uint32_t T = 0u;
  int posT = -1;                 // pivot; (0, -1) takes every candidate
  int sel_before[NU];            // taken candidates of bin b before each of this wave's cells
  int eq_before[NU];             // exact path: keys == T before each of this wave's cells
  bool exact = false;
  int need_eq = 0;
  const int* cells = sh.cell_nz;
#pragma unroll
  for (int u = 0; u < NU; ++u) { sel_before[u] = 0; eq_before[u] = 0; }
  if (kk < total) {
    const float lo = key_value(kmin);
    const float range = key_value(kmax) - lo;
    const float scale = static_cast<float>(kTkBins) / range;
    bool ok = range > 0.0f && range <= 3.0e38f && scale <= 3.0e38f;
    int b = 0, remain = 0;
    if (ok) {
      // ---- 2. histogram over equal-width bins of [min, max]
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (key[u][s] != 0u) {
            const int bn = min(kTkBins - 1, static_cast<int>((key_value(key[u][s]) - lo) * scale));
            atomicAdd(&sh.hist[hist_slot<kTkPB>(bn)], 1u);
          }
      __syncthreads();                                                // barrier 2
      int above;
      b = wave_threshold_bin<kTkPB>(sh.hist, kk, above);
      remain = kk - above;
      ok = static_cast<int>(sh.hist[hist_slot<kTkPB>(b)]) <= kTkCandCap;
    }
    if (ok) {
      // ---- 3. higher bins are taken (counted per cell); bin b goes to the list
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        int g = 0;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t kv = key[u][s];
          const int bn = kv != 0u ? min(kTkBins - 1, static_cast<int>((key_value(kv) - lo) * scale)) : -1;
          g += __popcll(__ballot(bn > b));
          const uint64_t m = __ballot(bn == b);
          if (m != 0) {
            int base = 0;
            const int leader = __ffsll(static_cast<long long>(m)) - 1;
            if (l == leader) base = atomicAdd(&sh.ncand, __popcll(m));
            base = __builtin_amdgcn_readlane(base, leader);
            if (bn == b) {
              const int p = base + lanes_below(m);
              sh.ckey[p] = kv;
              sh.cpos[p] = kTkChunk * u + 4 * tid + s;
            }
          }
        }
        if (l == 0) sh.cell[u * kTkWaves + w] = g;
      }
      __syncthreads();                                                // barrier 3
      cells = sh.cell;
      // ---- 4. rank the candidates; the remain-th is the pivot
      const int nc = __builtin_amdgcn_readfirstlane(sh.ncand);
      if (nc <= kWave) {
        // every wave ranks the list itself: candidate l in lane l, the others by readlane
        const uint32_t ki = l < nc ? sh.ckey[l] : 0u;
        const int pi = l < nc ? sh.cpos[l] : 0;
        int r = 0;
        for (int j = 0; j < nc; ++j) {
          const uint32_t kj = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ki), j));
          const int pj = __builtin_amdgcn_readlane(pi, j);
          r += (kj > ki || (kj == ki && pj < pi)) ? 1 : 0;
        }
        const bool sel = l < nc && r < remain;
        const int lp = __ffsll(static_cast<long long>(__ballot(l < nc && r == remain - 1))) - 1;
        T = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ki), lp));
        posT = __builtin_amdgcn_readlane(pi, lp);
#pragma unroll
        for (int u = 0; u < NU; ++u)
          sel_before[u] = __popcll(__ballot(sel && pi < kTkChunk * u + 256 * w));
      } else {
        for (int i = tid; i < nc; i += kTkThreads) {
          const uint32_t ki = sh.ckey[i];
          const int pi = sh.cpos[i];
          int r = 0;
          for (int j = 0; j < nc; ++j) {
            const uint32_t kj = sh.ckey[j];
            r += (kj > ki || (kj == ki && sh.cpos[j] < pi)) ? 1 : 0;
          }
          if (r < remain) atomicAdd(&sh.cell[cell_of(pi)], 1);
          if (r == remain - 1) { sh.T = ki; sh.posT = pi; }
        }
        __syncthreads();
        T = sh.T;
        posT = sh.posT;
      }
    } else {
      // ---- exact radix select over the three key digits
      uint32_t prefix = 0, mask = 0;
      int rem = kk;
      for (int pass = 0; pass < 3; ++pass) {
        const int shift = digit_shift(pass), nbins = digit_bins(pass);
        __syncthreads();
        for (int i = tid; i < kTkHistWords; i += kTkThreads) sh.hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const uint32_t kv = key[u][s];
            if (kv != 0u && (kv & mask) == prefix) {
              const int d = static_cast<int>((kv >> shift) & (nbins - 1));
              atomicAdd(&sh.hist[nbins == 2048 ? hist_slot<32>(d) : hist_slot<16>(d)], 1u);
            }
          }
        __syncthreads();
        int above, bb;
        if (nbins == 2048) bb = wave_threshold_bin<32>(sh.hist, rem, above);
        else bb = wave_threshold_bin<16>(sh.hist, rem, above);
        prefix |= static_cast<uint32_t>(bb) << shift;
        mask |= static_cast<uint32_t>(nbins - 1) << shift;
        rem -= above;
      }
      T = prefix;
      need_eq = rem;
      exact = true;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        int g = 0, e = 0;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          g += __popcll(__ballot(key[u][s] > T));
          e += __popcll(__ballot(key[u][s] == T));
        }
        if (l == 0) { sh.cell[u * kTkWaves + w] = g; sh.cell_eq[u * kTkWaves + w] = e; }
      }
      __syncthreads();
      cells = sh.cell;
      cells_before<NU>(sh.cell_eq, w, eq_before);
#pragma unroll
      for (int u = 0; u < NU; ++u) sel_before[u] = min(need_eq, eq_before[u]);
    }
  }
  // ---- 5. output slots: cells before this one, then lanes before this one
  int base[NU];
  cells_before<NU>(cells, w, base);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    int c = 0;
    if (exact) {
      int e = 0;
#pragma unroll
      for (int s = 0; s < 4; ++s) e += key[u][s] == T ? 1 : 0;
      int r = eq_before[u] + wave_incl_scan(e) - e;        // rank among keys == T
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t kv = key[u][s];
        bool t = kv > T;
        if (kv == T) t = r++ < need_eq;
        if (t) { taken |= 1ull << (4 * u + s); ++c; }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t kv = key[u][s];
        const int pos = kTkChunk * u + 4 * tid + s;
        if (kv > T || (kv == T && pos <= posT)) { taken |= 1ull << (4 * u + s); ++c; }
      }
    }
    obase[u] = base[u] + sel_before[u] + wave_incl_scan(c) - c;
  }
  return kk;
}

// Loads positions [0, n) of a score row as keys into registers (key 0 beyond n).
template <int NU>
__device__ __forceinline__ void load_score_keys(uint32_t (&key)[NU][4], const float* __restrict__ s, int n) {
  const bool vec = (reinterpret_cast<uintptr_t>(s) & 15u) == 0;
  float4 v[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int p = kTkChunk * u + 4 * static_cast<int>(threadIdx.x);
    if (vec && p + 3 < n) {
      v[u] = *reinterpret_cast<const float4*>(s + p);
    } else {
      v[u].x = p < n ? s[p] : -INFINITY;
      v[u].y = p + 1 < n ? s[p + 1] : -INFINITY;
      v[u].z = p + 2 < n ? s[p + 2] : -INFINITY;
      v[u].w = p + 3 < n ? s[p + 3] : -INFINITY;
    }
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    key[u][0] = score_key(v[u].x);
    key[u][1] = score_key(v[u].y);
    key[u][2] = score_key(v[u].z);
    key[u][3] = score_key(v[u].w);
  }
}

// ---------------------------------------------------------------------------------------
// One workgroup per row (Nc <= NU * 4096).
// ---------------------------------------------------------------------------------------
template <int NU>
__global__ __launch_bounds__(kTkThreads) void topk_rows(const float* __restrict__ scores, int Nc, int k,
                                                        int32_t* __restrict__ idx) {
  __shared__ TkShared sh;
  const size_t row = blockIdx.x;
  uint32_t key[NU][4];
  load_score_keys<NU>(key, scores + row * Nc, Nc);
  uint64_t taken;
  int obase[NU];
  const int kk = select_regs<NU>(sh, key, k, taken, obase);
  int32_t* out = idx + row * k;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    int o = obase[u];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if ((taken >> (4 * u + s)) & 1ull) out[o++] = kTkChunk * u + 4 * static_cast<int>(threadIdx.x) + s;
  }
  for (int p = kk + threadIdx.x; p < k; p += kTkThreads) out[p] = -1;
}

// ---------------------------------------------------------------------------------------
// Segmented schedule.  Workspace cand[rows][G][k] of (key, index) pairs, key 0 = empty,
// each segment's pairs in ascending index order.  Grid (rows, G).
// ---------------------------------------------------------------------------------------
template <int NU>
__global__ __launch_bounds__(kTkThreads) void topk_segments(const float* __restrict__ scores, int Nc, int k,
                                                            int seg, uint2* __restrict__ cand) {
  __shared__ TkShared sh;
  const size_t row = blockIdx.x;
  const int G = gridDim.y, g = blockIdx.y;
  const int j0 = g * seg;
  const int n = max(0, min(seg, Nc - j0));
  const float* sr = scores + row * Nc + min(j0, Nc);
  uint32_t key[NU][4];
  load_score_keys<NU>(key, sr, n);
  uint64_t taken;
  int obase[NU];
  const int kk = select_regs<NU>(sh, key, k, taken, obase);
  uint2* out = cand + (row * G + g) * static_cast<size_t>(k);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    int o = obase[u];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if ((taken >> (4 * u + s)) & 1ull) {      // the key is read again (cached) to keep registers low
        const int p = kTkChunk * u + 4 * static_cast<int>(threadIdx.x) + s;
        out[o++] = make_uint2(score_key(sr[p]), static_cast<uint32_t>(j0 + p));
      }
  }
  for (int p = kk + threadIdx.x; p < k; p += kTkThreads) out[p] = make_uint2(0u, 0u);
}

// One workgroup per row over the n = G*k pairs of its segments (n <= NU * 4096).  Only
// the keys are held in registers; the indices of the taken pairs are read again.
template <int NU>
__global__ __launch_bounds__(kTkThreads) void topk_merge(const uint2* __restrict__ cand, int n, int k,
                                                         int32_t* __restrict__ idx) {
  __shared__ TkShared sh;
  const size_t row = blockIdx.x;
  const uint2* c = cand + row * static_cast<size_t>(n);
  const bool vec = (reinterpret_cast<uintptr_t>(c) & 15u) == 0;
  uint32_t key[NU][4];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int p = kTkChunk * u + 4 * static_cast<int>(threadIdx.x);
    if (vec && p + 3 < n) {
      const uint4 a = *reinterpret_cast<const uint4*>(c + p);
      const uint4 b = *reinterpret_cast<const uint4*>(c + p + 2);
      key[u][0] = a.x;
      key[u][1] = a.z;
      key[u][2] = b.x;
      key[u][3] = b.z;
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) key[u][s] = p + s < n ? c[p + s].x : 0u;
    }
  }
  uint64_t taken;
  int obase[NU];
  const int kk = select_regs<NU>(sh, key, k, taken, obase);
  int32_t* out = idx + row * k;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    int o = obase[u];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if ((taken >> (4 * u + s)) & 1ull)
        out[o++] = static_cast<int32_t>(c[kTkChunk * u + 4 * static_cast<int>(threadIdx.x) + s].y);
  }
  for (int p = kk + threadIdx.x; p < k; p += kTkThreads) out[p] = -1;
}

// ---------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------
// Register chunks per workgroup for a set of n keys: 1, 2, 4 or 9.
static int chunks_for(int n) {
  const int c = cdiv(std::max(n, 1), kTkChunk);
  return c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : kTkMaxChunks;
}

// Segments per row: about sqrt(Nc / k), which balances the segment and merge work, with
// every segment and the G*k merged pairs within one workgroup.  0 = no valid split.
int topk_segments_per_row(int Nc, int k) {
  const int g_max = kTkMaxSet / k;
  const int g_min = cdiv(Nc, kTkMaxSet);
  if (g_max < 2 || g_min > g_max) return 0;
  int G = static_cast<int>(std::lround(std::sqrt(static_cast<double>(Nc) / k)));
  G = std::max(G, cdiv(Nc, 4 * kTkChunk));     // segments of <= 16384 keys where possible
  return std::min(g_max, std::max(std::max(G, g_min), 2));
}

static int topk_seg_len(int Nc, int G) { return 4 * cdiv(cdiv(Nc, G), 4); }

size_t topk_workspace_bytes(int rows, int Nc, int k) {
  const int G = topk_segments_per_row(Nc, k);
  return G < 2 ? 0 : static_cast<size_t>(rows) * G * k * sizeof(uint2);
}

// Whether a shape can run: with a workspace (any split allowed) or without one (the
// row must fit one workgroup).
bool topk_supported(int Nc, int k, bool with_ws) {
  if (Nc <= kTkMaxSet) return true;
  return with_ws && topk_segments_per_row(Nc, k) >= 2;
}

template <int NU>
static void launch_rows(const float* scores, int rows, int Nc, int k, int32_t* idx, hipStream_t st) {
  hipLaunchKernelGGL(topk_rows<NU>, dim3(rows), dim3(kTkThreads), 0, st, scores, Nc, k, idx);
}
template <int NU>
static void launch_segments(const float* scores, int rows, int G, int Nc, int k, int seg, uint2* cand,
                            hipStream_t st) {
  hipLaunchKernelGGL(topk_segments<NU>, dim3(rows, G), dim3(kTkThreads), 0, st, scores, Nc, k, seg, cand);
}
template <int NU>
static void launch_merge(const uint2* cand, int rows, int n, int k, int32_t* idx, hipStream_t st) {
  hipLaunchKernelGGL(topk_merge<NU>, dim3(rows), dim3(kTkThreads), 0, st, cand, n, k, idx);
}

// algo: 0 = automatic, 1 = one workgroup per row, 2 = segments + merge.  The caller has
// checked topk_supported() and the workspace size.
int launch_topk(const float* scores, int rows, int Nc, int k, int32_t* idx, void* ws, size_t ws_bytes,
                int algo, hipStream_t st) {
  const int G = topk_segments_per_row(Nc, k);
  const bool seg_ok = G >= 2 && ws != nullptr && ws_bytes >= topk_workspace_bytes(rows, Nc, k);
  const bool rows_ok = Nc <= kTkMaxSet;
  if (algo == 0) algo = (seg_ok && (!rows_ok || rows < 128)) ? 2 : 1;
  if (algo == 2 && !seg_ok) algo = 1;
  if (algo == 1 && !rows_ok) algo = 2;
  if (algo == 2 && !seg_ok) return CSA_ERR_WORKSPACE;
  if (algo == 1) {
    switch (chunks_for(Nc)) {
      case 1: launch_rows<1>(scores, rows, Nc, k, idx, st); break;
      case 2: launch_rows<2>(scores, rows, Nc, k, idx, st); break;
      case 4: launch_rows<4>(scores, rows, Nc, k, idx, st); break;
      default: launch_rows<kTkMaxChunks>(scores, rows, Nc, k, idx, st); break;
    }
    CSA_LAUNCH_CHECK();
    return CSA_OK;
  }
  const int seg = topk_seg_len(Nc, G);
  uint2* cand = static_cast<uint2*>(ws);
  switch (chunks_for(seg)) {
    case 1: launch_segments<1>(scores, rows, G, Nc, k, seg, cand, st); break;
    case 2: launch_segments<2>(scores, rows, G, Nc, k, seg, cand, st); break;
    case 4: launch_segments<4>(scores, rows, G, Nc, k, seg, cand, st); break;
    default: launch_segments<kTkMaxChunks>(scores, rows, G, Nc, k, seg, cand, st); break;
  }
  CSA_LAUNCH_CHECK();
  const int n = G * k;
  switch (chunks_for(n)) {
    case 1: launch_merge<1>(cand, rows, n, k, idx, st); break;
    case 2: launch_merge<2>(cand, rows, n, k, idx, st); break;
    case 4: launch_merge<4>(cand, rows, n, k, idx, st); break;
    default: launch_merge<kTkMaxChunks>(cand, rows, n, k, idx, st); break;
  }
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

}  // namespace csa
