// Selection of the k largest keys of a set held in registers by one workgroup: the core of
// the top-k stage (see topk.hip), also run by the fused indexer epilogue (segment top-k)
// and by the attention kernel that selects from segment candidates.
//
// Keys are order-preserving images of the scores (score_key); the order is (key
// descending, position ascending), a total order, and positions follow index order, so
// the first kk elements in this order are exactly the required selection:
//   1. candidate count and key range (block reduction);
//   2. histogram over 1024 equal-width bins of [min, max] of the candidate values (bin =
//      trunc((x-min)*scale), monotone in x because every rounding step is);
//   3. every wave finds the bin b holding the kk-th element from the padded histogram;
//      elements of higher bins are taken (a bit per element in registers), bin b goes to
//      an LDS candidate list;
//   4. the candidates are ranked in the total order (by readlane within one wave when
//      there are at most 64), giving the pivot (T, posT), the kk-th element; the list's
//      taken elements are marked in an LDS bitmap over positions;
//   5. an element is taken iff it precedes or equals the pivot: its bit from step 3 or
//      the bitmap; an ordered compaction (per-(chunk, wave) counts, one scan) gives every
//      taken element its output slot.
// Degenerate value ranges (all equal, infinities, or more than kTkCandCap keys in bin b)
// take an exact radix select over the three key digits (11, 11, 10 bits) and a tie rank
// among keys equal to T.
#pragma once

#include "common.hpp"

namespace csa {

constexpr int kTkMaxWaves = 16;                // largest workgroup: 1024 threads
constexpr int kTkMaxChunks = 9;                // largest register set: 9 chunks

constexpr int kTkBins = 1024;                  // equal-width bins of the fast path
constexpr int kTkPB = kTkBins / kWave;
constexpr int kTkHistWords = 2048 + 4 * 64;    // largest padded histogram (11-bit digit)
constexpr int kTkCandCap = 1024;
constexpr int kTkSelWords = kTkMaxChunks * 4096 / 32;   // bitmap of taken list elements

// radix digits, most significant first: bits 31..21, 20..10, 9..0
__host__ __device__ constexpr inline int digit_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__host__ __device__ constexpr inline int digit_bins(int pass) { return pass < 2 ? 2048 : 1024; }

struct alignas(16) TkShared {
  uint32_t hist[kTkHistWords];
  uint32_t ckey[kTkCandCap];
  uint32_t selbits[kTkSelWords];             // bit p: list element at position p taken
  int32_t cpos[kTkCandCap];
  int cell_nz[kTkMaxChunks * kTkMaxWaves];   // candidates per wave
  int cell[kTkMaxChunks * kTkMaxWaves];      // taken elements per (chunk, wave) above bin b / > T
  int cell_eq[kTkMaxChunks * kTkMaxWaves];   // exact path: keys equal to T per (chunk, wave)
  uint32_t red_lo[kTkMaxWaves], red_hi[kTkMaxWaves];   // smallest and largest candidate key per wave
  int ncand;
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
__device__ __forceinline__ int hist_slot(int bin) {
  const unsigned u = static_cast<unsigned>(bin);      // bins are >= 0
  return static_cast<int>(u + 4u * (u / PB));
}

// Threshold search run by every wave on its own over the complete histogram (no
// barrier): with 1 <= remain <= total, returns the bin b with
// (#keys in bins > b) < remain <= (#keys in bins >= b) and sets above = #keys in bins > b
// and count = #keys in bin b.
template <int PB>
__device__ __forceinline__ int wave_threshold_bin(const uint32_t* hist, int remain, int& above, int& count) {
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
  count = __builtin_amdgcn_readlane(c, J);
  return nbins - 1 - (PB * L + J);
}

// (chunk, wave) cell of a position: NT threads of KPT consecutive positions per chunk
template <int NT, int KPT>
__device__ __forceinline__ int cell_of(int pos) {
  return (pos / (KPT * NT)) * (NT / kWave) + (pos % (KPT * NT)) / (KPT * kWave);
}

// Exclusive prefix sums over the cells (chunk, wave) order, computed by every wave:
// returns the sum over the cells before cell (u, w) for each chunk u.
template <int NU, int W>
__device__ __forceinline__ void cells_before(const int* cells, int w, int (&out)[NU]) {
  constexpr int kCells = NU * W;
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
  for (int u = 0; u < NU; ++u)          // cell u*W + w: register (u*W)/64, lane (u*W)%64 + w (W divides 64)
    out[u] = cbase[(u * W) >> 6] + __builtin_amdgcn_readlane(cexcl[(u * W) >> 6], ((u * W) & 63) + w);
}

// Selection over the keys of one set held in registers by a workgroup of NT threads:
// key[u][s] is the key of position KPT*NT*u + KPT*threadIdx.x + s (0 = not a candidate).
// kPre: the caller has done step 1 itself, before a barrier: every wave w wrote its
// smallest candidate key - 1, largest key and candidate count to sh.red_lo[w],
// sh.red_hi[w], sh.cell_nz[w] (any partition of the set over the waves), and the
// histogram, the taken-element bitmap and sh.ncand were cleared (sel_clear).
// Returns kk = min(k, #candidates); sets bit KPT*u+s of `taken` for the taken elements and
// obase[u] to the output slot of this thread's first taken element of chunk u (taken
// elements fill slots 0..kk-1 in position order).
// Step 1's clears: the histogram, the first NPOS bits of the taken-element bitmap, the list.
template <int NT, int NPOS>
__device__ __forceinline__ void sel_clear(TkShared& sh) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kTkHistWords / 4; i += NT) reinterpret_cast<uint4*>(sh.hist)[i] = make_uint4(0u, 0u, 0u, 0u);
  for (int i = tid; i < NPOS / 128; i += NT) reinterpret_cast<uint4*>(sh.selbits)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (tid == 0) sh.ncand = 0;
}

// Step 1's per-wave partials (this lane's smallest candidate key - 1, largest key and
// candidate count, reduced over the wave) into wave w's LDS slots.
__device__ __forceinline__ void sel_wave_range(TkShared& sh, int w, int l, uint32_t kmin1, uint32_t kmax, int cnt) {
  kmax = wave_max_u32(kmax);
  kmin1 = ~wave_max_u32(~kmin1);
  cnt = __builtin_amdgcn_readlane(wave_incl_scan(cnt), 63);
  if (l == 0) { sh.red_lo[w] = kmin1; sh.red_hi[w] = kmax; sh.cell_nz[w] = cnt; }
}

template <int NT, int KPT, int NU, bool kPre = false>
__device__ int select_regs(TkShared& sh, const uint32_t (&key)[NU][KPT], int k, uint64_t& taken, int (&obase)[NU]) {
  static_assert(NT % kWave == 0 && kWave % (NT / kWave) == 0 && NU * KPT <= 64, "select_regs shape");
  static_assert(NU * KPT * NT <= 32 * kTkSelWords && 32 % KPT == 0, "taken-element bitmap");
  constexpr int W = NT / kWave;                 // waves
  constexpr int kChunk = KPT * NT;              // positions per chunk
  const int tid = threadIdx.x, w = wave_index();
  const int l = static_cast<int>(lane_id());
  // ---- 1. candidate count and key range, per thread and then per wave: no branches
  // (key 0 is the smallest key, and key - 1 wraps it to the largest)
  uint32_t kmin1 = 0xffffffffu, kmax = 0u;      // smallest candidate key - 1, largest key
  if constexpr (!kPre) {
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int s = 0; s < KPT; ++s) {
        const uint32_t kv = key[u][s];
        cnt += kv != 0u ? 1 : 0;
        kmax = max(kmax, kv);
        kmin1 = min(kmin1, kv - 1u);
      }
    sel_clear<NT, NU * KPT * NT>(sh);
    sel_wave_range(sh, w, l, kmin1, kmax, cnt);
    __syncthreads();                                                  // barrier 1
  }
  int total = 0;
  kmin1 = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    kmin1 = min(kmin1, sh.red_lo[i]);
    kmax = max(kmax, sh.red_hi[i]);
    total += sh.cell_nz[i];
  }
  const uint32_t kmin = kmin1 + 1u;             // used only when there are candidates
  const int kk = __builtin_amdgcn_readfirstlane(min(k, total));
  taken = 0;
#pragma unroll
  for (int u = 0; u < NU; ++u) obase[u] = 0;
  if (kk == 0) return 0;

  uint32_t T = 0u;               // exact path: the kk-th key
  int sel_before[NU];            // taken candidates of bin b before each of this wave's cells
  int eq_before[NU];             // exact path: keys == T before each of this wave's cells
  bool exact = false;
  int need_eq = 0;
  const int* cells = sh.cell;
#pragma unroll
  for (int u = 0; u < NU; ++u) { sel_before[u] = 0; eq_before[u] = 0; }
  if (kk < total) {
    const float lo = key_value(kmin);
    const float range = key_value(kmax) - lo;
    // any positive scale keeps the bins monotone in the value; the reciprocal is enough
    const float scale = static_cast<float>(kTkBins) * __builtin_amdgcn_rcpf(range);
    bool ok = range > 0.0f && range <= 3.0e38f && scale <= 3.0e38f;
    int b = 0, remain = 0;
    // each key's bin is kept from the histogram pass for the next one: as ints for small
    // register sets, two per register (bin + 1 in 16 bits, 0 = no candidate) for large ones
    constexpr bool kKeepBins = NU * KPT <= 16;
    constexpr int kPacked = kKeepBins ? 1 : (NU * KPT + 1) / 2;
    int bins[kKeepBins ? NU : 1][kKeepBins ? KPT : 1];
    uint32_t pbins[kPacked];
#pragma unroll
    for (int i = 0; i < kPacked; ++i) pbins[i] = 0u;
    auto bin_of = [&](uint32_t kv) __attribute__((always_inline)) {
      return kv != 0u ? min(kTkBins - 1, static_cast<int>((key_value(kv) - lo) * scale)) : -1;
    };
    if (ok) {
      // ---- 2. histogram over equal-width bins of [min, max]; a key that is not a
      // candidate adds to a padding word of its lane's bin group (never read), so the
      // pass has no branches
      const int junk = hist_slot<kTkPB>(kTkPB * l) + kTkPB;
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int s = 0; s < KPT; ++s) {
          const int bn = bin_of(key[u][s]);
          if constexpr (kKeepBins) {
            bins[u][s] = bn;
          } else {
            const int i = KPT * u + s;
            pbins[i >> 1] |= static_cast<uint32_t>(bn + 1) << (16 * (i & 1));
          }
          atomicAdd(&sh.hist[bn >= 0 ? hist_slot<kTkPB>(bn) : junk], 1u);
        }
      __syncthreads();                                                // barrier 2
      int above, cnt_b;
      b = wave_threshold_bin<kTkPB>(sh.hist, kk, above, cnt_b);
      remain = kk - above;
      ok = cnt_b <= kTkCandCap;
    }
    if (ok) {
      // ---- 3. higher bins are taken (counted per cell); bin b goes to the list
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        int g = 0;
#pragma unroll
        for (int s = 0; s < KPT; ++s) {
          const uint32_t kv = key[u][s];
          int bn;
          if constexpr (kKeepBins) {
            bn = bins[u][s];
          } else {
            const int i = KPT * u + s;
            bn = static_cast<int>((pbins[i >> 1] >> (16 * (i & 1))) & 0xffffu) - 1;
          }
          const bool above = bn > b;
          g += __popcll(__ballot(above));
          if (above) taken |= 1ull << (KPT * u + s);
          const uint64_t m = __ballot(bn == b);
          if (m != 0) {
            int base = 0;
            const int leader = __ffsll(static_cast<long long>(m)) - 1;
            if (l == leader) base = atomicAdd(&sh.ncand, __popcll(m));
            base = __builtin_amdgcn_readlane(base, leader);
            if (bn == b) {
              const int p = base + lanes_below(m);
              sh.ckey[p] = kv;
              sh.cpos[p] = kChunk * u + KPT * tid + s;
            }
          }
        }
        if (l == 0) sh.cell[u * W + w] = g;
      }
      __syncthreads();                                                // barrier 3
      cells = sh.cell;
      // ---- 4. rank the candidates; the first remain of them are taken
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
#pragma unroll
        for (int u = 0; u < NU; ++u)
          sel_before[u] = __popcll(__ballot(sel && pi < kChunk * u + KPT * kWave * w));
        // every wave marks the taken list elements among its own positions (the only
        // bitmap words it reads), so no barrier is needed
        if (sel && (pi % kChunk) / (KPT * kWave) == w) atomicOr(&sh.selbits[pi >> 5], 1u << (pi & 31));
      } else {
        for (int i = tid; i < nc; i += NT) {
          const uint32_t ki = sh.ckey[i];
          const int pi = sh.cpos[i];
          int r = 0;
          for (int j = 0; j < nc; ++j) {
            const uint32_t kj = sh.ckey[j];
            r += (kj > ki || (kj == ki && sh.cpos[j] < pi)) ? 1 : 0;
          }
          if (r < remain) {
            atomicAdd(&sh.cell[cell_of<NT, KPT>(pi)], 1);
            atomicOr(&sh.selbits[pi >> 5], 1u << (pi & 31));
          }
        }
        __syncthreads();
      }
    } else {
      // ---- exact radix select over the three key digits
      uint32_t prefix = 0, mask = 0;
      int rem = kk;
      for (int pass = 0; pass < 3; ++pass) {
        const int shift = digit_shift(pass), nbins = digit_bins(pass);
        __syncthreads();
        for (int i = tid; i < kTkHistWords / 4; i += NT) reinterpret_cast<uint4*>(sh.hist)[i] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int s = 0; s < KPT; ++s) {
            const uint32_t kv = key[u][s];
            if (kv != 0u && (kv & mask) == prefix) {
              const int d = static_cast<int>((kv >> shift) & (nbins - 1));
              atomicAdd(&sh.hist[nbins == 2048 ? hist_slot<32>(d) : hist_slot<16>(d)], 1u);
            }
          }
        __syncthreads();
        int above, bb, cnt_unused;
        if (nbins == 2048) bb = wave_threshold_bin<32>(sh.hist, rem, above, cnt_unused);
        else bb = wave_threshold_bin<16>(sh.hist, rem, above, cnt_unused);
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
        for (int s = 0; s < KPT; ++s) {
          g += __popcll(__ballot(key[u][s] > T));
          e += __popcll(__ballot(key[u][s] == T));
        }
        if (l == 0) { sh.cell[u * W + w] = g; sh.cell_eq[u * W + w] = e; }
      }
      __syncthreads();
      cells = sh.cell;
      cells_before<NU, W>(sh.cell_eq, w, eq_before);
#pragma unroll
      for (int u = 0; u < NU; ++u) sel_before[u] = min(need_eq, eq_before[u]);
    }
  } else {
    // every candidate is taken: candidates per (chunk, wave) give the output slots
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      int c = 0;
#pragma unroll
      for (int s = 0; s < KPT; ++s) {
        c += __popcll(__ballot(key[u][s] != 0u));
        if (key[u][s] != 0u) taken |= 1ull << (KPT * u + s);
      }
      if (l == 0) sh.cell[u * W + w] = c;
    }
    __syncthreads();
  }
  // ---- 5. output slots: cells before this one, then lanes before this one
  int base[NU];
  cells_before<NU, W>(cells, w, base);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    int c = 0;
    if (exact) {
      int e = 0;
#pragma unroll
      for (int s = 0; s < KPT; ++s) e += key[u][s] == T ? 1 : 0;
      int r = eq_before[u] + wave_incl_scan(e) - e;        // rank among keys == T
#pragma unroll
      for (int s = 0; s < KPT; ++s) {
        const uint32_t kv = key[u][s];
        bool t = kv > T;
        if (kv == T) t = r++ < need_eq;
        if (t) { taken |= 1ull << (KPT * u + s); ++c; }
      }
      obase[u] = base[u] + sel_before[u] + wave_incl_scan(c) - c;
    } else {
      // taken: the bits of step 3 (higher bins; every candidate when all are taken) and
      // the list elements marked in the bitmap (KPT consecutive positions in one word)
      const int p0 = kChunk * u + KPT * tid;
      const uint32_t lb = (sh.selbits[p0 >> 5] >> (p0 & 31)) & ((1u << KPT) - 1u);
      taken |= static_cast<uint64_t>(lb) << (KPT * u);
      obase[u] = __popc(static_cast<uint32_t>(taken >> (KPT * u)) & ((1u << KPT) - 1u));   // this lane's count for now
    }
  }
  if (!exact) {
    // lane prefixes of three chunks' counts per scan: a lane's count is <= KPT, so a
    // chunk's wave total (<= 64 * KPT <= 1023) fits a 10-bit field without carries
    static_assert(64 * KPT < 1024, "10-bit count fields");
#pragma unroll
    for (int u0 = 0; u0 < NU; u0 += 3) {
      int packed = 0;
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (u0 + j < NU) packed |= obase[u0 + j] << (10 * j);
      const int excl = wave_incl_scan(packed) - packed;
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (u0 + j < NU) obase[u0 + j] = base[u0 + j] + sel_before[u0 + j] + ((excl >> (10 * j)) & 1023);
    }
  }
  return kk;
}


}  // namespace csa
