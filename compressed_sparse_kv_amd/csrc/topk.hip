// Top-k selection (stage 3).
//
// Per row of Nc fp32 scores: the indices of the min(k, n_cand) largest candidate scores
// (candidates: not -inf, not NaN), ties to the lower index, ascending, padded with -1.
// [KV-COMP] sections 9.4 (S_t = TopK_k of the indexer scores) and 9.8 (invisible entries
// are -inf before the selection and -1 after it).
//
// Scores become order-preserving 32-bit keys (score_key).  A radix select over three
// digits (11, 11, 10 bits) finds the key T of the kk-th largest candidate and how many
// keys equal to T must be taken (need_eq).  The selection is then {key > T} plus the
// first need_eq entries with key == T in index order.
//
// Two schedules:
//  * one workgroup per row (1024 threads): the row's keys sit in LDS when they fit
//    (Nc <= kTkLdsKeys), otherwise each pass re-reads the scores; the output is written
//    in index order by a ballot compaction, so it needs no sort;
//  * few long rows: G workgroups per row build the first-digit histogram and collect
//    the entries above / inside the threshold bin; one workgroup per row then finishes
//    the select on the (small) candidate set and sorts the <= k chosen indices.
#include "common.hpp"

namespace csa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkLdsKeys = 36864;                 // 144 KiB of keys
constexpr int kTkBins = 2048;
// radix digits, most significant first: bits 31..21, 20..10, 9..0
__host__ __device__ constexpr inline int digit_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__host__ __device__ constexpr inline int digit_bins(int pass) { return pass < 2 ? 2048 : 1024; }

// ---- block-wide helpers for 1024 threads ---------------------------------------------
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = static_cast<int>(lane_id());
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(v, o, kWave);
    if (l >= o) v += y;
  }
  return v;
}

struct TkShared {
  uint32_t hist[kTkBins];
  int wtot[kTkWaves];
  int wgt[kTkWaves];
  int weq[kTkWaves];
  int bin;
  int above;
  int ncand;
};

// Given hist[0..nbins) and `remain` (>= 1, <= total), finds the bin b such that
// (#keys in bins > b) < remain <= (#keys in bins >= b).  Writes sh.bin, sh.above.
// Needs 1024 threads and nbins <= 2048.
__device__ void find_threshold_bin(TkShared& sh, int nbins, int remain) {
  const int tid = threadIdx.x, w = tid >> 6;
  // thread t owns the bins at descending positions r = 2t, 2t+1 (bin = nbins-1-r)
  int c0 = 0, c1 = 0;
  const int r0 = 2 * tid, r1 = 2 * tid + 1;
  if (r0 < nbins) c0 = static_cast<int>(sh.hist[nbins - 1 - r0]);
  if (r1 < nbins) c1 = static_cast<int>(sh.hist[nbins - 1 - r1]);
  const int incl = wave_incl_scan(c0 + c1);
  if (lane_id() == 63) sh.wtot[w] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += sh.wtot[i];
  const int p1 = before + incl;          // keys in bins at positions <= r1
  const int p0 = p1 - c1;                // keys in bins at positions <= r0
  const int pm = p0 - c0;                // keys in bins at positions < r0
  if (r0 < nbins && pm < remain && remain <= p0) { sh.bin = nbins - 1 - r0; sh.above = pm; }
  if (r1 < nbins && p0 < remain && remain <= p1) { sh.bin = nbins - 1 - r1; sh.above = p0; }
  __syncthreads();
}

// Radix select over all keys of a row held either in LDS (keys != nullptr) or re-read
// from `scores`.  Returns T and need_eq (keys == T to take); kk >= 1.
template <typename KeyAt>
__device__ void radix_select(TkShared& sh, KeyAt key_at, int n, int kk, uint32_t& T, int& need_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  int remain = kk;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = digit_shift(pass), nbins = digit_bins(pass);
    for (int i = tid; i < nbins; i += kTkThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < n; j += kTkThreads) {
      const uint32_t key = key_at(j);
      if (key != 0u && (key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (nbins - 1)], 1u);
    }
    __syncthreads();
    find_threshold_bin(sh, nbins, remain);
    prefix |= static_cast<uint32_t>(sh.bin) << shift;
    mask |= static_cast<uint32_t>(nbins - 1) << shift;
    remain -= sh.above;
    __syncthreads();
  }
  T = prefix;
  need_eq = remain;
}

// Writes the selection {key > T} + first need_eq of {key == T} in index order, then -1s.
template <typename KeyAt>
__device__ void ordered_compaction(TkShared& sh, KeyAt key_at, int n, int k, int kk, uint32_t T,
                                   int need_eq, int32_t* __restrict__ out) {
  const int tid = threadIdx.x, w = tid >> 6;
  const int l = static_cast<int>(lane_id());
  const int span = cdiv(cdiv(n, kTkWaves), kWave) * kWave;      // contiguous range per wave
  const int j0 = w * span, j1 = min(n, j0 + span);
  int gt = 0, eq = 0;
  for (int j = j0 + l; j - l < j1; j += kWave) {
    const uint32_t key = j < j1 ? key_at(j) : 0u;
    gt += __popcll(__ballot(key > T));
    eq += __popcll(__ballot(key == T && key != 0u));
  }
  if (l == 0) { sh.wgt[w] = gt; sh.weq[w] = eq; }
  __syncthreads();
  int eq_run = 0, pos = 0;
  for (int i = 0; i < w; ++i) {
    const int take = max(0, min(need_eq - eq_run, sh.weq[i]));
    pos += sh.wgt[i] + take;
    eq_run += sh.weq[i];
  }
  for (int j = j0 + l; j - l < j1; j += kWave) {
    const uint32_t key = j < j1 ? key_at(j) : 0u;
    const uint64_t em = __ballot(key == T && key != 0u);
    const bool sel = key > T || (key == T && key != 0u && eq_run + lanes_below(em) < need_eq);
    const uint64_t sm = __ballot(sel);
    if (sel) out[pos + lanes_below(sm)] = j;
    pos += __popcll(sm);
    eq_run += __popcll(em);
  }
  for (int p = kk + tid; p < k; p += kTkThreads) out[p] = -1;
}

__device__ int count_candidates(TkShared& sh, int local) {
  const int w = threadIdx.x >> 6;
  const int s = wave_sum_int(local);
  if (lane_id() == 0) sh.wtot[w] = s;
  __syncthreads();
  int tot = 0;
  for (int i = 0; i < kTkWaves; ++i) tot += sh.wtot[i];
  __syncthreads();
  return tot;
}

// One workgroup per row.  kInLds: the row's keys are cached in LDS.
template <bool kInLds>
__global__ __launch_bounds__(kTkThreads) void topk_rows(const float* __restrict__ scores, int Nc, int k,
                                                        int32_t* __restrict__ idx) {
  extern __shared__ uint32_t lkeys[];
  __shared__ TkShared sh;
  const size_t row = blockIdx.x;
  const float* sr = scores + row * Nc;
  int32_t* out = idx + row * k;
  int local = 0;
  for (int j = threadIdx.x; j < Nc; j += kTkThreads) {
    const uint32_t key = score_key(sr[j]);
    if (kInLds) lkeys[j] = key;
    local += key != 0u;
  }
  const int ncand = count_candidates(sh, local);
  const int kk = min(k, ncand);
  auto key_at = [&](int j) -> uint32_t { return kInLds ? lkeys[j] : score_key(sr[j]); };
  if (kk == 0) {
    for (int p = threadIdx.x; p < k; p += kTkThreads) out[p] = -1;
    return;
  }
  uint32_t T;
  int need_eq;
  radix_select(sh, key_at, Nc, kk, T, need_eq);
  ordered_compaction(sh, key_at, Nc, k, kk, T, need_eq, out);
}

// ---------------------------------------------------------------------------------------
// Multi-workgroup schedule for few long rows.
// Workspace per row: hist[2048] u32 | counters[4] (ncand, ngt, ncand_bin, pad) |
//                    gt[k] i32 | cand_key[cap] u32 | cand_idx[cap] i32
// ---------------------------------------------------------------------------------------
constexpr int kMwThreads = 256;
constexpr int kMwCap = 8192;                  // threshold-bin candidates kept per row
constexpr int kMwSegment = 4096;              // scores per workgroup in the parallel passes

struct MwRow {
  uint32_t* hist;
  int* counters;
  int32_t* gt;
  uint32_t* ckey;
  int32_t* cidx;
};

__host__ __device__ inline size_t mw_row_words(int k) { return kTkBins + 4 + k + 2 * kMwCap; }

__device__ inline MwRow mw_row(uint32_t* ws, int k, size_t row) {
  uint32_t* base = ws + row * mw_row_words(k);
  MwRow r;
  r.hist = base;
  r.counters = reinterpret_cast<int*>(base + kTkBins);
  r.gt = reinterpret_cast<int32_t*>(base + kTkBins + 4);
  r.ckey = base + kTkBins + 4 + k;
  r.cidx = reinterpret_cast<int32_t*>(base + kTkBins + 4 + k + kMwCap);
  return r;
}

__global__ void topk_mw_clear(uint32_t* __restrict__ ws, int k, int rows) {
  const size_t words = kTkBins + 4;
  for (size_t i = blockIdx.x * blockDim.x + threadIdx.x; i < rows * words; i += gridDim.x * blockDim.x) {
    const size_t r = i / words, o = i % words;
    ws[r * mw_row_words(k) + o] = 0u;
  }
}

__global__ __launch_bounds__(kMwThreads) void topk_mw_hist(const float* __restrict__ scores, int Nc, int k,
                                                           uint32_t* __restrict__ ws) {
  __shared__ uint32_t h[kTkBins];
  __shared__ int wcnt[kMwThreads / kWave];
  const size_t row = blockIdx.y;
  const MwRow R = mw_row(ws, k, row);
  const float* sr = scores + row * Nc;
  for (int i = threadIdx.x; i < kTkBins; i += kMwThreads) h[i] = 0u;
  __syncthreads();
  const int j0 = blockIdx.x * kMwSegment, j1 = min(Nc, j0 + kMwSegment);
  int local = 0;
  for (int j = j0 + threadIdx.x; j < j1; j += kMwThreads) {
    const uint32_t key = score_key(sr[j]);
    if (key != 0u) {
      atomicAdd(&h[key >> 21], 1u);
      ++local;
    }
  }
  local = wave_sum_int(local);
  if (lane_id() == 0) wcnt[threadIdx.x >> 6] = local;
  __syncthreads();
  for (int i = threadIdx.x; i < kTkBins; i += kMwThreads)
    if (h[i]) atomicAdd(&R.hist[i], h[i]);
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int i = 0; i < kMwThreads / kWave; ++i) tot += wcnt[i];
    if (tot) atomicAdd(&R.counters[0], tot);
  }
}

// First-digit threshold bin of a row from its global histogram (256 threads).
__device__ void mw_threshold(const MwRow& R, int k, uint32_t* lh, int* scratch, int& bin, int& above, int& kk) {
  const int ncand = R.counters[0];
  kk = min(k, ncand);
  for (int i = threadIdx.x; i < kTkBins; i += kMwThreads) lh[i] = R.hist[i];
  __syncthreads();
  // thread t owns 8 bins at descending positions 8t .. 8t+7
  int c[8], tot = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) { c[i] = static_cast<int>(lh[kTkBins - 1 - (8 * threadIdx.x + i)]); tot += c[i]; }
  const int incl = wave_incl_scan(tot);
  const int w = threadIdx.x >> 6;
  if (lane_id() == 63) scratch[w] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += scratch[i];
  int run = before + incl - tot;
  if (kk > 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (run < kk && kk <= run + c[i]) { scratch[4] = kTkBins - 1 - (8 * threadIdx.x + i); scratch[5] = run; }
      run += c[i];
    }
  }
  __syncthreads();
  bin = kk > 0 ? scratch[4] : 0;
  above = kk > 0 ? scratch[5] : 0;
  __syncthreads();
}

__global__ __launch_bounds__(kMwThreads) void topk_mw_filter(const float* __restrict__ scores, int Nc, int k,
                                                             uint32_t* __restrict__ ws) {
  __shared__ uint32_t lh[kTkBins];
  __shared__ int scratch[8];
  const size_t row = blockIdx.y;
  const MwRow R = mw_row(ws, k, row);
  int bin, above, kk;
  mw_threshold(R, k, lh, scratch, bin, above, kk);
  if (kk == 0) return;
  const float* sr = scores + row * Nc;
  const int j0 = blockIdx.x * kMwSegment, j1 = min(Nc, j0 + kMwSegment);
  for (int jb = j0; jb < j1; jb += kMwThreads) {
    const int j = jb + threadIdx.x;
    const uint32_t key = j < j1 ? score_key(sr[j]) : 0u;
    const int d = static_cast<int>(key >> 21);
    const bool is_gt = key != 0u && d > bin;
    const bool is_c = key != 0u && d == bin;
    const uint64_t gm = __ballot(is_gt), cm = __ballot(is_c);
    int gbase = 0, cbase = 0;
    if (lane_id() == 0) {
      if (gm) gbase = atomicAdd(&R.counters[1], __popcll(gm));
      if (cm) cbase = atomicAdd(&R.counters[2], __popcll(cm));
    }
    gbase = __shfl(gbase, 0, kWave);
    cbase = __shfl(cbase, 0, kWave);
    if (is_gt) R.gt[gbase + lanes_below(gm)] = j;               // < kk entries in total
    if (is_c) {
      const int p = cbase + lanes_below(cm);
      if (p < kMwCap) { R.ckey[p] = key; R.cidx[p] = j; }
    }
  }
}

// Ascending bitonic sort of n (power of two, <= 2*blockDim... any n <= buffer) int32 values
// in LDS; entries past `valid` must hold INT_MAX.
__device__ void bitonic_sort_lds(int32_t* v, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = threadIdx.x; i < n / 2; i += blockDim.x) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = ((lo & size) == 0);
        const int32_t a = v[lo], b = v[hi];
        if ((a > b) == up) { v[lo] = b; v[hi] = a; }
      }
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTkThreads) void topk_mw_final(const float* __restrict__ scores, int Nc, int k,
                                                            uint32_t* __restrict__ ws, int32_t* __restrict__ idx) {
  __shared__ TkShared sh;
  __shared__ uint32_t ckey[kMwCap];
  __shared__ int32_t cidx[kMwCap];
  __shared__ int32_t selv[2 * kTkThreads];
  __shared__ int nsel, neq;
  const size_t row = blockIdx.x;
  const MwRow R = mw_row(ws, k, row);
  int32_t* out = idx + row * k;
  const int ncand = R.counters[0];
  const int kk = min(k, ncand);
  if (kk == 0) {
    for (int p = threadIdx.x; p < k; p += kTkThreads) out[p] = -1;
    return;
  }
  const int nc = R.counters[2];
  const float* sr = scores + row * Nc;
  if (nc > kMwCap) {
    // threshold bin too crowded for the candidate buffer: finish this row the slow way
    auto key_at = [&](int j) -> uint32_t { return score_key(sr[j]); };
    uint32_t T;
    int need_eq;
    radix_select(sh, key_at, Nc, kk, T, need_eq);
    ordered_compaction(sh, key_at, Nc, k, kk, T, need_eq, out);
    return;
  }
  const int ngt = R.counters[1];
  for (int i = threadIdx.x; i < nc; i += kTkThreads) { ckey[i] = R.ckey[i]; cidx[i] = R.cidx[i]; }
  __syncthreads();
  // remaining digits (passes 2 and 3) over the candidates; their top digit is shared
  const int remain1 = kk - ngt;
  uint32_t T = ckey[0] & 0xffe00000u;   // placeholder when remain1 == 0 (no candidate taken)
  int need_eq = 0;
  if (remain1 > 0) {
    uint32_t prefix = ckey[0] & 0xffe00000u, mask = 0xffe00000u;
    int remain = remain1;
    for (int pass = 1; pass < 3; ++pass) {
      const int shift = digit_shift(pass), nbins = digit_bins(pass);
      for (int i = threadIdx.x; i < nbins; i += kTkThreads) sh.hist[i] = 0;
      __syncthreads();
      for (int j = threadIdx.x; j < nc; j += kTkThreads) {
        const uint32_t key = ckey[j];
        if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (nbins - 1)], 1u);
      }
      __syncthreads();
      find_threshold_bin(sh, nbins, remain);
      prefix |= static_cast<uint32_t>(sh.bin) << shift;
      mask |= static_cast<uint32_t>(nbins - 1) << shift;
      remain -= sh.above;
      __syncthreads();
    }
    T = prefix;
    need_eq = remain;
  }
  // gather: every gt entry, candidates with key > T, and the need_eq lowest-index key == T
  if (threadIdx.x == 0) { nsel = 0; neq = 0; }
  __syncthreads();
  for (int i = threadIdx.x; i < ngt; i += kTkThreads) selv[atomicAdd(&nsel, 1)] = R.gt[i];
  for (int i = threadIdx.x; i < nc; i += kTkThreads) {
    if (remain1 > 0 && ckey[i] > T) selv[atomicAdd(&nsel, 1)] = cidx[i];
  }
  __syncthreads();
  // equal-key candidates, sorted by index, reuse the candidate key buffer as int storage
  int32_t* eqv = reinterpret_cast<int32_t*>(ckey);
  __shared__ int32_t eqtmp[kMwCap];
  if (remain1 > 0) {
    for (int i = threadIdx.x; i < nc; i += kTkThreads)
      if (ckey[i] == T) eqtmp[atomicAdd(&neq, 1)] = cidx[i];
    __syncthreads();
    int n2 = 1;
    while (n2 < neq) n2 <<= 1;
    for (int i = threadIdx.x; i < n2; i += kTkThreads) eqv[i] = i < neq ? eqtmp[i] : 0x7fffffff;
    bitonic_sort_lds(eqv, n2);
    const int base = nsel;
    for (int i = threadIdx.x; i < need_eq; i += kTkThreads) selv[base + i] = eqv[i];
    __syncthreads();
    if (threadIdx.x == 0) nsel = base + need_eq;
  }
  __syncthreads();
  int n2 = 1;
  while (n2 < kk) n2 <<= 1;
  for (int i = nsel + threadIdx.x; i < n2; i += kTkThreads) selv[i] = 0x7fffffff;
  bitonic_sort_lds(selv, n2);
  for (int p = threadIdx.x; p < k; p += kTkThreads) out[p] = p < kk ? selv[p] : -1;
}

size_t topk_workspace_bytes(int rows, int Nc, int k) {
  (void)Nc;
  return static_cast<size_t>(rows) * mw_row_words(k) * sizeof(uint32_t);
}

// algo: 0 = automatic, 1 = one workgroup per row, 2 = several workgroups per row
int launch_topk(const float* scores, int rows, int Nc, int k, int32_t* idx, void* ws, size_t ws_bytes,
                int algo, hipStream_t st) {
  // several workgroups per row only when a row does not fit in LDS and rows are too few
  // to fill the chip (the 1M-context decode shape)
  if (algo == 0) algo = (rows < 64 && Nc > kTkLdsKeys) ? 2 : 1;
  if (algo == 2 && (ws == nullptr || ws_bytes < topk_workspace_bytes(rows, Nc, k))) algo = 1;
  if (algo == 1) {
    if (Nc <= kTkLdsKeys) {
      static bool attr_set = false;
      if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_rows<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, sizeof(uint32_t) * kTkLdsKeys);
        attr_set = true;
      }
      hipLaunchKernelGGL(topk_rows<true>, dim3(rows), dim3(kTkThreads), sizeof(uint32_t) * Nc, st,
                         scores, Nc, k, idx);
    } else {
      hipLaunchKernelGGL(topk_rows<false>, dim3(rows), dim3(kTkThreads), 0, st, scores, Nc, k, idx);
    }
    CSA_LAUNCH_CHECK();
    return CSA_OK;
  }
  uint32_t* w = static_cast<uint32_t*>(ws);
  const int segs = cdiv(Nc, kMwSegment);
  hipLaunchKernelGGL(topk_mw_clear, dim3(cdiv(rows * (kTkBins + 4), 256)), dim3(256), 0, st, w, k, rows);
  hipLaunchKernelGGL(topk_mw_hist, dim3(segs, rows), dim3(kMwThreads), 0, st, scores, Nc, k, w);
  hipLaunchKernelGGL(topk_mw_filter, dim3(segs, rows), dim3(kMwThreads), 0, st, scores, Nc, k, w);
  hipLaunchKernelGGL(topk_mw_final, dim3(rows), dim3(kTkThreads), 0, st, scores, Nc, k, w, idx);
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

}  // namespace csa
