// Top-k selection (stage 3).
//
// Per row of Nc fp32 scores: the indices of the min(k, n_cand) largest candidate scores
// (candidates: not -inf, not NaN), ties to the lower index, ascending, padded with -1.
// [KV-COMP] sections 9.4 (S_t = TopK_k of the indexer scores) and 9.8 (invisible entries
// are -inf before the selection and -1 after it).
//
// Scores become order-preserving 32-bit keys (score_key) and one workgroup of 1024
// threads selects over up to 9 x 4096 keys held in registers (4 consecutive positions
// per thread and 4096-position chunk) with select_regs (select.hpp).
//
// Schedules:
//   * one workgroup per row when the row fits one workgroup's registers;
//   * G segments per row: one workgroup per segment writes its local top-k as (key,
//     index) pairs in index order, then one workgroup per row selects the global top-k
//     among the G*k pairs.  The union of the local top-k sets holds the global top-k
//     (same total order), so the result is identical.
#include <algorithm>
#include <atomic>
#include <cmath>

#include "common.hpp"
#include "select.hpp"

namespace csa {

constexpr int kTkThreads = 1024;
constexpr int kTkChunk = 4 * kTkThreads;       // positions per register chunk
constexpr int kTkMaxSet = kTkMaxChunks * kTkChunk;   // 36864 keys per workgroup
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
  const int kk = select_regs<kTkThreads, 4, NU>(sh, key, k, taken, obase);
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
// Long rows (the largest register set), persistent: workgroup g takes rows g, g + G, ...
// (G = gridDim.x, one workgroup per compute unit).  While it selects over one row, the
// next row's scores stream into LDS (global_load_lds: one 1 KiB wave instruction per 256
// scores), so a row's memory time hides under the previous row's selection instead of
// adding to it.  The first kTkPfFloats scores of a row (whole 1 KiB pieces) take this
// path; the rest (rows longer than the buffer) are read directly.  Needs rows of a
// multiple of 4 scores at a 16-byte aligned base.
// ---------------------------------------------------------------------------------------
constexpr int kTkPfFloats = 34816;               // 139264 B: what LDS holds next to TkShared

// One 1 KiB piece from global memory (src, wave-uniform) into LDS at dst (wave-uniform):
// lane l moves bytes 16 l .. 16 l + 15.  Written as an instruction of its own so that the
// compiler, which cannot see that it writes LDS, does not wait for it at every LDS access
// or barrier of the selection: the kernel waits for these loads itself (vmcnt(0) and a
// barrier) before the buffer is read, and issues the next ones only after every wave has
// read it.  The asm provides the 5 wait states between a VALU write of the address SGPRs
// and the load (and the 1 after M0 is written).  nt: each score is read once.
__device__ __forceinline__ void tk_dma_piece(const void* src, void* dst, int voff) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst));
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(src), "{m0}"(lds) : "memory");
}

template <int NU>
__global__ __launch_bounds__(kTkThreads) void topk_rows_pf(const float* __restrict__ scores, int rows, int Nc, int k,
                                                           int32_t* __restrict__ idx) {
  static_assert(NU * kTkChunk >= kTkPfFloats, "the staged prefix lies inside the register set");
  __shared__ TkShared sh;
  __shared__ __attribute__((aligned(16))) float buf[kTkPfFloats];
  const int tid = static_cast<int>(threadIdx.x);
  const int w = wave_index();
  const int n_pc = min(Nc, kTkPfFloats) / 256;       // whole pieces staged through LDS
  const int p_lds = 256 * n_pc;                       // positions [0, p_lds) come from LDS
  auto issue = [&](int r) __attribute__((always_inline)) {
    const char* src = reinterpret_cast<const char*>(scores + static_cast<size_t>(r) * Nc);
    for (int j = w; j < n_pc; j += kTkThreads / kWave) tk_dma_piece(src + 1024 * j, buf + 256 * j, 16 * static_cast<int>(lane_id()));
  };
  int row = blockIdx.x;
  if (row < rows) issue(row);
  for (; row < rows; row += gridDim.x) {
    __builtin_amdgcn_s_waitcnt(0x0f70);              // vmcnt(0): this wave's pieces landed
    __syncthreads();                                  // and every other wave's
    const float* sr = scores + static_cast<size_t>(row) * Nc;
    uint32_t key[NU][4];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int p = kTkChunk * u + 4 * tid;           // 4 scores, all below p_lds or none
      float4 v;
      if (p < p_lds) {
        v = *reinterpret_cast<const float4*>(buf + p);
      } else if (p + 3 < Nc) {
        v = *reinterpret_cast<const float4*>(sr + p);
      } else {
        v.x = p < Nc ? sr[p] : -INFINITY;
        v.y = p + 1 < Nc ? sr[p + 1] : -INFINITY;
        v.z = p + 2 < Nc ? sr[p + 2] : -INFINITY;
        v.w = p + 3 < Nc ? sr[p + 3] : -INFINITY;
      }
      key[u][0] = score_key(v.x);
      key[u][1] = score_key(v.y);
      key[u][2] = score_key(v.z);
      key[u][3] = score_key(v.w);
    }
    // direct reads complete before the next pieces are issued (the compiler does not count
    // the pieces, so a later wait of its own for these reads would cover them too)
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();                                  // every wave has read the buffer
    if (row + static_cast<int>(gridDim.x) < rows) issue(row + gridDim.x);
    uint64_t taken;
    int obase[NU];
    const int kk = select_regs<kTkThreads, 4, NU>(sh, key, k, taken, obase);
    int32_t* out = idx + static_cast<size_t>(row) * k;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      int o = obase[u];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if ((taken >> (4 * u + s)) & 1ull) out[o++] = kTkChunk * u + 4 * tid + s;
    }
    for (int p = kk + tid; p < k; p += kTkThreads) out[p] = -1;
  }
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
  const int kk = select_regs<kTkThreads, 4, NU>(sh, key, k, taken, obase);
  uint2* out = cand + (row * G + g) * static_cast<size_t>(k);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    int o = obase[u];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if ((taken >> (4 * u + s)) & 1ull) {
        const int p = kTkChunk * u + 4 * static_cast<int>(threadIdx.x) + s;
        // the largest register set reads its key again (cached) to stay within 128 VGPRs
        const uint32_t kv = NU <= 4 ? key[u][s] : score_key(sr[p]);
        out[o++] = make_uint2(kv, static_cast<uint32_t>(j0 + p));
      }
  }
  for (int p = kk + threadIdx.x; p < k; p += kTkThreads) out[p] = make_uint2(0u, 0u);
}

// One workgroup per (row, group) over the pairs [grp * n_grp, min(n_row, (grp+1) * n_grp))
// of the row's n_row pairs at cand + row * row_stride (n_grp <= NU * 4096); gridDim.y
// groups per row.  The keys and
// (up to four register chunks) their entry indices stay in registers from the one read of
// the pairs; the largest set reads the indices of the taken pairs again.  kPairs: the k
// best are written as (key, entry) pairs in entry order to pairs_out[row][grp][k] (key 0
// = empty) at pairs_out + row * out_stride + grp * k, the input of a second merge; else as
// indices to idx[row][k] (one group).
// Groups of consecutive segments keep the pairs of a row in entry order at every level.
template <int NU, bool kPairs>
__global__ __launch_bounds__(kTkThreads) void topk_merge(const uint2* __restrict__ cand, size_t row_stride, int n_row,
                                                         int n_grp, int k, int32_t* __restrict__ idx,
                                                         uint2* __restrict__ pairs_out, size_t out_stride) {
  __shared__ TkShared sh;
  const size_t row = blockIdx.x;
  const int grp = blockIdx.y;
  const uint2* c = cand + row * row_stride + static_cast<size_t>(grp) * n_grp;
  const int n = min(n_grp, n_row - grp * n_grp);
  const bool vec = (reinterpret_cast<uintptr_t>(c) & 15u) == 0;
  constexpr int NE = NU <= 4 ? NU : 1;                 // register chunks of entry indices
  uint32_t key[NU][4], ent[NE][4];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int p = kTkChunk * u + 4 * static_cast<int>(threadIdx.x);
    if (vec && p + 3 < n) {
      const uint4 a = *reinterpret_cast<const uint4*>(c + p);
      const uint4 b = *reinterpret_cast<const uint4*>(c + p + 2);
      key[u][0] = a.x; key[u][1] = a.z; key[u][2] = b.x; key[u][3] = b.z;
      if (NU <= 4) { ent[u % NE][0] = a.y; ent[u % NE][1] = a.w; ent[u % NE][2] = b.y; ent[u % NE][3] = b.w; }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint2 v = p + s < n ? c[p + s] : make_uint2(0u, 0u);
        key[u][s] = v.x;
        if (NU <= 4) ent[u % NE][s] = v.y;
      }
    }
  }
  uint64_t taken;
  int obase[NU];
  const int kk = select_regs<kTkThreads, 4, NU>(sh, key, k, taken, obase);
  if constexpr (kPairs) {
    uint2* out = pairs_out + row * out_stride + static_cast<size_t>(grp) * k;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      int o = obase[u];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if ((taken >> (4 * u + s)) & 1ull)
          out[o++] = NU <= 4 ? make_uint2(key[u][s], ent[u % NE][s]) : c[kTkChunk * u + 4 * static_cast<int>(threadIdx.x) + s];
    }
    for (int p = kk + threadIdx.x; p < k; p += kTkThreads) out[p] = make_uint2(0u, 0u);
  } else {
    int32_t* out = idx + row * k;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      int o = obase[u];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if ((taken >> (4 * u + s)) & 1ull)
          out[o++] = static_cast<int32_t>(NU <= 4 ? ent[u % NE][s] : c[kTkChunk * u + 4 * static_cast<int>(threadIdx.x) + s].y);
    }
    for (int p = kk + threadIdx.x; p < k; p += kTkThreads) out[p] = -1;
  }
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
  if constexpr (NU == kTkMaxChunks) {
    // rows long enough to stage: the persistent kernel, one workgroup per compute unit
    // (the count is cached per device; any host thread may call)
    static std::atomic<int> n_cu[64];
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && Nc % 4 == 0 &&
        (reinterpret_cast<uintptr_t>(scores) & 15u) == 0 && rows > 1) {
      int cu = n_cu[dev].load(std::memory_order_relaxed);
      if (cu == 0 && hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cu > 0)
        n_cu[dev].store(cu, std::memory_order_relaxed);
      if (cu > 0) {
        hipLaunchKernelGGL(topk_rows_pf<NU>, dim3(std::min(rows, cu)), dim3(kTkThreads), 0, st, scores, rows, Nc, k,
                           idx);
        return;
      }
    }
  }
  hipLaunchKernelGGL(topk_rows<NU>, dim3(rows), dim3(kTkThreads), 0, st, scores, Nc, k, idx);
}
template <int NU>
static void launch_segments(const float* scores, int rows, int G, int Nc, int k, int seg, uint2* cand,
                            hipStream_t st) {
  hipLaunchKernelGGL(topk_segments<NU>, dim3(rows, G), dim3(kTkThreads), 0, st, scores, Nc, k, seg, cand);
}
template <int NU>
static void launch_merge(const uint2* cand, int rows, int n, int k, int32_t* idx, hipStream_t st) {
  hipLaunchKernelGGL((topk_merge<NU, false>), dim3(rows), dim3(kTkThreads), 0, st, cand, static_cast<size_t>(n), n, n,
                     k, idx, nullptr, size_t{0});
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

// Merge of G per-segment candidate lists (G*k (key, index) pairs per row, each list in
// index order, key 0 = empty) into the row's top-k.  When the G*k pairs of a row exceed one
// workgroup's set, a first level merges groups of M consecutive lists into k pairs each
// (in entry order, after the rows' G*k pairs in the same buffer), and the second level
// merges the ceil(G/M) group results.  M ~ sqrt(G) balances the two levels.
// Returns M, 0 for a single level, or -1 when two levels do not suffice.
int topk_merge_group(int G, int k) {
  if (G < 1 || k < 1 || k > kTkMaxSet) return -1;
  if (static_cast<long long>(G) * k <= kTkMaxSet) return 0;
  const int M = std::max(2, std::min(kTkMaxSet / k, static_cast<int>(std::lround(std::sqrt(static_cast<double>(G))))));
  return static_cast<long long>(cdiv(G, M)) * k <= kTkMaxSet ? M : -1;
}

int topk_merge_supported(int G, int k) { return topk_merge_group(G, k) >= 0; }

// Pairs per row of the candidate buffer: the G*k segment pairs and the first level's.
size_t topk_merge_pairs_per_row(int G, int k) {
  const int M = topk_merge_group(G, k);
  return static_cast<size_t>(G) * k + (M > 0 ? static_cast<size_t>(cdiv(G, M)) * k : 0);
}

template <bool kPairs>
static void launch_merge_level(const uint2* cand, size_t row_stride, int rows, int groups, int n_row, int n_grp,
                               int k, int32_t* idx, uint2* out, hipStream_t st) {
  const dim3 grid(rows, groups), block(kTkThreads);
#define CSA_MERGE_LAUNCH(NU_)                                                                                  \
  hipLaunchKernelGGL((topk_merge<NU_, kPairs>), grid, block, 0, st, cand, row_stride, n_row, n_grp, k, idx, out, \
                     row_stride)
  switch (chunks_for(n_grp)) {
    case 1: CSA_MERGE_LAUNCH(1); break;
    case 2: CSA_MERGE_LAUNCH(2); break;
    case 4: CSA_MERGE_LAUNCH(4); break;
    default: CSA_MERGE_LAUNCH(kTkMaxChunks); break;
  }
#undef CSA_MERGE_LAUNCH
}

// cand: rows x topk_merge_pairs_per_row(G, k) pairs (the first G*k of a row are the input).
int launch_topk_merge(uint2* cand, int rows, int G, int k, int32_t* idx, hipStream_t st) {
  const int M = topk_merge_group(G, k);
  if (M < 0) return CSA_ERR_UNSUPPORTED;
  const size_t per_row = topk_merge_pairs_per_row(G, k);
  if (M == 0) {
    launch_merge_level<false>(cand, per_row, rows, 1, G * k, G * k, k, idx, nullptr, st);
    CSA_LAUNCH_CHECK();
    return CSA_OK;
  }
  // rows are per_row pairs apart: the first level reads row r's G*k pairs at
  // cand + r * per_row and writes its G1 * k pairs right after them
  const int G1 = cdiv(G, M);
  uint2* lvl = cand + static_cast<size_t>(G) * k;
  launch_merge_level<true>(cand, per_row, rows, G1, G * k, M * k, k, nullptr, lvl, st);
  CSA_LAUNCH_CHECK();
  launch_merge_level<false>(lvl, per_row, rows, 1, G1 * k, G1 * k, k, idx, nullptr, st);
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

// The first merge level alone (for the fused selection + attention, which finishes the
// selection itself): writes the cdiv(G, M) * k level-one pairs of each row after its G * k
// segment pairs.  Returns the number of candidate pairs per row the caller selects from
// (G * k when one level is enough, nothing launched) and where they start, or < 0.
int launch_topk_merge_first(uint2* cand, int rows, int G, int k, size_t& offset, hipStream_t st) {
  const int M = topk_merge_group(G, k);
  if (M < 0) return -1;
  offset = 0;
  if (M == 0) return G * k;
  const size_t per_row = topk_merge_pairs_per_row(G, k);
  const int G1 = cdiv(G, M);
  uint2* lvl = cand + static_cast<size_t>(G) * k;
  launch_merge_level<true>(cand, per_row, rows, G1, G * k, M * k, k, nullptr, lvl, st);
  if (hipGetLastError() != hipSuccess) return -1;
  offset = static_cast<size_t>(G) * k;
  return G1 * k;
}

}  // namespace csa
