// Block compressor (stage 1).
//
// [HCA-CSA] sections "压缩算子：逐通道 softmax 的软池化" (per-token C and Z from one linear
// map, position bias B, per-channel softmax over the block's slots, weighted sum, then
// RMSNorm and RoPE), "CSA 的重叠窗口" (entry i pools the a-stream of block i and the
// b-stream of block i-1: 2m slots, stride m; for i = 0 the b-slots are -inf / 0 padding)
// and "HCA：同一个算子，关掉重叠" (one stream, m slots).  [ATTN-CMP] section "CSA（DeepSeek-V4）":
// RoPE at the block's first position.
//
// Two passes:
//   1. bf16 inputs with overlap and m = 4 (the CSA compressors): compress_fused, the
//      projection on MFMA v_mfma_f32_16x16x32_bf16 with the 2m-slot softmax pooling in its
//      epilogue, writing the pooled vectors u to the workspace.  Other shapes: the
//      projection GEMM P[r, :] = hidden_row(r) . w_proj^T alone (fp32 result in the
//      workspace; fp32 inputs on VALU), rows ordered per sequence as [previous block
//      (m rows, when given) | chunk (T rows)];
//   2. compress_pool: one workgroup per entry, one thread per channel pair (2p, 2p+1) so
//      the RoPE pair is thread-local; the pooling (unless pass 1 did it), block-wide RMS,
//      RoPE with the angle formed in double (positions reach 2^20 and beyond;
//      rope_cos_sin), output in fp32 / bf16 / e4m3 with the row scale amax/448 (row-major
//      or the 16-entry blocked key layout) or the low-precision types of entry_store.hpp.
#include <algorithm>

#include "common.hpp"
#include "entry_store.hpp"

namespace csa {

// ---------------------------------------------------------------------------------------
// bf16 MFMA GEMM, C[M,N] fp32 = A[M,K] . B[N,K]^T, K % 64 == 0.
// 128x128 tile, 4 waves in 2x2, each wave 64x64 (4x4 MFMA tiles), K step 64 via LDS
// (row stride 144 B).  A rows are gathered from (hidden_prev, hidden) per sequence.
// ---------------------------------------------------------------------------------------
constexpr int kGT = 128;
constexpr int kGK = 64;
constexpr int kGStride = kGK * 2 + 16;     // bytes per LDS row

struct GemmA {
  const uint16_t* hidden;
  const uint16_t* prev;      // may be null
  int T, m, d, rows_pb;      // rows per sequence in the projection buffer
};

__device__ __forceinline__ const uint16_t* a_row_bf16(const GemmA& A, int r) {
  const int bi = r / A.rows_pb, rr = r % A.rows_pb;
  if (A.prev) {
    if (rr < A.m) return A.prev + (static_cast<size_t>(bi) * A.m + rr) * A.d;
    return A.hidden + (static_cast<size_t>(bi) * A.T + rr - A.m) * A.d;
  }
  return A.hidden + (static_cast<size_t>(bi) * A.T + rr) * A.d;
}

__global__ __launch_bounds__(256) void proj_gemm_bf16(GemmA A, const uint16_t* __restrict__ Bw, int M, int N,
                                                      float* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) uint8_t la[2][kGT * kGStride];
  __shared__ __attribute__((aligned(16))) uint8_t lb[2][kGT * kGStride];
  const int tid = threadIdx.x, wave = tid >> 6, l = static_cast<int>(lane_id()), g = l >> 4;
  const int m0 = blockIdx.y * kGT, n0 = blockIdx.x * kGT;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int K = A.d;

  // loader: 128 rows x 128 bytes per operand = 16 KiB = 256 threads x 4 x 16 B
  // thread t moves row (t / 8) + 32*i, 16-byte piece t % 8
  const int lr = tid >> 3, lp = tid & 7;
  const uint16_t* arow[4];
  const uint16_t* brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    arow[i] = a_row_bf16(A, min(m0 + lr + 32 * i, M - 1));
    brow[i] = Bw + static_cast<size_t>(min(n0 + lr + 32 * i, N - 1)) * K;
  }
  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define CSA_GEMM_GLOAD(k0)                                                    \
  do {                                                                        \
    ra0 = *reinterpret_cast<const uint4*>(arow[0] + (k0) + 8 * lp);           \
    ra1 = *reinterpret_cast<const uint4*>(arow[1] + (k0) + 8 * lp);           \
    ra2 = *reinterpret_cast<const uint4*>(arow[2] + (k0) + 8 * lp);           \
    ra3 = *reinterpret_cast<const uint4*>(arow[3] + (k0) + 8 * lp);           \
    rb0 = *reinterpret_cast<const uint4*>(brow[0] + (k0) + 8 * lp);           \
    rb1 = *reinterpret_cast<const uint4*>(brow[1] + (k0) + 8 * lp);           \
    rb2 = *reinterpret_cast<const uint4*>(brow[2] + (k0) + 8 * lp);           \
    rb3 = *reinterpret_cast<const uint4*>(brow[3] + (k0) + 8 * lp);           \
  } while (0)
#define CSA_GEMM_SWRITE(buf)                                                                  \
  do {                                                                                        \
    *reinterpret_cast<uint4*>(&la[buf][(lr + 0) * kGStride + 16 * lp]) = ra0;                 \
    *reinterpret_cast<uint4*>(&la[buf][(lr + 32) * kGStride + 16 * lp]) = ra1;                \
    *reinterpret_cast<uint4*>(&la[buf][(lr + 64) * kGStride + 16 * lp]) = ra2;                \
    *reinterpret_cast<uint4*>(&la[buf][(lr + 96) * kGStride + 16 * lp]) = ra3;                \
    *reinterpret_cast<uint4*>(&lb[buf][(lr + 0) * kGStride + 16 * lp]) = rb0;                 \
    *reinterpret_cast<uint4*>(&lb[buf][(lr + 32) * kGStride + 16 * lp]) = rb1;                \
    *reinterpret_cast<uint4*>(&lb[buf][(lr + 64) * kGStride + 16 * lp]) = rb2;                \
    *reinterpret_cast<uint4*>(&lb[buf][(lr + 96) * kGStride + 16 * lp]) = rb3;                \
  } while (0)

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nk = K / kGK;
  CSA_GEMM_GLOAD(0);
  CSA_GEMM_SWRITE(0);
  __syncthreads();
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) CSA_GEMM_GLOAD((kt + 1) * kGK);
#pragma unroll
    for (int ks = 0; ks < kGK / 32; ++ks) {
      v8s af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const v8s*>(&la[buf][(wm + 16 * i + (l & 15)) * kGStride + 64 * ks + 16 * g]);
        bf[i] = *reinterpret_cast<const v8s*>(&lb[buf][(wn + 16 * i + (l & 15)) * kGStride + 64 * ks + 16 * g]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16_16x16x32(af[i], bf[j], acc[i][j]);
    }
    if (more) CSA_GEMM_SWRITE(buf ^ 1);
    __syncthreads();
  }
#undef CSA_GEMM_GLOAD
#undef CSA_GEMM_SWRITE
  // D tile (i, j): lane l holds rows 4*g + r, column l%16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn + 16 * j + (l & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm + 16 * i + 4 * g + r;
        if (row < M && col < N) C[static_cast<size_t>(row) * N + col] = acc[i][j][r];
      }
    }
}

// fp32 GEMM for small shapes: 16x16 output tile per 256 threads, K staged in 16-wide slabs.
__global__ __launch_bounds__(256) void proj_gemm_f32(const float* __restrict__ hidden, const float* __restrict__ prev,
                                                     int T, int m, int d, int rows_pb, const float* __restrict__ Bw,
                                                     int M, int N, float* __restrict__ C) {
  __shared__ float sa[16][17], sb[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int row = blockIdx.y * 16 + ty, col = blockIdx.x * 16 + tx;
  const int ra = min(blockIdx.y * 16 + tx, M - 1);     // loader roles
  const int bi = ra / rows_pb, rr = ra % rows_pb;
  const float* arow = prev ? (rr < m ? prev + (static_cast<size_t>(bi) * m + rr) * d
                                     : hidden + (static_cast<size_t>(bi) * T + rr - m) * d)
                           : hidden + (static_cast<size_t>(bi) * T + rr) * d;
  const float* brow = Bw + static_cast<size_t>(min(blockIdx.x * 16 + tx, N - 1)) * d;
  float acc = 0.0f;
  for (int k0 = 0; k0 < d; k0 += 16) {
    sa[tx][ty] = k0 + ty < d ? arow[k0 + ty] : 0.0f;
    sb[tx][ty] = k0 + ty < d ? brow[k0 + ty] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(sa[ty][kk], sb[tx][kk], acc);
    __syncthreads();
  }
  if (row < M && col < N) C[static_cast<size_t>(row) * N + col] = acc;
}

// ---------------------------------------------------------------------------------------
// Projection and overlapping pooling in one kernel (bf16 inputs, overlap, m = 4).
//
// A workgroup owns kTM consecutive tokens of one sequence and kTC channels, i.e. the
// 4*kTC projection columns (C^a | Z^a | C^b | Z^b) of those channels.  The b-stream
// products are formed from the token rows 4 earlier than the a-stream ones (the LDS tile
// holds 4 halo rows above the kTM tokens), so in the MFMA accumulator layout (lane holds 4
// consecutive rows of one column) every lane ends up holding, for one channel, the 4
// a-slots of block q and the 4 b-slots of block q-1: the whole 2m-slot softmax of entry q
// is lane-local and the projection never leaves the chip.  The halo rows of the first
// tile are hidden_prev (or padding, whose b-slots the epilogue drops).  The result per
// entry is the pooled vector u before RMSNorm, which compress_pool<true> finishes.
//
// Operands go from global memory straight into LDS (global_load_lds_dwordx4, no staging
// registers), two K=64 stages; LDS rows are 128 bytes with the 16-byte pieces XOR-swizzled
// by (row & 7), which keeps both the DMA writes and the fragment reads conflict-free.
// Tiles are handed out so that each XCD gets a contiguous range (shared rows and weights
// stay in that XCD's L2).
// ---------------------------------------------------------------------------------------
template <int kMI_, int kCG_, int kWM_, int kWN_, int kKS_, int kStages_>
struct FusedShape {
  static constexpr int kMI = kMI_;                   // 16-row MFMA tiles per wave (tokens)
  static constexpr int kCG = kCG_;                   // 16-channel groups per wave
  static constexpr int kWM = kWM_, kWN = kWN_;       // wave grid
  static constexpr int kKS = kKS_;                   // K per stage (32 or 64)
  static constexpr int kStages = kStages_;           // stages in the LDS ring
  static constexpr int kWaves = kWM * kWN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kTM = 16 * kMI * kWM;         // tokens per tile
  static constexpr int kTC = 16 * kCG * kWN;         // channels per tile
  static constexpr int kRowB = 2 * kKS;              // bytes per LDS row
  static constexpr int kPieces = kKS / 8;            // 16-byte pieces per row
  static constexpr int kRPC = 1024 / kRowB;          // rows per 1 KiB chunk (one wave-wide DMA)
  static constexpr int kAChunks = (kTM + 4 + kRPC - 1) / kRPC;   // 4 halo rows + kTM rows
  static constexpr int kARows = kRPC * kAChunks;
  static constexpr int kBRows = 4 * kTC;
  static constexpr int kChunks = kAChunks + kBRows / kRPC;
  static constexpr int kMaxCh = (kChunks + kWaves - 1) / kWaves;  // DMAs per wave and stage
  static constexpr int kStage = (kARows + kBRows) * kRowB;        // bytes per stage
  static_assert(kStages * kStage <= 160 * 1024, "LDS");
};
using FusedBig = FusedShape<4, 2, 4, 2, 64, 2>;     // 256 tokens x 64 channels, 130 KiB of LDS
using FusedSmall = FusedShape<1, 1, 4, 2, 64, 2>;   // 64 tokens x 32 channels, 50 KiB of LDS

struct FusedArgs {
  const uint16_t* hidden;    // [B, T, d]
  const uint16_t* prev;      // [B, 4, d] or null
  const uint16_t* w;         // [4c, d]
  const float* bias;         // [2, 4, c]
  float* u;                  // [B, T/4, c]
  int T, d, c, n_mt, n_nt, total;
};

// Tile of workgroup w: workgroups go to the 8 XCDs round robin, so XCD x runs w = x, x+8, ...;
// it gets the tile range [x*per + min(x, rem), ...) of the total = 8*per + rem tiles.
__device__ __forceinline__ int xcd_tile(int w, int total) {
  const int x = w & 7, j = w >> 3, per = total >> 3, rem = total & 7;
  return x * per + min(x, rem) + j;
}

// 16 bytes per lane from global memory into LDS at dst + 16 * lane (dst wave-uniform).
__device__ __forceinline__ void lds_dma16(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// Position of 16-byte piece `piece` of LDS row `row`.  The pieces are XOR-swizzled so that
// 8 consecutive rows read at one piece fall on 8 different 16-byte bank groups of the
// 256-byte bank line: 128-byte rows by row & 7, 64-byte rows (four per line, rows r and
// r + 4 on the same banks) by (row >> 2) & 3.
template <class Sh>
__device__ __forceinline__ int swz(int row, int piece) {
  return Sh::kKS == 64 ? piece ^ (row & 7) : piece ^ ((row >> 2) & 3);
}

template <class Sh>
__device__ __forceinline__ v8s lds_frag(const uint8_t* st, int row, int piece) {
  return *reinterpret_cast<const v8s*>(st + row * Sh::kRowB + 16 * swz<Sh>(row, piece));
}

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt not waited for)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <class Sh>
__global__ __launch_bounds__(Sh::kThreads) void compress_fused(FusedArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Sh::kStages * Sh::kStage];
  const int tile = xcd_tile(static_cast<int>(blockIdx.x), a.total);
  const int nt = tile % a.n_nt, mtg = tile / a.n_nt;
  const int b = mtg / a.n_mt, t0 = (mtg % a.n_mt) * Sh::kTM, j0 = nt * Sh::kTC;
  const int wave = threadIdx.x >> 6, l = static_cast<int>(lane_id()), g = l >> 4;
  const int wm = wave % Sh::kWM, wn = wave / Sh::kWM;
  const int d = a.d;

  // source rows of this lane's chunks: chunk ci = wave + 8k holds tile rows kRPC*ci .. +kRPC-1;
  // lane l fills 16-byte slot l of it.  Every wave issues kMaxCh DMAs per stage (a wave
  // with fewer chunks repeats its previous one: same bytes to the same place), so that
  // vmcnt counts whole stages.
  const uint16_t* src[Sh::kMaxCh];
  int dst[Sh::kMaxCh];
#pragma unroll
  for (int k = 0; k < Sh::kMaxCh; ++k) {
    const int ci = wave + Sh::kWaves * k < Sh::kChunks ? wave + Sh::kWaves * k : wave + Sh::kWaves * (k - 1);
    const int rho = Sh::kRPC * ci + l / Sh::kPieces;
    const uint16_t* r;
    if (ci < Sh::kAChunks) {
      const int tau = min(t0 - 4 + rho, a.T - 1);
      if (tau >= 0) r = a.hidden + (static_cast<size_t>(b) * a.T + tau) * d;
      else if (a.prev) r = a.prev + (static_cast<size_t>(b) * 4 + 4 + tau) * d;
      else r = a.hidden + static_cast<size_t>(b) * a.T * d;         // padding: b-slots dropped
    } else {
      const int n = rho - Sh::kARows, s = n / Sh::kTC;
      r = a.w + static_cast<size_t>(s * a.c + j0 + n % Sh::kTC) * d;
    }
    src[k] = r + 8 * swz<Sh>(rho, l % Sh::kPieces);
    dst[k] = ci * 1024;
  }
  auto issue = [&](int kt) {
    uint8_t* st = lds + (kt % Sh::kStages) * Sh::kStage;
#pragma unroll
    for (int k = 0; k < Sh::kMaxCh; ++k) lds_dma16(src[k] + Sh::kKS * kt, st + dst[k]);
  };

  v4f acc[Sh::kMI][4][Sh::kCG];
#pragma unroll
  for (int i = 0; i < Sh::kMI; ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int cg = 0; cg < Sh::kCG; ++cg) acc[i][s][cg] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nk = d / Sh::kKS;
  const int arow = 16 * Sh::kMI * wm + (l & 15);                     // + 4 for the a-stream
  const int brow = Sh::kARows + 16 * Sh::kCG * wn + (l & 15);       // + s*kTC + 16*cg
#pragma unroll
  for (int s = 0; s < Sh::kStages - 1; ++s)
    if (s < nk) issue(s);
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed once at most min(kStages - 2, nk - 1 - kt) later stages are in
    // flight; the barrier also frees the slot of stage kt - 1 for stage kt + kStages - 1
    const int ahead = min(Sh::kStages - 2, nk - 1 - kt);
    if (ahead >= 2) wait_vmcnt<2 * Sh::kMaxCh>();
    else if (ahead == 1) wait_vmcnt<Sh::kMaxCh>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (kt + Sh::kStages - 1 < nk) issue(kt + Sh::kStages - 1);
    const uint8_t* st = lds + (kt % Sh::kStages) * Sh::kStage;
#pragma unroll
    for (int h = 0; h < Sh::kKS / 32; ++h) {
      const int pc = 4 * h + g;
      v8s bf[4][Sh::kCG];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int cg = 0; cg < Sh::kCG; ++cg) bf[s][cg] = lds_frag<Sh>(st, brow + s * Sh::kTC + 16 * cg, pc);
#pragma unroll
      for (int i = 0; i < Sh::kMI; ++i) {
        const v8s fa = lds_frag<Sh>(st, arow + 16 * i + 4, pc);
        const v8s fb = lds_frag<Sh>(st, arow + 16 * i, pc);
#pragma unroll
        for (int cg = 0; cg < Sh::kCG; ++cg) {
          acc[i][0][cg] = mfma_bf16_16x16x32(fa, bf[0][cg], acc[i][0][cg]);
          acc[i][1][cg] = mfma_bf16_16x16x32(fa, bf[1][cg], acc[i][1][cg]);
          acc[i][2][cg] = mfma_bf16_16x16x32(fb, bf[2][cg], acc[i][2][cg]);
          acc[i][3][cg] = mfma_bf16_16x16x32(fb, bf[3][cg], acc[i][3][cg]);
        }
      }
    }
  }

  // pooling: lane (g, col) of tile i holds entry q = t0/4 + 4*(kMI*wm + i) + g, channel ch
  const int nent = a.T / 4;
#pragma unroll
  for (int i = 0; i < Sh::kMI; ++i) {
    const int q = t0 / 4 + 4 * (Sh::kMI * wm + i) + g;
#pragma unroll
    for (int cg = 0; cg < Sh::kCG; ++cg) {
      const int ch = j0 + 16 * (Sh::kCG * wn + cg) + (l & 15);
      if (q >= nent) continue;
      const bool bslots = q > 0 || a.prev != nullptr;
      float za[4], zb[4];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        za[r] = acc[i][1][cg][r] + a.bias[r * a.c + ch];
        mx = fmaxf(mx, za[r]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        zb[r] = acc[i][3][cg][r] + a.bias[(4 + r) * a.c + ch];
        if (bslots) mx = fmaxf(mx, zb[r]);
      }
      float den = 0.f, num = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = expf(za[r] - mx);
        den += e;
        num = fmaf(e, acc[i][0][cg][r], num);
      }
      if (bslots) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = expf(zb[r] - mx);
          den += e;
          num = fmaf(e, acc[i][2][cg][r], num);
        }
      }
      a.u[(static_cast<size_t>(b) * nent + q) * a.c + ch] = num / den;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Pooling + RMSNorm + RoPE (+ quantisation).  Grid (T/m, B); block = c/2 threads rounded
// up to whole waves (64 .. 512), one channel pair per thread.
// ---------------------------------------------------------------------------------------
struct PoolArgs {
  const float* P;            // projection [B*rows_pb, ns*c], or (pooled) u [B, T/m, c]
  const float* bias;         // [ns/2, m, c]
  int overlap, has_prev;
  int T, m, c, d_rope, rows_pb;
  double rope_r;             // theta^(-2/d_rope)
  float rms_eps;
  int64_t p0;
  int out_dtype, out_layout, Nc_max;
  void* out;
  float* out_scale;
};

// kPooled: P already holds the pooled vectors (compress_fused); only the normalisation,
// RoPE and the store remain.
template <bool kPooled>
__global__ __launch_bounds__(512) void compress_pool(PoolArgs a) {
  __shared__ float red[8];
  const int i = blockIdx.x, b = blockIdx.y;
  const int ns = a.overlap ? 4 : 2;
  const int N = ns * a.c;
  const int off = a.has_prev ? a.m : 0;              // buffer row of chunk token 0
  const float* Pb = a.P + static_cast<size_t>(b) * a.rows_pb * N;
  const int npairs = a.c / 2;
  const int pidx = threadIdx.x;                        // channel pair handled by this thread
  const bool live = pidx < npairs;
  float u[2] = {0.f, 0.f};
  if (kPooled) {
    if (live) {
      const float2 v = reinterpret_cast<const float2*>(a.P + (static_cast<size_t>(b) * (a.T / a.m) + i) * a.c)[pidx];
      u[0] = v.x;
      u[1] = v.y;
    }
  } else if (live) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = 2 * pidx + h;
      // slots: a-stream of block i, then (overlap) b-stream of block i-1
      float mx = -INFINITY;
      for (int j = 0; j < a.m; ++j) {
        const size_t r = static_cast<size_t>(off + a.m * i + j) * N;
        mx = fmaxf(mx, Pb[r + a.c + ch] + a.bias[j * a.c + ch]);
      }
      const bool bslots = a.overlap && (i > 0 || a.has_prev);
      if (bslots) {
        for (int j = 0; j < a.m; ++j) {
          const size_t r = static_cast<size_t>(off + a.m * (i - 1) + j) * N;
          mx = fmaxf(mx, Pb[r + 3 * a.c + ch] + a.bias[(a.m + j) * a.c + ch]);
        }
      }
      float den = 0.f, num = 0.f;
      for (int j = 0; j < a.m; ++j) {
        const size_t r = static_cast<size_t>(off + a.m * i + j) * N;
        const float e = expf(Pb[r + a.c + ch] + a.bias[j * a.c + ch] - mx);
        den += e;
        num = fmaf(e, Pb[r + ch], num);
      }
      if (bslots) {
        for (int j = 0; j < a.m; ++j) {
          const size_t r = static_cast<size_t>(off + a.m * (i - 1) + j) * N;
          const float e = expf(Pb[r + 3 * a.c + ch] + a.bias[(a.m + j) * a.c + ch] - mx);
          den += e;
          num = fmaf(e, Pb[r + 2 * a.c + ch], num);
        }
      }
      u[h] = num / den;
    }
  }
  // RMSNorm over the c channels
  float ss = u[0] * u[0] + u[1] * u[1];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
  if (lane_id() == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(a.c) + a.rms_eps);
  float x0 = u[0] * inv, x1 = u[1] * inv;
  // RoPE on the last d_rope channels, pair p = pidx - (c - d_rope)/2, position p0 + m*i
  const int p = pidx - (a.c - a.d_rope) / 2;
  if (live && p >= 0) {
    float cs, sn;
    rope_cos_sin(a.p0 + static_cast<int64_t>(a.m) * i, p, a.rope_r, cs, sn);
    const float y0 = fmaf(x0, cs, -x1 * sn), y1 = fmaf(x0, sn, x1 * cs);
    x0 = y0;
    x1 = y1;
  }
  const size_t orow = static_cast<size_t>(b) * (a.T / a.m) + i;
  if (a.out_dtype == CSA_F32) {
    if (live) reinterpret_cast<float2*>(static_cast<float*>(a.out) + orow * a.c)[pidx] = make_float2(x0, x1);
  } else if (a.out_dtype == CSA_BF16) {
    if (live) {
      const uint32_t v = static_cast<uint32_t>(f32_to_bf16(x0)) | (static_cast<uint32_t>(f32_to_bf16(x1)) << 16);
      reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + orow * a.c)[pidx] = v;
    }
  } else if (a.out_dtype != CSA_FP8_E4M3) {
    store_entry_lowp(a.out_dtype, a.out, reinterpret_cast<uint8_t*>(a.out_scale), orow, a.c, pidx, live, x0, x1, red);
  } else {
    float am = live ? fmaxf(fabsf(x0), fabsf(x1)) : 0.f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, kWave));
    __syncthreads();
    if (lane_id() == 0) red[threadIdx.x >> 6] = am;
    __syncthreads();
    float amax = 0.f;
    for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) amax = fmaxf(amax, red[w]);
    const float scale = amax / 448.0f;
    if (live) {
      uint8_t c0 = 0, c1 = 0;
      if (scale > 0.f) {
        c0 = f32_to_e4m3(x0 / scale);
        c1 = f32_to_e4m3(x1 / scale);
      }
      uint8_t* o8;
      size_t srow = orow;
      if (a.out_layout == CSA_LAYOUT_B16) {
        // cache entry e = p0/m + i of the sequence: block e/16, piece (2p)/32, slot e%16
        const size_t e = static_cast<size_t>(a.p0 / a.m) + i, nblk = static_cast<size_t>(cdiv(a.Nc_max, 16));
        o8 = static_cast<uint8_t*>(a.out) + (static_cast<size_t>(b) * nblk + e / 16) * (16 * 128) +
             ((2 * pidx) >> 5) * 512 + (e % 16) * 32 + ((2 * pidx) & 31);
        srow = static_cast<size_t>(b) * a.Nc_max + e;
      } else {
        o8 = static_cast<uint8_t*>(a.out) + orow * a.c + 2 * pidx;
      }
      o8[0] = c0;
      o8[1] = c1;
      if (threadIdx.x == 0) a.out_scale[srow] = scale;
    }
  }
}

size_t compress_workspace_bytes(int B, int T, int m, int c, int overlap, int has_prev) {
  const size_t rows = static_cast<size_t>(B) * (T + (has_prev ? m : 0));
  return rows * (overlap ? 4 : 2) * static_cast<size_t>(c) * sizeof(float);
}

// P[B*rows_pb, N] = rows of (hidden_prev | hidden) . w^T: the projection GEMM alone (also
// used by the CSA2 compressor).
int launch_proj_gemm(const void* hidden, const void* hidden_prev, int in_dtype, const void* w, int B, int T, int m,
                     int d, int N, float* P, hipStream_t st) {
  const int has_prev = hidden_prev != nullptr;
  const int rows_pb = T + (has_prev ? m : 0);
  const int M = B * rows_pb;
  if (in_dtype == CSA_BF16) {
    GemmA A{static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(hidden_prev), T, m, d, rows_pb};
    dim3 grid(cdiv(N, kGT), cdiv(M, kGT));
    hipLaunchKernelGGL(proj_gemm_bf16, grid, dim3(256), 0, st, A, static_cast<const uint16_t*>(w), M, N, P);
  } else {
    dim3 grid(cdiv(N, 16), cdiv(M, 16));
    hipLaunchKernelGGL(proj_gemm_f32, grid, dim3(256), 0, st, static_cast<const float*>(hidden),
                       static_cast<const float*>(hidden_prev), T, m, d, rows_pb, static_cast<const float*>(w), M, N, P);
  }
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

// The fused path: bf16 inputs, the overlapping compressor with m = 4, c a multiple of 64.
static bool fused_ok(int in_dtype, int overlap, int m, int c, int d) {
  return in_dtype == CSA_BF16 && overlap && m == 4 && c % 64 == 0 && d % 64 == 0;
}

template <class Sh>
static void launch_fused(const FusedArgs& base, int B, hipStream_t st) {
  FusedArgs fa = base;
  fa.n_mt = cdiv(fa.T, Sh::kTM);
  fa.n_nt = fa.c / Sh::kTC;
  fa.total = B * fa.n_mt * fa.n_nt;
  hipLaunchKernelGGL(compress_fused<Sh>, dim3(fa.total), dim3(Sh::kThreads), 0, st, fa);
}

int launch_compress(const void* hidden, const void* hidden_prev, int in_dtype, const void* w_proj, const float* bias,
                    int overlap, int B, int T, int d, int m, int c, int d_rope, float rope_theta, float rms_eps,
                    int64_t p0, void* out, float* out_scale, int out_dtype, int out_layout, int Nc_max, void* ws,
                    hipStream_t st) {
  const int has_prev = hidden_prev != nullptr;
  const int rows_pb = T + (has_prev ? m : 0);
  const int N = (overlap ? 4 : 2) * c;
  float* P = static_cast<float*>(ws);
  const bool fused = fused_ok(in_dtype, overlap, m, c, d);
  if (fused) {
    // the large tile when it still gives every CU a tile, else the small one
    FusedArgs fa{static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(hidden_prev),
                 static_cast<const uint16_t*>(w_proj), bias, P, T, d, c, 0, 0, 0};
    const int big_tiles = B * cdiv(T, FusedBig::kTM) * (c / FusedBig::kTC);
    if (big_tiles >= 192) launch_fused<FusedBig>(fa, B, st);
    else launch_fused<FusedSmall>(fa, B, st);
  } else {
    const int rc = launch_proj_gemm(hidden, hidden_prev, in_dtype, w_proj, B, T, m, d, N, P, st);
    if (rc != CSA_OK) return rc;
  }
  CSA_LAUNCH_CHECK();
  PoolArgs pa{P, bias, overlap, has_prev, T, m, c, d_rope, rows_pb, rope_ratio(rope_theta, d_rope), rms_eps, p0,
              out_dtype, out_layout, Nc_max, out, out_scale};
  const int threads = std::max(kWave, cdiv(c / 2, kWave) * kWave);
  if (fused) hipLaunchKernelGGL(compress_pool<true>, dim3(T / m, B), dim3(threads), 0, st, pa);
  else hipLaunchKernelGGL(compress_pool<false>, dim3(T / m, B), dim3(threads), 0, st, pa);
  CSA_LAUNCH_CHECK();
  return CSA_OK;
}

}  // namespace csa
