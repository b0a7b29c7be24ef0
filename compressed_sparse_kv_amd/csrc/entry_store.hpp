// Low-precision stores of one compressed entry, shared by the compressor epilogues (prefill,
// decode step, CSA2): thread p holds channels (2p, 2p+1) of the finished entry (normalised
// and rotated, fp32) and every thread of the workgroup calls the store, live or not, since
// the scales need reductions over 8 lanes, 16 lanes or the whole workgroup.
//
//   CSA_FP4_E2M1         MXFP4 rows ([V4-CSA2] section 16.2, indexer keys: E2M1 values with
//                        one E8M0 scale per 32): the block exponent is floor(log2 amax) - 2
//                        (the OCP microscaling rule: the block's largest value lands in
//                        [4, 8) before rounding); codes [rows, n/2] two per byte, the even
//                        channel in the low nibble; scale bytes [rows, n/32].
//   CSA_PACKED_FP4_E4M3  main-KV rows of 288 bytes ([V4-CSA2] section 16.1, [ATTN-CMP]
//                        section on CSA2: E2M1 with an E4M3 scale per 16 channels, the scale
//                        amax/6 rounded to E4M3): 256 code bytes, then 32 scale bytes.
//   CSA_PACKED_FP8_ROPE  main-KV rows of 584 bytes ([ATTN-CMP] section "CSA（DeepSeek-V4）":
//                        the 448 channels without RoPE in e4m3, the 64 RoPE channels in
//                        bf16): codes scaled by 2^e, e = ceil(log2(amax / 448)) over the 448
//                        channels (the smallest power of two that avoids saturation), then
//                        the bf16 channels, then the byte e + 127 and 7 zero bytes.
#pragma once
#include "common.hpp"

namespace csa {

// Nearest E2M1 code of v (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6): ties go to the code with
// an even mantissa bit, magnitudes above 6 saturate, the sign bit is kept (also for zero).
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  const float a = fabsf(v);
  const uint32_t mag = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                     : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return mag | ((__float_as_uint(v) >> 28) & 8u);
}

// Maximum over aligned groups of W lanes (W = 8 or 16).
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Maximum over the workgroup (every thread gets it); red holds one float per wave.
__device__ __forceinline__ float workgroup_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  __syncthreads();
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) t = fmaxf(t, red[w]);
  return t;
}

// Row bytes of a packed main-KV entry (c = 512).
__host__ __device__ constexpr inline int packed_row_bytes(int dtype) {
  return dtype == CSA_PACKED_FP4_E4M3 ? 288 : dtype == CSA_PACKED_FP8_ROPE ? 584 : 0;
}

// Stores pair p of row `row` (n channels) in one of the formats above; `live` = the thread
// holds a real pair of an entry that is written.  out: codes or packed rows; scale8: the
// MXFP4 scale bytes.  The packed formats need n = 512 (and 64 RoPE channels for the FP8 one).
__device__ __forceinline__ void store_entry_lowp(int dtype, void* out, uint8_t* scale8, size_t row, int n, int p,
                                                 bool live, float x0, float x1, float* red) {
  uint8_t* o8 = static_cast<uint8_t*>(out);
  const float am = live ? fmaxf(fabsf(x0), fabsf(x1)) : 0.f;
  if (dtype == CSA_FP4_E2M1) {
    const float amax = group_max<16>(am);
    int e2 = 0;
    frexpf(amax, &e2);                                         // amax in [2^(e2-1), 2^e2)
    const int ex = amax > 0.f ? max(-127, min(127, e2 - 1 - 2)) : -127;
    if (live) {
      const uint32_t c0 = f32_to_e2m1(ldexpf(x0, -ex)), c1 = f32_to_e2m1(ldexpf(x1, -ex));
      o8[row * (n / 2) + p] = static_cast<uint8_t>(c0 | (c1 << 4));
      if ((p & 15) == 0) scale8[row * (n / 32) + p / 16] = static_cast<uint8_t>(ex + 127);
    }
  } else if (dtype == CSA_PACKED_FP4_E4M3) {
    const float amax = group_max<8>(am);
    const uint32_t sc = f32_to_e4m3(amax / 6.0f);
    const float s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sc, 1.0f, false)[0];
    if (live) {
      const uint32_t c0 = s > 0.f ? f32_to_e2m1(x0 / s) : 0u, c1 = s > 0.f ? f32_to_e2m1(x1 / s) : 0u;
      uint8_t* r = o8 + row * 288;
      r[p] = static_cast<uint8_t>(c0 | (c1 << 4));
      if ((p & 7) == 0) r[256 + p / 8] = static_cast<uint8_t>(sc);
    }
  } else {                                                     // CSA_PACKED_FP8_ROPE, n = 512
    constexpr int kCodePairs = 224;                            // channels 0 .. 447
    const float amax = workgroup_max(p < kCodePairs ? am : 0.f, red);
    int e2 = 0;
    frexpf(amax, &e2);
    const int e0 = e2 - 1 - 8;                                 // amax in [2^(e0+8), 2^(e0+9))
    const int ex = amax > 0.f ? (amax <= ldexpf(1.75f, e0 + 8) ? e0 : e0 + 1) : -127;
    if (live) {
      uint8_t* r = o8 + row * 584;
      if (p < kCodePairs) {
        const uint32_t c0 = f32_to_e4m3(ldexpf(x0, -ex)), c1 = f32_to_e4m3(ldexpf(x1, -ex));
        *reinterpret_cast<uint16_t*>(r + 2 * p) = static_cast<uint16_t>(c0 | (c1 << 8));
      } else {
        *reinterpret_cast<uint32_t*>(r + 448 + 4 * (p - kCodePairs)) =
            static_cast<uint32_t>(f32_to_bf16(x0)) | (static_cast<uint32_t>(f32_to_bf16(x1)) << 16);
      }
      if (p == 0) *reinterpret_cast<uint2*>(r + 576) = make_uint2(static_cast<uint32_t>(ex + 127), 0u);
    }
  }
}

}  // namespace csa
