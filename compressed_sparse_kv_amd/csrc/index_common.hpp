// Pieces shared by the indexer kernels (index_score.hip, index_mx.hip): shapes, the
// decode workgroup geometry and the cross-lane head-sum of a 64-entry group.
#pragma once

#include "common.hpp"

namespace csa {

constexpr int kIH = 64;    // indexer heads handled by the FP8-input kernels
constexpr int kID = 128;   // indexer head dim handled by the FP8-input kernels


constexpr int kDecGroups = 8;                         // 64-entry groups per wave
// Waves per workgroup: 4 for scores alone (more workgroups for small grids), 8 with the
// top-k epilogue (4096-entry segments: half the candidates for the row merge).
template <bool kTopk> constexpr int dec_waves() { return kTopk ? 8 : 4; }
template <bool kTopk> constexpr int dec_entries() { return dec_waves<kTopk>() * 64 * kDecGroups; }


// p[nb] = partial head-sum of entry (lane&15) of block nb over this lane's heads.
// Returns, in lane l, the full sum for entry 16*(l>>4) + (l&15) = l of the 4 blocks.
// Two reduce-scatter steps on the gfx950 lane swaps, no LDS: v_permlane32_swap(x, y)
// leaves x = [x.lo, y.lo] and y = [x.hi, y.hi] (32-lane halves), so x + y is, in the low
// half, x + the high half's x and, in the high half, y + the low half's y; 16-lane rows
// pair up the same way under v_permlane16_swap.
__device__ __forceinline__ float reduce_scatter4(const float p[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]), false, false);
  const float q0 = __uint_as_float(a[0]) + __uint_as_float(a[1]);   // blocks 0 (low half), 2 (high half)
  const float q1 = __uint_as_float(b[0]) + __uint_as_float(b[1]);   // blocks 1, 3
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(q0), __float_as_uint(q1), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// ReLU as one instruction: med3(x, 0, 3e38) (fmaxf would also emit a NaN-quieting max).
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 3.0e38f); }

}  // namespace csa
