// Device helpers shared by the CSA/HCA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "csa.h"

namespace csa {

constexpr int kWave = 64;

// ---- vector types used as MFMA operands --------------------------------------------
typedef int v8i __attribute__((ext_vector_type(8)));          // 32 fp8 codes
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));        // 8 bf16 bit patterns
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));        // 4 bf16 bit patterns
typedef unsigned v4u __attribute__((ext_vector_type(4)));     // 16 raw bytes

// D(16x16, fp32) += A(16x32 bf16) * B(32x16 bf16); lane l: row/col l%16, k-group l/16.
__device__ __forceinline__ v4f mfma_bf16_16x16x32(const v8s& a, const v8s& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                 __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// LDS transpose read (ds_read_b64_tr_b16).  In each 16-lane group, output lane i' slot j'
// receives input lane 4j' + i'/4 slot i'%4 (each input lane names 4 consecutive 16-bit
// values at its address).
__device__ __forceinline__ v4s lds_read_tr16(const uint8_t* p) {
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
}

// ---- bfloat16 -------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ---- OCP e4m3fn encode: round to nearest even, saturate to +-448, NaN -> 0x7f --------
__device__ __forceinline__ uint8_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint8_t sign = static_cast<uint8_t>((u >> 24) & 0x80u);
  const float a = fabsf(v);
  if (a != a) return 0x7f;
  if (a >= 448.0f) return sign | 0x7e;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid of step 2^-9
    const int q = static_cast<int>(rintf(a * 512.0f));   // 0..8; 8 is the smallest normal
    return sign | static_cast<uint8_t>(q);
  }
  uint32_t ua = __float_as_uint(a);
  ua += 0x7ffffu + ((ua >> 20) & 1u);        // keep 3 mantissa bits, ties to even
  const int e = static_cast<int>((ua >> 23) & 0xffu) - 127 + 7;
  const uint32_t mnt = (ua >> 20) & 7u;
  return sign | static_cast<uint8_t>((e << 3) | mnt);
}

// ---- order-preserving keys for selection -----------------------------------------
// Larger float -> larger key.  -inf and NaN (not candidates) map to 0; -0 and +0
// share the key of +0.  Every candidate key is >= 0x00800000.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u || u == 0xff800000u) return 0u;
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- wave helpers ------------------------------------------------------------------
__device__ __forceinline__ float wave_xor(float v, int m) { return __shfl_xor(v, m, kWave); }

__device__ __forceinline__ unsigned lane_id() { return __lane_id(); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

__host__ __device__ constexpr inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// ---- RoPE angles -------------------------------------------------------------------
// cos and sin of the angle pos * r^p for pair p, with r = theta^(-2/d_rope) formed once on
// the host in double (rope_ratio).  r^p by square-and-multiply and the product with the
// position in double (positions reach 2^20 and beyond, where an fp32 angle would be off by
// tenths of a radian), the angle reduced to [-pi, pi] in double, then cos/sin in fp32.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, int p, double r, float& cs, float& sn) {
  double f = 1.0, base = r;
  for (int e = p; e != 0; e >>= 1) {
    if (e & 1) f *= base;
    base *= base;
  }
  const double ang = static_cast<double>(pos) * f;
  const double turns = rint(ang * 0.15915494309189535);         // 1 / (2 pi)
  const double red = fma(-turns, 6.283185307179586, ang);
  sincosf(static_cast<float>(red), &sn, &cs);
}

inline double rope_ratio(float theta, int d_rope) {
  return d_rope > 0 ? std::pow(static_cast<double>(theta), -2.0 / d_rope) : 1.0;
}

}  // namespace csa

// ---- host-side launch checking -------------------------------------------------------
#define CSA_LAUNCH_CHECK()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return CSA_ERR_HIP; \
  } while (0)
