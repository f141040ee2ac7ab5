// Pieces shared by the quantize kernels: the lane mapping of a wave over
// token rows and the in-register Walsh-Hadamard butterflies.
#pragma once

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

// One wave handles TPW token rows of one kv-head, D/8 lanes per row, 8
// channels per lane.  Lane bits {0,1,3,4} select the 8-channel chunk li
// (channel = 8*li + e), the remaining lane bits select the token tw, so the
// cross-lane butterfly stages (channel bits 3..6) run over lane xor 1, 2 (DPP
// quad_perm), xor 8 (DPP row_ror:8) and xor 16 (gfx950 permlane16 swap).
template <int D>
struct QMap;
template <>
struct QMap<128> {
  static constexpr int TPW = 4;  // token rows per wave
  __device__ static int li(int l) { return (l & 3) | ((l >> 1) & 0xC); }
  __device__ static int tw(int l) { return ((l >> 2) & 1) | ((l >> 4) & 2); }
};
template <>
struct QMap<64> {
  static constexpr int TPW = 8;
  __device__ static int li(int l) { return (l & 3) | ((l >> 1) & 0x4); }
  __device__ static int tw(int l) { return ((l >> 2) & 1) | ((l >> 3) & 2) | ((l >> 3) & 4); }
};

// exchange with the lane holding the token whose in-quad index differs in bit 1
// (lane bit 5 for D = 128, lane bit 4 for D = 64); bit 0 is lane bit 2 for both
template <int D>
__device__ __forceinline__ uint32_t quad_xor2(uint32_t x) {
  if constexpr (D == 128) return xor32u(x);
  else return xor16u(x);
}

// Unnormalized Walsh-Hadamard butterflies over the D channels of one token
// row, in the fixed stage order h = 1, 2, ..., D/2, fp32.
template <int D>
__device__ __forceinline__ void wht_rows(float (&x)[8], int lane) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (!(i & h)) {
        float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
  // lane holding a (bit clear) gets a + b, lane holding b gets a - b
  const float s1 = (lane & 1) ? -1.f : 1.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(s1, x[i], xor1(x[i]));
  const float s2 = (lane & 2) ? -1.f : 1.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(s2, x[i], xor2(x[i]));
  const float s8 = (lane & 8) ? -1.f : 1.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(s8, x[i], xor8(x[i]));
  if constexpr (D == 128) {
    const float s16 = (lane & 16) ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // even rows get (own, partner), odd rows (partner, own): a +- b = p0 +- p1
      auto p = __builtin_amdgcn_permlane16_swap(as_u(x[i]), as_u(x[i]), false, false);
      x[i] = __builtin_fmaf(s16, as_f(p[1]), as_f(p[0]));
    }
  }
}

}  // namespace tq
