// Device helpers shared by the gfx950 kernels: cross-lane exchanges, bf16 and
// fp16 bit handling, the exact fp16 rounding of an RMS, MFMA operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int8v __attribute__((ext_vector_type(8)));

constexpr int kBlock = 16;  // tokens per paged block

// ---- bit casts --------------------------------------------------------------
__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t as_u(half2v h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ uint16_t h_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }
__device__ __forceinline__ _Float16 h_from(uint16_t b) { return __builtin_bit_cast(_Float16, b); }

// bf16 halves of a packed word -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f(w & 0xffff0000u); }

// fp32 -> bf16 round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t b = as_u(x);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// fp32 -> fp16 RNE, infinities clamped to +-65504 (saturating conversion)
__device__ __forceinline__ _Float16 f16_sat(float x) {
  _Float16 h = (_Float16)x;
  uint16_t b = h_bits(h);
  if ((b & 0x7fffu) == 0x7c00u) b = (uint16_t)((b & 0x8000u) | 0x7bffu);
  return h_from(b);
}

// ---- cross-lane exchanges (wave64) -------------------------------------------
// DPP: quad_perm(1,0,3,2) = lane^1, quad_perm(2,3,0,1) = lane^2, row_ror:8 = lane^8
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float xor1(float x) { return as_f(dpp_u<0xB1>(as_u(x))); }
__device__ __forceinline__ float xor2(float x) { return as_f(dpp_u<0x4E>(as_u(x))); }
__device__ __forceinline__ float xor8(float x) { return as_f(dpp_u<0x128>(as_u(x))); }
__device__ __forceinline__ uint32_t xor1u(uint32_t x) { return dpp_u<0xB1>(x); }
__device__ __forceinline__ uint32_t xor2u(uint32_t x) { return dpp_u<0x4E>(x); }
__device__ __forceinline__ uint32_t xor8u(uint32_t x) { return dpp_u<0x128>(x); }
// ds_swizzle bit-mask mode within 32 lanes: lane ^ M (M < 32)
template <int M>
__device__ __forceinline__ uint32_t swz_xor_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, (M << 10) | 0x1F);
}
// gfx950 row swaps: returns the value of lane^16 (or lane^32)
__device__ __forceinline__ uint32_t xor16u(uint32_t x) {
  auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  // even rows receive the partner in p[1], odd rows in p[0]
  return (__lane_id() & 16) ? p[0] : p[1];
}
__device__ __forceinline__ uint32_t xor32u(uint32_t x) {
  auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (__lane_id() & 32) ? p[0] : p[1];
}
__device__ __forceinline__ float xor16(float x) { return as_f(xor16u(as_u(x))); }
__device__ __forceinline__ float xor32(float x) { return as_f(xor32u(as_u(x))); }
__device__ __forceinline__ uint32_t xor4u(uint32_t x) { return swz_xor_u<4>(x); }
__device__ __forceinline__ float xor4(float x) { return as_f(xor4u(as_u(x))); }

__device__ __forceinline__ double dpp64_xor1(double x) {
  uint64_t b = __builtin_bit_cast(uint64_t, x);
  uint32_t lo = xor1u((uint32_t)b), hi = xor1u((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double dpp64_xor2(double x) {
  uint64_t b = __builtin_bit_cast(uint64_t, x);
  uint32_t lo = xor2u((uint32_t)b), hi = xor2u((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double dpp64_xor8(double x) {
  uint64_t b = __builtin_bit_cast(uint64_t, x);
  uint32_t lo = xor8u((uint32_t)b), hi = xor8u((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double dpp64_xor16(double x) {
  uint64_t b = __builtin_bit_cast(uint64_t, x);
  uint32_t lo = xor16u((uint32_t)b), hi = xor16u((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// ---- exact fp16 rounding of sqrt(ms) ------------------------------------------
// h is the correctly rounded square root iff ms lies between the squares of the
// two midpoints around h (ties to the even significand).  Midpoints have <= 12
// significant bits, so their squares are exact in fp64.
__device__ __forceinline__ _Float16 f16_rne_sqrt(double ms) {
  if (ms >= 65520.0 * 65520.0) return (_Float16)65504.0f;
  _Float16 h = (_Float16)__builtin_sqrtf((float)ms);
  if (h_bits(h) >= 0x7c00u) h = h_from(0x7bffu);
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    uint16_t hb = h_bits(h);
    double hv = (double)(float)h;
    double up = (hb == 0x7bffu) ? 1e300 : (double)(float)h_from((uint16_t)(hb + 1));
    double mu = (hv + up) * 0.5;
    bool odd = hb & 1u;
    if (hb != 0x7bffu && (ms > mu * mu || (ms == mu * mu && odd))) {
      h = h_from((uint16_t)(hb + 1));
      continue;
    }
    if (hb != 0) {
      double dn = (double)(float)h_from((uint16_t)(hb - 1));
      double md = (dn + hv) * 0.5;
      if (ms < md * md || (ms == md * md && odd)) {
        h = h_from((uint16_t)(hb - 1));
        continue;
      }
    }
    break;
  }
  return h;
}

// ---- work-group id remap so that consecutive logical ids share an XCD -----------
// Work-groups are dispatched round-robin over the 8 XCDs (id % 8); this returns
// a logical id such that logical ids [k*n/8, (k+1)*n/8) all run on XCD k.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t id, uint32_t n) {
  uint32_t xcd = id & 7u, local = id >> 3;
  uint32_t per = n >> 3, rem = n & 7u;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

}  // namespace tq
