// Dequantization of the paged cache's records, shared by every kernel that
// reads them (decode, multi-token and cascade attention, and the test-only
// dequantize export), so that all of them consume the same values.
//
// "TurboQuant 在 AMD GPU 上把長上下文延遲壓下來", section 2: keys are coded
// against a 16-entry table after the rotation (k_hat = c[code] * s in the
// rotated domain), values by an asymmetric uniform code per 32 channels
// (v_hat = code * sc + mn).  "UltraQuant：4-bit KV 快取加速長代理", section
// "方法怎麼做，白話講": FP4 e2m1 elements with one UE8M0 exponent per 32
// channels (v_hat = e2m1 * 2^X).
//
// No value is rounded on the way into an MFMA operand:
//   * key table entries are fp16 and the key scale is applied to the fp32
//     logit, so k_hat = c * s is exact;
//   * a value code times its fp16 scale has at most 15 significant bits; it is
//     carried as the sum of two fp16 parts, hi = fp16_RNE(code * sc) and
//     lo = code * sc - hi, both exact (lo is a multiple of sc's last place,
//     at most 8 of them); the minimum enters through a separate product with
//     the probabilities, so v_hat = (hi + lo) + mn is never formed in low
//     precision.  code * sc overflows fp16 once sc >= 4368; scales of 4096 and
//     above are therefore taken as sc * 2^-7 (exact) and the matching
//     probability operand as p * 2^7;
//   * an e2m1 element times 2^X has two significant bits and is exact in
//     bf16 over the whole UE8M0 range.
#pragma once

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));

// Value scales at or above this (fp16 4096, bit pattern 0x6C00) are applied as
// sc * 2^-7 with the probabilities scaled by 2^7.
constexpr uint32_t kBigScaleBits = 0x6C00u;

// ---- the record reader -----------------------------------------------------------
template <int D>
struct KTile;
template <>
struct KTile<128> {
  typedef uint4 T;
};
template <>
struct KTile<64> {
  typedef uint2 T;
};

__device__ __forceinline__ uint32_t word(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ uint32_t word(const uint2 &v, int i) { return i == 0 ? v.x : v.y; }

// Value-code words per lane: 4-bit, one per 32-channel group; 2-bit (TQ4/2),
// one per group pair.
template <int D, int VB>
struct VTile {
  typedef typename KTile<D>::T T;
};
template <>
struct VTile<128, 2> {
  typedef uint2 T;
};
template <>
struct VTile<64, 2> {
  typedef uint32_t T;
};
__device__ __forceinline__ uint32_t word(uint32_t v, int) { return v; }

// One wave's loads of one (block, kv-head) record (TQ4/4 or TQ4/2, layout in
// tq.h), lane l = 16r + c:
//   kq   key codes of token l % 16, channels 32(l / 16) .. +31 (word s:
//        channels +8s .. +8s+7, the QK A operand of k-step s);
//   ks   the fp16 key scales of tokens 4r .. 4r+3;
//   vq   value codes of channel pairs 16gp + c of tokens 4r .. 4r+3 (word gp,
//        byte = token; 2-bit values: word gp / 2);
//   vmw  dword c % 4G of row r's 16G-byte (scale, min) tile: group c / 4 % G,
//        dwords 0-1 the scales of tokens 4r .. 4r+3, dwords 2-3 their minima.
template <int D, int VB>
struct Blk {
  typename KTile<D>::T kq;      // key codes: this lane's A-operand bytes
  uint2 ks;                     // key scales of tokens 4r .. 4r+3
  typename VTile<D, VB>::T vq;  // value codes: this lane's A-operand bytes
  uint32_t vmw;                 // one dword of the value (scale, min) tile; lane
                                // (r, c) holds dword c of row r's 16*G bytes
};

template <int D, int VB>
__device__ __forceinline__ void load_blk(Blk<D, VB> &o, const uint8_t *rec, int lane) {
  constexpr int G = D / 32, Q = D / 8;
  constexpr int VW = VB == 4 ? G : G / 2;  // value-code words per lane
  constexpr int OFF_KS = TqRec<D, VB>::KS, OFF_VC = TqRec<D, VB>::VC, OFF_VM = TqRec<D, VB>::VM;
  const int r = lane >> 4, c = lane & 15;
  o.kq = *reinterpret_cast<const typename KTile<D>::T *>(rec + TqRec<D, VB>::KC + lane * Q);
  o.ks = *reinterpret_cast<const uint2 *>(rec + OFF_KS + 8 * r);
  o.vq = *reinterpret_cast<const typename VTile<D, VB>::T *>(rec + OFF_VC + lane * (4 * VW));
  o.vmw = reinterpret_cast<const uint32_t *>(rec + OFF_VM)[r * (4 * G) + (c & (4 * G - 1))];
}

// ---- keys ----------------------------------------------------------------------
// Four code bytes (eight 4-bit codes) -> eight exact fp16 table entries through
// the byte-pair table (256 entries of two fp16 values) in LDS.
__device__ __forceinline__ uint4 key_entries(const uint32_t *s_lut, uint32_t w) {
  uint4 e;
  e.x = s_lut[w & 0xFF];
  e.y = s_lut[(w >> 8) & 0xFF];
  e.z = s_lut[(w >> 16) & 0xFF];
  e.w = s_lut[w >> 24];
  return e;
}

// ---- values: codes ---------------------------------------------------------------
// The value codes of channel group gp as bytes 0000cccc (bytes = tokens
// 4r + 0..3 of one channel pair): `lo` the even channel, `hi` the odd one.
// 4-bit: one word per group.  2-bit: one word per group pair, group 2w in bits
// 0-3 of each byte and 2w + 1 in bits 4-7, the even channel in the lower two.
template <int VB>
__device__ __forceinline__ void value_code_bytes(uint32_t w, int gp, uint32_t &lo, uint32_t &hi) {
  if constexpr (VB == 4) {
    lo = w & 0x0F0F0F0Fu;
    hi = (w >> 4) & 0x0F0F0F0Fu;
  } else {
    const uint32_t x = w >> (4 * (gp & 1));
    lo = x & 0x03030303u;
    hi = (x >> 2) & 0x03030303u;
  }
}

// Two code bytes (bytes 0-1, or 2-3 with HI_WORD) as exact fp16 integers:
// 0000cccc is the OCP e4m3 encoding of c * 2^-9, so the fp8 conversion with
// scale 2^9 gives c.
template <bool HI_WORD>
__device__ __forceinline__ half2v codes_f16(uint32_t bytes) {
  return __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bytes, 512.0f, HI_WORD));
}

// ---- values: code * scale as two exact fp16 parts ---------------------------------
struct ScaledPair {
  half2v hi, lo;  // hi + lo = code * sc exactly, per element
};
__device__ __forceinline__ ScaledPair scaled_codes(half2v code, half2v sc) {
  ScaledPair r;
  r.hi = code * sc;                                  // fp16 RNE of the exact product
  r.lo = __builtin_elementwise_fma(code, sc, -r.hi); // the exact remainder
  return r;
}

// Per fp16 scale of a pair: 1 where sc < 4096, 2^-7 where sc >= 4096 (the
// scale's own sign bit is clear: scales are >= 0).
__device__ __forceinline__ half2v big_scale_factor(half2v sc) {
  const uint32_t b = as_u(sc);
  const uint32_t lo = (b & 0xFFFFu) >= kBigScaleBits ? 0x2000u : 0x3C00u;  // 2^-7 : 1
  const uint32_t hi = (b >> 16) >= kBigScaleBits ? 0x2000u : 0x3C00u;
  return as_h2(lo | (hi << 16));
}
// The inverse factor for the probability operand: 2^7 where sc >= 4096.
__device__ __forceinline__ half2v big_prob_factor(half2v sc) {
  const uint32_t b = as_u(sc);
  const uint32_t lo = (b & 0xFFFFu) >= kBigScaleBits ? 0x5800u : 0x3C00u;  // 2^7 : 1
  const uint32_t hi = (b >> 16) >= kBigScaleBits ? 0x5800u : 0x3C00u;
  return as_h2(lo | (hi << 16));
}
// Nonzero when some fp16 scale of the dword is >= 4096 (scales are >= 0, so
// adding 0x1400 to each half sets its bit 15 exactly then, with no carry
// between the halves).
__device__ __forceinline__ uint32_t has_big_scale(uint32_t sc_pair_bits) {
  return (sc_pair_bits + 0x14001400u) & 0x80008000u;
}

// The exact fp32 dequantized value of (code, sc, mn): (hi + lo) is code * sc
// exactly (scaled back by 2^7 for big scales), then one rounding with mn -
// fp32(code * sc + mn).
__device__ __forceinline__ float value_f32(_Float16 hi, _Float16 lo, float back, _Float16 mn) {
  return __builtin_fmaf((float)hi + (float)lo, back, (float)mn);
}

// ---- probabilities as bf16 parts (MX-FP4 PV operand) --------------------------------
// hi = bf16_RNE(p) of two probabilities, packed.
__device__ __forceinline__ uint32_t prob_hi_bf16(float p0, float p1) {
  return __builtin_bit_cast(uint32_t, (bf16x2v){(__bf16)p0, (__bf16)p1});
}
// The operand part of this lane's column: the high part where lo_mask = 0,
// the low part bf16_RNE(p - hi) (the difference is exact) where lo_mask = 1.
__device__ __forceinline__ uint32_t prob_part_bf16(uint32_t hi, float p0, float p1, float lo_mask) {
  const float r0 = __builtin_fmaf(-lo_mask, as_f(hi << 16), p0);
  const float r1 = __builtin_fmaf(-lo_mask, as_f(hi & 0xFFFF0000u), p1);
  return __builtin_bit_cast(uint32_t, (bf16x2v){(__bf16)r0, (__bf16)r1});
}

// ---- MX-FP4 ------------------------------------------------------------------------
// The fp32 scale 2^X for a UE8M0 byte X + 127.  Byte 0 (X = -127) is the
// subnormal 2^-127.
__device__ __forceinline__ float ue8m0_scale(uint32_t byte) {
  return byte ? as_f(byte << 23) : as_f(0x00400000u);
}

// Two e2m1 elements (the pair at position `sel` of `word`) times 2^X, exact
// in bf16 (two significant bits; bf16 has the fp32 exponent range).
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair_bf16(uint32_t word, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, SEL));
}
// The same pair in fp32 (exact).
template <int SEL>
__device__ __forceinline__ float2v fp4_pair_f32(uint32_t word, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, SEL);
}

}  // namespace tq
