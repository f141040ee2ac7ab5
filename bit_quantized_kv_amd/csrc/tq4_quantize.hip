// TQ4/4 (and TQ4/2) quantize-and-append kernel for gfx950.
//
// Keys: Walsh-Hadamard rotation, per-(token, kv-head) RMS scale, nearest entry
// of a 16-entry table; values: per-32-channel asymmetric uniform 4-bit codes
// ("TurboQuant 在 AMD GPU 上把長上下文延遲壓下來", section 2: K = rotation +
// LUT, V = uniform; section 4: Walsh-Hadamard rotation).  The exact decision
// rules (fp32 operation order) and the record layout are stated in tq.h.
//
// The kernel is VALU-bound unless every step is lean, so:
//   * a lane holds 16 channels of one token row (two 128-bit loads of K and of
//     V); the three cross-lane butterfly stages are one DPP fmac each;
//   * the key scale comes from an fp32 sum of squares (bf16 dot2) and is
//     rounded to fp16 directly unless the RMS lies within a few ulps of an fp16
//     rounding boundary, where the exact fp64 rule decides (rare);
//   * 1/s and 1/sc are correctly rounded from a table of significand
//     reciprocals; sc = fp16(fp32(range/15)) likewise falls back to the exact
//     division only near a rounding boundary;
//   * key codes: one bin lookup (v_cvt_pk_u8 gives the clamped bin) plus one
//     comparison; value codes: v_cvt_pk_u8 rounds to nearest even and packs;
//   * persistent work-groups: each takes (32- or 64-token chunk, kv-head)
//     tasks, so one work-group writes whole 16-token records, and every wave
//     loads its next task before coding the current one.
#include <cstdlib>
#include <cstring>

#include "quant_common.h"

namespace tq {
namespace {

// Exact key scale of a token row (the rare path): fp64 sum of the bf16 squares
// over the row's LPT lanes (this lane's 16 channels in k0, k1), exact fp16 RMS.
template <int D>
__device__ __forceinline__ uint32_t key_scale_exact(const uint4 &k0, const uint4 &k1) {
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 &q = i < 4 ? k0 : k1;
    const uint32_t w = (i & 3) == 0 ? q.x : (i & 3) == 1 ? q.y : (i & 3) == 2 ? q.z : q.w;
    const double lo = (double)bf16_lo(w), hi = (double)bf16_hi(w);
    ss = __builtin_fma(lo, lo, ss);
    ss = __builtin_fma(hi, hi, ss);
  }
  ss += dpp64_xor1(ss);
  ss += dpp64_xor2(ss);
  if constexpr (D == 128) ss += dpp64_xor8(ss);
  return h_bits(f16_rne_sqrt(ss * (1.0 / D)));
}

// Quantize one token row held by the LPT lanes of this lane's token and write
// its codes and scales into the record of (slot / 16, h).
// VB: value code bits, 4 (TQ4/4) or 2 (TQ4/2: 2-bit values, the same
// per-group rule with 3 levels; four codes of one token per byte).
template <int D, int VB>
__device__ __forceinline__ void quantize_row(const QuantizeArgs &a, const RowLoad<D> &cur, int h, int lane,
                                             int li, int tq, const float2 *s_bins,
                                             const float *s_recip, float bin_a, float bin_b, float sigma) {
  constexpr int G = D / 32, Q = D / 8;
  constexpr int OFF_KC = TqRec<D, VB>::KC, OFF_KS = TqRec<D, VB>::KS, OFF_VC = TqRec<D, VB>::VC;
  constexpr int OFF_VM = TqRec<D, VB>::VM, REC = TqRec<D, VB>::BYTES;
  constexpr float LEVELS = VB == 4 ? 15.f : 3.f;
  const int slot = cur.valid ? cur.slot : -1;
  // ---- key scale: fp32 sum of squares, exact fp16 RMS -------------------------
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = kword<D>(cur, i);
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w), __builtin_bit_cast(bf2, w), ss, false);
  }
  ss = dpp_add<0xB1>(ss);
  ss = dpp_add<0x4E>(ss);
  if constexpr (D == 128) ss = dpp_add<0x128>(ss);
  // ss carries <= 12 roundings of <= 1 ulp; sqrt adds 1 ulp: 32 ulps is safe
  const float rms = __builtin_amdgcn_sqrtf(ss * (1.0f / D));
  uint32_t sb = h_bits((_Float16)rms);
  if (!(rms == 0.f || f16_round_safe(rms, 32))) sb = key_scale_exact<D>(cur.k0, cur.k1);

  // ---- rotation -------------------------------------------------------------------
  float z[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = kword<D>(cur, i);
    z[2 * i] = bf16_lo(w);
    z[2 * i + 1] = bf16_hi(w);
  }
  wht16<D>(z, lane);

  // ---- key codes: u = fp32(y * w), w = fp32(fp32(1/s) / sqrt(D)) ------------------
  const float w = recip_f16(sb, s_recip) * a.rsqrt_d * sigma;  // sigma: sign of z
  const float wa = w * bin_a;
  uint32_t kc0 = 0, kc1 = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float u = z[e] * w;
    const uint32_t bin = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(z[e], wa, bin_b), 0, 0);
    const float2 bt = s_bins[bin];
    const uint32_t code = (uint32_t)__float_as_int(bt.y) + (u > bt.x ? 1u : 0u);
    if (e < 8) kc0 |= code << (4 * e);
    else kc1 |= code << (4 * (e - 8));
  }

  // ---- value codes: the 32-channel group is this lane and lane ^ 1 -------------------
  float v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w2 = vword<D>(cur, i);
    v[2 * i] = bf16_lo(w2);
    v[2 * i + 1] = bf16_hi(w2);
  }
  float mn = min3f(v[0], v[1], v[2]), mx = max3f(v[0], v[1], v[2]);
#pragma unroll
  for (int e = 3; e < 15; e += 2) {
    mn = min3f(mn, v[e], v[e + 1]);
    mx = max3f(mx, v[e], v[e + 1]);
  }
  mn = __builtin_fminf(mn, v[15]);
  mx = __builtin_fmaxf(mx, v[15]);
  mn = __builtin_fminf(mn, xor1(mn));
  mx = __builtin_fmaxf(mx, xor1(mx));
  const float range = mx - mn;
  const float qs = range * (1.0f / LEVELS);  // within 2 ulps of fp32(range / levels)
  uint32_t scb = h_bits((_Float16)qs);
  if (!(qs == 0.f || f16_round_safe(qs, 4))) scb = h_bits(f16_sat(__fdiv_rn(range, LEVELS)));
  const _Float16 mn16 = (_Float16)__builtin_amdgcn_fmed3f(mn, -65504.0f, 65504.0f);  // saturating RNE
  const float mnv = (float)mn16;
  const float inv_sc = recip_f16(scb, s_recip);
  uint32_t ve0 = 0, ve1 = 0, vo0 = 0, vo1 = 0;  // bytes: even / odd channels
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float qv = __builtin_amdgcn_fmed3f((v[e] - mnv) * inv_sc, 0.f, LEVELS);
    const int bsel = (e & 7) >> 1;
    if (e < 8) {
      if (e & 1) vo0 = __builtin_amdgcn_cvt_pk_u8_f32(qv, bsel, vo0);
      else ve0 = __builtin_amdgcn_cvt_pk_u8_f32(qv, bsel, ve0);
    } else {
      if (e & 1) vo1 = __builtin_amdgcn_cvt_pk_u8_f32(qv, bsel, vo1);
      else ve1 = __builtin_amdgcn_cvt_pk_u8_f32(qv, bsel, ve1);
    }
  }
  // byte k: pair k's codes (pairs 0..3, 4..7 of this lane).  4-bit: even |
  // odd << 4.  2-bit: even | odd << 2 in the low nibble, and the same nibble of
  // the other group of the group pair (lane li ^ 2) in the high nibble, so both
  // lanes hold the full bytes (group 2w in the low nibble)
  uint32_t vc0, vc1;
  if constexpr (VB == 4) {
    vc0 = ve0 | (vo0 << 4);
    vc1 = ve1 | (vo1 << 4);
  } else {
    const uint32_t n0 = ve0 | (vo0 << 2), n1 = ve1 | (vo1 << 2);
    const uint32_t p0 = xor2u(n0), p1 = xor2u(n1);
    const bool odd_group = (li & 2) != 0;
    vc0 = odd_group ? (p0 | (n0 << 4)) : (n0 | (p0 << 4));
    vc1 = odd_group ? (p1 | (n1 << 4)) : (n1 | (p1 << 4));
  }

  // ---- placement ----------------------------------------------------------------------
  {
    // derived again from an opaque copy of the lane, so that the compiler
    // does not hold the store-address terms in registers through the task loop
    int l = lane;
    asm volatile("" : "+v"(l));
    li = QLanes<D>::li(l);
    tq = QLanes<D>::tw(l) & 3;
  }
  const bool aligned = quad_aligned<D>(slot, tq);
  const uint32_t vt0 = quad_transpose<D>(vc0, tq), vt1 = quad_transpose<D>(vc1, tq);
  const uint32_t scmn = scb | ((uint32_t)h_bits(mn16) << 16);
  const uint32_t scmn_p = tok_xor1(scmn);
  if (slot >= 0) {
    const int64_t blk = slot >> 4;
    const int t = slot & 15;
    uint8_t *rec = a.pool + ((int64_t)blk * a.hkv + h) * REC;
    // key codes: pairs 8*li .. 8*li+7 are contiguous in the key section
    const int p0 = 8 * li;
    *reinterpret_cast<uint2 *>(rec + OFF_KC + ((p0 / Q) * 16 + t) * Q + p0 % Q) = make_uint2(kc0, kc1);
    if (li == 0) *reinterpret_cast<uint16_t *>(rec + OFF_KS + 2 * t) = (uint16_t)sb;
    const int r = t >> 2, gp = li >> 1, j0 = 8 * (li & 1);
    // value-code word of pair j: 4-bit, one per group; 2-bit, one per group pair
    constexpr int VW = VB == 4 ? G : G / 2;
    const int wi = VB == 4 ? gp : gp >> 1;
    const bool v_store = VB == 4 || (li & 2) == 0;
    if (aligned) {
      // lane tq writes the quad's bytes of channel pairs j0 + tq and j0 + 4 + tq
      if (v_store) {
        *reinterpret_cast<uint32_t *>(rec + OFF_VC + ((r * 16 + j0 + tq) * VW + wi) * 4) = vt0;
        *reinterpret_cast<uint32_t *>(rec + OFF_VC + ((r * 16 + j0 + 4 + tq) * VW + wi) * 4) = vt1;
      }
      if ((li & 1) == 0 && (tq & 1) == 0) {
        // tokens tq, tq + 1: their scales form one dword, their minima another
        uint8_t *vm = rec + OFF_VM + (r * G + gp) * 16;
        *reinterpret_cast<uint32_t *>(vm + 2 * tq) = __builtin_amdgcn_perm(scmn_p, scmn, 0x05040100u);
        *reinterpret_cast<uint32_t *>(vm + 8 + 2 * tq) = __builtin_amdgcn_perm(scmn_p, scmn, 0x07060302u);
      }
    } else {
      const int tt = t & 3;
      if (v_store) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          rec[OFF_VC + ((r * 16 + j0 + k) * VW + wi) * 4 + tt] = (uint8_t)((k < 4 ? vc0 : vc1) >> (8 * (k & 3)));
      }
      if ((li & 1) == 0) {
        uint16_t *vm = reinterpret_cast<uint16_t *>(rec + OFF_VM) + (r * G + gp) * 8;
        vm[tt] = (uint16_t)scb;
        vm[4 + tt] = h_bits(mn16);
      }
    }
  }
}

template <int D, int VB, bool BAL>
__global__ __launch_bounds__(BAL ? kQuantThreadsBal : kQuantThreads) void tq4_quantize_kernel(QuantizeArgs a) {
  using L = QLanes<D>;
  __shared__ float2 s_bins[kMaxBins];
  __shared__ float s_recip[1024];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = L::li(lane), tw = L::tw(lane);
  const float bin_a = a.bins.a, bin_b = a.bins.b - 0.5f;  // v_cvt_pk_u8 rounds: floor via -0.5
  quantize_loop<D, BAL>(a, wv, tw, li,
                   [&] {
                     constexpr int NT = BAL ? kQuantThreadsBal : kQuantThreads;
                     for (int i = threadIdx.x; i < kMaxBins; i += NT) s_bins[i] = a.tables->bins[i];
                     for (int i = threadIdx.x; i < 1024; i += NT) s_recip[i] = a.tables->recip[i];
                     __syncthreads();
                   },
                   [&](const RowLoad<D> &row, int h) {
                     // the lane's indices through an opaque copy, derived
                     // again per row: held through the loop they would push
                     // the balanced loop's registers into spills
                     int l = lane;
                     asm volatile("" : "+v"(l));
                     const int li_r = L::li(l);
                     quantize_row<D, VB>(a, row, h, l, li_r, L::tw(l) & 3, s_bins, s_recip, bin_a, bin_b,
                                         wht16_sign(li_r));
                   });
}

}  // namespace

namespace {

// Work-groups of `kernel` (at `threads` per work-group) resident per compute
// unit, and the compute units of the current device; remembered per host
// thread, so a launch makes no runtime query after the first of its kind.
struct QuantOccupancy {
  int dev = -1, cus = 0;
  const void *kernel[8] = {};
  int per_cu[8] = {};
};

int resident_per_cu(QuantOccupancy &o, const void *kernel, int threads, int fallback) {
  for (int i = 0; i < 8; ++i)
    if (o.kernel[i] == kernel) return o.per_cu[i];
  int per = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess || per <= 0)
    per = fallback;
  for (int i = 0; i < 8; ++i)
    if (!o.kernel[i]) {
      o.kernel[i] = kernel;
      o.per_cu[i] = per;
      break;
    }
  return per;
}

}  // namespace

QuantGeometry quantize_geometry(const void *kernel_static, const void *kernel_balanced, int d, int64_t num_tokens,
                                int hkv) {
  thread_local QuantOccupancy occ;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev != occ.dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    occ = QuantOccupancy{};
    occ.dev = dev;
    occ.cus = cus;
  }
  const int tpw = d == 128 ? 8 : 16;
  const int64_t wave_tasks = (num_tokens + tpw - 1) / tpw * hkv;
  const int64_t slots = (int64_t)(kQuantThreadsBal / 64) * occ.cus;
  bool balanced = wave_tasks >= 8 * slots;
  int grain = wave_tasks >= 32 * slots ? 1 : 2;
  // override for tests: TQ_QUANT_LOOP=static, balanced (one by one) or
  // balanced-pairs
  if (const char *env = std::getenv("TQ_QUANT_LOOP")) {
    if (std::strcmp(env, "static") == 0) balanced = false;
    if (std::strcmp(env, "balanced") == 0) balanced = true, grain = 1;
    if (std::strcmp(env, "balanced-pairs") == 0) balanced = true, grain = 2;
  }
  QuantGeometry g;
  g.balanced = balanced;
  g.grain = grain;
  // override for tests: TQ_ITEM_WINDOW = tokens listed per pass of the
  // balanced loop (several passes per work-group at test sizes)
  g.window = kItemWindow;
  if (const char *env = std::getenv("TQ_ITEM_WINDOW")) {
    const long v = std::strtol(env, nullptr, 10);
    if (v >= 1 && v <= kItemWindow) g.window = (int)v;
  }
  if (balanced) {
    g.threads = kQuantThreadsBal;
    g.grid = occ.cus * resident_per_cu(occ, kernel_balanced, kQuantThreadsBal, 1);
    return g;
  }
  const int64_t wg_tasks = (num_tokens + 4 * tpw - 1) / (4 * tpw) * hkv;
  const int64_t cap = (int64_t)occ.cus * resident_per_cu(occ, kernel_static, kQuantThreads, 2);
  g.threads = kQuantThreads;
  g.grid = (int)(wg_tasks < cap ? wg_tasks : cap);
  return g;
}

template <int D, int VB>
void launch_q(const QuantizeArgs &a, hipStream_t s) {
  const QuantGeometry g = quantize_geometry((const void *)tq4_quantize_kernel<D, VB, false>,
                                            (const void *)tq4_quantize_kernel<D, VB, true>, D, a.num_tokens, a.hkv);
  QuantizeArgs b = a;
  b.grain = g.grain;
  b.window = g.window;
  if (g.balanced) hipLaunchKernelGGL((tq4_quantize_kernel<D, VB, true>), dim3(g.grid), dim3(g.threads), 0, s, b);
  else hipLaunchKernelGGL((tq4_quantize_kernel<D, VB, false>), dim3(g.grid), dim3(g.threads), 0, s, b);
}

hipError_t launch_tq4_quantize(int d, int vbits, const QuantizeArgs &a, hipStream_t s) {
  if (a.num_tokens <= 0) return hipSuccess;
  if (d == 128) vbits == 4 ? launch_q<128, 4>(a, s) : launch_q<128, 2>(a, s);
  else vbits == 4 ? launch_q<64, 4>(a, s) : launch_q<64, 2>(a, s);
  return hipGetLastError();
}

}  // namespace tq
