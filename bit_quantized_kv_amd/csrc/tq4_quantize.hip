// TQ4/4 quantize-and-append kernel for gfx950.
//
// Keys: Walsh-Hadamard rotation, per-(token, kv-head) RMS scale, nearest entry
// of a 16-entry table; values: per-32-channel asymmetric uniform 4-bit codes
// ("TurboQuant 在 AMD GPU 上把長上下文延遲壓下來", section 2: K = rotation +
// LUT, V = uniform; section 4: Walsh-Hadamard rotation).  The exact decision
// rules (fp32 operation order) and the record layout are stated in tq.h.
//
// One wave handles TPW token rows of one kv-head, D/8 lanes per row, 8
// channels per lane (one 128-bit load of K and of V).  Lane bits {0,1,3,4}
// select the 8-channel chunk, so the cross-lane butterfly stages (channel bits
// 3..6) run over lane xor 1, 2 (DPP quad_perm), xor 8 (DPP row_ror:8) and xor 16
// (gfx950 permlane16 swap); the remaining lane bits select the token.
#include "quant_common.h"

namespace tq {
namespace {

template <int D>
__global__ __launch_bounds__(256) void tq4_quantize_kernel(QuantizeArgs a) {
  constexpr int TPW = QMap<D>::TPW;
  constexpr int G = D / 32;
  constexpr int Q = D / 8;
  constexpr int P16 = 16 * (D / 2);
  constexpr int OFF_KS = P16;
  constexpr int OFF_VC = OFF_KS + 32;
  constexpr int OFF_VM = OFF_VC + P16;
  constexpr int REC = OFF_VM + 64 * G;

  __shared__ float2 s_bins[kMaxBins];
  for (int i = threadIdx.x; i < a.bins.nbins; i += blockDim.x) s_bins[i] = a.tables->bins[i];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t group = wave / a.hkv;
  const int h = (int)(wave - group * a.hkv);
  const int li = QMap<D>::li(lane);
  const int tw = QMap<D>::tw(lane);
  const int tq = tw & 3;  // token index within its quad
  const int64_t n = group * TPW + tw;
  if (group * TPW >= a.num_tokens) return;  // whole wave past the end

  const bool in_range = n < a.num_tokens;
  const int slot = in_range ? a.slots[n] : -1;

  uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
  if (in_range) {
    const int64_t base = (n * a.hkv + h) * D + li * 8;
    kr = *reinterpret_cast<const uint4 *>(a.k + base);
    vr = *reinterpret_cast<const uint4 *>(a.v + base);
  }
  float x[8], v[8];
  x[0] = bf16_lo(kr.x); x[1] = bf16_hi(kr.x); x[2] = bf16_lo(kr.y); x[3] = bf16_hi(kr.y);
  x[4] = bf16_lo(kr.z); x[5] = bf16_hi(kr.z); x[6] = bf16_lo(kr.w); x[7] = bf16_hi(kr.w);
  v[0] = bf16_lo(vr.x); v[1] = bf16_hi(vr.x); v[2] = bf16_lo(vr.y); v[3] = bf16_hi(vr.y);
  v[4] = bf16_lo(vr.z); v[5] = bf16_hi(vr.z); v[6] = bf16_lo(vr.w); v[7] = bf16_hi(vr.w);

  // ---- key scale: exact sum of bf16 squares in fp64, exact fp16 RMS ----------
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = __builtin_fma((double)x[e], (double)x[e], ss);
  ss += dpp64_xor1(ss);
  ss += dpp64_xor2(ss);
  ss += dpp64_xor8(ss);
  if constexpr (D == 128) ss += dpp64_xor16(ss);
  const _Float16 s16 = f16_rne_sqrt(ss * (1.0 / D));
  const float sf = (float)s16;

  // ---- key codes ---------------------------------------------------------------
  wht_rows<D>(x, lane);
  const float inv_s = sf > 0.f ? __fdiv_rn(1.0f, sf) : 0.0f;
  const float w = inv_s * a.rsqrt_d;
  const float nbm1 = (float)(a.bins.nbins - 1);
  uint32_t kw = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float u = x[e] * w;
    float fb = __builtin_fmaf(u, a.bins.a, a.bins.b);
    fb = __builtin_amdgcn_fmed3f(fb, 0.f, nbm1);
    const float2 bt = s_bins[(int)fb];
    const uint32_t code = (uint32_t)__float_as_int(bt.y) + (u > bt.x ? 1u : 0u);
    kw |= code << (4 * e);
  }

  // ---- value codes: 32-channel groups = 4 consecutive chunks (lane xor 1, 2) ----
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) {
    mn = __builtin_fminf(mn, v[e]);
    mx = __builtin_fmaxf(mx, v[e]);
  }
  mn = __builtin_fminf(mn, xor1(mn));
  mx = __builtin_fmaxf(mx, xor1(mx));
  mn = __builtin_fminf(mn, xor2(mn));
  mx = __builtin_fmaxf(mx, xor2(mx));
  const float range = mx - mn;
  const _Float16 sc16 = f16_sat(__fdiv_rn(range, 15.0f));
  const _Float16 mn16 = f16_sat(mn);
  const float scv = (float)sc16, mnv = (float)mn16;
  const float inv_sc = scv > 0.f ? __fdiv_rn(1.0f, scv) : 0.0f;
  uint32_t vw = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float d = v[e] - mnv;
    const float q = __builtin_rintf(d * inv_sc);
    vw |= (uint32_t)__builtin_amdgcn_fmed3f(q, 0.f, 15.f) << (4 * e);
  }

  // ---- does this quad of tokens fill four consecutive rows of one block? ------
  // (every exchange runs on all lanes: a cross-lane read under a divergent
  // exec mask would see inactive lanes)
  const int qid = (slot >= 0 && (slot & 3) == tq) ? (slot >> 2) : -1 - tq;
  const int qo = (int)xor4u((uint32_t)qid);
  const uint32_t pair_ok = (qid == qo && qid >= 0) ? 1u : 0u;
  const uint32_t other_ok = quad_xor2<D>(pair_ok);
  const int qp = (int)quad_xor2<D>((uint32_t)qid);
  const bool aligned = pair_ok && other_ok && qp == qid;

  // byte transposes among the quad (all lanes take part)
  uint32_t t1 = xor4u(vw);
  uint32_t vt = __builtin_amdgcn_perm(t1, vw, (tq & 1) ? 0x03070105u : 0x06020400u);
  uint32_t t2 = quad_xor2<D>(vt);
  vt = __builtin_amdgcn_perm(t2, vt, (tq & 2) ? 0x03020706u : 0x05040100u);
  const uint32_t scmn = (uint32_t)h_bits(sc16) | ((uint32_t)h_bits(mn16) << 16);
  const uint32_t scmn_p = quad_xor2<D>(scmn);

  if (slot < 0) return;
  const int64_t blk = slot >> 4;
  const int t = slot & 15;
  uint8_t *rec = a.pool + ((int64_t)blk * a.hkv + h) * REC;
  const int p0 = 4 * li;  // first channel pair of this lane
  *reinterpret_cast<uint32_t *>(rec + ((p0 / Q) * 16 + t) * Q + p0 % Q) = kw;
  if (li == 0) *reinterpret_cast<uint16_t *>(rec + OFF_KS + 2 * t) = h_bits(s16);
  const int r = t >> 2, gp = li >> 2, j0 = 4 * (li & 3);
  if (aligned) {
    // lane tq writes the 4 tokens' byte of channel pair j0 + tq
    *reinterpret_cast<uint32_t *>(rec + OFF_VC + ((r * 16 + j0 + tq) * G + gp) * 4) = vt;
    if ((li & 3) == 0 && tq < 2) {
      uint8_t *vm = rec + OFF_VM + (r * G + gp) * 16;
      *reinterpret_cast<uint32_t *>(vm + 4 * tq) = __builtin_amdgcn_perm(scmn_p, scmn, 0x05040100u);
      *reinterpret_cast<uint32_t *>(vm + 8 + 4 * tq) = __builtin_amdgcn_perm(scmn_p, scmn, 0x07060302u);
    }
  } else {
    const int tt = t & 3;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      rec[OFF_VC + ((r * 16 + j0 + k) * G + gp) * 4 + tt] = (uint8_t)(vw >> (8 * k));
    if ((li & 3) == 0) {
      const int pos = (tt == 1) ? 2 : (tt == 2) ? 1 : tt;
      uint16_t *vm = reinterpret_cast<uint16_t *>(rec + OFF_VM) + (r * G + gp) * 8;
      vm[pos] = h_bits(sc16);
      vm[4 + pos] = h_bits(mn16);
    }
  }
}

}  // namespace

hipError_t launch_tq4_quantize(int d, const QuantizeArgs &a, hipStream_t s) {
  if (a.num_tokens <= 0) return hipSuccess;
  const int tpw = (d == 128) ? 4 : 8;
  const int64_t waves = ((a.num_tokens + tpw - 1) / tpw) * a.hkv;
  const int64_t blocks = (waves + 3) / 4;
  if (d == 128)
    hipLaunchKernelGGL(tq4_quantize_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(tq4_quantize_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tq
