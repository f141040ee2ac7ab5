// TQ4/4 paged decode attention for gfx950, split-K with a log-sum-exp merge.
//
// One query token per sequence attends over the 4-bit paged cache; keys are
// compared in the rotated domain (the query is rotated instead, which leaves
// q . k unchanged: "TurboQuant 在 AMD GPU 上把長上下文延遲壓下來", section 4),
// values are dequantized in registers.
//
// Work-group = (sequence b, kv-head, split); its 4 waves take the split's
// blocks in turn, each keeping an online-softmax state, merged in LDS at the
// end.  Per 16-token block a wave does:
//   * one 128-bit load per lane of the key codes (the record places each lane's
//     MFMA A-operand bytes contiguously), a byte-pair LUT lookup in LDS giving
//     two exact fp16 table entries per byte;
//   * logits = K_hat (16 tokens x D) times the rotated query group (D x 16
//     columns: g columns of fp16 high parts, g of low parts) with
//     v_mfma_f32_16x16x32_f16, then the per-token key scale;
//   * online softmax in log2 units (the query carries log2(e));
//   * values dequantized to fp16 (code * scale + min, one rounding) and
//     out^T (channels x columns) += V_hat^T P with v_mfma_f32_16x16x16_f16,
//     P again split into fp16 high and low parts.
// Partials (max, sum, acc) per (sequence, query head, split) go to the
// workspace and a merge kernel combines them; a single split writes the output.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

template <int GQ>
__device__ __forceinline__ float xor_g(float x) {
  if constexpr (GQ == 1) return xor1(x);
  else if constexpr (GQ == 2) return xor2(x);
  else if constexpr (GQ == 4) return xor4(x);
  else return xor8(x);
}

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

// fp16 values of 4-bit codes: (w & 0x000F000F) | 0x6400_6400 = 1024 + code, exact
__device__ __forceinline__ half2v nib2(uint32_t w) {
  const half2v c = as_h2((w & 0x000F000Fu) | 0x64006400u);
  return c - (half2v){(_Float16)1024.0f, (_Float16)1024.0f};
}

template <int D, int GQ>
__global__ __launch_bounds__(256) void tq4_decode_kernel(DecodeArgs a) {
  constexpr int G = D / 32;
  constexpr int KS = D / 32;          // 32-channel k-steps of the QK product
  constexpr int Q = D / 8;            // key-code bytes per lane
  constexpr int P16 = 16 * (D / 2);
  constexpr int OFF_KS = P16;
  constexpr int OFF_VC = OFF_KS + 32;
  constexpr int OFF_VM = OFF_VC + P16;
  constexpr int REC = OFF_VM + 64 * G;
  typedef typename KTile<D>::T KT;

  __shared__ uint32_t s_lut[256];
  __shared__ float s_q[GQ][D];
  __shared__ float s_m[4][GQ], s_l[4][GQ];
  __shared__ float s_acc[4][GQ][D];

  const int tid = threadIdx.x;
  const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int b = (int)(wg % (uint32_t)a.batch);
  const uint32_t rest = wg / (uint32_t)a.batch;
  const int kvh = (int)(rest % (uint32_t)a.hkv);
  const int sp = (int)(rest / (uint32_t)a.hkv);

  const int T = a.ctx[b];
  const int nblk = (T + 15) >> 4;
  const int blk0 = sp * a.split_blocks;
  const bool single = a.nsplit == 1;
  const int qh0 = kvh * GQ;
  if (nblk == 0) {
    if (single && sp == 0) {
      for (int i = tid; i < GQ * D; i += 256) {
        const int64_t o = ((int64_t)b * a.hq + qh0) * D + i;
        if (a.out_bf16) reinterpret_cast<uint16_t *>(a.out)[o] = 0;
        else reinterpret_cast<float *>(a.out)[o] = 0.f;
      }
    }
    return;
  }
  if (blk0 >= nblk) return;
  const int blk1 = min(nblk, blk0 + a.split_blocks);

  // ---- stage the LUT and the rotated, scaled query group ----------------------
  s_lut[tid] = a.tables->lut2[tid];
  for (int i = tid; i < GQ * D; i += 256) {
    const uint16_t qb = a.q[((int64_t)b * a.hq + qh0) * D + i];
    s_q[i / D][i % D] = as_f((uint32_t)qb << 16);
  }
  __syncthreads();
#pragma unroll 1
  for (int hs = 1; hs < D; hs <<= 1) {
    for (int i = tid; i < GQ * D / 2; i += 256) {
      const int hh = i / (D / 2), pi = i % (D / 2);
      const int lo = (pi / hs) * (2 * hs) + (pi % hs);
      const float x0 = s_q[hh][lo], x1 = s_q[hh][lo + hs];
      s_q[hh][lo] = x0 + x1;
      s_q[hh][lo + hs] = x0 - x1;
    }
    __syncthreads();
  }

  const int lane = tid & 63, wv = tid >> 6;
  const int r = lane >> 4, n = lane & 15;

  // B operand of the QK product: column n < g is head n's high fp16 part,
  // g <= n < 2g head n-g's low part; lane (r, n) holds channels r*D/4 + 8s + i.
  half8v bq[KS];
  {
    const bool used = n < 2 * GQ;
    const bool is_lo = n >= GQ;
    const int hh = is_lo ? n - GQ : n;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xv = used ? s_q[used ? hh : 0][r * (D / 4) + 8 * s + i] * a.qscale : 0.f;
        const _Float16 hi = (_Float16)xv;
        const _Float16 lo = (_Float16)(xv - (float)hi);
        bq[s][i] = used ? (is_lo ? lo : hi) : (_Float16)0.f;
      }
    }
  }
  const bool col_lo = n >= GQ && n < 2 * GQ;
  const bool col_used = n < 2 * GQ;

  float m_run = kNegInf, l_run = 0.f;
  float4v acc[2 * G];
#pragma unroll
  for (int t = 0; t < 2 * G; ++t) acc[t] = (float4v){0.f, 0.f, 0.f, 0.f};

  const int32_t *btab = a.block_table + (int64_t)b * a.max_blocks;
#pragma unroll 1
  for (int lb = blk0 + wv; lb < blk1; lb += 4) {
    const int pid = btab[lb];
    const uint8_t *rec = a.pool + ((int64_t)pid * a.hkv + kvh) * REC;
    const KT kq = *reinterpret_cast<const KT *>(rec + lane * Q);
    const uint2 ksv = *reinterpret_cast<const uint2 *>(rec + OFF_KS + 8 * r);
    const KT vq = *reinterpret_cast<const KT *>(rec + OFF_VC + lane * (4 * G));
    uint4 vm[G];
#pragma unroll
    for (int gp = 0; gp < G; ++gp) vm[gp] = *reinterpret_cast<const uint4 *>(rec + OFF_VM + (r * G + gp) * 16);

    // ---- logits ---------------------------------------------------------------
    float4v qk = (float4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t w = word(kq, s);
      uint4 e;
      e.x = s_lut[w & 0xFF];
      e.y = s_lut[(w >> 8) & 0xFF];
      e.z = s_lut[(w >> 16) & 0xFF];
      e.w = s_lut[w >> 24];
      qk = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8v, e), bq[s], qk, 0, 0, 0);
    }
    const half2v s01 = as_h2(ksv.x), s23 = as_h2(ksv.y);
    const float ks[4] = {(float)s01[0], (float)s01[1], (float)s23[0], (float)s23[1]};
    float x[4];
    const int tok0 = lb * 16 + 4 * r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (qk[i] + xor_g<GQ>(qk[i])) * ks[i];
      if (tok0 + i >= T) x[i] = kNegInf;
    }

    // ---- online softmax ---------------------------------------------------------
    float bm = __builtin_fmaxf(__builtin_fmaxf(x[0], x[1]), __builtin_fmaxf(x[2], x[3]));
    bm = __builtin_fmaxf(bm, xor16(bm));
    bm = __builtin_fmaxf(bm, xor32(bm));
    const float m_new = __builtin_fmaxf(m_run, bm);
    if (m_new > m_run) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < 2 * G; ++t) acc[t] *= alpha;
      m_run = m_new;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - m_run);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    half4v bp;
    {
      // k-slot order of the value operand: tokens 4r + (0, 2, 1, 3)
      const float pk[4] = {p[0], p[2], p[1], p[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 hi = (_Float16)pk[i];
        const _Float16 lo = (_Float16)(pk[i] - (float)hi);
        bp[i] = col_used ? (col_lo ? lo : hi) : (_Float16)0.f;
      }
    }

    // ---- values -----------------------------------------------------------------
    const bool tail = (lb + 1) * 16 > T;
#pragma unroll
    for (int gp = 0; gp < G; ++gp) {
      const uint32_t w = word(vq, gp);
      const half2v sc02 = as_h2(vm[gp].x), sc13 = as_h2(vm[gp].y);
      const half2v mn02 = as_h2(vm[gp].z), mn13 = as_h2(vm[gp].w);
      half2v e02 = __builtin_elementwise_fma(nib2(w), sc02, mn02);
      half2v e13 = __builtin_elementwise_fma(nib2(w >> 8), sc13, mn13);
      half2v o02 = __builtin_elementwise_fma(nib2(w >> 4), sc02, mn02);
      half2v o13 = __builtin_elementwise_fma(nib2(w >> 12), sc13, mn13);
      if (tail) {
        // rows past the context may hold anything; zero them (p is 0 there)
        const bool v0 = tok0 + 0 < T, v1 = tok0 + 1 < T, v2 = tok0 + 2 < T, v3 = tok0 + 3 < T;
        const _Float16 z = (_Float16)0.f;
        e02 = (half2v){v0 ? e02[0] : z, v2 ? e02[1] : z};
        o02 = (half2v){v0 ? o02[0] : z, v2 ? o02[1] : z};
        e13 = (half2v){v1 ? e13[0] : z, v3 ? e13[1] : z};
        o13 = (half2v){v1 ? o13[0] : z, v3 ? o13[1] : z};
      }
      const half4v ae = (half4v){e02[0], e02[1], e13[0], e13[1]};
      const half4v ao = (half4v){o02[0], o02[1], o13[0], o13[1]};
      acc[2 * gp] = __builtin_amdgcn_mfma_f32_16x16x16f16(ae, bp, acc[2 * gp], 0, 0, 0);
      acc[2 * gp + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(ao, bp, acc[2 * gp + 1], 0, 0, 0);
    }
  }

  // ---- wave state -> LDS: combine high and low columns, sum over lane rows -------
  l_run += xor16(l_run);
  l_run += xor32(l_run);
#pragma unroll
  for (int t = 0; t < 2 * G; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] += xor_g<GQ>(acc[t][i]);
  }
  if (n < GQ) {
#pragma unroll
    for (int gp = 0; gp < G; ++gp) {
#pragma unroll
      for (int par = 0; par < 2; ++par) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s_acc[wv][n][32 * gp + 2 * (4 * r + i) + par] = acc[2 * gp + par][i];
      }
    }
    if (r == 0) {
      s_m[wv][n] = m_run;
      s_l[wv][n] = l_run;
    }
  }
  __syncthreads();

  // ---- merge the 4 waves ----------------------------------------------------------
  for (int i = tid; i < GQ * D; i += 256) {
    const int hh = i / D, c = i % D;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = __builtin_fmaxf(mx, s_m[w][hh]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (s_m[w][hh] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(s_m[w][hh] - mx);
      num += f * s_acc[w][hh][c];
      den += f * s_l[w][hh];
    }
    const int64_t row = (int64_t)b * a.hq + qh0 + hh;
    if (single) {
      const float o = den > 0.f ? num / den : 0.f;
      if (a.out_bf16) reinterpret_cast<uint16_t *>(a.out)[row * D + c] = f32_to_bf16(o);
      else reinterpret_cast<float *>(a.out)[row * D + c] = o;
    } else {
      const int64_t pi = row * a.nsplit + sp;
      a.part_acc[pi * D + c] = num;
      if (c == 0) {
        a.part_ml[pi * 2] = mx;
        a.part_ml[pi * 2 + 1] = den;
      }
    }
  }
}

// One wave per (sequence, query head): combine the split partials.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  constexpr int CPL = D / 64;  // channels per lane
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)a.batch * a.hq) return;
  const int lane = threadIdx.x & 63;
  const int b = (int)(row / a.hq);
  const int T = a.ctx[b];
  const int nblk = (T + 15) >> 4;
  const int ns = (nblk + a.split_blocks - 1) / a.split_blocks;
  const float *ml = a.part_ml + row * a.nsplit * 2;
  const float *pa = a.part_acc + row * a.nsplit * D;
  float mx = kNegInf;
  for (int s = 0; s < ns; ++s) mx = __builtin_fmaxf(mx, ml[2 * s]);
  float num[CPL] = {}, den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float m = ml[2 * s];
    const float f = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m - mx);
    den += f * ml[2 * s + 1];
#pragma unroll
    for (int c = 0; c < CPL; ++c) num[c] += f * pa[(int64_t)s * D + lane * CPL + c];
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const float o = den > 0.f ? num[c] / den : 0.f;
    const int64_t oi = row * D + lane * CPL + c;
    if (a.out_bf16) reinterpret_cast<uint16_t *>(a.out)[oi] = f32_to_bf16(o);
    else reinterpret_cast<float *>(a.out)[oi] = o;
  }
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s) {
  const int64_t wgs = (int64_t)a.batch * a.hkv * a.nsplit;
  switch (a.g) {
    case 1: hipLaunchKernelGGL((tq4_decode_kernel<D, 1>), dim3((unsigned)wgs), dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((tq4_decode_kernel<D, 2>), dim3((unsigned)wgs), dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((tq4_decode_kernel<D, 4>), dim3((unsigned)wgs), dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((tq4_decode_kernel<D, 8>), dim3((unsigned)wgs), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tq4_decode(int d, const DecodeArgs &a, hipStream_t s) {
  return d == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

hipError_t launch_decode_merge(int d, const DecodeArgs &a, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.hq;
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  if (d == 128) hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tq
