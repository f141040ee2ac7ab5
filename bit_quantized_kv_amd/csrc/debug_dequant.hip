// Test-only export of the dequantized cache: the values every attention
// kernel of this library consumes, written out in fp32 so that they can be
// compared bit for bit with an independent implementation.
//
// "TurboQuant 在 AMD GPU 上把長上下文延遲壓下來", section 2 (TQ4/4: keys by
// rotation + 16-entry table, k_hat = c[code] * s in the rotated domain; values
// uniform, v_hat = code * sc + mn); "UltraQuant：4-bit KV 快取加速長代理",
// section "方法怎麼做，白話講" (MX-FP4: e2m1 elements times 2^X per 32
// channels).
//
// One wave per (block, kv-head) record, with the decode kernels' record reader
// (load_blk), key table lookup (key_entries), code isolation
// (value_code_bytes, codes_f16), exact code * scale split (scaled_codes,
// including the 2^-7 pre-scaling of a block with a scale >= 4096) and FP4
// conversion (fp4_pair_bf16): v_hat = fp32((hi + lo) * back + mn) is
// fp32(code * sc + mn) exactly, as the MFMA consumes (hi + lo) * P + mn * P.
#include "decode_common.h"
#include "dequant.h"

namespace tq {
namespace {

// Output element (record i, kv-head h, token t, channel ch) of [n][hkv][16][D].
__device__ __forceinline__ int64_t out_idx(int64_t i, int h, int hkv, int t, int ch, int d) {
  return (((i * hkv + h) * 16) + t) * d + ch;
}

template <int D, int VB>
__global__ __launch_bounds__(64) void tq4_debug_dequant_kernel(const uint8_t *pool, int64_t num_blocks, int hkv,
                                                                const int32_t *ids, const DeviceTables *tables,
                                                                float *k_out, float *v_out) {
  constexpr int G = D / 32, KS = D / 32;
  constexpr int REC = TqRec<D, VB>::BYTES;
  __shared__ uint32_t s_lut[256];
  __shared__ __attribute__((aligned(16))) uint32_t s_vm[64];
  const int lane = threadIdx.x;
  const int64_t i = blockIdx.x / hkv;
  const int h = blockIdx.x % hkv;
  for (int j = lane; j < 256; j += 64) s_lut[j] = tables->lut2[j];
  const int64_t id = ids[i];
  const bool ok = id >= 0 && id < num_blocks;
  const uint8_t *rec = pool + ((ok ? id : 0) * hkv + h) * REC;
  Blk<D, VB> bk;
  load_blk<D, VB>(bk, rec, lane);
  const int r = lane >> 4, c = lane & 15;
  // the value (scale, min) tile as the decode kernel stages it, with its
  // per-block 2^-7 pre-scaling when some scale is >= 4096
  const uint32_t sc_lane = (lane & 2) ? 0u : 0xFFFFFFFFu;
  uint32_t vmw = bk.vmw;
  const bool big = __builtin_amdgcn_ballot_w64(has_big_scale(vmw & sc_lane) != 0) != 0;
  if (big && sc_lane) vmw = as_u(as_h2(vmw) * (half2v){(_Float16)0x1p-7f, (_Float16)0x1p-7f});
  s_vm[r * (4 * G) + (c & (4 * G - 1))] = vmw;
  __syncthreads();
  const float back = big ? 128.f : 1.f;

  // keys: lane l holds token l % 16, channels (D / 4) (l / 16) + 8 s + (0..7)
  // in word s
  const int kt = lane & 15;
  const float s = (float)h_from(reinterpret_cast<const uint16_t *>(rec + TqRec<D, VB>::KS)[kt]);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint4 e = key_entries(s_lut, word(bk.kq, ks));
    const half8v c8 = __builtin_bit_cast(half8v, e);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float kv = ok ? (float)c8[j] * s : 0.f;
      k_out[out_idx(i, h, hkv, kt, (D / 4) * (lane >> 4) + 8 * ks + j, D)] = kv;
    }
  }
  // values: lane (r, c) holds channels 32 gp + 2c (+1) of tokens 4r .. 4r+3
  const uint4 *vm_row = reinterpret_cast<const uint4 *>(s_vm) + r * G;
#pragma unroll
  for (int gp = 0; gp < G; ++gp) {
    const uint4 vm = vm_row[gp];
    uint32_t lo, hi;
    value_code_bytes<VB>(VB == 4 ? word(bk.vq, gp) : word(bk.vq, gp >> 1), gp, lo, hi);
    const half2v sc01 = as_h2(vm.x), sc23 = as_h2(vm.y), mn01 = as_h2(vm.z), mn23 = as_h2(vm.w);
    const ScaledPair e01 = scaled_codes(codes_f16<false>(lo), sc01);
    const ScaledPair e23 = scaled_codes(codes_f16<true>(lo), sc23);
    const ScaledPair o01 = scaled_codes(codes_f16<false>(hi), sc01);
    const ScaledPair o23 = scaled_codes(codes_f16<true>(hi), sc23);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const ScaledPair &ev = tt < 2 ? e01 : e23, &ov = tt < 2 ? o01 : o23;
      const _Float16 mn = tt < 2 ? mn01[tt] : mn23[tt - 2];
      const int t = 4 * r + tt;
      const float ve = value_f32(ev.hi[tt & 1], ev.lo[tt & 1], back, mn);
      const float vo = value_f32(ov.hi[tt & 1], ov.lo[tt & 1], back, mn);
      v_out[out_idx(i, h, hkv, t, 32 * gp + 2 * c, D)] = ok ? ve : 0.f;
      v_out[out_idx(i, h, hkv, t, 32 * gp + 2 * c + 1, D)] = ok ? vo : 0.f;
    }
  }
}

// MX-FP4 (D = 128): keys as e2m1 * 2^X in fp32 (the decode's scaled MFMA
// applies the same exponent bytes), values through the decode's bf16 path.
__global__ __launch_bounds__(64) void mxfp4_debug_dequant_kernel(const uint8_t *pool, int64_t num_blocks, int hkv,
                                                                  const int32_t *ids, float *k_out, float *v_out) {
  constexpr int D = 128, G = 4, REC = MxRec::BYTES, OFF_KS = MxRec::KS, OFF_VC = MxRec::VC, OFF_VS = MxRec::VS;
  const int lane = threadIdx.x;
  const int64_t i = blockIdx.x / hkv;
  const int h = blockIdx.x % hkv;
  const int64_t id = ids[i];
  const bool ok = id >= 0 && id < num_blocks;
  const uint8_t *rec = pool + ((ok ? id : 0) * hkv + h) * REC;
  const uint4 kq = *reinterpret_cast<const uint4 *>(rec + MxRec::KC + lane * 16);
  const uint32_t kx = rec[OFF_KS + lane];  // (token lane % 16, group lane / 16)
  const uint4 vq = *reinterpret_cast<const uint4 *>(rec + OFF_VC + lane * 16);
  const int r = lane >> 4, c = lane & 15, kt = lane & 15;
  // keys: word s holds channels 32 (l / 16) + 8 s + (0..7), byte j of it
  // channels + 2j, + 2j + 1
  const float ksc = ue8m0_scale(kx);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t w = word(kq, s);
    const float2v p0 = fp4_pair_f32<0>(w, ksc), p1 = fp4_pair_f32<1>(w, ksc);
    const float2v p2 = fp4_pair_f32<2>(w, ksc), p3 = fp4_pair_f32<3>(w, ksc);
    const float kv[8] = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      k_out[out_idx(i, h, hkv, kt, 32 * (lane >> 4) + 8 * s + j, D)] = ok ? kv[j] : 0.f;
  }
  // values: lane (r, c) holds channels 32 gp + 2c (+1) of tokens 4r .. 4r+3
#pragma unroll
  for (int gp = 0; gp < G; ++gp) {
    const uint32_t w = word(vq, gp);
    const uint32_t xs = *reinterpret_cast<const uint32_t *>(rec + OFF_VS + (r * G + gp) * 4);
    const uint32_t h4[4] = {fp4_pair_bf16<0>(w, ue8m0_scale(xs & 0xFFu)),
                            fp4_pair_bf16<1>(w, ue8m0_scale((xs >> 8) & 0xFFu)),
                            fp4_pair_bf16<2>(w, ue8m0_scale((xs >> 16) & 0xFFu)),
                            fp4_pair_bf16<3>(w, ue8m0_scale(xs >> 24))};
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int t = 4 * r + tt;
      v_out[out_idx(i, h, hkv, t, 32 * gp + 2 * c, D)] = ok ? as_f(h4[tt] << 16) : 0.f;
      v_out[out_idx(i, h, hkv, t, 32 * gp + 2 * c + 1, D)] = ok ? as_f(h4[tt] & 0xFFFF0000u) : 0.f;
    }
  }
}

}  // namespace

hipError_t launch_debug_dequant(int format, int d, const uint8_t *pool, int64_t num_blocks, int hkv,
                                const int32_t *ids, int64_t n, const DeviceTables *tables, float *k_out,
                                float *v_out, hipStream_t s) {
  const dim3 grid((unsigned)(n * hkv)), block(64);
  if (format == 1) {
    hipLaunchKernelGGL(mxfp4_debug_dequant_kernel, grid, block, 0, s, pool, num_blocks, hkv, ids, k_out, v_out);
  } else if (format == 0) {
    if (d == 128) hipLaunchKernelGGL((tq4_debug_dequant_kernel<128, 4>), grid, block, 0, s, pool, num_blocks, hkv, ids, tables, k_out, v_out);
    else hipLaunchKernelGGL((tq4_debug_dequant_kernel<64, 4>), grid, block, 0, s, pool, num_blocks, hkv, ids, tables, k_out, v_out);
  } else {
    if (d == 128) hipLaunchKernelGGL((tq4_debug_dequant_kernel<128, 2>), grid, block, 0, s, pool, num_blocks, hkv, ids, tables, k_out, v_out);
    else hipLaunchKernelGGL((tq4_debug_dequant_kernel<64, 2>), grid, block, 0, s, pool, num_blocks, hkv, ids, tables, k_out, v_out);
  }
  return hipGetLastError();
}

}  // namespace tq
