// TQ4/4 paged decode attention for gfx950, split-K with a log-sum-exp merge.
//
// One query token per sequence attends over the 4-bit paged cache; keys are
// compared in the rotated domain (the query is rotated instead, which leaves
// q . k unchanged: "TurboQuant 在 AMD GPU 上把長上下文延遲壓下來", section 4),
// values are dequantized in registers.
//
// Work-group = (sequence b, kv-head, split) with NW waves.  Each wave takes
// every NW-th block of the split, four blocks of loads in flight, and keeps an
// online-softmax state; the waves are merged in LDS at the end.  Per 16-token
// block a wave does:
//   * one 128-bit load per lane of the key codes (the record places each lane's
//     MFMA A-operand bytes contiguously), a byte-pair LUT lookup in LDS giving
//     two exact fp16 table entries per byte;
//   * logits = K_hat (16 tokens x D) times the rotated query group (D x 16
//     columns: g columns of fp16 high parts, g of low parts) with
//     v_mfma_f32_16x16x32_f16, then the per-token key scale;
//   * online softmax in log2 units (the query carries log2(e)), rescaling the
//     accumulators only when the running maximum moves by more than 2^8;
//   * values dequantized to fp16 (code * scale + min, one rounding) and
//     out^T (channels x columns) += V_hat^T P with v_mfma_f32_16x16x16_f16,
//     P again split into fp16 high and low parts.
// Split partials (max, sum, acc) go to the workspace; decode_merge combines them.
#include "decode_common.h"

namespace tq {
namespace {

constexpr int kWaves = 8;

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

// Two 4-bit codes, each alone in a byte of `bytes` (word `hi_word`), as exact
// fp16 values: 0000cccc is the OCP e4m3 encoding of c * 2^-9.
template <bool HI_WORD>
__device__ __forceinline__ half2v codes_f16(uint32_t bytes) {
  return __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bytes, 512.0f, HI_WORD));
}

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
  constexpr int G = D / 32, Q = D / 8, P16 = 16 * (D / 2);
  constexpr int VW = VB == 4 ? G : G / 2;  // value-code words per lane
  constexpr int OFF_KS = P16, OFF_VC = OFF_KS + 32, OFF_VM = OFF_VC + 64 * 4 * VW;
  const int r = lane >> 4, c = lane & 15;
  o.kq = *reinterpret_cast<const typename KTile<D>::T *>(rec + lane * Q);
  o.ks = *reinterpret_cast<const uint2 *>(rec + OFF_KS + 8 * r);
  o.vq = *reinterpret_cast<const typename VTile<D, VB>::T *>(rec + OFF_VC + lane * (4 * VW));
  o.vmw = reinterpret_cast<const uint32_t *>(rec + OFF_VM)[r * (4 * G) + (c & (4 * G - 1))];
}

// vm_slot: this wave's 16*D/8-byte LDS slot for the value (scale, min) tile.
// vm_keep: per-lane mask clearing the (scale, min) halves of rows past the
// context, so those rows dequantize to exactly 0 whatever the pool holds
// (applied here, at the use, so that no wait on the block's loads is forced
// earlier).
// tail: the block is the partial last one of its sequence (rows past the
// context are masked: -inf logits, zero value scale and minimum).
template <int D, int GQ, int VB>
__device__ __forceinline__ void do_block(const Blk<D, VB> &bk, const half8v (&bq)[D / 32], const uint32_t *s_lut,
                                         uint32_t *vm_slot, WaveState<2 * D / 32> &st, float lo_mask, int lane,
                                         int tok0, int T, bool tail, uint32_t vm_keep) {
  constexpr int G = D / 32, KS = D / 32;
  // the value (scale, min) tile goes through LDS: lane (r, c) wrote dword c of
  // row r; every lane reads its row's 16*G bytes back (broadcast reads)
  // (the tail fix-ups sit behind real branches: an if-converted select would
  // cost every block several instructions)
  uint32_t vmw = bk.vmw;
  if (tail) {
    __asm__ volatile("");
    vmw &= vm_keep;
  }
  vm_slot[(lane >> 4) * (4 * G) + (lane & (4 * G - 1))] = vmw;
  // ---- logits ---------------------------------------------------------------
  float4v qk = (float4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const uint32_t w = word(bk.kq, s);
    uint4 e;
    e.x = s_lut[w & 0xFF];
    e.y = s_lut[(w >> 8) & 0xFF];
    e.z = s_lut[(w >> 16) & 0xFF];
    e.w = s_lut[w >> 24];
    qk = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8v, e), bq[s], qk, 0, 0, 0);
  }
  const half2v s01 = as_h2(bk.ks.x), s23 = as_h2(bk.ks.y);
  // logit = (high + low column) * key scale, one v_fma_mix each (the fp16
  // scale taken directly; the +0 addend only turns a -0 product into +0)
  float x[4];
  x[0] = __builtin_fmaf(qk[0] + xor_g<GQ>(qk[0]), (float)s01[0], 0.0f);
  x[1] = __builtin_fmaf(qk[1] + xor_g<GQ>(qk[1]), (float)s01[1], 0.0f);
  x[2] = __builtin_fmaf(qk[2] + xor_g<GQ>(qk[2]), (float)s23[0], 0.0f);
  x[3] = __builtin_fmaf(qk[3] + xor_g<GQ>(qk[3]), (float)s23[1], 0.0f);
  if (tail) {
    __asm__ volatile("");
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (tok0 + i >= T) x[i] = kNegInf;
  }
  float p[4];
  softmax_block<2 * G>(x, st, p);
  // B operand: tokens 4r + 0..3 in k order; high part on columns < g, low
  // part (p - high) on columns g .. 2g-1; other columns are never read
  half4v bp;
  {
    const half2v h01 = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(p[0], p[1]));
    const half2v h23 = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(p[2], p[3]));
    const float r0 = __builtin_fmaf(-lo_mask, (float)h01[0], p[0]);
    const float r1 = __builtin_fmaf(-lo_mask, (float)h01[1], p[1]);
    const float r2 = __builtin_fmaf(-lo_mask, (float)h23[0], p[2]);
    const float r3 = __builtin_fmaf(-lo_mask, (float)h23[1], p[3]);
    const half2v a01 = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(r0, r1));
    const half2v a23 = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(r2, r3));
    bp = (half4v){a01[0], a01[1], a23[0], a23[1]};
  }

  // ---- values -----------------------------------------------------------------
  // A nibble isolated in a byte, 0000cccc, is the OCP e4m3 encoding of
  // c * 2^-9 (codes 0..7 subnormal, 8..15 with exponent field 1), so the fp8
  // conversion with scale 2^9 turns two such bytes into two exact fp16 codes;
  // one fma with the fp16 (scale, min) pair then dequantizes with one rounding.
  const uint4 *vm_row = reinterpret_cast<const uint4 *>(vm_slot) + (lane >> 4) * G;
#pragma unroll
  for (int gp = 0; gp < G; ++gp) {
    const uint4 vm = vm_row[gp];
    // bytes = tokens 4r + 0..3 of one channel pair; lo / hi = the even / odd
    // channel's codes, each alone in its byte (2-bit: the group pair's word,
    // group 2w in bits 0-3 of each byte, 2w + 1 in bits 4-7)
    uint32_t lo, hi;
    if constexpr (VB == 4) {
      const uint32_t w = word(bk.vq, gp);
      lo = w & 0x0F0F0F0Fu;
      hi = (w >> 4) & 0x0F0F0F0Fu;
    } else {
      const uint32_t w = word(bk.vq, gp >> 1) >> (4 * (gp & 1));
      lo = w & 0x03030303u;
      hi = (w >> 2) & 0x03030303u;
    }
    const half2v sc01 = as_h2(vm.x), sc23 = as_h2(vm.y);
    const half2v mn01 = as_h2(vm.z), mn23 = as_h2(vm.w);
    const half2v e01 = __builtin_elementwise_fma(codes_f16<false>(lo), sc01, mn01);
    const half2v e23 = __builtin_elementwise_fma(codes_f16<true>(lo), sc23, mn23);
    const half2v o01 = __builtin_elementwise_fma(codes_f16<false>(hi), sc01, mn01);
    const half2v o23 = __builtin_elementwise_fma(codes_f16<true>(hi), sc23, mn23);
    const half4v ae = __builtin_bit_cast(half4v, make_uint2(as_u(e01), as_u(e23)));
    const half4v ao = __builtin_bit_cast(half4v, make_uint2(as_u(o01), as_u(o23)));
    st.acc[2 * gp] = __builtin_amdgcn_mfma_f32_16x16x16f16(ae, bp, st.acc[2 * gp], 0, 0, 0);
    st.acc[2 * gp + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(ao, bp, st.acc[2 * gp + 1], 0, 0, 0);
  }
}

template <int D, int GQ, bool CASCADE, int VB = 4>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void tq4_decode_kernel(
    DecodeArgs a) {
  constexpr int G = D / 32, KS = D / 32;
  constexpr int REC = 16 * (D / 2) + 32 + (VB == 4 ? 16 * (D / 2) : 16 * (D / 4)) + 64 * G;
  constexpr int NW = kWaves;

  __shared__ uint32_t s_lut[256];
  __shared__ __attribute__((aligned(16))) uint32_t s_vm[NW][64];
  __shared__ __attribute__((aligned(16))) _Float16 s_bq[16][D];
  __shared__ float s_m[NW][GQ], s_l[NW][GQ];
  __shared__ float s_acc[NW][GQ][D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: block ids load as scalars
  const WgTask task = decode_task(a);
  const int b = task.b, kvh = task.kvh, sp = task.sp;
  const int qh0 = kvh * GQ;

  const int T = a.ctx[b];  // a scalar load: nothing is written before it
  // this wave's block ids, fetched before the context length is known (the
  // index is clamped into the table row; entries past the context are never
  // used): blocks blk0 + wv + k * NW, lane k holds the id of the k-th
  // cascade: the splits start at the sequence's first block of its own
  const int blk0 = (CASCADE ? a.first_blk[b] : 0) + sp * a.split_blocks;
  const int32_t *btab = a.block_table + (int64_t)b * a.max_blocks;
  const int my_id_raw = btab[min(blk0 + wv + lane * NW, a.max_blocks - 1)];
  // set-up loads next (table word, query word): they complete while the block
  // ids are fetched, so the set-up below waits on nothing
  const uint32_t lut_w = tid < 256 ? a.tables->lut2[tid] : 0u;
  const uint32_t q_w = wv < GQ ? load_query_word<D>(a.q + ((int64_t)b * a.hq + qh0 + wv) * D, lane) : 0u;
  __asm__ volatile("" ::: "memory");
  const int nblk = (T + 15) >> 4;
  if (nblk == 0) {
    if (!CASCADE && a.nsplit == 1 && sp == 0) write_zero_rows<D>(a, b, qh0, GQ);
    return;
  }
  if (blk0 >= nblk) return;
  const int blk1 = min(nblk, blk0 + a.split_blocks);

  // ---- first loads go out before the set-up work -----------------------------
  const uint8_t *base = a.pool + (int64_t)kvh * REC;
  const int64_t stride = (int64_t)a.hkv * REC;
  // this wave's blocks: blk0 + wv + k * NW, k < mine (mine <= 64); lane k
  // holds block id k, read back with readlane.  Four blocks stay in flight:
  // every step refills its buffer unconditionally (past the end with the
  // wave's last block again, an L2 hit), so the number of loads in flight is
  // the same on every path and the waits stay partial.
  const int mine = blk1 - blk0 > wv ? (blk1 - blk0 - wv + NW - 1) / NW : 0;
  const int my_id = settled(my_id_raw);
  auto rec_of = [&](int k) {
    const int kk = k < mine ? k : mine - 1;
    return base + (int64_t)__builtin_amdgcn_readlane(my_id, kk) * stride;
  };
  // rows of the partial last block past the context get zero (scale, min)
  const int tail_blk = (T & 15) ? nblk - 1 : nblk;
  uint32_t tail_keep;
  {
    // dword w of a group's 16 bytes: (sc t0, t1) (sc t2, t3) (mn t0, t1) (mn t2, t3)
    const int r0 = 4 * (lane >> 4), w = lane & 3;
    const int ta = (T & 15) - (r0 + 2 * (w & 1)), tb = ta - 1;
    tail_keep = (ta > 0 ? 0x0000FFFFu : 0u) | (tb > 0 ? 0xFFFF0000u : 0u);
  }
  Blk<D, VB> b0, b1, b2, b3;
  if (mine > 0) {
    // issued block by block, as the loop's refills are, so that the
    // compiler's wait counts inside the loop stay partial on its first pass
    load_blk<D, VB>(b0, rec_of(0), lane);
    __asm__ volatile("" ::: "memory");
    load_blk<D, VB>(b1, rec_of(1), lane);
    __asm__ volatile("" ::: "memory");
    load_blk<D, VB>(b2, rec_of(2), lane);
    __asm__ volatile("" ::: "memory");
    load_blk<D, VB>(b3, rec_of(3), lane);
  }

  // ---- LUT and the rotated, scaled query group (wave w < g rotates head w) ------
  if (tid < 256) s_lut[tid] = lut_w;
  for (int i = tid; i < (16 - 2 * GQ) * D; i += NW * 64) s_bq[2 * GQ + i / D][i % D] = (_Float16)0.f;
  if (wv < GQ) {
    float x0, x1;
    rotate_row<D>(q_w, lane, x0, x1);
#pragma unroll
    for (int e = 0; e < (D == 128 ? 2 : 1); ++e) {
      const float xs = (e ? x1 : x0) * a.qscale;
      const _Float16 hi = (_Float16)xs;
      const _Float16 lo = (_Float16)(xs - (float)hi);
      const int c = rotated_channel<D>(lane, e);
      s_bq[wv][c] = hi;
      s_bq[wv + GQ][c] = lo;
    }
  }
  __syncthreads();

  const int r = lane >> 4, n = lane & 15;
  half8v bq[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) bq[s] = *reinterpret_cast<const half8v *>(&s_bq[n][r * (D / 4) + 8 * s]);
  const float lo_mask = (n >= GQ && n < 2 * GQ) ? 1.f : 0.f;

  WaveState<2 * G> st;
  st.m = kNegInf;
  st.l = 0.f;
#pragma unroll
  for (int t = 0; t < 2 * G; ++t) st.acc[t] = (float4v){0.f, 0.f, 0.f, 0.f};

  // process buffer k (if it is one of this wave's blocks), then refill it
  uint32_t *vm_slot = s_vm[wv];
  auto run = [&](Blk<D, VB> &buf, int k) {
    if (k < mine) {
      const int blk = blk0 + wv + k * NW;
      do_block<D, GQ, VB>(buf, bq, s_lut, vm_slot, st, lo_mask, lane, blk * 16 + 4 * r, T, blk == tail_blk,
                          tail_keep);
    }
    load_blk<D, VB>(buf, rec_of(k + 4), lane);
  };
#pragma unroll 1
  for (int k = 0; k < mine; k += 4) {
    run(b0, k);
    run(b1, k + 1);
    run(b2, k + 2);
    run(b3, k + 3);
  }

  finish_workgroup<D, GQ, NW, CASCADE>(a, st, b, qh0, sp, s_m, s_l, s_acc);
}

// One work-group per (sequence, query head) (grid x, y): combine the split
// partials.  Every slot below nsplit is in the row's workspace, so the first
// partials are loaded while the context length is still on its way.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const int b = blockIdx.x;
  const int64_t row = (int64_t)b * a.hq + blockIdx.y;
  merge_row_impl<D>(MergeView{a.part_ml, a.part_acc, a.out, a.nsplit, a.out_bf16}, row, a.nsplit,
                    [&]() {
                      const int nblk = (a.ctx[b] + 15) >> 4;
                      return (nblk + a.split_blocks - 1) / a.split_blocks;
                    },
                    SlotsDirect());
}

// Cascade: one work-group per (sequence, query head) combines the row's own
// splits (slots 0 .. its split count - 1) with the partials of the
// shared-block groups it is in (slot nsplit + d for the group at depth d).
template <int D>
__global__ __launch_bounds__(256) void cascade_merge_kernel(DecodeArgs a) {
  const int64_t row = blockIdx.x;
  const int b = (int)(row / a.hq);
  const int T = a.ctx[b];
  const int fb = a.first_blk[b];
  const int nblk = (T + 15) >> 4;
  const int own = nblk > fb ? (nblk - fb + a.split_blocks - 1) / a.split_blocks : 0;
  const int pre = a.depth[b];
  merge_row<D>(MergeView{a.part_ml, a.part_acc, a.out, a.part_stride, a.out_bf16}, row, own + pre,
               SlotsTwoRuns{own, a.nsplit});
}

template <int D, bool CASCADE, int VB = 4>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s) {
  const int64_t wgs = (int64_t)a.batch * a.hkv * a.nsplit;
  const dim3 grid((unsigned)wgs), block(kWaves * 64);
  switch (a.g) {
    case 1: hipLaunchKernelGGL((tq4_decode_kernel<D, 1, CASCADE, VB>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((tq4_decode_kernel<D, 2, CASCADE, VB>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((tq4_decode_kernel<D, 4, CASCADE, VB>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((tq4_decode_kernel<D, 8, CASCADE, VB>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tq4_decode(int d, int vbits, const DecodeArgs &a, hipStream_t s) {
  if (vbits == 2) return d == 128 ? launch_d<128, false, 2>(a, s) : launch_d<64, false, 2>(a, s);
  return d == 128 ? launch_d<128, false>(a, s) : launch_d<64, false>(a, s);
}

hipError_t launch_tq4_cascade_decode(int d, int vbits, const DecodeArgs &a, hipStream_t s) {
  if (vbits == 2) return d == 128 ? launch_d<128, true, 2>(a, s) : launch_d<64, true, 2>(a, s);
  return d == 128 ? launch_d<128, true>(a, s) : launch_d<64, true>(a, s);
}

hipError_t launch_cascade_merge(int d, const DecodeArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.batch * a.hq)), block(256);
  if (d == 128) hipLaunchKernelGGL(cascade_merge_kernel<128>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(cascade_merge_kernel<64>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_merge(int d, const DecodeArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)a.batch, (unsigned)a.hq), block(256);
  if (d == 128) hipLaunchKernelGGL(decode_merge_kernel<128>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(decode_merge_kernel<64>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace tq
