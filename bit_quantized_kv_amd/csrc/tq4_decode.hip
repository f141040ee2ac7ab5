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
//   * values: out^T (channels x columns) += V_hat^T P with P split into fp16
//     high and low parts, V_hat = code * scale + min consumed exactly: code *
//     scale as two exact fp16 parts on the 32-deep v_mfma_f32_16x16x32_f16
//     (k = token and part), the minimum through one v_mfma_f32_16x16x16_f16
//     of the group minima with P, added at the end.
// Split partials (max, sum, acc) go to the workspace; decode_merge combines them.
#include "decode_common.h"
#include "dequant.h"

namespace tq {
namespace {

constexpr int kWaves = 8;

// Block slots of one 16-column logit tile.  A block's logits take 2g columns
// (g query heads, each with the high and the low part of the query), so 16 /
// 2g blocks share one tile (at most 4, the depth of the load ring): their
// softmax, probability split and sums run once for all of them.
template <int GQ>
constexpr int decode_slots() {
  return GQ >= 8 ? 1 : GQ == 4 ? 2 : 4;
}

template <int N>
__device__ __forceinline__ float xor_n(float x) {
  if constexpr (N == 1) return xor1(x);
  else if constexpr (N == 2) return xor2(x);
  else if constexpr (N == 4) return xor4(x);
  else if constexpr (N == 8) return xor8(x);
  else if constexpr (N == 16) return xor16(x);
  else return xor32(x);
}

// Sum (or max) of a column's value over the SL block slots of its head: the
// lanes whose columns differ in the slot bits (column / 2g).
template <int GQ, int SL>
__device__ __forceinline__ float slot_sum(float x) {
  if constexpr (SL >= 2) x += xor_n<2 * GQ>(x);
  if constexpr (SL >= 4) x += xor_n<4 * GQ>(x);
  return x;
}
template <int GQ, int SL>
__device__ __forceinline__ float slot_max(float x) {
  if constexpr (SL >= 2) x = __builtin_fmaxf(x, xor_n<2 * GQ>(x));
  if constexpr (SL >= 4) x = __builtin_fmaxf(x, xor_n<4 * GQ>(x));
  return x;
}

// Online softmax over one tile (this lane's four logits, log2 units) with the
// lazy rescale of softmax_block; the running maximum is shared by the block
// slots of a head (raised over all of them together), so their accumulators
// add up at the end without rescaling.
template <int GQ, int SL, int NA>
__device__ __forceinline__ void softmax_tile(const float (&x)[4], WaveState<NA> &st, float (&p)[4]) {
  float lm;
  __asm__("v_max3_f32 %0, %1, %2, %3\n\tv_max_f32 %0, %0, %4"
          : "=&v"(lm)
          : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
  if (__builtin_amdgcn_ballot_w64(lm > st.m + kLazyRescale) != 0) {
    float bm = __builtin_fmaxf(lm, xor16(lm));
    bm = __builtin_fmaxf(bm, xor32(bm));
    bm = slot_max<GQ, SL>(bm);
    const bool raise = bm > st.m + kLazyRescale;
    const float m_new = raise ? bm : st.m;
    const float alpha = (st.m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int t = 0; t < NA; ++t) st.acc[t] *= alpha;
    st.m = m_new;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - st.m);
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
}

// The value (scale, min) tile of a block goes through LDS (vm_slot): lane
// (r, c) writes dword c of row r, every lane reads its row back.  `tail`:
// the (scale, min) halves of rows past the context T are cleared, so those
// rows dequantize to exactly 0 whatever the pool holds.  A block holding a scale >= 4096 gets every scale applied as
// sc * 2^-7 (rare; code * sc < 65520 then holds for every scale, and the
// split below stays exact for scales >= 2^-7).  Returns that flag.
template <int D, int VB>
__device__ __forceinline__ bool stage_vm(const Blk<D, VB> &bk, uint32_t *vm_slot, int lane, bool tail, int T) {
  constexpr int G = D / 32;
  uint32_t vmw = bk.vmw;
  if (tail) {
    // dword w of a group's 16 bytes: (sc t0, t1) (sc t2, t3) (mn t0, t1) (mn t2, t3)
    __asm__ volatile("");
    const int r0 = 4 * (lane >> 4), w = lane & 3;
    const int ta = (T & 15) - (r0 + 2 * (w & 1)), tb = ta - 1;
    vmw &= (ta > 0 ? 0x0000FFFFu : 0u) | (tb > 0 ? 0xFFFF0000u : 0u);
  }
  // lanes whose dword holds scales
  const uint32_t sc_lane = (lane & 2) ? 0u : 0xFFFFFFFFu;
  const bool big = __builtin_amdgcn_ballot_w64(has_big_scale(vmw & sc_lane) != 0) != 0;
  if (big) {
    __asm__ volatile("");
    if (sc_lane) vmw = as_u(as_h2(vmw) * (half2v){(_Float16)0x1p-7f, (_Float16)0x1p-7f});
  }
  vm_slot[(lane >> 4) * (4 * G) + (lane & (4 * G - 1))] = vmw;
  return big;
}

// P times one block's values into the output tiles.  bpj: the probabilities
// of this block's slot columns (zero on the other columns).  The minima: tile
// 2G gets sum_t mn(t, g) P(t, col) (A rows c hold group c % G, so row 4r' + i
// of the result is group i % G).  code * scale: A operand of tile (group gp,
// parity): k = 8r + j holds token 4r + (j & 3) of the lane's channel, the
// high fp16 part of code * sc for j < 4 and the low part for j >= 4; the B
// operand repeats P for both halves, so one 32-deep MFMA adds (hi + lo) * P
// = code * sc * P exactly (up to the fp32 accumulation).
template <int D, int VB>
__device__ __forceinline__ void block_values(const Blk<D, VB> &bk, const uint32_t *vm_slot, half4v bpj, bool big,
                                             WaveState<2 * D / 32 + 1> &st, int lane) {
  constexpr int G = D / 32;
  {
    const uint2 mnw = *reinterpret_cast<const uint2 *>(vm_slot + (lane >> 4) * (4 * G) + 4 * (lane & (G - 1)) + 2);
    st.acc[2 * G] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4v, mnw), bpj, st.acc[2 * G], 0, 0, 0);
  }
  if (big) {
    __asm__ volatile("");
    bpj = bpj * (half4v){(_Float16)128.f, (_Float16)128.f, (_Float16)128.f, (_Float16)128.f};
  }
  const uint4 *vm_row = reinterpret_cast<const uint4 *>(vm_slot) + (lane >> 4) * G;
  const half8v bp8 = (half8v){bpj[0], bpj[1], bpj[2], bpj[3], bpj[0], bpj[1], bpj[2], bpj[3]};
#pragma unroll
  for (int gp = 0; gp < G; ++gp) {
    const uint2 scw = *reinterpret_cast<const uint2 *>(&vm_row[gp]);
    // bytes = tokens 4r + 0..3 of one channel pair; lo / hi = the even / odd
    // channel's codes, each alone in its byte
    uint32_t lo, hi;
    value_code_bytes<VB>(VB == 4 ? word(bk.vq, gp) : word(bk.vq, gp >> 1), gp, lo, hi);
    const half2v sc01 = as_h2(scw.x), sc23 = as_h2(scw.y);
    const ScaledPair e01 = scaled_codes(codes_f16<false>(lo), sc01);
    const ScaledPair e23 = scaled_codes(codes_f16<true>(lo), sc23);
    const ScaledPair o01 = scaled_codes(codes_f16<false>(hi), sc01);
    const ScaledPair o23 = scaled_codes(codes_f16<true>(hi), sc23);
    const half8v ae = __builtin_bit_cast(half8v, make_uint4(as_u(e01.hi), as_u(e23.hi), as_u(e01.lo), as_u(e23.lo)));
    const half8v ao = __builtin_bit_cast(half8v, make_uint4(as_u(o01.hi), as_u(o23.hi), as_u(o01.lo), as_u(o23.lo)));
    st.acc[2 * gp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ae, bp8, st.acc[2 * gp], 0, 0, 0);
    st.acc[2 * gp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao, bp8, st.acc[2 * gp + 1], 0, 0, 0);
  }
}

template <int D, int GQ, bool CASCADE, int VB = 4>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void tq4_decode_kernel(
    DecodeArgs a) {
  constexpr int G = D / 32, KS = D / 32;
  constexpr int REC = TqRec<D, VB>::BYTES;
  constexpr int NW = kWaves;
  constexpr int SL = decode_slots<GQ>();  // block slots per logit tile
  constexpr int CW = 2 * GQ;              // columns per slot

  __shared__ uint32_t s_lut[256];
  __shared__ __attribute__((aligned(16))) uint32_t s_vm[NW][SL][64];
  // query operand rows, padded by 16 bytes so that the 16 columns' reads of
  // one k-step fall on different LDS banks
  __shared__ __attribute__((aligned(16))) _Float16 s_bq[16][D + 8];
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
  // every step refills its buffers unconditionally (past the end with the
  // wave's last block again, an L2 hit), so the number of loads in flight is
  // the same on every path and the waits stay partial.
  const int mine = blk1 - blk0 > wv ? (blk1 - blk0 - wv + NW - 1) / NW : 0;
  const int my_id = settled(my_id_raw);
  auto rec_of = [&](int k) {
    const int kk = k < mine ? k : mine - 1;
    return base + (int64_t)__builtin_amdgcn_readlane(my_id, kk) * stride;
  };
  // the partial last block of the sequence (its rows past the context are masked)
  const int tail_blk = (T & 15) ? nblk - 1 : nblk;
  Blk<D, VB> ring[4];
  if (mine > 0) {
    // issued block by block, as the loop's refills are, so that the
    // compiler's wait counts inside the loop stay partial on its first pass
    load_blk<D, VB>(ring[0], rec_of(0), lane);
    __asm__ volatile("" ::: "memory");
    load_blk<D, VB>(ring[1], rec_of(1), lane);
    __asm__ volatile("" ::: "memory");
    load_blk<D, VB>(ring[2], rec_of(2), lane);
    __asm__ volatile("" ::: "memory");
    load_blk<D, VB>(ring[3], rec_of(3), lane);
  }

  // ---- LUT and the rotated, scaled query group (wave w < g rotates head w) ------
  // query operand rows (tile columns): column j * 2g + h is head h's high
  // part for block slot j, column j * 2g + g + h its low part; columns past
  // the slots are zero
  if (tid < 256) s_lut[tid] = lut_w;
  for (int i = tid; i < (16 - SL * CW) * D; i += NW * 64) s_bq[SL * CW + i / D][i % D] = (_Float16)0.f;
  if (wv < GQ) {
    float x0, x1;
    rotate_row<D>(q_w, lane, x0, x1);
#pragma unroll
    for (int e = 0; e < (D == 128 ? 2 : 1); ++e) {
      const float xs = (e ? x1 : x0) * a.qscale;
      const _Float16 hi = (_Float16)xs;
      const _Float16 lo = (_Float16)(xs - (float)hi);
      const int c = rotated_channel<D>(lane, e);
#pragma unroll
      for (int j = 0; j < SL; ++j) {
        s_bq[j * CW + wv][c] = hi;
        s_bq[j * CW + GQ + wv][c] = lo;
      }
    }
  }
  __syncthreads();

  const int r = lane >> 4, n = lane & 15;
  // this lane's query operand (k-step s at bq[s]), read from LDS per block
  const half8v *bq = reinterpret_cast<const half8v *>(&s_bq[n][r * (D / 4)]);
  const int js = n / CW;  // this lane's block slot (>= SL: a column past the slots)
  const float lo_mask = (n % CW) >= GQ ? 1.f : 0.f;

  // tiles 0 .. 2G-1: out^T per (group, parity); tile 2G: the minima's product
  WaveState<2 * G + 1> st;
  st.m = kNegInf;
  st.l = 0.f;
#pragma unroll
  for (int t = 0; t < 2 * G + 1; ++t) st.acc[t] = (float4v){0.f, 0.f, 0.f, 0.f};
  // one tile: ring buffers j0 .. j0 + SL - 1 hold the wave's blocks k .. k +
  // SL - 1 (those past `mine` are not its blocks); then every buffer of the
  // tile is refilled with the block four further on
  auto tile = [&](int j0, int k) {
    float4v qk[SL];
    bool big[SL];
    // the query operand, read once for the tile's blocks
    half8v bqr[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) bqr[s] = bq[s];
#pragma unroll
    for (int j = 0; j < SL; ++j) {
      qk[j] = (float4v){0.f, 0.f, 0.f, 0.f};
      big[j] = false;
      if (k + j < mine) {
        const int blk = blk0 + wv + (k + j) * NW;
        big[j] = stage_vm<D, VB>(ring[j0 + j], s_vm[wv][j], lane, blk == tail_blk, T);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const uint4 e = key_entries(s_lut, word(ring[j0 + j].kq, s));
          qk[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8v, e), bqr[s], qk[j], 0, 0, 0);
        }
      }
    }
    // this lane's slot: its logits and key scales
    float4v q = qk[0];
    uint2 ks = ring[j0].ks;
#pragma unroll
    for (int j = 1; j < SL; ++j) {
      if (js == j) {
        q = qk[j];
        ks = ring[j0 + j].ks;
      }
    }
    const half2v s01 = as_h2(ks.x), s23 = as_h2(ks.y);
    // logit = (high + low column) * key scale, one v_fma_mix each (the fp16
    // scale taken directly; the +0 addend only turns a -0 product into +0)
    float x[4];
    x[0] = __builtin_fmaf(q[0] + xor_g<GQ>(q[0]), (float)s01[0], 0.0f);
    x[1] = __builtin_fmaf(q[1] + xor_g<GQ>(q[1]), (float)s01[1], 0.0f);
    x[2] = __builtin_fmaf(q[2] + xor_g<GQ>(q[2]), (float)s23[0], 0.0f);
    x[3] = __builtin_fmaf(q[3] + xor_g<GQ>(q[3]), (float)s23[1], 0.0f);
    // a slot past the wave's blocks, or the partial last block of the
    // sequence: the rows past the context get -inf (a wave-uniform test first)
    const int kl = k + SL - 1;
    if (kl >= mine || blk0 + wv + kl * NW >= tail_blk) {
      __asm__ volatile("");
      const int kj = k + (js < SL ? js : 0);
      const int tok0 = (blk0 + wv + kj * NW) * 16 + 4 * r;
      const bool none = kj >= mine || js >= SL;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (none || tok0 + i >= T) x[i] = kNegInf;
    }
    float p[4];
    softmax_tile<GQ, SL>(x, st, p);
    // B operand: tokens 4r + 0..3 in k order; high part on the slot's first
    // g columns, low part (p - high) on its next g
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
#pragma unroll
    for (int j = 0; j < SL; ++j) {
      if (k + j < mine) {
        // the lane's probabilities are kept on its own slot's columns only
        const uint2 w = __builtin_bit_cast(uint2, bp);
        const half4v bpj = __builtin_bit_cast(half4v, js == j ? w : make_uint2(0u, 0u));
        block_values<D, VB>(ring[j0 + j], s_vm[wv][j], bpj, big[j], st, lane);
      }
    }
#pragma unroll
    for (int j = 0; j < SL; ++j) load_blk<D, VB>(ring[j0 + j], rec_of(k + j + 4), lane);
  };
#pragma unroll 1
  for (int k = 0; k < mine; k += 4) {
#pragma unroll
    for (int j0 = 0; j0 < 4; j0 += SL) tile(j0, k + j0);
  }

  // the slots of a head add up (one running maximum), then the minima's
  // contribution goes to every channel of their group
  st.l = slot_sum<GQ, SL>(st.l);
#pragma unroll
  for (int t = 0; t < 2 * G + 1; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st.acc[t][i] = slot_sum<GQ, SL>(st.acc[t][i]);
  }
#pragma unroll
  for (int gp = 0; gp < G; ++gp) {
    st.acc[2 * gp] += st.acc[2 * G][gp];
    st.acc[2 * gp + 1] += st.acc[2 * G][gp];
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
