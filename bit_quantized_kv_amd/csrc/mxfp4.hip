// MX-FP4 path for gfx950: FP4 (e2m1) keys and values with one UE8M0 exponent
// per 32 channels, FP8 (e4m3) queries, QK on the scaled MFMA.
//
// "UltraQuant：4-bit KV 快取加速長代理", section "方法怎麼做，白話講": FP8
// queries, FP4 KV tensors and UE8M0 group scales, with dequantization absorbed
// into CDNA4's native scaled MFMA; keys keep the Walsh-Hadamard rotation.  The
// conversion rules (OCP MX) and the record layout are stated in tq.h.
//
// Quantize: as the TQ4/4 kernel, with the rotated key y = fp32(x * fp32(1/sqrt(D)))
// and per-group X = floor(log2(amax)) - 2; v_cvt_scalef32_pk_fp4_f32 gives
// e2m1_RNE(value / 2^X) (ties to even, saturating, sign kept) two at a time.
//
// Decode: logits = K (FP4, A operand: lane = token row and one 32-channel
// group, its own UE8M0 byte as the A scale) times q8 (FP8, B operand; lane
// group gb carries channels 16gb..+15 and 64+16gb..+15) with
// v_mfma_scale_f32_16x16x128_f8f6f4, one instruction per 16-token block.
// Values are dequantized to bf16 exactly (v_cvt_scalef32_pk_bf16_fp4 with the
// scale 2^X: an e2m1 element times 2^X has two significant bits, and bf16 has
// the fp32 exponent range) and PV runs on v_mfma_f32_16x16x16_bf16 with P
// split into bf16 high and low parts (16 significant bits).
#include "decode_common.h"
#include "dequant.h"
#include "quant_common.h"

namespace tq {
namespace {

constexpr int kD = 128, kG = 4, kRec = MxRec::BYTES;
constexpr int kOffKc = MxRec::KC, kOffKs = MxRec::KS, kOffVc = MxRec::VC, kOffVs = MxRec::VS;

// ---- quantize -----------------------------------------------------------------

// Shared exponent and e2m1 codes of one lane's 16 values (two words, channel
// e in nibble e % 8 of word e / 8); the group's amax is reduced over the two
// lanes of a 32-channel group (lane ^ 1).  Keys (KEY): y = fp32(z * mul) with
// mul = 1/sqrt(D) times the butterflies' sign, computed as fma(z, mul, +0) so
// that an exact zero is +0 (the record format stores rotated zeros as +0);
// values are encoded as they are, zero signs kept.
template <bool KEY>
__device__ __forceinline__ uint2 mx_encode16(const float (&y)[16], float mul, int &xexp) {
  float t[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) t[e] = KEY ? __builtin_fmaf(y[e], mul, 0.0f) : y[e];
  float am = __builtin_fabsf(t[0]);
#pragma unroll
  for (int e = 1; e < 16; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(t[e]));
  am = __builtin_fmaxf(am, xor1(am));
  int x = -127;
  if (am > 0.f) x = __builtin_amdgcn_frexp_expf(am) - 1 - 2;  // floor(log2 amax) - 2
  x = x < -127 ? -127 : (x > 127 ? 127 : x);
  xexp = x;
  // 2^-127 is not a normal fp32 scale: pre-multiply by 2^127 instead (exact;
  // only tiny groups take this path)
  float scale = as_f((uint32_t)(x + 127) << 23);
  if (x == -127) {
#pragma unroll
    for (int e = 0; e < 16; ++e) t[e] *= 0x1p127f;
    scale = 1.0f;
  }
  uint2 w = make_uint2(0, 0);
#define TQ_CVT(J)                                                                                    \
  w.x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w.x, t[2 * J], t[2 * J + 1], scale, J);               \
  w.y = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w.y, t[8 + 2 * J], t[9 + 2 * J], scale, J);
  TQ_CVT(0)
  TQ_CVT(1)
  TQ_CVT(2)
  TQ_CVT(3)
#undef TQ_CVT
  return w;
}

// Quantize one token row (keys rotated, both MX-FP4) into its record.
__device__ __forceinline__ void mx_quantize_row(const QuantizeArgs &a, const RowLoad<kD> &cur, int h, int lane,
                                                int li, int tq, float ksign) {
  constexpr int Q = kD / 8;
  const int slot = cur.valid ? cur.slot : -1;
  float z[16], v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t kw = kword<kD>(cur, i), vw = vword<kD>(cur, i);
    z[2 * i] = bf16_lo(kw);
    z[2 * i + 1] = bf16_hi(kw);
    v[2 * i] = bf16_lo(vw);
    v[2 * i + 1] = bf16_hi(vw);
  }
  wht16<kD>(z, lane);
  int kx, vx;
  const uint2 kc = mx_encode16<true>(z, ksign, kx);  // y = fp32(x * fp32(1/sqrt(D)))
  const uint2 vc = mx_encode16<false>(v, 1.0f, vx);

  const bool aligned = quad_aligned<kD>(slot, tq);
  const uint32_t vt0 = quad_transpose<kD>(vc.x, tq), vt1 = quad_transpose<kD>(vc.y, tq);
  // the quad's four value exponents as one dword [t0, t1, t2, t3]
  const uint32_t xb = (uint32_t)(vx + 127) & 0xFFu;
  const uint32_t xp1 = tok_xor1(xb);
  const uint32_t pr = (tq & 1) ? (xp1 | (xb << 8)) : (xb | (xp1 << 8));
  const uint32_t xp2 = tok_xor2<kD>(pr);
  const uint32_t xq = (tq & 2) ? (xp2 | (pr << 16)) : (pr | (xp2 << 16));
  if (slot < 0) return;
  const int64_t blk = slot >> 4;
  const int t = slot & 15;
  uint8_t *rec = a.pool + ((int64_t)blk * a.hkv + h) * kRec;
  const int p0 = 8 * li;
  *reinterpret_cast<uint2 *>(rec + kOffKc + ((p0 / Q) * 16 + t) * Q + p0 % Q) = kc;
  const int r = t >> 2, gp = li >> 1, j0 = 8 * (li & 1);
  if ((li & 1) == 0) rec[kOffKs + gp * 16 + t] = (uint8_t)(kx + 127);
  if (aligned) {
    *reinterpret_cast<uint32_t *>(rec + kOffVc + ((r * 16 + j0 + tq) * kG + gp) * 4) = vt0;
    *reinterpret_cast<uint32_t *>(rec + kOffVc + ((r * 16 + j0 + 4 + tq) * kG + gp) * 4) = vt1;
    if ((li & 1) == 0 && tq == 0) *reinterpret_cast<uint32_t *>(rec + kOffVs + (r * kG + gp) * 4) = xq;
  } else {
    const int tt = t & 3;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      rec[kOffVc + ((r * 16 + j0 + k) * kG + gp) * 4 + tt] = (uint8_t)((k < 4 ? vc.x : vc.y) >> (8 * (k & 3)));
    if ((li & 1) == 0) rec[kOffVs + (r * kG + gp) * 4 + tt] = (uint8_t)xb;
  }
}

template <bool BAL>
__global__ __launch_bounds__(BAL ? kQuantThreadsBal : kQuantThreads) void mxfp4_quantize_kernel(QuantizeArgs a) {
  using L = QLanes<kD>;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = L::li(lane), tw = L::tw(lane), tq = tw & 3;
  // keys leave the butterflies with the sign (-1)^popcount(li); folding it into
  // the 1/sqrt(D) factor is exact
  const float ksign = a.rsqrt_d * wht16_sign(li);
  quantize_loop<kD, BAL>(a, wv, tw, li, [] {},
                    [&](const RowLoad<kD> &row, int h) { mx_quantize_row(a, row, h, lane, li, tq, ksign); });
}

// ---- decode -------------------------------------------------------------------

constexpr int kWaves = 8;

// OCP e4m3fn encode of an fp32 value: round to nearest even on the binade
// grid (spacing 2^(e-3), 2^-9 below 2^-6), saturating to +-448.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const float a = __builtin_fminf(__builtin_fabsf(y), 448.f);
  uint32_t code;
  if (a < 0x1p-6f) {
    code = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    int e = (int)(as_u(a) >> 23) - 127;
    const float m = a * as_f((uint32_t)(127 - e) << 23);  // a / 2^e, exact
    float q = __builtin_rintf(m * 8.f);
    if (q == 16.f) {
      ++e;
      q = 8.f;
    }
    code = ((uint32_t)(e + 7) << 3) | (uint32_t)((int)q - 8);
  }
  return code | ((as_u(y) >> 24) & 0x80u);
}

struct Blk4 {
  uint4 kq;       // e2m1 key codes: this lane's 32 channels of one token
  uint32_t ksb;   // UE8M0 byte of (token lane % 16, group lane / 16)
  uint4 vq;       // e2m1 value codes, laid out as in the TQ4/4 record
  uint32_t vsw;   // one dword of the value exponent tile (lane (r, c): dword c & 3 of row r)
};

__device__ __forceinline__ void load_blk4(Blk4 &o, const uint8_t *rec, int lane) {
  const int r = lane >> 4, c = lane & 15;
  o.kq = *reinterpret_cast<const uint4 *>(rec + kOffKc + lane * 16);
  o.ksb = rec[kOffKs + lane];
  o.vq = *reinterpret_cast<const uint4 *>(rec + kOffVc + lane * 16);
  o.vsw = reinterpret_cast<const uint32_t *>(rec + kOffVs)[4 * r + (c & 3)];
}

__device__ __forceinline__ uint32_t word4(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// tail: the partial last block of its sequence (rows past the context masked).
template <int GQ>
__device__ __forceinline__ void do_block4(const Blk4 &bk, const int8v &bq8, uint32_t *vs_slot, WaveState<8> &st,
                                          float qscale, float lo_mask, int lane, int tok0, int T, bool tail,
                                          uint32_t vs_keep) {
  // exponent bytes of rows past the context are cleared (those rows then
  // dequantize to exactly 0), at the use so no early wait on the loads is
  // forced; the tail fix-ups sit behind real branches
  uint32_t vsw = bk.vsw;
  if (tail) {
    __asm__ volatile("");
    vsw &= vs_keep;
  }
  vs_slot[(lane >> 4) * 4 + (lane & 3)] = vsw;
  // ---- logits: one scaled MFMA per block ------------------------------------------
  const int8v ak = (int8v){(int)bk.kq.x, (int)bk.kq.y, (int)bk.kq.z, (int)bk.kq.w, 0, 0, 0, 0};
  float4v qk = (float4v){0.f, 0.f, 0.f, 0.f};
  qk = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ak, bq8, qk, 4, 0, 0, (int)bk.ksb, 0, 127);
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = qk[i] * qscale;
  if (tail) {
    __asm__ volatile("");
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (tok0 + i >= T) x[i] = kNegInf;
  }
  float p[4];
  softmax_block<8>(x, st, p);
  // B operand: tokens in the order 0, 2, 1, 3 (the A operand's order below);
  // bf16 high part on columns < g, bf16 low part (p - high, exact, then
  // rounded to nearest) on columns g .. 2g-1
  bf16x4v bp;
  {
    const uint32_t h02 = prob_hi_bf16(p[0], p[2]), h13 = prob_hi_bf16(p[1], p[3]);
    const uint32_t a02 = prob_part_bf16(h02, p[0], p[2], lo_mask);
    const uint32_t a13 = prob_part_bf16(h13, p[1], p[3], lo_mask);
    bp = __builtin_bit_cast(bf16x4v, make_uint2(a02, a13));
  }
  // ---- values: exact bf16 dequantization, then PV on bf16 MFMA --------------------
  const uint4 vs = reinterpret_cast<const uint4 *>(vs_slot)[lane >> 4];
#pragma unroll
  for (int gp = 0; gp < kG; ++gp) {
    const uint32_t w = word4(bk.vq, gp);
    const uint32_t xs = word4(vs, gp);  // exponent bytes of tokens 4r + 0..3
    const uint32_t h0 = fp4_pair_bf16<0>(w, ue8m0_scale(xs & 0xFFu));
    const uint32_t h1 = fp4_pair_bf16<1>(w, ue8m0_scale((xs >> 8) & 0xFFu));
    const uint32_t h2 = fp4_pair_bf16<2>(w, ue8m0_scale((xs >> 16) & 0xFFu));
    const uint32_t h3 = fp4_pair_bf16<3>(w, ue8m0_scale(xs >> 24));
    const uint32_t e02 = __builtin_amdgcn_perm(h2, h0, 0x05040100u), o02 = __builtin_amdgcn_perm(h2, h0, 0x07060302u);
    const uint32_t e13 = __builtin_amdgcn_perm(h3, h1, 0x05040100u), o13 = __builtin_amdgcn_perm(h3, h1, 0x07060302u);
    const bf16x4v ae = __builtin_bit_cast(bf16x4v, make_uint2(e02, e13));
    const bf16x4v ao = __builtin_bit_cast(bf16x4v, make_uint2(o02, o13));
    st.acc[2 * gp] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ae, bp, st.acc[2 * gp], 0, 0, 0);
    st.acc[2 * gp + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ao, bp, st.acc[2 * gp + 1], 0, 0, 0);
  }
}

// CASCADE: the own-token pass of cascade decode (the splits start at the
// sequence's first block of its own; always split partials, at slot sp of
// rows of a.part_stride slots).
template <int GQ, bool CASCADE>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void mxfp4_decode_kernel(
    DecodeArgs a) {
  constexpr int NW = kWaves;
  __shared__ __attribute__((aligned(16))) uint32_t s_vs[NW][16];
  __shared__ __attribute__((aligned(16))) uint8_t s_q8[16][kD];
  __shared__ float s_m[NW][GQ], s_l[NW][GQ];
  __shared__ float s_acc[NW][GQ][kD];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const WgTask task = decode_task(a);
  const int b = task.b, kvh = task.kvh, sp = task.sp;
  const int qh0 = kvh * GQ;
  const int T = a.ctx[b];  // a scalar load: nothing is written before it
  // this wave's block ids, fetched before the context length is known (index
  // clamped into the table row; entries past the context are never used)
  const int blk0 = (CASCADE ? a.first_blk[b] : 0) + sp * a.split_blocks;
  const int32_t *btab = a.block_table + (int64_t)b * a.max_blocks;
  const int my_id_raw = btab[min(blk0 + wv + lane * NW, a.max_blocks - 1)];
  // the query word next: it completes while the block ids are fetched
  const uint32_t q_w = wv < GQ ? load_query_word<kD>(a.q + ((int64_t)b * a.hq + qh0 + wv) * kD, lane) : 0u;
  __asm__ volatile("" ::: "memory");
  const int nblk = (T + 15) >> 4;
  if (nblk == 0) {
    if (!CASCADE && a.nsplit == 1 && sp == 0) write_zero_rows<kD>(a, b, qh0, GQ);
    return;
  }
  if (blk0 >= nblk) return;
  const int blk1 = min(nblk, blk0 + a.split_blocks);

  const uint8_t *base = a.pool + (int64_t)kvh * kRec;
  const int64_t stride = (int64_t)a.hkv * kRec;
  const int mine = blk1 - blk0 > wv ? (blk1 - blk0 - wv + NW - 1) / NW : 0;
  const int my_id = settled(my_id_raw);
  auto rec_of = [&](int k) {
    const int kk = k < mine ? k : mine - 1;
    return base + (int64_t)__builtin_amdgcn_readlane(my_id, kk) * stride;
  };
  const int tail_blk = (T & 15) ? nblk - 1 : nblk;
  uint32_t tail_keep = 0;
  {
    const int r0 = 4 * (lane >> 4), rem = (T & 15) - r0;  // exponent bytes: tokens r0 + 0..3
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) tail_keep |= (rem > tt ? 0xFFu : 0u) << (8 * tt);
  }
  Blk4 b0, b1, b2, b3;
  if (mine > 0) {
    // issued block by block, as the loop's refills are, so that the
    // compiler's wait counts inside the loop stay partial on its first pass
    load_blk4(b0, rec_of(0), lane);
    __asm__ volatile("" ::: "memory");
    load_blk4(b1, rec_of(1), lane);
    __asm__ volatile("" ::: "memory");
    load_blk4(b2, rec_of(2), lane);
    __asm__ volatile("" ::: "memory");
    load_blk4(b3, rec_of(3), lane);
  }

  // ---- the query group as e4m3 bytes: rows h and g + h both hold head h --------
  for (int i = tid; i < (16 - 2 * GQ) * kD; i += NW * 64) s_q8[2 * GQ + i / kD][i % kD] = 0;
  if (wv < GQ) {
    float x0, x1;
    rotate_row<kD>(q_w, lane, x0, x1);
    const uint32_t c0 = e4m3_rne(x0 * a.rsqrt_d), c1 = e4m3_rne(x1 * a.rsqrt_d);
    s_q8[wv][2 * lane] = (uint8_t)c0;
    s_q8[wv][2 * lane + 1] = (uint8_t)c1;
    s_q8[wv + GQ][2 * lane] = (uint8_t)c0;
    s_q8[wv + GQ][2 * lane + 1] = (uint8_t)c1;
  }
  __syncthreads();
  const int r = lane >> 4, n = lane & 15;
  int8v bq8;
  {
    const uint4 lo = *reinterpret_cast<const uint4 *>(&s_q8[n][16 * r]);
    const uint4 hi = *reinterpret_cast<const uint4 *>(&s_q8[n][64 + 16 * r]);
    bq8 = (int8v){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  const float lo_mask = (n >= GQ && n < 2 * GQ) ? 1.f : 0.f;

  WaveState<8> st;
  st.m = kNegInf;
  st.l = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) st.acc[t] = (float4v){0.f, 0.f, 0.f, 0.f};
  uint32_t *vs_slot = s_vs[wv];
  auto run = [&](Blk4 &buf, int k) {
    if (k < mine) {
      const int blk = blk0 + wv + k * NW;
      do_block4<GQ>(buf, bq8, vs_slot, st, a.qscale, lo_mask, lane, blk * 16 + 4 * r, T, blk == tail_blk, tail_keep);
    }
    load_blk4(buf, rec_of(k + 4), lane);
  };
#pragma unroll 1
  for (int k = 0; k < mine; k += 4) {
    run(b0, k);
    run(b1, k + 1);
    run(b2, k + 2);
    run(b3, k + 3);
  }
  // the low-part columns are real columns here too: combine as in TQ4/4
  finish_workgroup<kD, GQ, NW, CASCADE>(a, st, b, qh0, sp, s_m, s_l, s_acc);
}

// ---- multi-token attention ------------------------------------------------------
// Several query tokens per sequence (chunked prefill, verification), and the
// shared-block pass of cascade decode, over MX-FP4 records.  Rows are (query
// token, query head) pairs of one kv-head, token-major, with the causal limits,
// row tiles and partial slots of the TQ4/4 multi-token kernels.  A work-group
// of kMtWavesMx waves takes 16 RT rows (row tile rt) and one split of the key
// blocks (at most 64 per wave: lane k holds the id of the wave's k-th block);
// wave w takes every NW-th block of the split, four blocks of loads in flight,
// and runs all its rows against each block:
//   * logits: one scaled MFMA per 16 rows, the keys as the A operand (e2m1,
//     the token's UE8M0 byte per 32 channels as the A scale), the rows' e4m3
//     rotated queries as the B operand;
//   * online softmax per row with its causal limit (the running maximum starts
//     finite, so a row that sees no token yet gets p = 0);
//   * out^T += V_hat^T P on v_mfma_f32_16x16x32_bf16, k = token and part: the
//     values exact in bf16 (e2m1 * 2^X) in both halves of the A operand, P as
//     its bf16 high part and the bf16 rounding of p - high (exact) in the B
//     operand, so every p enters with 16 significant bits.
// The waves' states merge in LDS by halving rounds; wave 0 writes the rows or
// their split partials.  PREFIX: the rows are the (member, head) pairs of one
// group, every row sees the group's blocks, and the results are partials at
// slot slot0 + the group's depth.
constexpr int kMtWavesMx = 4;
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

template <int RT, bool PREFIX>
__global__ __launch_bounds__(kMtWavesMx * 64) __attribute__((amdgpu_waves_per_eu(2))) void mxfp4_mt_kernel(
    MultiTokenArgs a) {
  constexpr int NW = kMtWavesMx;
  constexpr int NT = kD / 16;  // output tiles: (group, channel parity)
  constexpr int QJ = 16 * RT / NW;  // query rows staged per wave
  __shared__ __attribute__((aligned(16))) uint32_t s_vs[NW][16];
  // the rows' e4m3 queries, then the wave-merge area
  constexpr size_t kQBytes = (size_t)RT * 16 * kD;
  constexpr size_t kMBytes = (size_t)(NW / 2) * RT * NT * 64 * sizeof(float4v);
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[kQBytes > kMBytes ? kQBytes : kMBytes];
  __shared__ float s_wm[NW / 2][RT][16], s_wl[NW / 2][RT][16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const MtTask task = mt_task(a);
  const int b = task.b, kvh = task.kvh, sp = task.sp;
  // causal: b is a sequence with query tokens q0 .. q0 + M - 1, the last of
  // which sees all T keys; prefix: b is a group, q0 its first member's index
  // into group_seqs, M its size, and every row sees blocks blk_lo .. T/16 - 1
  int q0, M, T, tab_seq, blk_lo = 0, slot = sp;
  if constexpr (PREFIX) {
    q0 = a.group_start[b];
    M = a.group_start[b + 1] - q0;
    if (M <= 0) return;
    tab_seq = a.group_seqs[q0];
    blk_lo = a.group_blocks[2 * b];
    T = 16 * a.group_blocks[2 * b + 1];
    slot = a.slot0 + a.group_depth[b];
  } else {
    q0 = a.q_start[b];
    M = a.q_start[b + 1] - q0;
    T = a.ctx[b];
    tab_seq = b;
  }
  const int R = M * a.g;
  const int row0 = 16 * RT * task.rt;
  if (row0 >= R) return;
  const int nrow = min(R - row0, 16 * RT);
  auto q_row = [&](int row) -> int64_t {
    const int who = row / a.g, j = row % a.g;
    const int64_t tok = PREFIX ? (int64_t)a.group_seqs[q0 + who] : (int64_t)(q0 + who);
    return tok * a.hq + kvh * a.g + j;
  };
  const int nblk = (T + 15) >> 4;
  const int blk0 = blk_lo + sp * a.split_blocks;
  if (blk0 >= nblk) {
    if constexpr (PREFIX) {
      // an empty group range: empty partials (max -inf, sum 0), which the
      // merge weighs 0
      for (int i = tid; i < nrow * (kD + 2); i += NW * 64) {
        const int64_t pi = q_row(row0 + i / (kD + 2)) * a.part_stride + slot;
        const int c = i % (kD + 2);
        if (c < kD) a.part_acc[pi * kD + c] = 0.f;
        else a.part_ml[pi * 2 + (c - kD)] = c == kD ? kNegInf : 0.f;
      }
    }
    return;
  }
  const int blk1 = min(nblk, blk0 + a.split_blocks);
  // the tile's smallest visible-key count: blocks below it need no mask
  const int lmin = PREFIX ? T : T - M + 1 + row0 / a.g;

  const int r = lane >> 4, n = lane & 15;
  int lim[RT];  // this lane's column's visible-key count in tile t (0: no row)
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int row = row0 + 16 * t + n;
    lim[t] = row < R ? (PREFIX ? T : T - M + row / a.g + 1) : 0;
  }

  // ---- block ids, query words, the first loads --------------------------------------
  const int32_t *btab = a.block_table + (int64_t)tab_seq * a.max_blocks;
  const int my_id_raw = btab[min(blk0 + wv + lane * NW, a.max_blocks - 1)];
  uint32_t qw[QJ];  // rows wv + j NW of the tile
#pragma unroll
  for (int j = 0; j < QJ; ++j) qw[j] = load_query_word<kD>(a.q + q_row(min(row0 + wv + j * NW, R - 1)) * kD, lane);
  __asm__ volatile("" ::: "memory");
  const uint8_t *base = a.pool + (int64_t)kvh * kRec;
  const int64_t stride = (int64_t)a.hkv * kRec;
  const int mine = blk1 - blk0 > wv ? (blk1 - blk0 - wv + NW - 1) / NW : 0;
  const int my_id = settled(my_id_raw);
  // block k of this wave (k >= mine: its last block again, an L2 hit); only
  // called when mine > 0
  auto rec_of = [&](int k) {
    const int kk = k < mine ? k : mine - 1;
    return base + (int64_t)__builtin_amdgcn_readlane(my_id, kk) * stride;
  };
  const int tail_blk = (T & 15) ? nblk - 1 : nblk;
  uint32_t tail_keep = 0;  // exponent bytes of tokens 4r + 0..3 inside the context
  {
    const int rem = (T & 15) - 4 * r;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) tail_keep |= (rem > tt ? 0xFFu : 0u) << (8 * tt);
  }
  Blk4 b0, b1, b2, b3;
  if (mine > 0) {
    load_blk4(b0, rec_of(0), lane);
    __asm__ volatile("" ::: "memory");
    load_blk4(b1, rec_of(1), lane);
    __asm__ volatile("" ::: "memory");
    load_blk4(b2, rec_of(2), lane);
    __asm__ volatile("" ::: "memory");
    load_blk4(b3, rec_of(3), lane);
  }

  // ---- the rows' rotated queries as e4m3 bytes (rows past R: zero) ------------------
  uint8_t(*s_q8)[kD] = reinterpret_cast<uint8_t(*)[kD]>(s_buf);
#pragma unroll
  for (int j = 0; j < QJ; ++j) {
    const int i = wv + j * NW;
    float x0, x1;
    rotate_row<kD>(qw[j], lane, x0, x1);
    const bool live = row0 + i < R;
    const uint32_t c0 = live ? e4m3_rne(x0 * a.rsqrt_d) : 0u, c1 = live ? e4m3_rne(x1 * a.rsqrt_d) : 0u;
    reinterpret_cast<uint16_t *>(s_q8[i])[lane] = (uint16_t)(c0 | (c1 << 8));
  }
  __syncthreads();
  int8v bq8[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const uint4 lo = *reinterpret_cast<const uint4 *>(&s_q8[16 * t + n][16 * r]);
    const uint4 hi = *reinterpret_cast<const uint4 *>(&s_q8[16 * t + n][64 + 16 * r]);
    bq8[t] = (int8v){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }

  WaveState<NT> st[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    st[t].m = kMtFloor;
    st[t].l = 0.f;
#pragma unroll
    for (int c = 0; c < NT; ++c) st[t].acc[c] = (float4v){0.f, 0.f, 0.f, 0.f};
  }
  uint32_t *vs_slot = s_vs[wv];
  auto block = [&](const Blk4 &bk, int k) {
    const int blk = blk0 + wv + k * NW;
    const int tok0 = 16 * blk + 4 * r;
    // exponent bytes of rows past the context are cleared (those rows then
    // dequantize to finite values whatever the pool holds; their p is 0)
    uint32_t vsw = bk.vsw;
    if (blk == tail_blk) {
      __asm__ volatile("");
      vsw &= tail_keep;
    }
    vs_slot[r * 4 + (lane & 3)] = vsw;
    const int8v ak = (int8v){(int)bk.kq.x, (int)bk.kq.y, (int)bk.kq.z, (int)bk.kq.w, 0, 0, 0, 0};
    const bool masked = 16 * blk + 16 > lmin;
    bf16x8v bp[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      float4v qk = (float4v){0.f, 0.f, 0.f, 0.f};
      qk = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ak, bq8[t], qk, 4, 0, 0, (int)bk.ksb, 0, 127);
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = qk[i] * a.qscale;
      if (masked) {
        __asm__ volatile("");
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + i >= lim[t]) x[i] = kNegInf;
      }
      float p[4];
      softmax_block<NT>(x, st[t], p);
      // k = 8r + j: tokens 4r + (0, 2, 1, 3) for j = 0..3 (high parts), the
      // same tokens' low parts for j = 4..7
      const uint32_t h02 = prob_hi_bf16(p[0], p[2]), h13 = prob_hi_bf16(p[1], p[3]);
      const uint32_t l02 = prob_part_bf16(h02, p[0], p[2], 1.f), l13 = prob_part_bf16(h13, p[1], p[3], 1.f);
      bp[t] = __builtin_bit_cast(bf16x8v, make_uint4(h02, h13, l02, l13));
    }
    const uint4 vs = reinterpret_cast<const uint4 *>(vs_slot)[r];
#pragma unroll
    for (int gp = 0; gp < kG; ++gp) {
      const uint32_t w = word4(bk.vq, gp);
      const uint32_t xs = word4(vs, gp);  // exponent bytes of tokens 4r + 0..3
      const uint32_t h0 = fp4_pair_bf16<0>(w, ue8m0_scale(xs & 0xFFu));
      const uint32_t h1 = fp4_pair_bf16<1>(w, ue8m0_scale((xs >> 8) & 0xFFu));
      const uint32_t h2 = fp4_pair_bf16<2>(w, ue8m0_scale((xs >> 16) & 0xFFu));
      const uint32_t h3 = fp4_pair_bf16<3>(w, ue8m0_scale(xs >> 24));
      const uint32_t e02 = __builtin_amdgcn_perm(h2, h0, 0x05040100u), o02 = __builtin_amdgcn_perm(h2, h0, 0x07060302u);
      const uint32_t e13 = __builtin_amdgcn_perm(h3, h1, 0x05040100u), o13 = __builtin_amdgcn_perm(h3, h1, 0x07060302u);
      const bf16x8v ae = __builtin_bit_cast(bf16x8v, make_uint4(e02, e13, e02, e13));
      const bf16x8v ao = __builtin_bit_cast(bf16x8v, make_uint4(o02, o13, o02, o13));
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        st[t].acc[2 * gp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ae, bp[t], st[t].acc[2 * gp], 0, 0, 0);
        st[t].acc[2 * gp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, bp[t], st[t].acc[2 * gp + 1], 0, 0, 0);
      }
    }
  };
  auto run = [&](Blk4 &buf, int k) {
    if (k < mine) block(buf, k);
    load_blk4(buf, rec_of(k + 4), lane);
  };
#pragma unroll 1
  for (int k = 0; k < mine; k += 4) {
    run(b0, k);
    run(b1, k + 1);
    run(b2, k + 2);
    run(b3, k + 3);
  }

  // ---- merge the waves' states: halving rounds through LDS ------------------------
  float l[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    l[t] = st[t].l;
    l[t] += xor16(l[t]);
    l[t] += xor32(l[t]);
  }
  float4v(*s_fa)[RT][NT][64] = reinterpret_cast<float4v(*)[RT][NT][64]>(s_buf);
#pragma unroll 1
  for (int h = NW / 2; h >= 1; h >>= 1) {
    __syncthreads();  // the area is free (queries read, or the last round's reads done)
    if (wv >= h && wv < 2 * h) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int c = 0; c < NT; ++c) s_fa[wv - h][t][c][lane] = st[t].acc[c];
        if (r == 0) {
          s_wm[wv - h][t][n] = st[t].m;
          s_wl[wv - h][t][n] = l[t];
        }
      }
    }
    __syncthreads();
    if (wv < h) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const float m2 = s_wm[wv][t][n];
        const float mx = __builtin_fmaxf(st[t].m, m2);
        const float f1 = __builtin_amdgcn_exp2f(st[t].m - mx), f2 = __builtin_amdgcn_exp2f(m2 - mx);
        l[t] = l[t] * f1 + s_wl[wv][t][n] * f2;
#pragma unroll
        for (int c = 0; c < NT; ++c) st[t].acc[c] = st[t].acc[c] * f1 + s_fa[wv][t][c][lane] * f2;
        st[t].m = mx;
      }
    }
  }
  if (wv != 0) return;

  // ---- wave 0 writes the rows: output, or the split partial --------------------------
  // lane (r, n) of tile (gp, parity) holds channels 32 gp + 8 r + 2 i + parity
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int row = row0 + 16 * t + n;
    if (row >= R) continue;
    const int64_t orow = q_row(row);
    if (!PREFIX && a.nsplit == 1) {
      const float inv = l[t] > 0.f ? 1.f / l[t] : 0.f;
#pragma unroll
      for (int gp = 0; gp < kG; ++gp) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[2 * i] = st[t].acc[2 * gp][i] * inv;
          o[2 * i + 1] = st[t].acc[2 * gp + 1][i] * inv;
        }
        const int64_t oi = orow * kD + 32 * gp + 8 * r;
        if (a.out_bf16) {
          uint4 w;
          w.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
          w.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
          w.z = (uint32_t)f32_to_bf16(o[4]) | ((uint32_t)f32_to_bf16(o[5]) << 16);
          w.w = (uint32_t)f32_to_bf16(o[6]) | ((uint32_t)f32_to_bf16(o[7]) << 16);
          *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.out) + oi) = w;
        } else {
          float4 *dst = reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + oi);
          dst[0] = make_float4(o[0], o[1], o[2], o[3]);
          dst[1] = make_float4(o[4], o[5], o[6], o[7]);
        }
      }
    } else {
      const int64_t pi = orow * a.part_stride + slot;
#pragma unroll
      for (int gp = 0; gp < kG; ++gp) {
        float4 *dst = reinterpret_cast<float4 *>(a.part_acc + pi * kD + 32 * gp + 8 * r);
        dst[0] = make_float4(st[t].acc[2 * gp][0], st[t].acc[2 * gp + 1][0], st[t].acc[2 * gp][1],
                             st[t].acc[2 * gp + 1][1]);
        dst[1] = make_float4(st[t].acc[2 * gp][2], st[t].acc[2 * gp + 1][2], st[t].acc[2 * gp][3],
                             st[t].acc[2 * gp + 1][3]);
      }
      if (r == 0) {
        a.part_ml[pi * 2] = st[t].m;
        a.part_ml[pi * 2 + 1] = l[t];
      }
    }
  }
}

template <bool CASCADE>
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.batch * a.hkv * a.nsplit)), block(kWaves * 64);
  switch (a.g) {
    case 1: hipLaunchKernelGGL((mxfp4_decode_kernel<1, CASCADE>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((mxfp4_decode_kernel<2, CASCADE>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((mxfp4_decode_kernel<4, CASCADE>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((mxfp4_decode_kernel<8, CASCADE>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool PREFIX>
hipError_t launch_mt(const MultiTokenArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.batch * a.hkv * a.row_tiles * a.nsplit)), block(kMtWavesMx * 64);
  switch (a.rows_per_wg) {
    case 16: hipLaunchKernelGGL((mxfp4_mt_kernel<1, PREFIX>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((mxfp4_mt_kernel<2, PREFIX>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mxfp4_quantize(const QuantizeArgs &a, hipStream_t s) {
  if (a.num_tokens <= 0) return hipSuccess;
  const QuantGeometry g = quantize_geometry((const void *)mxfp4_quantize_kernel<false>,
                                            (const void *)mxfp4_quantize_kernel<true>, kD, a.num_tokens, a.hkv);
  QuantizeArgs b = a;
  b.grain = g.grain;
  b.window = g.window;
  if (g.balanced) hipLaunchKernelGGL(mxfp4_quantize_kernel<true>, dim3(g.grid), dim3(g.threads), 0, s, b);
  else hipLaunchKernelGGL(mxfp4_quantize_kernel<false>, dim3(g.grid), dim3(g.threads), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_mxfp4_decode(const DecodeArgs &a, hipStream_t s) { return launch_decode<false>(a, s); }

hipError_t launch_mxfp4_cascade_decode(const DecodeArgs &a, hipStream_t s) { return launch_decode<true>(a, s); }

hipError_t launch_mxfp4_multitoken(const MultiTokenArgs &a, hipStream_t s) {
  const hipError_t e = launch_mt<false>(a, s);
  if (e != hipSuccess || a.nsplit == 1) return e;
  return launch_multitoken_merge(kD, a, s);
}

hipError_t launch_mxfp4_prefix_attention(const MultiTokenArgs &a, hipStream_t s) { return launch_mt<true>(a, s); }

}  // namespace tq
