// TQ4/4 (and TQ4/2) attention of several query tokens per sequence over the
// 4-bit-key paged cache: chunked prefill of new tokens, or the verification of
// proposed tokens.
// The query tokens are the last M_b of sequence b's context of T_b tokens and
// see the keys causally: query token i sees positions t < T_b - M_b + i + 1.
//
// Rows are (query token, query head) pairs of one kv-head, token-major.  Two
// kernels, chosen by the number of rows of a (sequence, kv-head):
//   * up to 32 (verification of a few tokens): the direct kernel below, where
//     every wave runs all rows against its own block pairs, dequantizing keys
//     and values in registers as the decode kernel does;
//   * more (chunked prefill), and the shared-block pass of cascade decode: the
//     staged kernel.  A work-group of 8 waves takes 32 to 256 rows of one
//     (sequence, kv-head) and one split of the key blocks, which are
//     dequantized once per work-group and shared through LDS.  Stage k: wave w
//     loads block 8k + w of the split (a ring of four blocks of 128-bit loads
//     in flight per wave), unpacks it into the work-group's stage buffer
//     (keys: the fp16 table entries in the QK A-operand order; values: the
//     codes as exact fp16 integers in the PV A-operand order and the block's
//     (scale, min) tile; key scales), and after one barrier every wave runs
//     its rows against its pairs of blocks of the stage.  Two stage buffers
//     alternate, so one barrier per stage suffices.
// Per pair of blocks and 16-row tile: logits = K_hat (16 tokens x D) times the
// rotated query rows (D x 16 rows) on v_mfma_f32_16x16x32_f16, the query split
// into fp16 high and low parts (two MFMAs into one accumulator); the key
// scale; the causal mask; online softmax in log2 units with lazy rescale;
// out^T (channels x rows) += V_hat^T P over the pair's 32 tokens on
// v_mfma_f32_16x16x32_f16: code * scale as two exact fp16 parts (one MFMA
// each) and the minima through a separate product with P, so V_hat enters
// exactly; P is rounded once to fp16.
// With one split the rows are written directly; otherwise split partials
// (max, sum, acc) go to the workspace and a merge kernel combines them per row.
#include "decode_common.h"
#include "dequant.h"

namespace tq {
namespace {

constexpr int kMtWaves = 8;
// block ids of one split staged in LDS: split_blocks <= kMtMaxIds
constexpr int kMtMaxIds = 4096;
constexpr int kDirMaxIds = 1024;

template <int D>
struct MtTile;
template <>
struct MtTile<128> {
  typedef uint4 T;
};
template <>
struct MtTile<64> {
  typedef uint2 T;
};

__device__ __forceinline__ uint32_t mt_word(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ uint32_t mt_word(const uint2 &v, int i) { return i == 0 ? v.x : v.y; }
__device__ __forceinline__ uint32_t mt_word(uint32_t v, int) { return v; }

// Value-code words per lane: 4-bit values, one per 32-channel group; 2-bit
// values (TQ4/2), one per group pair.
template <int D, int VB>
struct MtVTile {
  typedef typename MtTile<D>::T T;
};
template <>
struct MtVTile<128, 2> {
  typedef uint2 T;
};
template <>
struct MtVTile<64, 2> {
  typedef uint32_t T;
};

// Record bytes of one (block, kv-head).
template <int D, int VB>
constexpr int mt_rec_bytes() {
  return TqRec<D, VB>::BYTES;
}

template <int D, int VB>
struct MtBlk {
  typename MtTile<D>::T kq;
  uint2 ks;
  typename MtVTile<D, VB>::T vq;
  uint32_t vmw;
};

template <int D, int VB>
__device__ __forceinline__ void mt_load_blk(MtBlk<D, VB> &o, const uint8_t *rec, int lane) {
  constexpr int G = D / 32, Q = D / 8;
  constexpr int VW = VB == 4 ? G : G / 2;  // value-code words per lane
  constexpr int OFF_KS = TqRec<D, VB>::KS, OFF_VC = TqRec<D, VB>::VC, OFF_VM = TqRec<D, VB>::VM;
  const int r = lane >> 4, c = lane & 15;
  o.kq = *reinterpret_cast<const typename MtTile<D>::T *>(rec + TqRec<D, VB>::KC + lane * Q);
  o.ks = *reinterpret_cast<const uint2 *>(rec + OFF_KS + 8 * r);
  o.vq = *reinterpret_cast<const typename MtVTile<D, VB>::T *>(rec + OFF_VC + lane * (4 * VW));
  o.vmw = reinterpret_cast<const uint32_t *>(rec + OFF_VM)[r * (4 * G) + (c & (4 * G - 1))];
}

// LDS image of a pair of blocks (per lane: its MFMA A operands).  The PV
// operand of a lane holds its 4 value codes of the first block, then its 4 of
// the second (exact fp16 integers), so one 16-byte read gives the 32-token
// operand; the consumers form code * scale from them and the blocks' (scale,
// min) tiles.
template <int D>
struct MtPair {
  uint4 k[2][D / 32][64];  // QK A operand of block h, k-step s: 8 fp16 table entries
  uint4 v[D / 16][64];     // PV A operand of tile t: 4 + 4 fp16 value codes
  uint32_t vm[2][64];      // block h's (scale, min) tile as in the record (row r,
                           // group gp: 4 scales then 4 minima, fp16), the scales
                           // times 2^-7 when big[h]
  uint2 ks[2][4];          // fp16 key scales of tokens 4r .. 4r+3 of block h
  uint32_t big[2];         // block h holds a value scale >= 4096
};

// Producer: this wave's loaded block into half `half` of its LDS pair: key
// table entries, value codes as exact fp16, the (scale, min) tile (the scales
// pre-multiplied by 2^-7 when one of them is >= 4096, flagged in big[half]);
// `lone`: the block is the last of the stage and unpaired, so the other
// half's codes and (scale, min) tile are cleared (its probabilities are 0,
// and 0 * NaN would not be).
template <int D, int VB>
__device__ __forceinline__ void mt_produce(const MtBlk<D, VB> &bk, MtPair<D> &slot, int half, bool lone,
                                           const uint32_t *s_lut, int lane, bool tail, uint32_t vm_keep,
                                           uint32_t sc_lane) {
  constexpr int G = D / 32, KS = D / 32;
  uint32_t vmw = bk.vmw;
  if (tail) {
    __asm__ volatile("");
    vmw &= vm_keep;
  }
  const bool big = __builtin_amdgcn_ballot_w64(has_big_scale(vmw & sc_lane) != 0) != 0;
  if (big) {
    __asm__ volatile("");
    if (sc_lane) vmw = as_u(as_h2(vmw) * (half2v){(_Float16)0x1p-7f, (_Float16)0x1p-7f});
  }
  slot.vm[half][(lane >> 4) * (4 * G) + (lane & (4 * G - 1))] = vmw;
  if (lane == 0) slot.big[half] = big ? 1u : 0u;
  if (lone) {
    __asm__ volatile("");
    slot.vm[1][(lane >> 4) * (4 * G) + (lane & (4 * G - 1))] = 0u;
    if (lane == 0) slot.big[1] = 0u;
  }
#pragma unroll
  for (int s = 0; s < KS; ++s) slot.k[half][s][lane] = key_entries(s_lut, mt_word(bk.kq, s));
  if ((lane & 15) == 0) slot.ks[half][lane >> 4] = bk.ks;
#pragma unroll
  for (int gp = 0; gp < G; ++gp) {
    uint32_t lo, hi;
    value_code_bytes<VB>(VB == 4 ? mt_word(bk.vq, gp) : mt_word(bk.vq, gp >> 1), gp, lo, hi);
    uint2 *ve = reinterpret_cast<uint2 *>(&slot.v[2 * gp][lane]);
    uint2 *vo = reinterpret_cast<uint2 *>(&slot.v[2 * gp + 1][lane]);
    ve[half] = make_uint2(as_u(codes_f16<false>(lo)), as_u(codes_f16<true>(lo)));
    vo[half] = make_uint2(as_u(codes_f16<false>(hi)), as_u(codes_f16<true>(hi)));
    if (lone) {
      __asm__ volatile("");
      ve[1] = make_uint2(0u, 0u);
      vo[1] = make_uint2(0u, 0u);
    }
  }
}

// The probabilities of a pair of blocks as the PV B operand: each rounded once
// to fp16, to nearest even (v_cvt_pk_f16_f32).  The relative error is at most
// 2^-11 and unbiased, the same bound as the fp16 rounding of the dequantized
// values; the running sum of the softmax stays in fp32.
__device__ __forceinline__ half8v mt_p_f16(const float (&p)[8]) {
  typedef float float8v __attribute__((ext_vector_type(8)));
  const float8v f = {p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]};
  return __builtin_convertvector(f, half8v);
}

// Online softmax over a pair of blocks (8 logits per lane: tokens 4r..4r+3 of
// each block, column n = lane % 16), with the lazy rescale of softmax_block.
template <int NT>
__device__ __forceinline__ void mt_softmax8(const float (&x)[8], WaveState<NT> &st, float (&p)[8]) {
  // v_max3 written out: the logits need no canonicalizing first
  float lm;
  __asm__("v_max3_f32 %0, %1, %2, %3\n\tv_max3_f32 %0, %0, %4, %5\n\tv_max3_f32 %0, %0, %6, %7\n\t"
          "v_max_f32 %0, %0, %8"
          : "=&v"(lm)
          : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]));
  if (__builtin_amdgcn_ballot_w64(lm > st.m + kLazyRescale) != 0) {
    float bm = __builtin_fmaxf(lm, xor16(lm));
    bm = __builtin_fmaxf(bm, xor32(bm));
    const bool raise = bm > st.m + kLazyRescale;
    const float m_new = raise ? bm : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int t = 0; t < NT; ++t) st.acc[t] *= alpha;
    st.m = m_new;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - st.m);
  st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

// Consumer: this wave's TR tiles of 16 rows against a pair of blocks (has_b
// false: a lone last block, whose second half gets p = 0).  The PV product
// contracts over the pair's 32 tokens on v_mfma_f32_16x16x32_f16: operand
// index 8r + j is token 4r + j of the first block for j < 4 and token
// 4r + j - 4 of the second, which is how both the QK accumulators (B operand)
// and the LDS value slots (A operand) hold them.  Every LDS operand read feeds
// all TR tiles, and the tiles' and blocks' MFMA chains are independent and
// interleaved.  lim[t]: this lane's column's visible-key count in tile t;
// masked: the pair reaches past some column's limit.
template <int D, int TR>
__device__ __forceinline__ void mt_consume_pair(const MtPair<D> &sp, bool has_b,
                                                const half8v (&bq_hi)[TR][D / 32],
                                                const half8v (&bq_lo)[TR][D / 32], WaveState<D / 16 + 1> (&st)[TR],
                                                int lane, int tok0, const int (&lim)[TR], bool masked) {
  constexpr int G = D / 32, KS = D / 32, NT = D / 16;
  const int r = lane >> 4;
  float4v qa[TR], qb[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) qa[t] = qb[t] = (float4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const half8v ka = __builtin_bit_cast(half8v, sp.k[0][s][lane]);
    const half8v kb = __builtin_bit_cast(half8v, sp.k[1][s][lane]);
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      qa[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, bq_hi[t][s], qa[t], 0, 0, 0);
      qb[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb, bq_hi[t][s], qb[t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      qa[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, bq_lo[t][s], qa[t], 0, 0, 0);
      qb[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb, bq_lo[t][s], qb[t], 0, 0, 0);
    }
  }
  const uint2 ka_s = sp.ks[0][r], kb_s = sp.ks[1][r];
  const half2v a01 = as_h2(ka_s.x), a23 = as_h2(ka_s.y), b01 = as_h2(kb_s.x), b23 = as_h2(kb_s.y);
  half8v ph[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    float x[8];
    x[0] = __builtin_fmaf(qa[t][0], (float)a01[0], 0.0f);
    x[1] = __builtin_fmaf(qa[t][1], (float)a01[1], 0.0f);
    x[2] = __builtin_fmaf(qa[t][2], (float)a23[0], 0.0f);
    x[3] = __builtin_fmaf(qa[t][3], (float)a23[1], 0.0f);
    x[4] = __builtin_fmaf(qb[t][0], (float)b01[0], 0.0f);
    x[5] = __builtin_fmaf(qb[t][1], (float)b01[1], 0.0f);
    x[6] = __builtin_fmaf(qb[t][2], (float)b23[0], 0.0f);
    x[7] = __builtin_fmaf(qb[t][3], (float)b23[1], 0.0f);
    if (!has_b) {
      __asm__ volatile("");
#pragma unroll
      for (int i = 4; i < 8; ++i) x[i] = kNegInf;
    }
    if (masked) {
      __asm__ volatile("");
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (tok0 + (i >> 2) * 16 + 4 * r + (i & 3) >= lim[t]) x[i] = kNegInf;
    }
    float p[8];
    mt_softmax8<NT + 1>(x, st[t], p);
    ph[t] = mt_p_f16(p);
  }
  // the minima: tile NT gets sum_t mn(t, g) P(t, row) (A row c: group c % G)
  {
    const int mi = r * (4 * G) + 4 * (lane & (G - 1)) + 2;
    const half8v amn = __builtin_bit_cast(half8v, make_uint4(sp.vm[0][mi], sp.vm[0][mi + 1], sp.vm[1][mi],
                                                             sp.vm[1][mi + 1]));
#pragma unroll
    for (int t = 0; t < TR; ++t) st[t].acc[NT] = __builtin_amdgcn_mfma_f32_16x16x32_f16(amn, ph[t], st[t].acc[NT], 0, 0, 0);
  }
  const uint32_t big_a = __builtin_amdgcn_readfirstlane(sp.big[0]), big_b = __builtin_amdgcn_readfirstlane(sp.big[1]);
  if (big_a | big_b) {
    __asm__ volatile("");
    const _Float16 fa = big_a ? (_Float16)128.f : (_Float16)1.f, fb = big_b ? (_Float16)128.f : (_Float16)1.f;
#pragma unroll
    for (int t = 0; t < TR; ++t) ph[t] = ph[t] * (half8v){fa, fa, fa, fa, fb, fb, fb, fb};
  }
  // code * scale as two exact fp16 parts (scales of this lane's 4 + 4 tokens
  // of the group), one MFMA each
#pragma unroll
  for (int gp = 0; gp < G; ++gp) {
    const int si = r * (4 * G) + 4 * gp;
    const half8v sc = __builtin_bit_cast(half8v, make_uint4(sp.vm[0][si], sp.vm[0][si + 1], sp.vm[1][si],
                                                            sp.vm[1][si + 1]));
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const half8v code = __builtin_bit_cast(half8v, sp.v[2 * gp + par][lane]);
      const half8v hi = code * sc;
      const half8v lo = __builtin_elementwise_fma(code, sc, -hi);
#pragma unroll
      for (int t = 0; t < TR; ++t) {
        st[t].acc[2 * gp + par] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, ph[t], st[t].acc[2 * gp + par], 0, 0, 0);
        st[t].acc[2 * gp + par] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, ph[t], st[t].acc[2 * gp + par], 0, 0, 0);
      }
    }
  }
}

// NRG row groups of 16 TR rows (TR tiles of 16 per wave) times NBG = 8 / NRG
// block groups: wave w takes rows 16 TR (w % NRG) .. + 16 TR - 1 of the
// work-group's tile and, of the four block pairs of every stage, those with
// index w / NRG (mod NBG); the block groups of a row group are merged in LDS at
// the end.  Every wave loads and dequantizes one block per stage.
//
// PREFIX (the shared-prefix pass of cascade decode): the work-group's rows are
// the (member sequence, query head) pairs of one group of sequences that share
// their leading blocks; every row sees all the shared tokens, which are read
// once for the whole group; the results are always partials.
template <int D, int NRG, int TR, bool PREFIX, int VB>
__global__ __launch_bounds__(kMtWaves * 64) void tq4_multitoken_kernel(MultiTokenArgs a) {
  constexpr int G = D / 32, KS = D / 32, NT = D / 16;
  constexpr int REC = mt_rec_bytes<D, VB>();
  constexpr int NW = kMtWaves;
  constexpr int NBG = NW / NRG;
  constexpr int RW = 16 * TR * NRG;  // rows per work-group

  __shared__ uint32_t s_lut[256];
  // two stage buffers of NW block slots; the query staging area and the final
  // block-group merge overlay them
  __shared__ __attribute__((aligned(16))) MtPair<D> s_stage[2][NW / 2];
  __shared__ float s_fm[NW][TR][16], s_fl[NW][TR][16];
  __shared__ int32_t s_ids[kMtMaxIds];  // the split's block ids
  static_assert(sizeof(s_stage) >= (size_t)NRG * TR * 32 * D * sizeof(_Float16), "query staging overlay");
  static_assert(NBG == 1 || sizeof(s_stage) >= (size_t)NW * TR * NT * 64 * sizeof(float4v), "merge overlay");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wv % NRG, bg = wv / NRG;
  const MtTask task = mt_task(a);
  const int b = task.b, kvh = task.kvh, sp = task.sp;

  // causal: b is a sequence, its query tokens q0 .. q0 + M - 1; prefix: b is a
  // group, q0 its first member's index into group_seqs, M its size
  int q0, M, T, tab_seq, blk_lo = 0, slot = sp;
  if constexpr (PREFIX) {
    q0 = a.group_start[b];
    M = a.group_start[b + 1] - q0;
    if (M <= 0) return;
    tab_seq = a.group_seqs[q0];
    blk_lo = a.group_blocks[2 * b];
    T = 16 * a.group_blocks[2 * b + 1];
    slot = a.slot0 + a.group_depth[b];  // one split per group (split_blocks covers it)
  } else {
    q0 = a.q_start[b];
    M = a.q_start[b + 1] - q0;
    T = a.ctx[b];
    tab_seq = b;
  }
  const int R = M * a.g;
  const int row0 = task.rt * RW;
  if (row0 >= R) return;
  const int rlast = min(R, row0 + RW) - 1;
  // keys the work-group's last row sees (prefix: every row sees all T)
  const int lmax_wg = PREFIX ? T : T - M + rlast / a.g + 1;
  const int nblk = (lmax_wg + 15) >> 4;
  const int blk0 = blk_lo + sp * a.split_blocks;
  if (blk0 >= nblk) {
    if constexpr (PREFIX) {
      // an empty group range: its rows get empty partials (max -inf, sum 0),
      // which the merge weighs 0
      for (int i = threadIdx.x; i < RW * (D + 2); i += NW * 64) {
        const int row = row0 + i / (D + 2), c = i % (D + 2);
        if (row >= R) continue;
        const int who = row / a.g, j = row % a.g;
        const int64_t pi = ((int64_t)a.group_seqs[q0 + who] * a.hq + kvh * a.g + j) * a.part_stride + slot;
        if (c < D) a.part_acc[pi * D + c] = 0.f;
        else a.part_ml[pi * 2 + (c - D)] = c == D ? kNegInf : 0.f;
      }
    }
    return;
  }
  const int blk1 = min(nblk, blk0 + a.split_blocks);
  const int nb = blk1 - blk0;

  // this lane's column (row) of each tile and its visible-key count; rows past
  // R see none
  const int n = lane & 15, r = lane >> 4;
  const int w_first = row0 + 16 * TR * rg;
  int myrow[TR], lim[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    myrow[t] = w_first + 16 * t + n;
    lim[t] = myrow[t] < R ? (PREFIX ? T : T - M + myrow[t] / a.g + 1) : 0;
  }
  // the wave's smallest and largest visible-key counts (its first and last rows)
  const int w_last = min(R, w_first + 16 * TR) - 1;
  const int lmin_w = w_first < R ? (PREFIX ? T : T - M + w_first / a.g + 1) : 0;
  const int lmax_w = w_first < R ? (PREFIX ? T : T - M + w_last / a.g + 1) : 0;
  // query / output row of tile row `row`: (token or member, head)
  auto q_row = [&](int row) -> int64_t {
    const int who = row / a.g, j = row % a.g;
    const int64_t tok = PREFIX ? (int64_t)a.group_seqs[q0 + who] : (int64_t)(q0 + who);
    return tok * a.hq + kvh * a.g + j;
  };

  // ---- block ids and the first loads ---------------------------------------------
  // lane k < 4 holds the id of this wave's block k (the first loads); the
  // split's ids (nb <= kMtMaxIds) go to LDS for the ring's refills, so that no
  // load is issued on a path of its own inside the loop (the compiler would
  // then wait for every load in flight before each refill)
  const int32_t *btab = a.block_table + (int64_t)tab_seq * a.max_blocks;
  const int my_id_raw = btab[min(blk0 + wv + (lane & 3) * NW, a.max_blocks - 1)];
  const uint32_t lut_w = tid < 256 ? a.tables->lut2[tid] : 0u;
  int ids[kMtMaxIds / (NW * 64)];
#pragma unroll
  for (int i = 0; i < kMtMaxIds / (NW * 64); ++i) ids[i] = btab[min(blk0 + tid + i * NW * 64, a.max_blocks - 1)];
  __asm__ volatile("" ::: "memory");
  const uint8_t *base = a.pool + (int64_t)kvh * REC;
  const int64_t stride = (int64_t)a.hkv * REC;
  const int mine = nb > wv ? (nb - wv + NW - 1) / NW : 0;
  const int my_id = settled(my_id_raw);
  // block k of this wave (k >= mine: its last block again, an L2 hit; a wave
  // with no block of this split refills from block 0's record, never used)
  auto first_rec = [&](int k) {
    const int kk = k < mine ? k : mine - 1;
    if (kk < 0) return base;
    return base + (int64_t)__builtin_amdgcn_readlane(my_id, kk) * stride;
  };
  auto rec_of = [&](int k) {
    const int kk = k < mine ? k : mine - 1;
    if (kk < 0) return base;
    return base + (int64_t)__builtin_amdgcn_readfirstlane(s_ids[wv + kk * NW]) * stride;
  };
  const int seq_nblk = (T + 15) >> 4;
  const int tail_blk = (T & 15) ? seq_nblk - 1 : seq_nblk;
  uint32_t tail_keep;
  {
    const int rr = 4 * (lane >> 4), w = lane & 3;
    const int ta = (T & 15) - (rr + 2 * (w & 1)), tb = ta - 1;
    tail_keep = (ta > 0 ? 0x0000FFFFu : 0u) | (tb > 0 ? 0xFFFF0000u : 0u);
  }
  MtBlk<D, VB> b0, b1, b2, b3;
  if (mine > 0) {
    mt_load_blk<D, VB>(b0, first_rec(0), lane);
    __asm__ volatile("" ::: "memory");
    mt_load_blk<D, VB>(b1, first_rec(1), lane);
    __asm__ volatile("" ::: "memory");
    mt_load_blk<D, VB>(b2, first_rec(2), lane);
    __asm__ volatile("" ::: "memory");
    mt_load_blk<D, VB>(b3, first_rec(3), lane);
  }

  // ---- the row group's 16 TR rotated, scaled query rows: fp16 high and low ------
  if (tid < 256) s_lut[tid] = lut_w;
#pragma unroll
  for (int i = 0; i < kMtMaxIds / (NW * 64); ++i)
    if (tid + i * NW * 64 < nb) s_ids[tid + i * NW * 64] = ids[i];
  _Float16(*s_q)[TR][2][16][D] = reinterpret_cast<_Float16(*)[TR][2][16][D]>(&s_stage[0][0]);
  if (bg == 0) {
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      uint32_t qw[16];  // all 16 query loads in flight before the first rotation
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        qw[j] = load_query_word<D>(a.q + q_row(min(w_first + 16 * t + j, R - 1)) * D, lane);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x0 = 0.f, x1 = 0.f;
        if (w_first + 16 * t + j < R) rotate_row<D>(qw[j], lane, x0, x1);
#pragma unroll
        for (int e = 0; e < (D == 128 ? 2 : 1); ++e) {
          const float xs = (e ? x1 : x0) * a.qscale;
          const _Float16 hi = (_Float16)xs;
          const _Float16 lo = (_Float16)(xs - (float)hi);
          const int c = rotated_channel<D>(lane, e);
          s_q[rg][t][0][j][c] = hi;
          s_q[rg][t][1][j][c] = lo;
        }
      }
    }
  }
  __syncthreads();
  half8v bq_hi[TR][KS], bq_lo[TR][KS];
#pragma unroll
  for (int t = 0; t < TR; ++t) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bq_hi[t][s] = *reinterpret_cast<const half8v *>(&s_q[rg][t][0][n][r * (D / 4) + 8 * s]);
      bq_lo[t][s] = *reinterpret_cast<const half8v *>(&s_q[rg][t][1][n][r * (D / 4) + 8 * s]);
    }
  }
  __syncthreads();  // the staging area becomes stage buffer 0

  // tiles 0 .. NT-1: out^T per (group, parity); tile NT: the minima's product
  WaveState<NT + 1> st[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    st[t].m = kMtFloor;
    st[t].l = 0.f;
#pragma unroll
    for (int c = 0; c < NT + 1; ++c) st[t].acc[c] = (float4v){0.f, 0.f, 0.f, 0.f};
  }
  // lanes whose dword of a group's 16-byte (scale, min) tile holds scales
  const uint32_t sc_lane = (lane & 2) ? 0u : 0xFFFFFFFFu;

  const int nstage = (nb + NW - 1) / NW;
  auto stage = [&](MtBlk<D, VB> &buf, int k) {
    MtPair<D>(&cur)[NW / 2] = s_stage[k & 1];
    const int first = blk0 + k * NW;
    const int cnt = min(NW, blk1 - first);
    if (k < mine) {
      const int blk = first + wv;
      mt_produce<D, VB>(buf, cur[wv >> 1], wv & 1, (wv & 1) == 0 && wv + 1 == cnt, s_lut, lane, blk == tail_blk,
                        tail_keep, sc_lane);
    }
    mt_load_blk<D, VB>(buf, rec_of(k + 4), lane);
    __syncthreads();
#pragma unroll 1
    for (int j = 2 * bg; j < cnt; j += 2 * NBG) {
      const int tok0 = (first + j) * 16;
      if (tok0 >= lmax_w) break;  // this pair and the later ones are masked for every row
      mt_consume_pair<D, TR>(cur[j >> 1], j + 1 < cnt, bq_hi, bq_lo, st, lane, tok0, lim, tok0 + 32 > lmin_w);
    }
  };
  // the four stages of an iteration run unconditionally (a stage past the
  // last has no block and no pair: one barrier), so every path through the
  // loop issues the same loads and the waits stay partial
#pragma unroll 1
  for (int k = 0; k < nstage; k += 4) {
    stage(b0, k);
    stage(b1, k + 1);
    stage(b2, k + 2);
    stage(b3, k + 3);
  }

  // the minima's contribution to every channel of their group
#pragma unroll
  for (int t = 0; t < TR; ++t) {
#pragma unroll
    for (int gp = 0; gp < G; ++gp) {
      st[t].acc[2 * gp] += st[t].acc[NT][gp];
      st[t].acc[2 * gp + 1] += st[t].acc[NT][gp];
    }
  }

  // ---- merge the block groups of each row group ---------------------------------
  float l[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    l[t] = st[t].l;
    l[t] += xor16(l[t]);
    l[t] += xor32(l[t]);
  }
  if constexpr (NBG > 1) {
    float4v(*s_fa)[TR][NT][64] = reinterpret_cast<float4v(*)[TR][NT][64]>(&s_stage[0][0]);
    __syncthreads();  // every wave is done with the stage buffers
#pragma unroll
    for (int t = 0; t < TR; ++t) {
#pragma unroll
      for (int c = 0; c < NT; ++c) s_fa[wv][t][c][lane] = st[t].acc[c];
      if (r == 0) {
        s_fm[wv][t][n] = st[t].m;
        s_fl[wv][t][n] = l[t];
      }
    }
    __syncthreads();
    if (bg != 0) return;
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      float mx = st[t].m;
#pragma unroll
      for (int q = 1; q < NBG; ++q) mx = __builtin_fmaxf(mx, s_fm[rg + NRG * q][t][n]);
      const float f0 = __builtin_amdgcn_exp2f(st[t].m - mx);
      l[t] *= f0;
#pragma unroll
      for (int c = 0; c < NT; ++c) st[t].acc[c] *= f0;
#pragma unroll
      for (int q = 1; q < NBG; ++q) {
        const int w2 = rg + NRG * q;
        const float f = __builtin_amdgcn_exp2f(s_fm[w2][t][n] - mx);
        l[t] += f * s_fl[w2][t][n];
#pragma unroll
        for (int c = 0; c < NT; ++c) st[t].acc[c] += f * s_fa[w2][t][c][lane];
      }
      st[t].m = mx;
    }
  }

  // ---- this wave's rows: output, or the split partial ------------------------------
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    if (myrow[t] >= R) continue;
    const int64_t orow = q_row(myrow[t]);
    if (!PREFIX && a.nsplit == 1) {
      const float inv = l[t] > 0.f ? 1.f / l[t] : 0.f;
#pragma unroll
      for (int gp = 0; gp < G; ++gp) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[2 * i] = st[t].acc[2 * gp][i] * inv;
          o[2 * i + 1] = st[t].acc[2 * gp + 1][i] * inv;
        }
        const int64_t oi = orow * D + 32 * gp + 8 * r;
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
      for (int gp = 0; gp < G; ++gp) {
        float4 *dst = reinterpret_cast<float4 *>(a.part_acc + pi * D + 32 * gp + 8 * r);
        dst[0] = make_float4(st[t].acc[2 * gp][0], st[t].acc[2 * gp + 1][0], st[t].acc[2 * gp][1],
                             st[t].acc[2 * gp + 1][1]);
        dst[1] = make_float4(st[t].acc[2 * gp][2], st[t].acc[2 * gp + 1][2], st[t].acc[2 * gp][3],
                             st[t].acc[2 * gp + 1][3]);
      }
      if (r == 0) {
        // a row none of whose keys fall in this split keeps the floor maximum
        // and a zero sum; the merge gives it weight 0
        a.part_ml[pi * 2] = st[t].m;
        a.part_ml[pi * 2 + 1] = l[t];
      }
    }
  }
}

// Direct kernel for up to 32 rows per (sequence, kv-head) (verification of a
// few proposed tokens): every row of the sequence's kv-head sees every block,
// so staging the blocks through LDS (above) would share each dequantized block
// among only two waves.  Here a work-group of 4 waves takes one split of the
// key blocks, and every wave runs all RT 16-row tiles against its own pairs of
// blocks (pair p = blocks 2p, 2p + 1 of the split, p = wave + 4k), as the
// decode kernel does for one query token: no barrier in the main loop, keys
// through the byte-pair table in LDS straight into the QK A operand, values
// dequantized in registers straight into the PV A operand (the pair's 32
// tokens: operand index 8r + j is token 4r + j of the first block for j < 4 and
// of the second otherwise, the QK accumulators' order).  Two pairs of loads
// stay in flight per wave, and the query operands stay in registers (two
// waves per SIMD: two work-groups per CU).  The 4 waves' softmax states are
// merged in LDS at the end (two halving rounds).
constexpr int kDirWaves = 4;

// PREFIX (the shared-block pass of cascade decode, groups of at most 32
// rows): the rows are the (member sequence, query head) pairs of one group,
// every row sees all the group's blocks, and the results are always partials
// (at slot slot0 + the group's depth).
template <int D, int RT, bool PREFIX, int VB>
__global__ __launch_bounds__(kDirWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void tq4_mt_direct_kernel(
    MultiTokenArgs a) {
  constexpr int G = D / 32, KS = D / 32, NT = D / 16;
  constexpr int REC = mt_rec_bytes<D, VB>();
  constexpr int NW = kDirWaves;

  __shared__ uint32_t s_lut[256];
  __shared__ __attribute__((aligned(16))) uint32_t s_vm[NW][2][64];
  // the query staging area, then the wave-merge area
  constexpr size_t kQBytes = (size_t)RT * 2 * 16 * D * sizeof(_Float16);
  constexpr size_t kMBytes = (size_t)(NW / 2) * RT * NT * 64 * sizeof(float4v);
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[kQBytes > kMBytes ? kQBytes : kMBytes];
  __shared__ float s_wm[NW / 2][RT][16], s_wl[NW / 2][RT][16];
  __shared__ int32_t s_ids[kDirMaxIds];  // the split's block ids

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const MtTask task = mt_task(a);
  const int b = task.b, kvh = task.kvh, sp = task.sp;
  // causal: b is a sequence, its query tokens q0 .. q0 + M - 1, and the last
  // row sees all T keys, the first T - M + 1; prefix: b is a group, q0 its
  // first member's index into group_seqs, M its size, and every row sees the
  // group's blocks blk_lo .. T / 16 - 1
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
  if (R <= 0) return;
  auto q_row = [&](int row) -> int64_t {
    const int who = row / a.g, j = row % a.g;
    const int64_t tok = PREFIX ? (int64_t)a.group_seqs[q0 + who] : (int64_t)(q0 + who);
    return tok * a.hq + kvh * a.g + j;
  };
  const int nblk = (T + 15) >> 4;
  const int blk0 = blk_lo + sp * a.split_blocks;
  if (blk0 >= nblk) {
    if constexpr (PREFIX) {
      // an empty group range: its rows get empty partials (max -inf, sum 0),
      // which the merge weighs 0
      for (int i = tid; i < R * (D + 2); i += NW * 64) {
        const int64_t pi = q_row(i / (D + 2)) * a.part_stride + slot;
        const int c = i % (D + 2);
        if (c < D) a.part_acc[pi * D + c] = 0.f;
        else a.part_ml[pi * 2 + (c - D)] = c == D ? kNegInf : 0.f;
      }
    }
    return;
  }
  const int blk1 = min(nblk, blk0 + a.split_blocks);
  const int npair = (blk1 - blk0 + 1) >> 1;
  const int lmin = PREFIX ? T : T - M + 1;

  const int n = lane & 15, r = lane >> 4;
  int myrow[RT], lim[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    myrow[t] = 16 * t + n;
    lim[t] = myrow[t] < R ? (PREFIX ? T : T - M + myrow[t] / a.g + 1) : 0;
  }

  // ---- block ids and the first loads ---------------------------------------------
  // lane j < 4 holds the id of block j & 1 of this wave's pair j / 2 (the first
  // loads); the split's ids (at most kDirMaxIds) go to LDS for the refills
  const int32_t *btab = a.block_table + (int64_t)tab_seq * a.max_blocks;
  const int my_id_raw = btab[min(blk0 + 2 * (wv + ((lane & 3) >> 1) * NW) + (lane & 1), a.max_blocks - 1)];
  const uint32_t lut_w = tid < 256 ? a.tables->lut2[tid] : 0u;
  int ids[kDirMaxIds / (NW * 64)];
#pragma unroll
  for (int i = 0; i < kDirMaxIds / (NW * 64); ++i) ids[i] = btab[min(blk0 + tid + i * NW * 64, a.max_blocks - 1)];
  __asm__ volatile("" ::: "memory");
  const uint8_t *base = a.pool + (int64_t)kvh * REC;
  const int64_t stride = (int64_t)a.hkv * REC;
  const int mine = npair > wv ? (npair - wv + NW - 1) / NW : 0;
  const int my_id = settled(my_id_raw);
  // block h of this wave's pair k (k >= mine: its last pair again, an L2 hit;
  // the missing second block of a lone last pair: the first again; a wave
  // without pairs refills from block 0's record, never used)
  auto first_rec = [&](int k, int h) {
    const int kk = k < mine ? k : mine - 1;
    if (kk < 0) return base;
    const int hh = blk0 + 2 * (wv + kk * NW) + h < blk1 ? h : 0;
    return base + (int64_t)__builtin_amdgcn_readlane(my_id, 2 * kk + hh) * stride;
  };
  auto rec_of = [&](int k, int h) {
    const int kk = k < mine ? k : mine - 1;
    if (kk < 0) return base;
    const int hh = blk0 + 2 * (wv + kk * NW) + h < blk1 ? h : 0;
    return base + (int64_t)__builtin_amdgcn_readfirstlane(s_ids[2 * (wv + kk * NW) + hh]) * stride;
  };
  const int tail_blk = (T & 15) ? nblk - 1 : nblk;
  uint32_t tail_keep;
  {
    const int rr = 4 * (lane >> 4), w = lane & 3;
    const int ta = (T & 15) - (rr + 2 * (w & 1)), tb = ta - 1;
    tail_keep = (ta > 0 ? 0x0000FFFFu : 0u) | (tb > 0 ? 0xFFFF0000u : 0u);
  }
  MtBlk<D, VB> a0, b0, a1, b1;
  if (mine > 0) {
    mt_load_blk<D, VB>(a0, first_rec(0, 0), lane);
    mt_load_blk<D, VB>(b0, first_rec(0, 1), lane);
    __asm__ volatile("" ::: "memory");
    mt_load_blk<D, VB>(a1, first_rec(1, 0), lane);
    mt_load_blk<D, VB>(b1, first_rec(1, 1), lane);
  }

  // ---- the RT 16-row tiles of rotated, scaled query rows: fp16 high and low -----
  if (tid < 256) s_lut[tid] = lut_w;
#pragma unroll
  for (int i = 0; i < kDirMaxIds / (NW * 64); ++i)
    if (tid + i * NW * 64 < blk1 - blk0) s_ids[tid + i * NW * 64] = ids[i];
  _Float16(*s_q)[2][16][D] = reinterpret_cast<_Float16(*)[2][16][D]>(s_buf);
  if (wv < RT) {
    uint32_t qw[16];  // all 16 query loads in flight before the first rotation
#pragma unroll
    for (int j = 0; j < 16; ++j) qw[j] = load_query_word<D>(a.q + q_row(min(16 * wv + j, R - 1)) * D, lane);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float x0 = 0.f, x1 = 0.f;
      if (16 * wv + j < R) rotate_row<D>(qw[j], lane, x0, x1);
#pragma unroll
      for (int e = 0; e < (D == 128 ? 2 : 1); ++e) {
        const float xs = (e ? x1 : x0) * a.qscale;
        const _Float16 hi = (_Float16)xs;
        const _Float16 lo = (_Float16)(xs - (float)hi);
        const int c = rotated_channel<D>(lane, e);
        s_q[wv][0][j][c] = hi;
        s_q[wv][1][j][c] = lo;
      }
    }
  }
  __syncthreads();
  // the query operands (B of the QK product) stay in registers
  half8v bq[RT][2][KS];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int hl = 0; hl < 2; ++hl)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        bq[t][hl][s] = *reinterpret_cast<const half8v *>(&s_q[t][hl][n][r * (D / 4) + 8 * s]);

  // tiles 0 .. NT-1: out^T per (group, parity); tile NT: the minima's product
  WaveState<NT + 1> st[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    st[t].m = kMtFloor;
    st[t].l = 0.f;
#pragma unroll
    for (int c = 0; c < NT + 1; ++c) st[t].acc[c] = (float4v){0.f, 0.f, 0.f, 0.f};
  }
  // lanes whose dword of a group's 16-byte (scale, min) tile holds scales
  const uint32_t sc_lane = (lane & 2) ? 0u : 0xFFFFFFFFu;

  uint32_t *vm_a = s_vm[wv][0], *vm_b = s_vm[wv][1];
  const int vm_i = (lane >> 4) * (4 * G) + (lane & (4 * G - 1));
  auto pair = [&](const MtBlk<D, VB> &ba, const MtBlk<D, VB> &bb, int k) {
    const int blk = blk0 + 2 * (wv + k * NW);
    const bool has_b = blk + 1 < blk1;
    const int tok0 = 16 * blk;
    // the value (scale, min) tiles go through LDS (rows of the partial last
    // block past the context get zero scale and minimum)
    uint32_t vma = ba.vmw, vmb = bb.vmw;
    if (blk == tail_blk) {
      __asm__ volatile("");
      vma &= tail_keep;
    }
    if (blk + 1 == tail_blk) {
      __asm__ volatile("");
      vmb &= tail_keep;
    }
    // a block holding a value scale >= 4096 gets every scale applied as
    // sc * 2^-7 and its tokens' probabilities as P * 2^7 (rare)
    const bool big_a = __builtin_amdgcn_ballot_w64(has_big_scale(vma & sc_lane) != 0) != 0;
    const bool big_b = __builtin_amdgcn_ballot_w64(has_big_scale(vmb & sc_lane) != 0) != 0;
    if (big_a || big_b) {
      __asm__ volatile("");
      const half2v f = (half2v){(_Float16)0x1p-7f, (_Float16)0x1p-7f};
      if (big_a && sc_lane) vma = as_u(as_h2(vma) * f);
      if (big_b && sc_lane) vmb = as_u(as_h2(vmb) * f);
    }
    vm_a[vm_i] = vma;
    vm_b[vm_i] = vmb;
    // ---- logits of both blocks for every tile ----
    float4v qa[RT], qb[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) qa[t] = qb[t] = (float4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t wa = mt_word(ba.kq, s), wb = mt_word(bb.kq, s);
      uint4 ea, eb;
      ea.x = s_lut[wa & 0xFF];
      ea.y = s_lut[(wa >> 8) & 0xFF];
      ea.z = s_lut[(wa >> 16) & 0xFF];
      ea.w = s_lut[wa >> 24];
      eb.x = s_lut[wb & 0xFF];
      eb.y = s_lut[(wb >> 8) & 0xFF];
      eb.z = s_lut[(wb >> 16) & 0xFF];
      eb.w = s_lut[wb >> 24];
      const half8v ka = __builtin_bit_cast(half8v, ea), kb = __builtin_bit_cast(half8v, eb);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const half8v qh = bq[t][0][s];
        qa[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qh, qa[t], 0, 0, 0);
        qb[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb, qh, qb[t], 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const half8v ql = bq[t][1][s];
        qa[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, ql, qa[t], 0, 0, 0);
        qb[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb, ql, qb[t], 0, 0, 0);
      }
    }
    const half2v a01 = as_h2(ba.ks.x), a23 = as_h2(ba.ks.y), b01 = as_h2(bb.ks.x), b23 = as_h2(bb.ks.y);
    const bool masked = tok0 + 32 > lmin;
    half8v ph[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      float x[8];
      x[0] = __builtin_fmaf(qa[t][0], (float)a01[0], 0.0f);
      x[1] = __builtin_fmaf(qa[t][1], (float)a01[1], 0.0f);
      x[2] = __builtin_fmaf(qa[t][2], (float)a23[0], 0.0f);
      x[3] = __builtin_fmaf(qa[t][3], (float)a23[1], 0.0f);
      x[4] = __builtin_fmaf(qb[t][0], (float)b01[0], 0.0f);
      x[5] = __builtin_fmaf(qb[t][1], (float)b01[1], 0.0f);
      x[6] = __builtin_fmaf(qb[t][2], (float)b23[0], 0.0f);
      x[7] = __builtin_fmaf(qb[t][3], (float)b23[1], 0.0f);
      if (!has_b) {
        __asm__ volatile("");
#pragma unroll
        for (int i = 4; i < 8; ++i) x[i] = kNegInf;
      }
      if (masked) {
        __asm__ volatile("");
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (tok0 + (i >> 2) * 16 + 4 * r + (i & 3) >= lim[t]) x[i] = kNegInf;
      }
      float p[8];
      mt_softmax8<NT + 1>(x, st[t], p);
      ph[t] = mt_p_f16(p);
    }
    // ---- values ----
    // the minima: the bias tile gets sum_t mn(t, g) P(t, row); A rows c hold
    // group c % G of the pair's 32 tokens (operand index 8r + j: token 4r + j
    // of the first block for j < 4, of the second otherwise), so row 4r' + i
    // of the result is group i % G
    {
      const uint2 mna = *reinterpret_cast<const uint2 *>(vm_a + (lane >> 4) * (4 * G) + 4 * (lane & (G - 1)) + 2);
      const uint2 mnb = *reinterpret_cast<const uint2 *>(vm_b + (lane >> 4) * (4 * G) + 4 * (lane & (G - 1)) + 2);
      const half8v amn = __builtin_bit_cast(half8v, make_uint4(mna.x, mna.y, mnb.x, mnb.y));
#pragma unroll
      for (int t = 0; t < RT; ++t)
        st[t].acc[NT] = __builtin_amdgcn_mfma_f32_16x16x32_f16(amn, ph[t], st[t].acc[NT], 0, 0, 0);
    }
    if (big_a || big_b) {
      __asm__ volatile("");
      const _Float16 fa = big_a ? (_Float16)128.f : (_Float16)1.f, fb = big_b ? (_Float16)128.f : (_Float16)1.f;
#pragma unroll
      for (int t = 0; t < RT; ++t) ph[t] = ph[t] * (half8v){fa, fa, fa, fa, fb, fb, fb, fb};
    }
    // code * scale as two exact fp16 parts per element, both blocks into one
    // 32-token operand; the high and the low parts each take one MFMA
    const uint4 *vra = reinterpret_cast<const uint4 *>(vm_a) + (lane >> 4) * G;
    const uint4 *vrb = reinterpret_cast<const uint4 *>(vm_b) + (lane >> 4) * G;
#pragma unroll
    for (int gp = 0; gp < G; ++gp) {
      const uint2 sa = *reinterpret_cast<const uint2 *>(&vra[gp]), sb = *reinterpret_cast<const uint2 *>(&vrb[gp]);
      uint32_t la, ha, lb, hb;
      value_code_bytes<VB>(VB == 4 ? mt_word(ba.vq, gp) : mt_word(ba.vq, gp >> 1), gp, la, ha);
      value_code_bytes<VB>(VB == 4 ? mt_word(bb.vq, gp) : mt_word(bb.vq, gp >> 1), gp, lb, hb);
      const ScaledPair ea01 = scaled_codes(codes_f16<false>(la), as_h2(sa.x));
      const ScaledPair ea23 = scaled_codes(codes_f16<true>(la), as_h2(sa.y));
      const ScaledPair oa01 = scaled_codes(codes_f16<false>(ha), as_h2(sa.x));
      const ScaledPair oa23 = scaled_codes(codes_f16<true>(ha), as_h2(sa.y));
      const ScaledPair eb01 = scaled_codes(codes_f16<false>(lb), as_h2(sb.x));
      const ScaledPair eb23 = scaled_codes(codes_f16<true>(lb), as_h2(sb.y));
      const ScaledPair ob01 = scaled_codes(codes_f16<false>(hb), as_h2(sb.x));
      const ScaledPair ob23 = scaled_codes(codes_f16<true>(hb), as_h2(sb.y));
      const half8v veh = __builtin_bit_cast(half8v, make_uint4(as_u(ea01.hi), as_u(ea23.hi), as_u(eb01.hi), as_u(eb23.hi)));
      const half8v vel = __builtin_bit_cast(half8v, make_uint4(as_u(ea01.lo), as_u(ea23.lo), as_u(eb01.lo), as_u(eb23.lo)));
      const half8v voh = __builtin_bit_cast(half8v, make_uint4(as_u(oa01.hi), as_u(oa23.hi), as_u(ob01.hi), as_u(ob23.hi)));
      const half8v vol = __builtin_bit_cast(half8v, make_uint4(as_u(oa01.lo), as_u(oa23.lo), as_u(ob01.lo), as_u(ob23.lo)));
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        st[t].acc[2 * gp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(veh, ph[t], st[t].acc[2 * gp], 0, 0, 0);
        st[t].acc[2 * gp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(voh, ph[t], st[t].acc[2 * gp + 1], 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        st[t].acc[2 * gp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vel, ph[t], st[t].acc[2 * gp], 0, 0, 0);
        st[t].acc[2 * gp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vol, ph[t], st[t].acc[2 * gp + 1], 0, 0, 0);
      }
    }
  };
  // process ring slot (pair k, if it is one of this wave's), then refill it
  auto run = [&](MtBlk<D, VB> &ba, MtBlk<D, VB> &bb, int k) {
    if (k < mine) pair(ba, bb, k);
    mt_load_blk<D, VB>(ba, rec_of(k + 2, 0), lane);
    mt_load_blk<D, VB>(bb, rec_of(k + 2, 1), lane);
  };
#pragma unroll 1
  for (int k = 0; k < mine; k += 2) {
    run(a0, b0, k);
    run(a1, b1, k + 1);
  }

  // the minima's contribution to every channel of their group
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int gp = 0; gp < G; ++gp) {
      st[t].acc[2 * gp] += st[t].acc[NT][gp];
      st[t].acc[2 * gp + 1] += st[t].acc[NT][gp];
    }
  }

  // ---- merge the waves' states: halving rounds through LDS -----------------------
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
    __syncthreads();  // the area is free (query staging read, or the last round's reads done)
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

  // ---- wave 0 writes the rows: output, or the split partial ---------------------------
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    if (myrow[t] >= R) continue;
    const int64_t orow = q_row(myrow[t]);
    if (!PREFIX && a.nsplit == 1) {
      const float inv = l[t] > 0.f ? 1.f / l[t] : 0.f;
#pragma unroll
      for (int gp = 0; gp < G; ++gp) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[2 * i] = st[t].acc[2 * gp][i] * inv;
          o[2 * i + 1] = st[t].acc[2 * gp + 1][i] * inv;
        }
        const int64_t oi = orow * D + 32 * gp + 8 * r;
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
      for (int gp = 0; gp < G; ++gp) {
        float4 *dst = reinterpret_cast<float4 *>(a.part_acc + pi * D + 32 * gp + 8 * r);
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

// One wave per (sequence, query token, query head) slot, four per work-group:
// combine the split partials of the row, if the slot holds a query token.
// Multi-token rows are many and their splits few, so a wave takes a row: the
// lanes find the largest partial maximum together, then every lane adds the
// weighted accumulators of its D / 64 channels over the splits.
template <int D>
__global__ __launch_bounds__(256) void multitoken_merge_kernel(MultiTokenArgs a) {
  constexpr int CPL = D / 64;  // channels per lane
  const int lane = threadIdx.x & 63;
  const int64_t slot = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (slot >= (int64_t)a.batch * a.max_query_len * a.hq) return;
  const int h = (int)(slot % a.hq);
  const int64_t rest = slot / a.hq;
  const int i = (int)(rest % a.max_query_len);
  const int b = (int)(rest / a.max_query_len);
  const int q0 = a.q_start[b];
  const int M = a.q_start[b + 1] - q0;
  if (i >= M) return;
  const int T = a.ctx[b];
  const int lim = T - M + i + 1;
  const int nblk = (lim + 15) >> 4;
  const int ns = (nblk + a.split_blocks - 1) / a.split_blocks;
  const int64_t row = (int64_t)(q0 + i) * a.hq + h;
  const float2 *ml = reinterpret_cast<const float2 *>(a.part_ml + row * a.nsplit * 2);
  const float *pa = a.part_acc + row * a.nsplit * D + CPL * lane;
  float mx = kNegInf;
  for (int sp = lane; sp < ns; sp += 64) mx = __builtin_fmaxf(mx, ml[sp].x);
  mx = __builtin_fmaxf(mx, xor1(mx));
  mx = __builtin_fmaxf(mx, xor2(mx));
  mx = __builtin_fmaxf(mx, xor4(mx));
  mx = __builtin_fmaxf(mx, xor8(mx));
  mx = __builtin_fmaxf(mx, xor16(mx));
  mx = __builtin_fmaxf(mx, xor32(mx));
  float den = 0.f, num[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) num[c] = 0.f;
#pragma unroll 4
  for (int sp = 0; sp < ns; ++sp) {
    const float2 m_l = ml[sp];  // the same address on every lane
    const float f = m_l.x == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_l.x - mx);
    den += f * m_l.y;
#pragma unroll
    for (int c = 0; c < CPL; ++c) num[c] += f * pa[(int64_t)sp * D + c];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int64_t oi = row * D + CPL * lane + c;
    if (a.out_bf16) reinterpret_cast<uint16_t *>(a.out)[oi] = f32_to_bf16(num[c] * inv);
    else reinterpret_cast<float *>(a.out)[oi] = num[c] * inv;
  }
}

template <int D>
hipError_t launch_merge(const MultiTokenArgs &a, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.max_query_len * a.hq;
  hipLaunchKernelGGL(multitoken_merge_kernel<D>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, int VB>
hipError_t launch_mt(const MultiTokenArgs &a, hipStream_t s) {
  const int64_t wgs = (int64_t)a.batch * a.hkv * a.row_tiles * a.nsplit;
  const dim3 grid((unsigned)wgs), block(kMtWaves * 64);
  switch (a.rows_per_wg) {
    case 16: hipLaunchKernelGGL((tq4_mt_direct_kernel<D, 1, false, VB>), grid, dim3(kDirWaves * 64), 0, s, a); break;
    case 32: hipLaunchKernelGGL((tq4_mt_direct_kernel<D, 2, false, VB>), grid, dim3(kDirWaves * 64), 0, s, a); break;
    case 64: hipLaunchKernelGGL((tq4_multitoken_kernel<D, 4, 1, false, VB>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((tq4_multitoken_kernel<D, 8, 1, false, VB>), grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL((tq4_multitoken_kernel<D, 8, 2, false, VB>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  return launch_merge<D>(a, s);
}

template <int D, int VB>
hipError_t launch_prefix(const MultiTokenArgs &a, hipStream_t s) {
  const int64_t wgs = (int64_t)a.batch * a.hkv * a.row_tiles * a.nsplit;
  const dim3 grid((unsigned)wgs), block(kMtWaves * 64);
  switch (a.rows_per_wg) {
    case 16: hipLaunchKernelGGL((tq4_mt_direct_kernel<D, 1, true, VB>), grid, dim3(kDirWaves * 64), 0, s, a); break;
    case 32: hipLaunchKernelGGL((tq4_mt_direct_kernel<D, 2, true, VB>), grid, dim3(kDirWaves * 64), 0, s, a); break;
    case 64: hipLaunchKernelGGL((tq4_multitoken_kernel<D, 4, 1, true, VB>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((tq4_multitoken_kernel<D, 8, 1, true, VB>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tq4_multitoken(int d, int vbits, const MultiTokenArgs &a, hipStream_t s) {
  if (vbits == 2) return d == 128 ? launch_mt<128, 2>(a, s) : launch_mt<64, 2>(a, s);
  return d == 128 ? launch_mt<128, 4>(a, s) : launch_mt<64, 4>(a, s);
}

hipError_t launch_prefix_attention(int d, int vbits, const MultiTokenArgs &a, hipStream_t s) {
  if (vbits == 2) return d == 128 ? launch_prefix<128, 2>(a, s) : launch_prefix<64, 2>(a, s);
  return d == 128 ? launch_prefix<128, 4>(a, s) : launch_prefix<64, 4>(a, s);
}

// The split merge of multi-token attention (any format: the partials have one
// layout).
hipError_t launch_multitoken_merge(int d, const MultiTokenArgs &a, hipStream_t s) {
  return d == 128 ? launch_merge<128>(a, s) : launch_merge<64>(a, s);
}

}  // namespace tq
