// Pieces shared by the quantize kernels: the lane mapping of a wave over token
// rows, the in-register Walsh-Hadamard butterflies, the quad byte transposes
// and the persistent launch geometry.
#pragma once

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

// A wave handles TPW token rows of one kv-head; a row is spread over LPT lanes
// with 16 channels per lane (channel = 16*li + e).  The lane bits that carry
// the chunk index li are those whose exchanges are single DPP operations:
// lane bits 0, 1 (quad_perm) and 3 (row_ror:8).  The token index tw takes the
// remaining lane bits; its bit 0 is lane bit 2 and its bit 1 is lane bit TB1.
template <int D>
struct QLanes;
template <>
struct QLanes<128> {
  static constexpr int LPT = 8, TPW = 8, TB1 = 4;
  __device__ static int li(int l) { return (l & 3) | ((l >> 1) & 4); }
  __device__ static int tw(int l) { return ((l >> 2) & 1) | ((l >> 3) & 6); }
};
template <>
struct QLanes<64> {
  static constexpr int LPT = 4, TPW = 16, TB1 = 3;
  __device__ static int li(int l) { return l & 3; }
  __device__ static int tw(int l) { return l >> 2; }
};

// Exchange with the lane of the token whose in-quad index differs in bit 0 /
// bit 1 (ds_swizzle: these run in the LDS pipe, not on the VALU).
__device__ __forceinline__ uint32_t tok_xor1(uint32_t x) { return swz_xor_u<4>(x); }
template <int D>
__device__ __forceinline__ uint32_t tok_xor2(uint32_t x) {
  return swz_xor_u<(1 << QLanes<D>::TB1)>(x);
}

// fp32 x + partner(x) on all lanes, partner = lane ^ 1, ^ 2, ^ 8 (DPP, one op)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(x), CTRL, 0xF, 0xF, true));
}

// Unnormalized Walsh-Hadamard butterflies over one token row, fp32, in the
// stage order h = 1, 2, ..., D/2 ((a, b) -> (a + b, a - b)).  Stages h = 1..8
// are in-lane.  The cross-lane stages (h = 16, 32, 64: chunk bits 0, 1, 2 =
// lane bits 0, 1, 3) are one v_fmac_f32_dpp each: z += s * z[partner] with
// s = -1 on the lane whose chunk bit is set.  That lane then holds -(a - b)
// instead of a - b; the values leave this function as sigma * y with
// sigma = (-1)^popcount(li), which the caller folds into its scale (the
// rounding of each stage is symmetric in sign, so sigma * y is exactly the
// negation of the correctly rounded stage result).
template <int D>
__device__ __forceinline__ void wht16(float (&z)[16], int lane) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (!(i & h)) {
        const float a = z[i], b = z[i + h];
        z[i] = a + b;
        z[i + h] = a - b;
      }
    }
  }
  const float s0 = (lane & 1) ? -1.f : 1.f;
  const float s1 = (lane & 2) ? -1.f : 1.f;
  // s_nop 1: a DPP source must not be written by the two preceding VALU ops
#define TQ_F16(ctl, s)                                                                              \
  "v_fmac_f32_dpp %0, %0, " s " " ctl "\n\tv_fmac_f32_dpp %1, %1, " s " " ctl "\n\t"                \
  "v_fmac_f32_dpp %2, %2, " s " " ctl "\n\tv_fmac_f32_dpp %3, %3, " s " " ctl "\n\t"                \
  "v_fmac_f32_dpp %4, %4, " s " " ctl "\n\tv_fmac_f32_dpp %5, %5, " s " " ctl "\n\t"                \
  "v_fmac_f32_dpp %6, %6, " s " " ctl "\n\tv_fmac_f32_dpp %7, %7, " s " " ctl "\n\t"                \
  "v_fmac_f32_dpp %8, %8, " s " " ctl "\n\tv_fmac_f32_dpp %9, %9, " s " " ctl "\n\t"                \
  "v_fmac_f32_dpp %10, %10, " s " " ctl "\n\tv_fmac_f32_dpp %11, %11, " s " " ctl "\n\t"            \
  "v_fmac_f32_dpp %12, %12, " s " " ctl "\n\tv_fmac_f32_dpp %13, %13, " s " " ctl "\n\t"            \
  "v_fmac_f32_dpp %14, %14, " s " " ctl "\n\tv_fmac_f32_dpp %15, %15, " s " " ctl "\n\t"
#define TQ_ZOPS                                                                                     \
  "+v"(z[0]), "+v"(z[1]), "+v"(z[2]), "+v"(z[3]), "+v"(z[4]), "+v"(z[5]), "+v"(z[6]), "+v"(z[7]),  \
      "+v"(z[8]), "+v"(z[9]), "+v"(z[10]), "+v"(z[11]), "+v"(z[12]), "+v"(z[13]), "+v"(z[14]),     \
      "+v"(z[15])
  if constexpr (D == 128) {
    const float s3 = (lane & 8) ? -1.f : 1.f;
    asm volatile("s_nop 1\n\t" TQ_F16("quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf", "%16")
                     TQ_F16("quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf", "%17")
                         TQ_F16("row_ror:8 row_mask:0xf bank_mask:0xf", "%18")
                 : TQ_ZOPS
                 : "v"(s0), "v"(s1), "v"(s3));
  } else {
    asm volatile("s_nop 1\n\t" TQ_F16("quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf", "%16")
                     TQ_F16("quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf", "%17")
                 : TQ_ZOPS
                 : "v"(s0), "v"(s1));
  }
#undef TQ_F16
#undef TQ_ZOPS
}

// sigma of wht16: (-1)^popcount(li)
__device__ __forceinline__ float wht16_sign(int li) { return (__builtin_popcount(li) & 1) ? -1.f : 1.f; }

// 4 x 4 byte transpose among the quad of tokens (tq = in-quad token index):
// lane tq receives byte tq of each of the four tokens' words, token order.
template <int D>
__device__ __forceinline__ uint32_t quad_transpose(uint32_t w, int tq) {
  const uint32_t t1 = tok_xor1(w);
  uint32_t t = __builtin_amdgcn_perm(t1, w, (tq & 1) ? 0x03070105u : 0x06020400u);
  const uint32_t t2 = tok_xor2<D>(t);
  return __builtin_amdgcn_perm(t2, t, (tq & 2) ? 0x03020706u : 0x05040100u);
}

// Is this lane's token one of four consecutive rows r*4 .. r*4+3 of one block,
// with the quad's tokens in order?  Every exchange runs on all lanes (a
// cross-lane read under a divergent mask would see inactive lanes).
template <int D>
__device__ __forceinline__ bool quad_aligned(int slot, int tq) {
  const int qid = (slot >= 0 && (slot & 3) == tq) ? (slot >> 2) : -1 - tq;
  const int qo = (int)tok_xor1((uint32_t)qid);
  const uint32_t pair_ok = (qid == qo && qid >= 0) ? 1u : 0u;
  const uint32_t other_ok = tok_xor2<D>(pair_ok);
  const int qp = (int)tok_xor2<D>((uint32_t)qid);
  return pair_ok && other_ok && qp == qid;
}

// Correctly rounded fp32 1/h for an fp16 h >= 0 given by its bits, from the
// table of significand reciprocals (recip[f] = fp32(1 / (1 + f/1024))); 1/h of
// a normal h is that entry times 2^(15 - E), an exact scaling.  Zero gives 0;
// subnormal h takes the division.
__device__ __forceinline__ float recip_f16(uint32_t hb, const float *s_recip) {
  if (hb == 0) return 0.f;
  if (hb < 0x400u) return __fdiv_rn(1.0f, (float)h_from((uint16_t)hb));
  return __builtin_amdgcn_ldexpf(s_recip[hb & 0x3FFu], 15 - (int)(hb >> 10));
}

// fp32 r -> fp16 RNE is decided safely from an approximation of r within a
// few ulps unless r lies near an fp16 rounding boundary (the low 13 bits of a
// normal fp16-range fp32 value near 0x1000) or outside the normal fp16 range.
__device__ __forceinline__ bool f16_round_safe(float r, uint32_t ulps) {
  const uint32_t b = as_u(r);
  const uint32_t m13 = b & 0x1FFFu;
  return r >= 0x1p-14f && r < 65504.0f && (m13 + ulps - 0x1000u) > 2u * ulps;
}

// v_min3 / v_max3 of finite values (written out so that bit-cast inputs need
// no canonicalizing instruction first)
__device__ __forceinline__ float min3f(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

template <int D>
struct RowLoad {
  uint4 k0, k1, v0, v1;  // 16 bf16 channels of K and of V
  int slot;
  bool valid;            // the lane's token exists
};

// Loads of the rows of one wave: tokens n0 + tw (n0 wave-uniform).  Tokens past
// the end are clamped to the last token, so every load is valid and
// unconditional; `valid` says whether the lane's token exists.  Addresses are a
// wave-uniform base plus a 32-bit lane offset.
template <int D>
__device__ __forceinline__ void load_row(RowLoad<D> &o, const QuantizeArgs &a, int64_t n0, int h, int tw, int li) {
  const int64_t last = a.num_tokens - 1;
  const int64_t b0 = n0 < last ? n0 : last;
  const int64_t span = last - b0;
  const int lim = span < 64 ? (int)span : 64;
  const int t = tw < lim ? tw : lim;
  const int64_t ubase = (b0 * a.hkv + h) * D;
  const uint32_t loff = ((uint32_t)t * (uint32_t)a.hkv * D + (uint32_t)li * 16u) * 2u;
  const uint8_t *kb = reinterpret_cast<const uint8_t *>(a.k + ubase);
  const uint8_t *vb = reinterpret_cast<const uint8_t *>(a.v + ubase);
  o.k0 = *reinterpret_cast<const uint4 *>(kb + loff);
  o.k1 = *reinterpret_cast<const uint4 *>(kb + loff + 16);
  o.v0 = *reinterpret_cast<const uint4 *>(vb + loff);
  o.v1 = *reinterpret_cast<const uint4 *>(vb + loff + 16);
  o.slot = (a.slots + b0)[t];
  o.valid = n0 <= last && tw <= span;
}

template <int D>
__device__ __forceinline__ uint32_t kword(const RowLoad<D> &r, int i) {
  const uint4 &q = i < 4 ? r.k0 : r.k1;
  const int j = i & 3;
  return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
}
template <int D>
__device__ __forceinline__ uint32_t vword(const RowLoad<D> &r, int i) {
  const uint4 &q = i < 4 ? r.v0 : r.v1;
  const int j = i & 3;
  return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
}

constexpr int kQuantThreads = 256;       // static loop: four waves per work-group
constexpr int kQuantThreadsBal = 1024;   // balanced loop: one work-group per compute unit

// The static persistent loop (launches with few tasks per wave).  A
// work-group task is (chunk of 4 * TPW tokens, kv-head): wave wv codes tokens
// chunk * 4 * TPW + wv * TPW + tw, so one work-group writes whole 16-token
// records.  The grid strides through the tasks, tracked as (chunk, head) pairs
// so the loop needs no 64-bit division.  Two row buffers: every step loads the
// next task into one (clamped to a valid task, so the loads are unconditional)
// while coding the other.  `stage` runs once, after the first loads are issued
// (table staging); `code(row, h)` codes one row.
template <int D, class Stage, class Code>
__device__ __forceinline__ void quantize_loop_static(const QuantizeArgs &a, int wv, int tw, int li, Stage stage,
                                                     Code code) {
  constexpr int TPW = QLanes<D>::TPW, WG_TOK = 4 * TPW;
  const int64_t chunks = (a.num_tokens + WG_TOK - 1) / WG_TOK;
  const int hkv = a.hkv;
  const int64_t gq = gridDim.x / hkv;
  const int gr = (int)(gridDim.x % hkv);
  auto advance = [&](int64_t &c, int &h) {
    c += gq;
    h += gr;
    if (h >= hkv) {
      h -= hkv;
      ++c;
    }
  };
  int64_t c = blockIdx.x / hkv;
  int h = (int)(blockIdx.x % hkv);
  RowLoad<D> ra, rb;
  load_row<D>(ra, a, c * WG_TOK + wv * TPW, h, tw, li);
  stage();
  while (c < chunks) {
    int64_t c2 = c;
    int h2 = h;
    advance(c2, h2);
    load_row<D>(rb, a, (c2 < chunks ? c2 : c) * WG_TOK + wv * TPW, c2 < chunks ? h2 : h, tw, li);
    code(ra, h);
    if (c2 >= chunks) break;
    c = c2;
    h = h2;
    advance(c2, h2);
    load_row<D>(ra, a, (c2 < chunks ? c2 : c) * WG_TOK + wv * TPW, c2 < chunks ? h2 : h, tw, li);
    code(rb, h);
    c = c2;
    h = h2;
  }
}

// Rows of one task of the balanced loop: the item of `len` tokens starting at
// token tb, whose first row sits at `lead` of its TPW-row span.  Lane token
// index tw takes token tb + tw - lead, so each row lands on the lanes of its
// own position in the span; the other lanes load a token of the item again
// (every load is valid) and are not `valid`.
template <int D>
__device__ __forceinline__ void load_item_row(RowLoad<D> &o, const QuantizeArgs &a, int64_t tb, int lead, int len,
                                              int h, int tw, int li) {
  const int j = tw - lead;
  const int t = j < 0 ? 0 : (j >= len ? len - 1 : j);
  const int64_t ubase = (tb * a.hkv + h) * D;
  const uint32_t loff = ((uint32_t)t * (uint32_t)a.hkv * D + (uint32_t)li * 16u) * 2u;
  const uint8_t *kb = reinterpret_cast<const uint8_t *>(a.k + ubase);
  const uint8_t *vb = reinterpret_cast<const uint8_t *>(a.v + ubase);
  o.k0 = *reinterpret_cast<const uint4 *>(kb + loff);
  o.k1 = *reinterpret_cast<const uint4 *>(kb + loff + 16);
  o.v0 = *reinterpret_cast<const uint4 *>(vb + loff);
  o.v1 = *reinterpret_cast<const uint4 *>(vb + loff + 16);
  o.slot = (a.slots + tb)[t];
  o.valid = j >= 0 && j < len;
}

// Most tokens one pass of the balanced loop lists (6 bytes of LDS each).
constexpr int kItemWindow = 8192;
static_assert(3 * kQuantThreadsBal <= kItemWindow, "the first round's slots are parked in the item list");

// The balanced persistent loop (launches with many tasks per wave).  One
// work-group of 16 waves per compute unit takes an equal contiguous range of
// the tokens and cuts it into items: the longest runs of tokens whose slots are
// consecutive rows of one aligned TPW-row span of a block (half a block at
// D = 128, the block at D = 64).  Tokens with a negative slot belong to no
// item.  A task is (item, kv-head), numbered item * Hkv + head; wave w starts
// with task w * grain and every later task (or pair of tasks) goes to the wave
// that asks first (an LDS counter), so the waves of a unit end together (with
// fixed shares per work-group, the unit's arbiter favours the oldest).  A
// wave puts row r of a span on its lanes of token index r mod TPW, so the rows
// of a whole item of four aligned rows sit where the record's four-row words
// want them, however the launch's token order is cut into sequences.  The
// range is listed in windows of at most a.window tokens (a work-group-wide
// ballot scan; items are cut at window edges).  Two row buffers: every step
// loads the next task into one (past the window's tasks, its first task again)
// while coding the other.  `stage` runs once (table staging); `code(row, h)`
// codes one row.
template <int D, class Stage, class Code>
__device__ __forceinline__ void quantize_loop_balanced(const QuantizeArgs &a, int wv, int tw, int li, Stage stage,
                                                       Code code) {
  constexpr int TPW = QLanes<D>::TPW;
  constexpr int NWAVE = kQuantThreadsBal / 64;
  __shared__ uint32_t s_first[kItemWindow];  // item k: window offset of its first token | its lead << 16
  __shared__ uint16_t s_last[kItemWindow];   // item k: window offset of its last token
  __shared__ int s_cnt[2][NWAVE];            // item starts and ends found by each wave in one round
  __shared__ int s_next;
  const int lane = (int)(threadIdx.x & 63);
  const int hkv = a.hkv;
  const int64_t n_tok = a.num_tokens, g = gridDim.x, b = blockIdx.x;
  const int64_t t_lo = n_tok * b / g, t_hi = n_tok * (b + 1) / g;
  const int win = a.window >= 1 && a.window <= kItemWindow ? a.window : kItemWindow;
  const int grain = a.grain;
  auto grab = [&]() {
    int x = 0;
    if (lane == 0) x = __hip_atomic_fetch_add(&s_next, grain, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return __builtin_amdgcn_readfirstlane(x);
  };
  // slots of window token i and of its neighbours (-1 past the window's
  // ends); the three loads are independent and always in range (0 <= i < wn)
  auto slots3 = [&](int64_t w0, int wn, int i, uint32_t &sl, uint32_t &sp, uint32_t &sn) {
    const int32_t *p = a.slots + w0;
    sl = (uint32_t)p[i];
    const uint32_t lp = (uint32_t)p[i > 0 ? i - 1 : 0], ln1 = (uint32_t)p[i + 1 < wn ? i + 1 : i];
    sp = i > 0 ? lp : 0xFFFFFFFFu;
    sn = i + 1 < wn ? ln1 : 0xFFFFFFFFu;
  };
  // the first round's slots are loaded before the table staging (the two
  // waits overlap) and parked in LDS, where each thread reads its own back
  {
    const int wn0 = (int)(t_hi - t_lo < win ? t_hi - t_lo : win);
    const int t0 = (int)threadIdx.x;
    uint32_t sl = 0, sp = 0, sn = 0;
    if (t0 < wn0) slots3(t_lo, wn0, t0, sl, sp, sn);
    stage();
    if (t0 < wn0) {
      s_first[3 * t0] = sl;
      s_first[3 * t0 + 1] = sp;
      s_first[3 * t0 + 2] = sn;
    }
  }
  for (int64_t w0 = t_lo; w0 < t_hi; w0 += win) {
    const int wn = (int)(t_hi - w0 < win ? t_hi - w0 : win);
    __syncthreads();  // the previous window's lists and counter are no longer used
    // ---- the window's items, in token order ------------------------------------
    // the thread index through an opaque copy, so that nothing the listing
    // derives from it is kept in registers through the task loop
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int ln = tid & 63;
    // items listed so far: by their starts and by their ends (an item can
    // start in one round and end in the next, so the two differ between rounds)
    int items = 0, ended = 0;
    for (int r0 = 0; r0 < wn; r0 += kQuantThreadsBal) {
      const int i = r0 + tid;
      bool st = false, en = false;
      uint32_t lead = 0;
      if (i < wn) {
        uint32_t sl, sp, sn;
        if (w0 == t_lo && r0 == 0) {  // parked above (i = this thread's index)
          sl = s_first[3 * i];
          sp = s_first[3 * i + 1];
          sn = s_first[3 * i + 2];
        } else {
          slots3(w0, wn, i, sl, sp, sn);
        }
        if ((int)sl >= 0) {
          // a row continues the item of the row before it when its slot is
          // the next one and not the first of a span
          st = (int)sp < 0 || sl != sp + 1u || (sl & (TPW - 1)) == 0;
          en = (int)sn < 0 || sn != sl + 1u || (sn & (TPW - 1)) == 0;
          lead = sl & (TPW - 1);
        }
      }
      const uint64_t bs = __builtin_amdgcn_ballot_w64(st), be = __builtin_amdgcn_ballot_w64(en);
      if (ln == 0) {
        s_cnt[0][wv] = __builtin_popcountll(bs);
        s_cnt[1][wv] = __builtin_popcountll(be);
      }
      __syncthreads();
      // the starts (ends) of the waves before this one and of all waves: lane
      // w < NWAVE holds wave w's counts, summed over lanes 0 .. NWAVE - 1
      static_assert(NWAVE == 16, "the sums below cover 16 lanes");
      const int cw = ln < NWAVE ? ln : 0;
      const int c_s = ln < NWAVE ? s_cnt[0][cw] : 0, c_e = ln < NWAVE ? s_cnt[1][cw] : 0;
      uint32_t pre_s = ln < wv ? c_s : 0, pre_e = ln < wv ? c_e : 0, tot_s = c_s, tot_e = c_e;
      pre_s += swz_xor_u<1>(pre_s);
      pre_e += swz_xor_u<1>(pre_e);
      tot_s += swz_xor_u<1>(tot_s);
      tot_e += swz_xor_u<1>(tot_e);
      pre_s += swz_xor_u<2>(pre_s);
      pre_e += swz_xor_u<2>(pre_e);
      tot_s += swz_xor_u<2>(tot_s);
      tot_e += swz_xor_u<2>(tot_e);
      pre_s += swz_xor_u<4>(pre_s);
      pre_e += swz_xor_u<4>(pre_e);
      tot_s += swz_xor_u<4>(tot_s);
      tot_e += swz_xor_u<4>(tot_e);
      pre_s += swz_xor_u<8>(pre_s);
      pre_e += swz_xor_u<8>(pre_e);
      tot_s += swz_xor_u<8>(tot_s);
      tot_e += swz_xor_u<8>(tot_e);
      // item number of this lane's start (end): the starts (ends) listed
      // before it.  Every item has one start and one end, so both lists end
      // with the same count, at most wn <= kItemWindow
      const int ps = items + __builtin_amdgcn_readfirstlane((int)pre_s) +
                     (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bs >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bs, 0u));
      const int pe = ended + __builtin_amdgcn_readfirstlane((int)pre_e) +
                     (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0u));
      if (st) s_first[ps] = (uint32_t)i | (lead << 16);
      if (en) s_last[pe] = (uint16_t)i;
      items += __builtin_amdgcn_readfirstlane((int)tot_s);
      ended += __builtin_amdgcn_readfirstlane((int)tot_e);
      __syncthreads();  // the counts are read before the next round writes them; the lists are complete
    }
    const int ntask = items * hkv;
    if (ntask == 0) continue;  // work-group-uniform
    if (tid == 0) s_next = grain * NWAVE;
    __syncthreads();
    // ---- the window's tasks ---------------------------------------------------------
    // task n (past the window's tasks: task 0) as (first token, lead, length, head)
    auto locate = [&](int n, int64_t &tb, int &lead, int &len, int &h) {
      const int m = n < ntask ? n : 0;
      const int k = m / hkv;
      h = m - k * hkv;
      const uint32_t e = (uint32_t)__builtin_amdgcn_readfirstlane((int)s_first[k]);
      const int i0 = (int)(e & 0xFFFFu);
      lead = (int)(e >> 16);
      const int l = __builtin_amdgcn_readfirstlane((int)s_last[k]) - i0 + 1;
      len = l < 1 ? 1 : l;  // always >= 1 for a complete list; kept so for every load
      tb = w0 + i0;
    };
    int n = grain * wv, h, lead, len;
    int64_t tb;
    locate(n, tb, lead, len, h);
    RowLoad<D> ra, rb;
    load_item_row<D>(ra, a, tb, lead, len, h, tw, li);
    while (n < ntask) {
      const int n2 = grain == 2 ? n + 1 : grab();  // the pair's second task, or the next one
      int h2, lead2, len2;
      int64_t tb2;
      locate(n2, tb2, lead2, len2, h2);
      load_item_row<D>(rb, a, tb2, lead2, len2, h2, tw, li);
      code(ra, h);
      if (n2 >= ntask) break;
      n = grab();
      locate(n, tb, lead, len, h);
      load_item_row<D>(ra, a, tb, lead, len, h, tw, li);
      code(rb, h2);
    }
  }
}

// The loop a launch runs: BAL selects the balanced one.
template <int D, bool BAL, class Stage, class Code>
__device__ __forceinline__ void quantize_loop(const QuantizeArgs &a, int wv, int tw, int li, Stage stage, Code code) {
  if constexpr (BAL) quantize_loop_balanced<D>(a, wv, tw, li, stage, code);
  else quantize_loop_static<D>(a, wv, tw, li, stage, code);
}

// Launch geometry of a quantize launch, by wave tasks (TPW tokens, one
// kv-head) per wave slot of the chip (16 per compute unit):
// * under 8: the static loop: work-group tasks of 4 * TPW tokens and one
//   kv-head, as many 4-wave work-groups as fit at once (at most one per task);
// * 8 to 31: the balanced loop, one 16-wave work-group per compute unit,
//   tasks handed out in pairs;
// * 32 and more: the balanced loop, tasks handed out one by one.
// Measured: single hand-outs take 8% off launches with 50 and more tasks per
// wave and cost 4% at 8, where pairs (half the counter's round trips) take 2%
// off instead; pairs cost 1.5% on the long launches (coarser balance).
struct QuantGeometry {
  bool balanced;
  int grain;   // balanced loop: tasks per hand-out
  int window;  // balanced loop: tokens listed per pass
  int grid, threads;
};
QuantGeometry quantize_geometry(const void *kernel_static, const void *kernel_balanced, int d, int64_t num_tokens,
                                int hkv);

}  // namespace tq
