// Pieces shared by the TQ4/4 and MX-FP4 decode kernels: the query rotation,
// the online-softmax state and the end-of-work-group merge.
#pragma once

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

constexpr float kNegInf = -__builtin_huge_valf();
// A running maximum is only raised when a block's maximum exceeds it by more
// than this (log2 units), so most blocks skip the accumulator rescale; the
// probabilities then stay below 2^kLazyRescale.
constexpr float kLazyRescale = 8.0f;

// A copy of a loaded value made by a VALU move the compiler cannot see
// through.  Reading the copy later (v_readlane in the block loop) then carries
// no dependency on an outstanding vector load, so the compiler's wait before
// it does not drain the loads in flight (it emits vmcnt(0) for the loaded
// register itself).
__device__ __forceinline__ int settled(int x) {
  int y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
  return y;
}

template <int GQ>
__device__ __forceinline__ float xor_g(float x) {
  if constexpr (GQ == 1) return xor1(x);
  else if constexpr (GQ == 2) return xor2(x);
  else if constexpr (GQ == 4) return xor4(x);
  else return xor8(x);
}

// a + b on the lane holding a, a - b on the lane holding b, for lane xor 16 / 32
__device__ __forceinline__ float bfly16(float x, float sgn) {
  auto p = __builtin_amdgcn_permlane16_swap(as_u(x), as_u(x), false, false);
  return __builtin_fmaf(sgn, as_f(p[1]), as_f(p[0]));
}
__device__ __forceinline__ float bfly32(float x, float sgn) {
  auto p = __builtin_amdgcn_permlane32_swap(as_u(x), as_u(x), false, false);
  return __builtin_fmaf(sgn, as_f(p[1]), as_f(p[0]));
}

// One wave rotates one query row of D channels: unnormalized Walsh-Hadamard
// butterflies in fp32 in the stage order h = 1, 2, ..., D/2 (the order the
// record format fixes).  D = 128: lane l holds channels 2l, 2l+1 (stage h = 1
// in-lane, h = 2..64 over lane xor 1..32); D = 64: lane l holds channel l.
// `w` is this lane's query word (load_query_word).
template <int D>
__device__ __forceinline__ uint32_t load_query_word(const uint16_t *q, int lane) {
  if constexpr (D == 128) return reinterpret_cast<const uint32_t *>(q)[lane];
  else return (uint32_t)q[lane];
}
template <int D>
__device__ __forceinline__ void rotate_row(uint32_t w, int lane, float &x0, float &x1) {
  if constexpr (D == 128) {
    const float a = bf16_lo(w), b = bf16_hi(w);
    x0 = a + b;
    x1 = a - b;
  } else {
    x0 = as_f(w << 16);
    x1 = 0.f;
  }
  const float s1 = (lane & 1) ? -1.f : 1.f, s2 = (lane & 2) ? -1.f : 1.f, s4 = (lane & 4) ? -1.f : 1.f;
  const float s8 = (lane & 8) ? -1.f : 1.f, s16 = (lane & 16) ? -1.f : 1.f, s32 = (lane & 32) ? -1.f : 1.f;
  x0 = __builtin_fmaf(s1, x0, xor1(x0));
  x1 = __builtin_fmaf(s1, x1, xor1(x1));
  x0 = __builtin_fmaf(s2, x0, xor2(x0));
  x1 = __builtin_fmaf(s2, x1, xor2(x1));
  x0 = __builtin_fmaf(s4, x0, xor4(x0));
  x1 = __builtin_fmaf(s4, x1, xor4(x1));
  x0 = __builtin_fmaf(s8, x0, xor8(x0));
  x1 = __builtin_fmaf(s8, x1, xor8(x1));
  x0 = bfly16(x0, s16);
  x1 = bfly16(x1, s16);
  x0 = bfly32(x0, s32);
  x1 = bfly32(x1, s32);
}

// Channel of element e (0 or 1) of lane l after rotate_row.
template <int D>
__device__ __forceinline__ int rotated_channel(int lane, int e) {
  return D == 128 ? 2 * lane + e : lane;
}

// Work-group -> (sequence, kv-head, split).  Logical ids (after the XCD remap,
// which gives each XCD a contiguous range) run split-fastest, then sequence,
// then kv-head: each XCD gets whole kv-heads (every split of every sequence),
// so the XCDs carry equal work whatever the context lengths, and sequences
// that share prefix blocks read them through the same L2.
struct WgTask {
  int b, kvh, sp;
};
__device__ __forceinline__ WgTask decode_task(const DecodeArgs &a) {
  const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
  WgTask t;
  t.sp = (int)(wg % (uint32_t)a.nsplit);
  const uint32_t rest = wg / (uint32_t)a.nsplit;
  t.b = (int)(rest % (uint32_t)a.batch);
  t.kvh = (int)(rest / (uint32_t)a.batch);
  return t;
}

// A running maximum that starts finite, so that a column whose tokens are all
// masked so far gets p = 2^(-inf - m) = 0 rather than 2^(-inf + inf).
constexpr float kMtFloor = -1.0e30f;

// Multi-token work-group -> (sequence or group, kv-head, row tile, split).
struct MtTask {
  int b, kvh, rt, sp;
};

__device__ __forceinline__ MtTask mt_task(const MultiTokenArgs &a) {
  // row tiles fastest, then splits, sequences, kv-heads; each XCD gets a
  // contiguous range, so the work-groups that read the same blocks share an L2
  const uint32_t wg = xcd_logical_id(blockIdx.x, gridDim.x);
  MtTask t;
  t.rt = (int)(wg % (uint32_t)a.row_tiles);
  uint32_t rest = wg / (uint32_t)a.row_tiles;
  t.sp = (int)(rest % (uint32_t)a.nsplit);
  rest /= (uint32_t)a.nsplit;
  t.b = (int)(rest % (uint32_t)a.batch);
  t.kvh = (int)(rest / (uint32_t)a.batch);
  return t;
}

// Per-wave online-softmax state for the 16 operand columns.  Column n < g is
// query head n (high fp16 part), g <= n < 2g the same head's low part.
template <int G2>  // number of PV accumulator tiles (2 * D / 32)
struct WaveState {
  float m;          // running reference maximum (log2 units), per column
  float l;          // running sum of probabilities over this lane's tokens
  float4v acc[G2];  // out^T tiles: rows = channels, columns = operand columns
};

// Online softmax over one 16-token block with lazy rescale.  x: this lane's
// four logits (log2 units; -inf for rows past the context), column n = lane %
// 16; the four lanes n, n+16, n+32, n+48 of a column share its running max.
// The common case needs no cross-lane work: a lane only checks whether one of
// its own logits exceeds the running max by more than kLazyRescale; when some
// lane does, the columns' block maxima are reduced and the raised columns
// rescale their accumulators.  Leaves p = 2^(x - m) and adds them to st.l.
template <int G2>
__device__ __forceinline__ void softmax_block(const float (&x)[4], WaveState<G2> &st, float (&p)[4]) {
  // v_max3 + v_max written out: the logits need no canonicalizing first
  float lm;
  __asm__("v_max3_f32 %0, %1, %2, %3\n\tv_max_f32 %0, %0, %4"
          : "=&v"(lm)
          : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
  if (__builtin_amdgcn_ballot_w64(lm > st.m + kLazyRescale) != 0) {
    float bm = __builtin_fmaxf(lm, xor16(lm));
    bm = __builtin_fmaxf(bm, xor32(bm));
    const bool raise = bm > st.m + kLazyRescale;
    const float m_new = raise ? bm : st.m;
    const float alpha = (st.m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int t = 0; t < G2; ++t) st.acc[t] *= alpha;
    st.m = m_new;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - st.m);
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
}

// Combine the NW waves of a work-group and write either the output (single
// split) or a split partial.  s_m / s_l / s_acc are LDS scratch.  CASCADE:
// always a partial, at slot sp of rows of a.part_stride slots.
// Tiles 0 .. 2D/32 - 1 of st are the output tiles (a state may carry more).
template <int D, int GQ, int NW, bool CASCADE = false, int NA>
__device__ __forceinline__ void finish_workgroup(const DecodeArgs &a, WaveState<NA> &st, int b, int qh0,
                                                 int sp, float (*s_m)[GQ], float (*s_l)[GQ],
                                                 float (*s_acc)[GQ][D]) {
  constexpr int G = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane >> 4, n = lane & 15;
  float l = st.l;
  l += xor16(l);
  l += xor32(l);
#pragma unroll
  for (int t = 0; t < 2 * G; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st.acc[t][i] += xor_g<GQ>(st.acc[t][i]);
  }
  if (n < GQ) {
#pragma unroll
    for (int gp = 0; gp < G; ++gp) {
#pragma unroll
      for (int par = 0; par < 2; ++par) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s_acc[wv][n][32 * gp + 2 * (4 * r + i) + par] = st.acc[2 * gp + par][i];
      }
    }
    if (r == 0) {
      s_m[wv][n] = st.m;
      s_l[wv][n] = l;
    }
  }
  __syncthreads();
  for (int i = tid; i < GQ * D; i += NW * 64) {
    const int hh = i / D, c = i % D;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = __builtin_fmaxf(mx, s_m[w][hh]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_m[w][hh];
      const float f = (mw == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(mw - mx);
      num += f * s_acc[w][hh][c];
      den += f * s_l[w][hh];
    }
    const int64_t row = (int64_t)b * a.hq + qh0 + hh;
    if (!CASCADE && a.nsplit == 1) {
      const float o = den > 0.f ? num / den : 0.f;
      if (a.out_bf16) reinterpret_cast<uint16_t *>(a.out)[row * D + c] = f32_to_bf16(o);
      else reinterpret_cast<float *>(a.out)[row * D + c] = o;
    } else {
      const int64_t pi = row * (CASCADE ? a.part_stride : a.nsplit) + sp;
      a.part_acc[pi * D + c] = num;
      if (c == 0) {
        a.part_ml[pi * 2] = mx;
        a.part_ml[pi * 2 + 1] = den;
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void write_zero_rows(const DecodeArgs &a, int b, int qh0, int gq) {
  for (int i = threadIdx.x; i < gq * D; i += blockDim.x) {
    const int64_t o = ((int64_t)b * a.hq + qh0) * D + i;
    if (a.out_bf16) reinterpret_cast<uint16_t *>(a.out)[o] = 0;
    else reinterpret_cast<float *>(a.out)[o] = 0.f;
  }
}

// Combine the split partials of one output row (one work-group of 256 threads)
// in one pass over them.  Thread (cq, sl) takes channels 4*cq .. 4*cq+3 of
// splits sl, sl + SL, ..., in chunks of 8 splits whose loads (maxima, sums,
// accumulators) are all issued before any is used, and keeps a running
// maximum m with its sum and accumulators scaled to 2^-m (an online softmax
// over partials); the SL slices are rescaled to the largest maximum when they
// are added in LDS.  The first chunk may be loaded before the row's count of
// partials is known (it waits on a context length): it reads slots below
// nload, which are inside the row's workspace whether or not they hold one of
// its partials, and the ones at or past ns are dropped by selection (their
// contents may be anything, NaN included).
struct MergeView {
  const float *part_ml;   // [rows][nsplit][2]: (max, sum) in log2 units
  const float *part_acc;  // [rows][nsplit][d]
  void *out;              // fp32 / bf16 [rows][d]
  int32_t nsplit;         // partial slots per row
  int32_t out_bf16;
};

// The partial slots of a row in order: the first ns (plain split-K).
struct SlotsDirect {
  __device__ __forceinline__ int operator()(int k) const { return k; }
};
// Two runs of slots: [0, n0), then [lo1, lo1 + ns - n0) (cascade: the
// sequence's own splits, then its shared-prefix splits).
struct SlotsTwoRuns {
  int n0, lo1;
  __device__ __forceinline__ int operator()(int k) const { return k < n0 ? k : lo1 + (k - n0); }
};

// nload >= 1: chunk 0 reads slots slot(k), k < nload, before the row's count
// of partials ns = ns_fn() is asked for (slot(k) for k < nload must lie in
// the row's workspace); ns = 0 writes a zero row.
template <int D, typename NsFn, typename Slots>
__device__ __forceinline__ void merge_row_impl(const MergeView &v, int64_t row, int nload, NsFn ns_fn,
                                               Slots slot) {
  constexpr int CQ = D / 4;          // channel quads
  constexpr int SL = 256 / CQ;       // split lanes
  constexpr int CH = 8;              // splits per thread per chunk
  __shared__ float s_m[SL][CQ], s_l[SL][CQ];
  __shared__ float4 s_acc[SL][CQ];
  const int tid = threadIdx.x, cq = tid % CQ, sl = tid / CQ;
  const float2 *ml = reinterpret_cast<const float2 *>(v.part_ml + row * v.nsplit * 2);
  const float *pa = v.part_acc + row * v.nsplit * D;
  float2 c_ml[CH];
  float4 c_v[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int sp = min(sl + j * SL, nload - 1);
    c_ml[j] = ml[slot(sp)];
    c_v[j] = *reinterpret_cast<const float4 *>(pa + (int64_t)slot(sp) * D + 4 * cq);
  }
  // chunk 0 is processed unconditionally (no partial in it counts when ns = 0,
  // which then writes zeros), so its loads stay ahead of the use of ns
  const int ns = ns_fn();
  float m = kNegInf, den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  auto take = [&](int base) {
    bool in[CH];
    float cm = m;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      in[j] = base + sl + j * SL < ns && c_ml[j].x != kNegInf;
      if (in[j]) cm = __builtin_fmaxf(cm, c_ml[j].x);
    }
    if (cm != m) {  // the running maximum rises (from -inf on the first partial)
      const float r = m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - cm);
      den *= r;
      num.x *= r;
      num.y *= r;
      num.z *= r;
      num.w *= r;
      m = cm;
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (in[j]) {
        const float f = __builtin_amdgcn_exp2f(c_ml[j].x - m);
        den = __builtin_fmaf(f, c_ml[j].y, den);
        num.x = __builtin_fmaf(f, c_v[j].x, num.x);
        num.y = __builtin_fmaf(f, c_v[j].y, num.y);
        num.z = __builtin_fmaf(f, c_v[j].z, num.z);
        num.w = __builtin_fmaf(f, c_v[j].w, num.w);
      }
    }
  };
  take(0);
  for (int base = CH * SL; base < ns; base += CH * SL) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int sp = min(base + sl + j * SL, ns - 1);
      c_ml[j] = ml[slot(sp)];
      c_v[j] = *reinterpret_cast<const float4 *>(pa + (int64_t)slot(sp) * D + 4 * cq);
    }
    take(base);
  }
  s_m[sl][cq] = m;
  s_l[sl][cq] = den;
  s_acc[sl][cq] = num;
  __syncthreads();
  if (sl == 0) {
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < SL; ++i) M = __builtin_fmaxf(M, s_m[i][cq]);
    float L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      const float mi = s_m[i][cq];
      const float w = mi == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mi - M);
      L = __builtin_fmaf(w, s_l[i][cq], L);
      o.x = __builtin_fmaf(w, s_acc[i][cq].x, o.x);
      o.y = __builtin_fmaf(w, s_acc[i][cq].y, o.y);
      o.z = __builtin_fmaf(w, s_acc[i][cq].z, o.z);
      o.w = __builtin_fmaf(w, s_acc[i][cq].w, o.w);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const float ov[4] = {o.x * inv, o.y * inv, o.z * inv, o.w * inv};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t oi = row * D + 4 * cq + c;
      if (v.out_bf16) reinterpret_cast<uint16_t *>(v.out)[oi] = f32_to_bf16(ov[c]);
      else reinterpret_cast<float *>(v.out)[oi] = ov[c];
    }
  }
}

// ns: partials that hold this row's tokens (0: the row attends to nothing and
// is written as zeros); slot(k) is the slot of the k-th.
template <int D, typename Slots = SlotsDirect>
__device__ __forceinline__ void merge_row(const MergeView &v, int64_t row, int ns, Slots slot = Slots()) {
  if (ns == 0) {  // no partial exists to read
    for (int c = threadIdx.x; c < D; c += 256) {
      if (v.out_bf16) reinterpret_cast<uint16_t *>(v.out)[row * D + c] = 0;
      else reinterpret_cast<float *>(v.out)[row * D + c] = 0.f;
    }
    return;
  }
  merge_row_impl<D>(v, row, ns, [ns]() { return ns; }, slot);
}

}  // namespace tq
