// Internal declarations shared by the host library and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tq {

constexpr int kMaxBins = 256;    // key-coder bins (indexed by a saturating byte conversion)
constexpr int kMaxGqa = 8;       // query heads per kv-head handled by one work-group

// Device-side tables of one cache (one allocation, laid out in this order).
struct DeviceTables {
  uint32_t lut2[256];            // byte -> (fp16 c[lo nibble], fp16 c[hi nibble])
  float2 bins[kMaxBins];         // key coder: (threshold inside the bin or +inf, code below as int bits)
  float recip[1024];             // fp32(1 / (1 + f/1024)), correctly rounded: 1/x of fp16 significands
};

// Key-coder bin parameters: bin(u) = clamp(floor(u * a + b), 0, nbins - 1).
struct BinParams {
  float a, b;
  int nbins;
};

struct QuantizeArgs {
  const uint16_t *k, *v;         // bf16 [n][hkv][d]
  const int32_t *slots;          // [n]
  int64_t num_tokens;
  int32_t hkv;
  uint8_t *pool;
  int64_t num_blocks;
  const DeviceTables *tables;
  BinParams bins;
  float rsqrt_d;                 // fp32(1/sqrt(d))
  int32_t grain;                 // balanced quantize loop: tasks per hand-out (1 or 2)
  int32_t window;                // balanced quantize loop: tokens listed per pass (1 .. kItemWindow)
};

struct DecodeArgs {
  const uint16_t *q;             // bf16 [batch][hq][d]
  void *out;                     // fp32 / bf16 [batch][hq][d]
  const int32_t *block_table;    // [batch][max_blocks]
  const int32_t *ctx;            // [batch]
  const uint8_t *pool;
  const DeviceTables *tables;
  float *part_ml;                // [batch][hq][nsplit][2] (max, sum) in log2 units
  float *part_acc;               // [batch][hq][nsplit][d]
  float qscale;                  // TQ4/4: softmax_scale * log2(e) * fp32(1/sqrt(d)); MX-FP4: softmax_scale * log2(e)
  float rsqrt_d;                 // fp32(1/sqrt(d)), the rotation's normalization (MX-FP4 query)
  int32_t max_blocks, batch, hq, hkv, g;
  int32_t split_blocks;          // blocks per work-group
  int32_t nsplit;                // splits per (sequence, kv-head)
  int32_t out_bf16;
  // cascade decode only: the sequence's first block of its own (after the
  // shared prefix), and partial slots per row (own splits, then the prefix's)
  const int32_t *first_blk;      // [batch]
  const int32_t *depth;          // [batch]: shared-block groups the sequence is in
  int32_t part_stride;
};

struct MultiTokenArgs {
  const uint16_t *q;             // bf16 [num_tokens][hq][d]
  void *out;                     // fp32 / bf16 [num_tokens][hq][d]
  const int32_t *q_start;        // [batch + 1]: query tokens of sequence b are q_start[b] .. q_start[b+1]-1
  const int32_t *block_table;    // [batch][max_blocks]
  const int32_t *ctx;            // [batch]: context lengths, query tokens included
  const uint8_t *pool;
  const DeviceTables *tables;
  float *part_ml;                // [num_tokens][hq][nsplit][2]
  float *part_acc;               // [num_tokens][hq][nsplit][d]
  float qscale;                  // TQ4: softmax_scale * log2(e) * fp32(1/sqrt(d)); MX-FP4: softmax_scale * log2(e)
  float rsqrt_d;                 // fp32(1/sqrt(d)) (MX-FP4: the query's scale before e4m3)
  int32_t max_blocks, batch, hq, hkv, g;
  int32_t max_query_len;         // bound on q_start[b+1] - q_start[b]
  int32_t rows_per_wg;           // 16 or 32 (direct kernel), 64, 128 or 256 query rows per work-group
  int32_t row_tiles;             // row tiles per (sequence, kv-head)
  int32_t split_blocks, nsplit;
  int32_t out_bf16;
  // shared-prefix mode (the prefix pass of cascade decode): work-groups walk
  // groups instead of sequences (batch = number of groups, max_query_len =
  // largest group); group i's members are group_seqs[group_start[i] ..
  // group_start[i+1]), its shared blocks group_blocks[2i] .. group_blocks[2i+1]
  // - 1 of its first member's table, its depth group_depth[i]; one split per
  // group (split_blocks >= the largest group), whose partial goes to slot
  // slot0 + depth of rows of part_stride slots
  const int32_t *group_start;
  const int32_t *group_seqs;
  const int32_t *group_blocks;
  const int32_t *group_depth;
  int32_t part_stride, slot0;
};

// The fixed device scratch of tq_decode_attention_noalloc (noalloc.hip):
// its size, and its address on the current device (looked up on the first
// call per device).
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void **ptr);

// Launchers (defined next to their kernels).
hipError_t launch_tq4_quantize(int d, int vbits, const QuantizeArgs &a, hipStream_t s);
hipError_t launch_tq4_decode(int d, int vbits, const DecodeArgs &a, hipStream_t s);
hipError_t launch_mxfp4_quantize(const QuantizeArgs &a, hipStream_t s);
hipError_t launch_mxfp4_decode(const DecodeArgs &a, hipStream_t s);
hipError_t launch_mxfp4_cascade_decode(const DecodeArgs &a, hipStream_t s);
hipError_t launch_mxfp4_multitoken(const MultiTokenArgs &a, hipStream_t s);
hipError_t launch_mxfp4_prefix_attention(const MultiTokenArgs &a, hipStream_t s);
hipError_t launch_decode_merge(int d, const DecodeArgs &a, hipStream_t s);
hipError_t launch_tq4_multitoken(int d, int vbits, const MultiTokenArgs &a, hipStream_t s);
hipError_t launch_prefix_attention(int d, int vbits, const MultiTokenArgs &a, hipStream_t s);
hipError_t launch_multitoken_merge(int d, const MultiTokenArgs &a, hipStream_t s);
hipError_t launch_tq4_cascade_decode(int d, int vbits, const DecodeArgs &a, hipStream_t s);
hipError_t launch_cascade_merge(int d, const DecodeArgs &a, hipStream_t s);
hipError_t launch_debug_dequant(int format, int d, const uint8_t *pool, int64_t num_blocks, int hkv,
                                const int32_t *ids, int64_t n, const DeviceTables *tables, float *k_out,
                                float *v_out, hipStream_t s);
size_t calibrate_workspace_bytes(int64_t layers, int64_t rows, int d);
hipError_t launch_calibrate(int d, int layers, int64_t rows, const uint16_t *k, const uint16_t init_f16[16],
                            int max_iters, float rsqrt_d, void *workspace, uint16_t *tables, double *levels,
                            double *mse, int32_t *updates, hipStream_t stream);

// Host table construction (pure C++, no HIP calls).
void lloyd_max_gaussian16(double out[16]);
uint16_t f64_to_f16_rne(double x);
double f16_to_f64(uint16_t h);
// Builds lut2, the key-coder bins and the reciprocal table from an fp16 table;
// false if the table's midpoints are too close for kMaxBins bins.
bool build_key_tables(const uint16_t table_f16[16], DeviceTables *t, BinParams *bp);

// Byte offsets of the sections of one (16-token block, kv-head) record (the
// layout tq.h states).  TQ4/4 and TQ4/2 (VB = value bits): key codes, value
// codes, value (scale, min), key scales; at D = 128 the record is padded to
// whole 128-byte lines, so that records and their large sections start on a
// line and the quantize writes whole lines.
template <int D, int VB>
struct TqRec {
  static constexpr int KC = 0;
  static constexpr int VC = KC + 16 * (D / 2);
  static constexpr int VM = VC + 16 * (D / 2) * VB / 4;
  static constexpr int KS = VM + 16 * (D / 32) * 4;
  static constexpr int END = KS + 32;
  static constexpr int BYTES = D == 128 ? (END + 127) / 128 * 128 : END;
};
// MX-FP4 (D = 128): key codes, value codes, key exponents, value exponents
// (2176 bytes: whole lines).
struct MxRec {
  static constexpr int KC = 0, VC = 1024, KS = 2048, VS = 2112, BYTES = 2176;
};

// Record sizes.
inline size_t tq4_record_bytes(int d) { return d == 128 ? TqRec<128, 4>::BYTES : TqRec<64, 4>::BYTES; }
inline size_t tq4v2_record_bytes(int d) { return d == 128 ? TqRec<128, 2>::BYTES : TqRec<64, 2>::BYTES; }
inline size_t mxfp4_record_bytes(int) { return MxRec::BYTES; }

// Split-K plan shared by the workspace query and the launch.
struct SplitPlan {
  int split_blocks, nsplit;
};
SplitPlan plan_split(int batch, int hkv, int max_context_len);
// Multi-token attention: `units` work-groups per split (sequences x kv-heads x
// row tiles); splits only when the units alone leave compute units idle, at
// most max_split_blocks blocks per work-group.
SplitPlan plan_split_multitoken(int64_t units, int max_context_len, int max_split_blocks);

}  // namespace tq
