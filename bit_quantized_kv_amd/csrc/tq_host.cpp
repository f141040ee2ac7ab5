// C-ABI of the 4-bit KV-cache library: argument checks, handle and table
// management, launch planning.  Every compute step runs in the HIP kernels.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/tq.h"
#include "tq_internal.h"

struct tq_cache {
  tq_cache_desc desc;
  size_t record_bytes;
  size_t pool_bytes;
  uint8_t *pool;
  bool owns_pool;
  tq::DeviceTables *tables;  // device
  tq::BinParams bins;
  uint16_t table_f16[16];
  // cascade decode: a second stream (default priority) on which the
  // shared-block pass runs beside the decode of the sequences' own tokens,
  // forked from and joined to the caller's stream with two events; created on
  // first use
  hipStream_t aux = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

namespace {

thread_local std::string g_last_error;

tq_status fail(tq_status st, const std::string &msg) {
  g_last_error = msg;
  return st;
}

tq_status hip_fail(hipError_t e, const char *what) {
  return fail(TQ_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

tq_status check_desc(const tq_cache_desc *d, size_t *record) {
  if (!d) return fail(TQ_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->block_size != 16) return fail(TQ_ERR_INVALID_ARG, "block_size must be 16");
  if (d->num_kv_heads < 1 || d->num_kv_heads > 65536)
    return fail(TQ_ERR_INVALID_ARG, "num_kv_heads must be in [1, 65536]");
  if (d->num_blocks < 1) return fail(TQ_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (d->format == TQ_FORMAT_TQ4 || d->format == TQ_FORMAT_TQ4V2) {
    if (d->head_dim != 64 && d->head_dim != 128)
      return fail(TQ_ERR_UNSUPPORTED, "TQ4/4 and TQ4/2 support head_dim 64 and 128");
    *record = d->format == TQ_FORMAT_TQ4 ? tq::tq4_record_bytes(d->head_dim) : tq::tq4v2_record_bytes(d->head_dim);
  } else if (d->format == TQ_FORMAT_MXFP4) {
    if (d->head_dim != 128) return fail(TQ_ERR_UNSUPPORTED, "MX-FP4 supports head_dim 128");
    if (d->key_table) return fail(TQ_ERR_INVALID_ARG, "MX-FP4 takes no key table");
    *record = tq::mxfp4_record_bytes(d->head_dim);
  } else {
    return fail(TQ_ERR_INVALID_ARG, "unknown format");
  }
  const double total = (double)*record * (double)d->num_blocks * (double)d->num_kv_heads;
  if (total > 9.0e18) return fail(TQ_ERR_INVALID_ARG, "pool size overflows");
  return TQ_OK;
}

}  // namespace

extern "C" {

const char *tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported";
    case TQ_ERR_OOM: return "out of device memory";
    case TQ_ERR_WORKSPACE: return "workspace too small";
    case TQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *tq_last_error(void) { return g_last_error.c_str(); }

tq_status tq_record_bytes(const tq_cache_desc *desc, size_t *bytes) {
  if (!bytes) return fail(TQ_ERR_INVALID_ARG, "bytes is NULL");
  size_t rec;
  tq_status st = check_desc(desc, &rec);
  if (st != TQ_OK) return st;
  *bytes = rec;
  return TQ_OK;
}

tq_status tq_pool_bytes(const tq_cache_desc *desc, size_t *bytes) {
  if (!bytes) return fail(TQ_ERR_INVALID_ARG, "bytes is NULL");
  size_t rec;
  tq_status st = check_desc(desc, &rec);
  if (st != TQ_OK) return st;
  *bytes = rec * (size_t)desc->num_blocks * (size_t)desc->num_kv_heads;
  return TQ_OK;
}

tq_status tq_default_key_table(uint16_t out_f16[16]) {
  if (!out_f16) return fail(TQ_ERR_INVALID_ARG, "output is NULL");
  double c[16];
  tq::lloyd_max_gaussian16(c);
  for (int i = 0; i < 16; ++i) out_f16[i] = tq::f64_to_f16_rne(c[i]);
  return TQ_OK;
}

tq_status tq_create_cache(const tq_cache_desc *desc, void *pool, size_t pool_bytes, tq_cache **out) {
  if (!out) return fail(TQ_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  size_t rec;
  tq_status st = check_desc(desc, &rec);
  if (st != TQ_OK) return st;
  const size_t need = rec * (size_t)desc->num_blocks * (size_t)desc->num_kv_heads;
  if (pool && pool_bytes < need) return fail(TQ_ERR_INVALID_ARG, "pool smaller than tq_pool_bytes");

  tq_cache c{};
  c.desc = *desc;
  c.desc.key_table = nullptr;
  c.record_bytes = rec;
  c.pool_bytes = need;
  tq::DeviceTables host_tables{};
  if (desc->format != TQ_FORMAT_MXFP4) {
    if (desc->key_table) {
      for (int i = 0; i < 16; ++i) {
        if (!std::isfinite(desc->key_table[i])) return fail(TQ_ERR_INVALID_ARG, "key table entries must be finite");
        c.table_f16[i] = tq::f64_to_f16_rne((double)desc->key_table[i]);
        if ((c.table_f16[i] & 0x7c00u) == 0x7c00u) return fail(TQ_ERR_INVALID_ARG, "key table entry overflows fp16");
      }
      for (int i = 0; i < 15; ++i)
        if (!(tq::f16_to_f64(c.table_f16[i]) < tq::f16_to_f64(c.table_f16[i + 1])))
          return fail(TQ_ERR_INVALID_ARG, "key table must be strictly ascending after rounding to fp16");
    } else {
      tq_default_key_table(c.table_f16);
    }
    if (!tq::build_key_tables(c.table_f16, &host_tables, &c.bins))
      return fail(TQ_ERR_UNSUPPORTED, "key table midpoints are too close for the coder's bin table");
  }

  hipError_t e;
  if (pool) {
    c.pool = static_cast<uint8_t *>(pool);
    c.owns_pool = false;
  } else {
    e = hipMalloc(&c.pool, need);
    if (e != hipSuccess) return fail(TQ_ERR_OOM, std::string("pool allocation failed: ") + hipGetErrorString(e));
    c.owns_pool = true;
    e = hipMemset(c.pool, 0, need);
    if (e != hipSuccess) {
      (void)hipFree(c.pool);
      return hip_fail(e, "hipMemset(pool)");
    }
  }
  e = hipMalloc(&c.tables, sizeof(tq::DeviceTables));
  if (e != hipSuccess) {
    if (c.owns_pool) (void)hipFree(c.pool);
    return fail(TQ_ERR_OOM, "table allocation failed");
  }
  e = hipMemcpy(c.tables, &host_tables, sizeof host_tables, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(c.tables);
    if (c.owns_pool) (void)hipFree(c.pool);
    return hip_fail(e, "hipMemcpy(tables)");
  }
  *out = new tq_cache(c);
  return TQ_OK;
}

tq_status tq_cache_info(const tq_cache *cache, void **pool, size_t *pool_bytes, uint16_t *key_table_f16) {
  if (!cache) return fail(TQ_ERR_INVALID_ARG, "cache is NULL");
  if (pool) *pool = cache->pool;
  if (pool_bytes) *pool_bytes = cache->pool_bytes;
  if (key_table_f16) std::memcpy(key_table_f16, cache->table_f16, sizeof cache->table_f16);
  return TQ_OK;
}

tq_status tq_quantize_append(tq_cache *cache, const void *k, const void *v, const int32_t *slot_mapping,
                             int64_t num_tokens, void *stream) {
  if (!cache) return fail(TQ_ERR_INVALID_ARG, "cache is NULL");
  if (num_tokens < 0) return fail(TQ_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (num_tokens == 0) return TQ_OK;
  if (!k || !v || !slot_mapping) return fail(TQ_ERR_INVALID_ARG, "k, v and slot_mapping must be non-NULL");
  if (((uintptr_t)k | (uintptr_t)v) & 15) return fail(TQ_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  if (num_tokens > ((int64_t)1 << 36)) return fail(TQ_ERR_INVALID_ARG, "num_tokens too large");
  tq::QuantizeArgs a{};
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.hkv = cache->desc.num_kv_heads;
  a.pool = cache->pool;
  a.num_blocks = cache->desc.num_blocks;
  a.tables = cache->tables;
  a.bins = cache->bins;
  a.rsqrt_d = (float)(1.0 / std::sqrt((double)cache->desc.head_dim));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = cache->desc.format != TQ_FORMAT_MXFP4
                     ? tq::launch_tq4_quantize(cache->desc.head_dim, cache->desc.format == TQ_FORMAT_TQ4 ? 4 : 2, a, s)
                                                      : tq::launch_mxfp4_quantize(a, s);
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return TQ_OK;
}

tq_status tq_decode_workspace_bytes(const tq_cache *cache, int32_t batch, int32_t num_q_heads,
                                    int32_t max_context_len, size_t *bytes) {
  if (!cache || !bytes) return fail(TQ_ERR_INVALID_ARG, "cache and bytes must be non-NULL");
  if (batch < 0 || num_q_heads < 1 || max_context_len < 0)
    return fail(TQ_ERR_INVALID_ARG, "batch, num_q_heads or max_context_len out of range");
  const tq::SplitPlan p = tq::plan_split(batch, cache->desc.num_kv_heads, max_context_len);
  // (max, sum) pairs, then the accumulators from a 256-byte boundary
  const size_t rows = (size_t)batch * num_q_heads * p.nsplit;
  *bytes = p.nsplit > 1 ? ((rows * 2 * 4 + 255) / 256) * 256 + rows * (size_t)cache->desc.head_dim * 4 : 0;
  return TQ_OK;
}

namespace {

// Decode attention with the workspace given (the caller's, or the fixed
// scratch of the no-allocation entry point).
tq_status decode_impl(tq_cache *cache, const void *q, void *out, int32_t out_dtype, const int32_t *block_table,
                      int32_t max_blocks, const int32_t *context_lens, int32_t batch, int32_t num_q_heads,
                      int32_t max_context_len, float softmax_scale, void *workspace, size_t workspace_bytes,
                      void *stream, bool fixed_scratch);

}  // namespace

tq_status tq_decode_attention(tq_cache *cache, const void *q, void *out, int32_t out_dtype,
                              const int32_t *block_table, int32_t max_blocks, const int32_t *context_lens,
                              int32_t batch, int32_t num_q_heads, int32_t max_context_len, float softmax_scale,
                              void *workspace, size_t workspace_bytes, void *stream) {
  return decode_impl(cache, q, out, out_dtype, block_table, max_blocks, context_lens, batch, num_q_heads,
                     max_context_len, softmax_scale, workspace, workspace_bytes, stream, false);
}

tq_status tq_decode_attention_noalloc(tq_cache *cache, const void *q, void *out, int32_t out_dtype,
                                      const int32_t *block_table, int32_t max_blocks, const int32_t *context_lens,
                                      int32_t batch, int32_t num_q_heads, int32_t max_context_len,
                                      float softmax_scale, void *stream) {
  return decode_impl(cache, q, out, out_dtype, block_table, max_blocks, context_lens, batch, num_q_heads,
                     max_context_len, softmax_scale, nullptr, 0, stream, true);
}

namespace {

tq_status decode_impl(tq_cache *cache, const void *q, void *out, int32_t out_dtype, const int32_t *block_table,
                      int32_t max_blocks, const int32_t *context_lens, int32_t batch, int32_t num_q_heads,
                      int32_t max_context_len, float softmax_scale, void *workspace, size_t workspace_bytes,
                      void *stream, bool fixed_scratch) {
  if (!cache) return fail(TQ_ERR_INVALID_ARG, "cache is NULL");
  if (batch < 0) return fail(TQ_ERR_INVALID_ARG, "batch must be >= 0");
  if (batch == 0) return TQ_OK;
  if (!q || !out || !block_table || !context_lens)
    return fail(TQ_ERR_INVALID_ARG, "q, out, block_table and context_lens must be non-NULL");
  if (out_dtype != TQ_OUT_F32 && out_dtype != TQ_OUT_BF16) return fail(TQ_ERR_INVALID_ARG, "bad out_dtype");
  const int hkv = cache->desc.num_kv_heads;
  if (num_q_heads < hkv || num_q_heads % hkv)
    return fail(TQ_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  const int g = num_q_heads / hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(TQ_ERR_UNSUPPORTED, "query heads per kv-head must be 1, 2, 4 or 8");
  if (max_context_len < 0) return fail(TQ_ERR_INVALID_ARG, "max_context_len must be >= 0");
  if (max_blocks < (max_context_len + 15) / 16 || max_blocks < 1)
    return fail(TQ_ERR_INVALID_ARG, "max_blocks must cover max_context_len");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(TQ_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
  const tq::SplitPlan p = tq::plan_split(batch, hkv, max_context_len);
  size_t need = 0;
  tq_decode_workspace_bytes(cache, batch, num_q_heads, max_context_len, &need);
  if (fixed_scratch && need) {
    if (need > tq::kNoallocScratchBytes)
      return fail(TQ_ERR_WORKSPACE, "these sizes need " + std::to_string(need) +
                                        " bytes of split partials, more than the fixed scratch of " +
                                        std::to_string(tq::kNoallocScratchBytes) + " bytes");
    hipError_t e = tq::noalloc_scratch(&workspace);
    if (e != hipSuccess) return hip_fail(e, "fixed scratch lookup");
    workspace_bytes = tq::kNoallocScratchBytes;
  }
  if (need && (!workspace || workspace_bytes < need))
    return fail(TQ_ERR_WORKSPACE, "workspace smaller than tq_decode_workspace_bytes (" + std::to_string(need) + ")");

  tq::DecodeArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.out = out;
  a.block_table = block_table;
  a.ctx = context_lens;
  a.pool = cache->pool;
  a.tables = cache->tables;
  const int d = cache->desc.head_dim;
  if (p.nsplit > 1) {
    a.part_ml = static_cast<float *>(workspace);
    a.part_acc = a.part_ml + (((size_t)batch * num_q_heads * p.nsplit * 2 + 63) / 64) * 64;
  }
  const double log2e = 1.4426950408889634074;
  a.rsqrt_d = (float)(1.0 / std::sqrt((double)d));
  a.qscale = cache->desc.format != TQ_FORMAT_MXFP4
                 ? (float)((double)softmax_scale * log2e * (1.0 / std::sqrt((double)d)))
                 : (float)((double)softmax_scale * log2e);
  a.max_blocks = max_blocks;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = hkv;
  a.g = g;
  a.split_blocks = p.split_blocks;
  a.nsplit = p.nsplit;
  a.out_bf16 = out_dtype == TQ_OUT_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = cache->desc.format == TQ_FORMAT_MXFP4 ? tq::launch_mxfp4_decode(a, s)
                 : tq::launch_tq4_decode(d, cache->desc.format == TQ_FORMAT_TQ4 ? 4 : 2, a, s);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (p.nsplit > 1) {
    e = tq::launch_decode_merge(d, a, s);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return TQ_OK;
}

}  // namespace

namespace {

struct MtPlan {
  tq::SplitPlan split;
  int rows_per_wg;
  int row_tiles;
};

tq_status multitoken_plan(const tq_cache *cache, int32_t batch, int32_t num_q_heads, int64_t num_tokens,
                          int32_t max_query_len, int32_t max_context_len, MtPlan *p) {
  if (!cache) return fail(TQ_ERR_INVALID_ARG, "cache is NULL");
  const bool mx = cache->desc.format == TQ_FORMAT_MXFP4;
  const int hkv = cache->desc.num_kv_heads;
  if (batch < 0 || num_tokens < 0 || max_query_len < 0 || max_context_len < 0)
    return fail(TQ_ERR_INVALID_ARG, "batch, num_tokens, max_query_len and max_context_len must be >= 0");
  if (num_q_heads < hkv || num_q_heads % hkv)
    return fail(TQ_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (max_query_len > max_context_len)
    return fail(TQ_ERR_INVALID_ARG, "max_query_len must be <= max_context_len");
  if (num_tokens > (int64_t)batch * max_query_len)
    return fail(TQ_ERR_INVALID_ARG, "num_tokens must be <= batch * max_query_len");
  const int64_t g = num_q_heads / hkv;
  // rows of one (sequence, kv-head): up to 16 or 32 in the direct kernel
  // (every wave runs all rows against its own block pairs), up to 64 in a
  // staged work-group of 4 row groups x 2 block groups, up to 128 in 8 x 1,
  // more in tiles of 256 (8 x 1, two 16-row tiles per wave)
  // MX-FP4: work-groups of 16 or 32 rows, more rows as more row tiles; a
  // wave keeps at most 64 block ids (one per lane), 256 per work-group
  const int64_t rows = (int64_t)max_query_len * g;
  const int rows_per_wg = rows <= 16 ? 16 : rows <= 32 || mx ? 32 : rows <= 64 ? 64 : rows <= 128 ? 128 : 256;
  const int64_t row_tiles = (rows + rows_per_wg - 1) / rows_per_wg;
  // prefill-sized tiles (MFMA-heavy per block) walk whole contexts; smaller
  // ones split long contexts at 512 blocks so uneven lengths balance
  const int max_split = mx ? 256 : rows_per_wg >= 256 ? 4096 : 512;
  tq::SplitPlan sp = tq::plan_split_multitoken((int64_t)batch * hkv * std::max<int64_t>(1, row_tiles),
                                               max_context_len, max_split);
  // a work-group stages its split's block ids in LDS: at most 4096 (staged
  // kernel) or 1024 (direct kernel)
  const int max_ids = mx ? 256 : rows_per_wg <= 32 ? 1024 : 4096;
  if (sp.split_blocks > max_ids) {
    sp.split_blocks = max_ids;
    sp.nsplit = (int)std::max<int64_t>(1, (((int64_t)max_context_len + 15) / 16 + max_ids - 1) / max_ids);
  }
  if ((int64_t)batch * hkv * row_tiles * sp.nsplit >= (int64_t(1) << 31) ||
      (int64_t)batch * max_query_len * num_q_heads >= (int64_t(1) << 31))
    return fail(TQ_ERR_INVALID_ARG, "launch grid too large");
  p->split = sp;
  p->rows_per_wg = rows_per_wg;
  p->row_tiles = (int)row_tiles;
  return TQ_OK;
}

}  // namespace

tq_status tq_multitoken_workspace_bytes(const tq_cache *cache, int32_t batch, int32_t num_q_heads,
                                        int64_t num_tokens, int32_t max_query_len, int32_t max_context_len,
                                        size_t *bytes) {
  if (!bytes) return fail(TQ_ERR_INVALID_ARG, "bytes is NULL");
  MtPlan p;
  tq_status st = multitoken_plan(cache, batch, num_q_heads, num_tokens, max_query_len, max_context_len, &p);
  if (st != TQ_OK) return st;
  const size_t rows = (size_t)num_tokens * num_q_heads * p.split.nsplit;
  *bytes = p.split.nsplit > 1 ? ((rows * 2 * 4 + 255) / 256) * 256 + rows * (size_t)cache->desc.head_dim * 4 : 0;
  return TQ_OK;
}

tq_status tq_multitoken_attention(tq_cache *cache, const void *q, void *out, int32_t out_dtype,
                                  const int32_t *q_start, int64_t num_tokens, int32_t max_query_len,
                                  const int32_t *block_table, int32_t max_blocks, const int32_t *context_lens,
                                  int32_t batch, int32_t num_q_heads, int32_t max_context_len,
                                  float softmax_scale, void *workspace, size_t workspace_bytes, void *stream) {
  MtPlan p;
  tq_status st = multitoken_plan(cache, batch, num_q_heads, num_tokens, max_query_len, max_context_len, &p);
  if (st != TQ_OK) return st;
  if (batch == 0 || num_tokens == 0 || max_query_len == 0) return TQ_OK;
  if (!q || !out || !q_start || !block_table || !context_lens)
    return fail(TQ_ERR_INVALID_ARG, "q, out, q_start, block_table and context_lens must be non-NULL");
  if (out_dtype != TQ_OUT_F32 && out_dtype != TQ_OUT_BF16) return fail(TQ_ERR_INVALID_ARG, "bad out_dtype");
  if (max_blocks < (max_context_len + 15) / 16 || max_blocks < 1)
    return fail(TQ_ERR_INVALID_ARG, "max_blocks must cover max_context_len");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(TQ_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
  size_t need = 0;
  tq_multitoken_workspace_bytes(cache, batch, num_q_heads, num_tokens, max_query_len, max_context_len, &need);
  if (need && (!workspace || workspace_bytes < need))
    return fail(TQ_ERR_WORKSPACE,
                "workspace smaller than tq_multitoken_workspace_bytes (" + std::to_string(need) + ")");
  const int d = cache->desc.head_dim;
  tq::MultiTokenArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.out = out;
  a.q_start = q_start;
  a.block_table = block_table;
  a.ctx = context_lens;
  a.pool = cache->pool;
  a.tables = cache->tables;
  if (p.split.nsplit > 1) {
    a.part_ml = static_cast<float *>(workspace);
    a.part_acc = a.part_ml + (((size_t)num_tokens * num_q_heads * p.split.nsplit * 2 + 63) / 64) * 64;
  }
  const double log2e = 1.4426950408889634074;
  const bool mx = cache->desc.format == TQ_FORMAT_MXFP4;
  // MX-FP4 queries carry 1/sqrt(d) before their e4m3 rounding
  a.qscale = (float)((double)softmax_scale * log2e * (mx ? 1.0 : 1.0 / std::sqrt((double)d)));
  a.rsqrt_d = (float)(1.0 / std::sqrt((double)d));
  a.max_blocks = max_blocks;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = cache->desc.num_kv_heads;
  a.g = num_q_heads / a.hkv;
  a.max_query_len = max_query_len;
  a.rows_per_wg = p.rows_per_wg;
  a.row_tiles = p.row_tiles;
  a.split_blocks = p.split.split_blocks;
  a.nsplit = p.split.nsplit;
  a.part_stride = p.split.nsplit;
  a.slot0 = 0;
  a.out_bf16 = out_dtype == TQ_OUT_BF16;
  hipError_t e = mx ? tq::launch_mxfp4_multitoken(a, static_cast<hipStream_t>(stream))
                    : tq::launch_tq4_multitoken(d, cache->desc.format == TQ_FORMAT_TQ4 ? 4 : 2, a,
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "multi-token attention launch");
  return TQ_OK;
}

namespace {

struct CascadePlan {
  tq::SplitPlan own, prefix;
  int rows_per_wg, row_tiles;
  int part_stride;
};

tq_status cascade_plan(const tq_cache *cache, int32_t batch, int32_t num_q_heads, int32_t max_context_len,
                       int32_t num_groups, int32_t max_group_size, int32_t max_group_blocks, int32_t max_depth,
                       CascadePlan *p) {
  if (!cache) return fail(TQ_ERR_INVALID_ARG, "cache is NULL");
  const bool mx = cache->desc.format == TQ_FORMAT_MXFP4;
  const int hkv = cache->desc.num_kv_heads;
  if (batch < 0 || max_context_len < 0 || num_groups < 0 || max_group_blocks < 0 || max_depth < 0)
    return fail(TQ_ERR_INVALID_ARG,
                "batch, max_context_len, num_groups, max_group_blocks and max_depth must be >= 0");
  if (num_q_heads < hkv || num_q_heads % hkv)
    return fail(TQ_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  const int g = num_q_heads / hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(TQ_ERR_UNSUPPORTED, "query heads per kv-head must be 1, 2, 4 or 8");
  if (num_groups > 0 && (max_group_size < 1 || max_group_size > batch))
    return fail(TQ_ERR_INVALID_ARG, "max_group_size must be in [1, batch]");
  if (num_groups > 0 && (max_depth < 1 || max_depth > num_groups))
    return fail(TQ_ERR_INVALID_ARG, "max_depth must be in [1, num_groups]");
  if ((int64_t)16 * max_group_blocks > max_context_len)
    return fail(TQ_ERR_INVALID_ARG, "16 * max_group_blocks must be <= max_context_len");
  if (max_group_blocks > (mx ? 256 : 4096))
    return fail(TQ_ERR_UNSUPPORTED, mx ? "an MX-FP4 group's shared range is at most 256 blocks (cut longer ones into "
                                         "chained groups)"
                                       : "a group's shared range is at most 4096 blocks (cut longer ones into chained "
                                         "groups)");
  p->own = tq::plan_split(batch, hkv, max_context_len);
  // groups of at most 32 rows take the direct kernel (every wave runs all rows
  // against its own blocks; the group's block ids, at most 1024, in LDS),
  // larger ones the staged kernel; MX-FP4 groups take work-groups of 16 or 32
  // rows (more rows: more row tiles)
  const int64_t rows = (int64_t)std::max(1, max_group_size) * g;
  const bool direct = mx || (rows <= 32 && max_group_blocks <= 1024);
  p->rows_per_wg = direct ? (rows <= 16 ? 16 : 32) : rows <= 64 ? 64 : 128;
  p->row_tiles = (int)((rows + p->rows_per_wg - 1) / p->rows_per_wg);
  // one split per group: a group is the unit of parallel work (callers cut
  // long shared ranges into chained groups)
  p->prefix.split_blocks = std::max(1, max_group_blocks);
  p->prefix.nsplit = 1;
  const int64_t stride = (int64_t)p->own.nsplit + (num_groups > 0 ? max_depth : 0);
  if (stride > (1 << 20)) return fail(TQ_ERR_INVALID_ARG, "too many partial slots per row");
  p->part_stride = (int)stride;
  return TQ_OK;
}

}  // namespace

tq_status tq_cascade_workspace_bytes(const tq_cache *cache, int32_t batch, int32_t num_q_heads,
                                     int32_t max_context_len, int32_t num_groups, int32_t max_group_size,
                                     int32_t max_group_blocks, int32_t max_depth, size_t *bytes) {
  if (!bytes) return fail(TQ_ERR_INVALID_ARG, "bytes is NULL");
  CascadePlan p;
  tq_status st = cascade_plan(cache, batch, num_q_heads, max_context_len, num_groups, max_group_size,
                              max_group_blocks, max_depth, &p);
  if (st != TQ_OK) return st;
  const size_t rows = (size_t)batch * num_q_heads * p.part_stride;
  *bytes = ((rows * 2 * 4 + 255) / 256) * 256 + rows * (size_t)cache->desc.head_dim * 4;
  return TQ_OK;
}

tq_status tq_cascade_decode_attention(tq_cache *cache, const void *q, void *out, int32_t out_dtype,
                                      const int32_t *block_table, int32_t max_blocks, const int32_t *context_lens,
                                      int32_t batch, int32_t num_q_heads, int32_t max_context_len,
                                      float softmax_scale, const int32_t *seq_prefix_blocks,
                                      const int32_t *seq_depth, const int32_t *group_start,
                                      const int32_t *group_seqs, const int32_t *group_blocks,
                                      const int32_t *group_depth, int32_t num_groups, int32_t max_group_size,
                                      int32_t max_group_blocks, int32_t max_depth, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  CascadePlan p;
  tq_status st = cascade_plan(cache, batch, num_q_heads, max_context_len, num_groups, max_group_size,
                              max_group_blocks, max_depth, &p);
  if (st != TQ_OK) return st;
  if (batch == 0) return TQ_OK;
  if (!q || !out || !block_table || !context_lens || !seq_prefix_blocks || !seq_depth)
    return fail(TQ_ERR_INVALID_ARG,
                "q, out, block_table, context_lens, seq_prefix_blocks and seq_depth must be non-NULL");
  if (num_groups > 0 && (!group_start || !group_seqs || !group_blocks || !group_depth))
    return fail(TQ_ERR_INVALID_ARG, "group_start, group_seqs, group_blocks and group_depth must be non-NULL");
  if (out_dtype != TQ_OUT_F32 && out_dtype != TQ_OUT_BF16) return fail(TQ_ERR_INVALID_ARG, "bad out_dtype");
  if (max_blocks < (max_context_len + 15) / 16 || max_blocks < 1)
    return fail(TQ_ERR_INVALID_ARG, "max_blocks must cover max_context_len");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(TQ_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
  size_t need = 0;
  tq_cascade_workspace_bytes(cache, batch, num_q_heads, max_context_len, num_groups, max_group_size,
                             max_group_blocks, max_depth, &need);
  if (!workspace || workspace_bytes < need)
    return fail(TQ_ERR_WORKSPACE, "workspace smaller than tq_cascade_workspace_bytes (" + std::to_string(need) + ")");
  const int d = cache->desc.head_dim;
  const int hkv = cache->desc.num_kv_heads;
  float *part_ml = static_cast<float *>(workspace);
  float *part_acc = part_ml + (((size_t)batch * num_q_heads * p.part_stride * 2 + 63) / 64) * 64;
  const double log2e = 1.4426950408889634074;
  const bool mx = cache->desc.format == TQ_FORMAT_MXFP4;
  // MX-FP4 queries carry 1/sqrt(d) before their e4m3 rounding
  const float qscale = (float)((double)softmax_scale * log2e * (mx ? 1.0 : 1.0 / std::sqrt((double)d)));
  const float rsqrt_d = (float)(1.0 / std::sqrt((double)d));
  hipStream_t s = static_cast<hipStream_t>(stream);

  hipError_t e;
  if (num_groups > 0 && !cache->aux) {
    e = hipStreamCreateWithFlags(&cache->aux, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&cache->fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&cache->join, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "cascade stream set-up");
  }
  if (num_groups > 0) {
    tq::MultiTokenArgs m{};
    m.q = static_cast<const uint16_t *>(q);
    m.block_table = block_table;
    m.pool = cache->pool;
    m.tables = cache->tables;
    m.part_ml = part_ml;
    m.part_acc = part_acc;
    m.qscale = qscale;
    m.rsqrt_d = rsqrt_d;
    m.max_blocks = max_blocks;
    m.batch = num_groups;
    m.hq = num_q_heads;
    m.hkv = hkv;
    m.g = num_q_heads / hkv;
    m.max_query_len = max_group_size;
    m.rows_per_wg = p.rows_per_wg;
    m.row_tiles = p.row_tiles;
    m.split_blocks = p.prefix.split_blocks;
    m.nsplit = p.prefix.nsplit;
    m.group_start = group_start;
    m.group_seqs = group_seqs;
    m.group_blocks = group_blocks;
    m.group_depth = group_depth;
    m.part_stride = p.part_stride;
    m.slot0 = p.own.nsplit;
    e = hipEventRecord(cache->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(cache->aux, cache->fork, 0);
    if (e != hipSuccess) return hip_fail(e, "cascade fork");
    e = mx ? tq::launch_mxfp4_prefix_attention(m, cache->aux)
           : tq::launch_prefix_attention(d, cache->desc.format == TQ_FORMAT_TQ4 ? 4 : 2, m, cache->aux);
    if (e != hipSuccess) return hip_fail(e, "shared-block attention launch");
    e = hipEventRecord(cache->join, cache->aux);
    if (e != hipSuccess) return hip_fail(e, "cascade join record");
  }
  tq::DecodeArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.out = out;
  a.block_table = block_table;
  a.ctx = context_lens;
  a.pool = cache->pool;
  a.tables = cache->tables;
  a.part_ml = part_ml;
  a.part_acc = part_acc;
  a.qscale = qscale;
  a.rsqrt_d = rsqrt_d;
  a.max_blocks = max_blocks;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = hkv;
  a.g = num_q_heads / hkv;
  a.split_blocks = p.own.split_blocks;
  a.nsplit = p.own.nsplit;
  a.out_bf16 = out_dtype == TQ_OUT_BF16;
  a.first_blk = seq_prefix_blocks;
  a.depth = seq_depth;
  a.part_stride = p.part_stride;
  e = mx ? tq::launch_mxfp4_cascade_decode(a, s)
         : tq::launch_tq4_cascade_decode(d, cache->desc.format == TQ_FORMAT_TQ4 ? 4 : 2, a, s);
  if (e != hipSuccess) return hip_fail(e, "cascade decode launch");
  if (num_groups > 0) {
    e = hipStreamWaitEvent(s, cache->join, 0);
    if (e != hipSuccess) return hip_fail(e, "cascade join");
  }
  e = tq::launch_cascade_merge(d, a, s);
  if (e != hipSuccess) return hip_fail(e, "cascade merge launch");
  return TQ_OK;
}

tq_status tq_calibrate_workspace_bytes(int32_t num_layers, int64_t rows, int32_t head_dim, size_t *bytes) {
  if (!bytes) return fail(TQ_ERR_INVALID_ARG, "bytes is NULL");
  if (head_dim != 64 && head_dim != 128) return fail(TQ_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (num_layers < 0 || num_layers > 65535) return fail(TQ_ERR_INVALID_ARG, "num_layers must be in [0, 65535]");
  if (rows < 0 || rows > (int64_t(1) << 30) / head_dim)
    return fail(TQ_ERR_INVALID_ARG, "rows must be in [0, 2^30 / head_dim]");
  *bytes = tq::calibrate_workspace_bytes(num_layers, rows, head_dim);
  return TQ_OK;
}

tq_status tq_calibrate_key_tables(const void *k, int32_t num_layers, int64_t rows, int32_t head_dim,
                                  const float *init_table, int32_t max_iters, uint16_t *tables_f16,
                                  double *levels, double *mse, int32_t *updates, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  size_t need = 0;
  tq_status st = tq_calibrate_workspace_bytes(num_layers, rows, head_dim, &need);
  if (st != TQ_OK) return st;
  if (max_iters < 0 || max_iters > 1000000) return fail(TQ_ERR_INVALID_ARG, "max_iters must be in [0, 1e6]");
  uint16_t init[16];
  if (init_table) {
    for (int i = 0; i < 16; ++i) {
      if (!std::isfinite(init_table[i])) return fail(TQ_ERR_INVALID_ARG, "init table entries must be finite");
      init[i] = tq::f64_to_f16_rne((double)init_table[i]);
      if ((init[i] & 0x7c00u) == 0x7c00u) return fail(TQ_ERR_INVALID_ARG, "init table entry overflows fp16");
    }
    for (int i = 0; i < 15; ++i)
      if (!(tq::f16_to_f64(init[i]) < tq::f16_to_f64(init[i + 1])))
        return fail(TQ_ERR_INVALID_ARG, "init table must be strictly ascending after rounding to fp16");
  } else {
    tq_default_key_table(init);
  }
  if (num_layers == 0) return TQ_OK;
  if (!tables_f16) return fail(TQ_ERR_INVALID_ARG, "tables_f16 is NULL");
  if (rows > 0 && !k) return fail(TQ_ERR_INVALID_ARG, "k is NULL");
  if (!workspace || workspace_bytes < need)
    return fail(TQ_ERR_WORKSPACE, "workspace smaller than tq_calibrate_workspace_bytes (" + std::to_string(need) + ")");
  const float rsqrt_d = (float)(1.0 / std::sqrt((double)head_dim));
  hipError_t e = tq::launch_calibrate(head_dim, num_layers, rows, static_cast<const uint16_t *>(k), init, max_iters,
                                      rsqrt_d, workspace, tables_f16, levels, mse, updates,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "calibrate launch");
  return TQ_OK;
}

tq_status tq_select_layers(const double *mse, int32_t num_layers, int32_t percent, uint8_t *chosen) {
  if (num_layers < 0) return fail(TQ_ERR_INVALID_ARG, "num_layers must be >= 0");
  if (percent < 0 || percent > 100) return fail(TQ_ERR_INVALID_ARG, "percent must be in [0, 100]");
  if (num_layers == 0) return TQ_OK;
  if (!mse || !chosen) return fail(TQ_ERR_INVALID_ARG, "mse or chosen is NULL");
  for (int i = 0; i < num_layers; ++i)
    if (std::isnan(mse[i])) return fail(TQ_ERR_INVALID_ARG, "mse holds a NaN");
  // rank of layer i: layers with a larger MSE, or an equal MSE and a lower index
  for (int i = 0; i < num_layers; ++i) {
    int64_t rank = 0;
    for (int j = 0; j < num_layers; ++j)
      if (mse[j] > mse[i] || (mse[j] == mse[i] && j < i)) ++rank;
    chosen[i] = 100 * rank < (int64_t)percent * num_layers ? 1 : 0;
  }
  return TQ_OK;
}

tq_status tq_debug_dequantize(tq_cache *cache, const int32_t *block_ids, int32_t n, float *k_out, float *v_out,
                              void *stream) {
  if (!cache) return fail(TQ_ERR_INVALID_ARG, "cache is NULL");
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return TQ_OK;
  if (!block_ids || !k_out || !v_out) return fail(TQ_ERR_INVALID_ARG, "block_ids, k_out and v_out must be non-NULL");
  if ((int64_t)n * cache->desc.num_kv_heads >= (int64_t(1) << 31))
    return fail(TQ_ERR_INVALID_ARG, "n * num_kv_heads must be < 2^31");
  hipError_t e = tq::launch_debug_dequant(cache->desc.format, cache->desc.head_dim, cache->pool,
                                          cache->desc.num_blocks, cache->desc.num_kv_heads, block_ids, n,
                                          cache->tables, k_out, v_out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dequantize launch");
  return TQ_OK;
}

void tq_free(tq_cache *cache) {
  if (!cache) return;
  (void)hipDeviceSynchronize();
  if (cache->fork) (void)hipEventDestroy(cache->fork);
  if (cache->join) (void)hipEventDestroy(cache->join);
  if (cache->aux) (void)hipStreamDestroy(cache->aux);
  if (cache->tables) (void)hipFree(cache->tables);
  if (cache->owns_pool && cache->pool) (void)hipFree(cache->pool);
  delete cache;
}

}  // extern "C"
