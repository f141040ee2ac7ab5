// Host-side tables: the default 16-entry key table (Lloyd-Max quantizer of
// N(0,1)), fp16 rounding, the decode LUT and the quantizer's bin table.
// Pure C++ (no HIP calls), so it runs without a GPU.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <limits>

#include "tq_internal.h"

namespace tq {

// ---------------------------------------------------------------------------
// 16-level Lloyd-Max quantizer of the standard normal ("UltraQuant：4-bit KV
// 快取加速長代理", section "方法怎麼做，白話講": the 16-entry table starts
// from the theoretical Lloyd-Max centroids).  Lloyd's conditions, iterated in
// fp64: thresholds are midpoints of neighbouring levels; each level is the
// conditional mean of N(0,1) on its cell, (pdf(a) - pdf(b)) / (cdf(b) - cdf(a)).
// ---------------------------------------------------------------------------
static double npdf(double x) {
  if (std::isinf(x)) return 0.0;
  return std::exp(-0.5 * x * x) * 0.39894228040143267794;  // 1/sqrt(2 pi)
}
static double ncdf(double x) {
  if (x == -std::numeric_limits<double>::infinity()) return 0.0;
  if (x == std::numeric_limits<double>::infinity()) return 1.0;
  return 0.5 * std::erfc(-x * 0.70710678118654752440);
}

void lloyd_max_gaussian16(double out[16]) {
  double c[16];
  for (int i = 0; i < 16; ++i) c[i] = -2.0 + 4.0 * (i + 0.5) / 16.0;
  const double inf = std::numeric_limits<double>::infinity();
  for (int it = 0; it < 200000; ++it) {
    double edges[17];
    edges[0] = -inf;
    edges[16] = inf;
    for (int i = 0; i < 15; ++i) edges[i + 1] = 0.5 * (c[i] + c[i + 1]);
    double moved = 0.0;
    for (int i = 0; i < 16; ++i) {
      const double a = edges[i], b = edges[i + 1];
      const double nc = (npdf(a) - npdf(b)) / (ncdf(b) - ncdf(a));
      moved = std::fmax(moved, std::fabs(nc - c[i]));
      c[i] = nc;
    }
    if (moved <= 1e-15) break;
  }
  for (int i = 0; i < 16; ++i) out[i] = c[i];
}

// ---------------------------------------------------------------------------
// fp16 <-> fp64, round to nearest even, written from the IEEE binary16 format
// (1 sign, 5 exponent bits, bias 15, 10 fraction bits; subnormal spacing 2^-24).
// ---------------------------------------------------------------------------
uint16_t f64_to_f16_rne(double x) {
  const uint16_t sign = std::signbit(x) ? 0x8000u : 0u;
  if (std::isnan(x)) return 0x7e00u;
  double a = std::fabs(x);
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);           // a = m * 2^e, m in [0.5, 1): binade exponent e - 1
  int be = e - 1;
  if (be < -14) be = -14;      // subnormal range shares the 2^-24 spacing
  const double step = std::ldexp(1.0, be - 10);
  double q = std::nearbyint(a / step);       // exact scaling, ties to even
  double v = q * step;
  if (v >= 65520.0) return (uint16_t)(sign | 0x7c00u);  // overflow -> inf
  if (v == 0.0) return sign;
  // encode v
  int ve;
  std::frexp(v, &ve);
  int vbe = ve - 1;
  if (vbe < -14) {             // subnormal
    return (uint16_t)(sign | (uint16_t)std::lround(v / std::ldexp(1.0, -24)));
  }
  const int frac = (int)std::lround((v / std::ldexp(1.0, vbe) - 1.0) * 1024.0);
  return (uint16_t)(sign | (uint16_t)((vbe + 15) << 10) | (uint16_t)frac);
}

double f16_to_f64(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0) v = std::ldexp((double)f, -24);
  else if (e == 31) v = f ? std::numeric_limits<double>::quiet_NaN() : std::numeric_limits<double>::infinity();
  else v = std::ldexp(1.0 + f / 1024.0, e - 15);
  return s ? -v : v;
}

// ---------------------------------------------------------------------------
// Tables for the kernels.
//   lut2[byte] = fp16 c[byte & 15] | fp16 c[byte >> 4] << 16 (decode dequant).
//   Key coder: code(u) = #{ j : u > t_j }, t_j = fp32((c_j + c_{j+1}) * 0.5).
//   The kernel finds the bin of u on a uniform grid and adds one comparison:
//   code = below[bin] + (u > inside[bin]).  That is exact when every bin,
//   widened by a margin that covers the rounding of the bin computation, holds
//   at most one threshold; `below` counts the thresholds under the widened bin.
// ---------------------------------------------------------------------------
bool build_key_tables(const uint16_t table_f16[16], DeviceTables *t, BinParams *bp) {
  // recip[f] = fp32 RNE of 1024 / (1024 + f), by exact integer long division
  for (int f = 0; f < 1024; ++f) {
    const uint64_t den = 1024 + (uint64_t)f;
    if (f == 0) {
      t->recip[0] = 1.0f;
      continue;
    }
    // 1024/den lies in (0.5, 1): its 24-bit significand is floor(2^24 * 1024 / den)
    const uint64_t num = (uint64_t)1024 << 24;
    uint64_t q = num / den, r = num % den;
    if (2 * r > den || (2 * r == den && (q & 1))) ++q;  // round to nearest even
    t->recip[f] = (float)std::ldexp((double)q, -24);
  }
  for (int e = 0; e < 256; ++e) t->lut2[e] = (uint32_t)table_f16[e & 15] | ((uint32_t)table_f16[e >> 4] << 16);

  float th[15];
  for (int j = 0; j < 15; ++j) {
    const float cj = (float)f16_to_f64(table_f16[j]);
    const float cn = (float)f16_to_f64(table_f16[j + 1]);
    volatile float sum = cj + cn;  // fp32 sum, then exact halving
    th[j] = sum * 0.5f;
  }
  const double span = (double)th[14] - (double)th[0];
  const float inf = std::numeric_limits<float>::infinity();
  for (int nb = kMaxBins; nb <= kMaxBins; nb *= 2) {
    const double width = span > 0 ? span / (nb - 8) : 1.0;
    for (int shift = 0; shift < 8; ++shift) {
      const double origin = (double)th[0] - 4.0 * width - shift * width / 8.0;
      const float a = (float)(1.0 / width);
      const float b = (float)(-origin / width);
      // actual bin edges implied by the fp32 (a, b): u maps to bin k when
      // k <= u*a + b < k+1, i.e. u in [(k - b)/a, (k + 1 - b)/a)
      const double margin = width / 16.0;
      bool ok = true;
      for (int k = 0; k < nb && ok; ++k) {
        const double lo = (k == 0) ? -1e300 : ((double)k - (double)b) / (double)a - margin;
        const double hi = (k == nb - 1) ? 1e300 : ((double)k + 1.0 - (double)b) / (double)a + margin;
        int below = 0, inside = 0;
        float thr = inf;
        for (int j = 0; j < 15; ++j) {
          if ((double)th[j] < lo) ++below;
          else if ((double)th[j] < hi) {
            ++inside;
            thr = th[j];
          }
        }
        if (inside > 1) ok = false;
        float2 v;
        v.x = thr;
        int bi = below;
        std::memcpy(&v.y, &bi, sizeof bi);
        t->bins[k] = v;
      }
      if (ok) {
        bp->a = a;
        bp->b = b;
        bp->nbins = nb;
        return true;
      }
    }
  }
  return false;
}

// Split-K plan: blocks per work-group S (a multiple of its 8 waves, 16..256).
// Measured on MI355X across the workloads: about one work-group per compute
// unit (256) is best (fewer, longer work-groups pay the block-id fetch, query
// rotation and wave merge fewer times, and leave fewer partials to merge),
// while more than 256 blocks per work-group unbalances ragged batches (short
// sequences leave their later splits empty).  So: nsplit = the larger of
// ceil(256 / units) and ceil(blocks / 256), S = ceil(blocks / nsplit) rounded up
// to a multiple of 8.  A grid of 256 to 512 work-groups is resident at once
// (two per compute unit), and its units that hold two work-groups finish
// last, each of their work-groups running about 0.6 times as fast as a lone
// one (measured); when the units divide 256 the split count is then
// raised so that every compute unit holds two (448 -> 512 work-groups at 8
// sequences x 8 kv-heads measured 3% faster end to end).
SplitPlan plan_split(int batch, int hkv, int max_context_len) {
  const int64_t max_nblk = std::max<int64_t>(1, ((int64_t)max_context_len + 15) / 16);
  const int64_t units = std::max<int64_t>(1, (int64_t)batch * hkv);
  int64_t want = std::max((256 + units - 1) / units, (max_nblk + 255) / 256);
  if (256 % units == 0 && units * want > 256 && units * want < 512) want = 512 / units;
  int64_t best_s = (max_nblk + want - 1) / want;
  best_s = std::min<int64_t>(256, std::max<int64_t>(16, ((best_s + 7) / 8) * 8));
  int64_t s = best_s;
  // override for tests; a wave keeps at most 64 block ids (one per lane), so a
  // work-group of 8 waves takes at most 512 blocks
  if (const char *env = std::getenv("TQ_SPLIT_BLOCKS")) {
    const long v = std::strtol(env, nullptr, 10);
    if (v >= 1 && v <= 512) s = v;
  }
  SplitPlan p;
  p.split_blocks = (int)s;
  p.nsplit = (int)std::max<int64_t>(1, (max_nblk + s - 1) / s);
  return p;
}

SplitPlan plan_split_multitoken(int64_t units, int max_context_len, int max_split_blocks) {
  const int64_t max_nblk = std::max<int64_t>(1, ((int64_t)max_context_len + 15) / 16);
  units = std::max<int64_t>(1, units);
  const int64_t want = (256 + units - 1) / units;
  int64_t s = (max_nblk + want - 1) / want;
  s = std::min<int64_t>(max_split_blocks, std::max<int64_t>(16, ((s + 7) / 8) * 8));
  if (const char *env = std::getenv("TQ_SPLIT_BLOCKS")) {
    const long v = std::strtol(env, nullptr, 10);
    if (v >= 1 && v <= 4096) s = v;
  }
  SplitPlan p;
  p.split_blocks = (int)s;
  p.nsplit = (int)std::max<int64_t>(1, (max_nblk + s - 1) / s);
  return p;
}

}  // namespace tq
