// Calibrated key tables: a Lloyd fit of the 16 key-table entries on captured
// keys, per layer, and the per-element key-quantization MSE of the layer under
// the table in use and under the fitted one.
//
// [UQ] "方法怎麼做，白話講": the 16-entry table is refit on captured
// activations, about 20 vectors per rotated layer, and used only on the tenth
// of the layers whose per-element key MSE is highest.
//
// One work-group of 1024 threads per layer.  The layer's calibration set is
// small (about 20 tokens times the kv-heads), so the fit is a latency problem:
// the whole Lloyd loop runs inside one work-group, with the samples read from
// L2 each iteration and every reduction in a fixed order (deterministic).
#include "decode_common.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kCalThreads = 1024;
constexpr int kCalWaves = kCalThreads / 64;

__device__ __forceinline__ double shfl_xor_f64(double x, int m) { return __shfl_xor(x, m, 64); }

template <typename T>
__device__ __forceinline__ T wave_sum(T x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// fp64 -> fp16, round to nearest even, directly (no double rounding through
// fp32): scale to units of the target ulp, round to an integer, scale back.
__device__ __forceinline__ uint16_t f64_to_f16_bits(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const uint64_t mag = b & 0x7fffffffffffffffull;
  if (mag >= 0x7ff0000000000000ull) return sign | (mag > 0x7ff0000000000000ull ? 0x7e00u : 0x7c00u);
  const double ax = __builtin_bit_cast(double, mag);
  if (ax >= 65520.0) return sign | 0x7c00u;
  const int e = (int)(mag >> 52) - 1023;
  const int ulp_e = e < -14 ? -24 : e - 10;  // fp16 ulp exponent of ax's binade
  const double r = __builtin_rint(__builtin_ldexp(ax, -ulp_e));
  const float v = (float)__builtin_ldexp(r, ulp_e);  // exact: <= 11 significant bits
  return sign | h_bits((_Float16)v);
}

// fp64 unnormalized Walsh-Hadamard butterflies of one row, the same lane layout
// as rotate_row (D = 128: lane l holds channels 2l, 2l+1; D = 64: channel l).
template <int D>
__device__ __forceinline__ void rotate_row_f64(uint32_t w, int lane, double &x0, double &x1) {
  if constexpr (D == 128) {
    const double a = bf16_lo(w), b = bf16_hi(w);
    x0 = a + b;
    x1 = a - b;
  } else {
    x0 = (double)as_f(w << 16);
    x1 = 0.0;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const double p0 = shfl_xor_f64(x0, m), p1 = shfl_xor_f64(x1, m);
    x0 = (lane & m) ? p0 - x0 : x0 + p0;
    x1 = (lane & m) ? p1 - x1 : x1 + p1;
  }
}

struct CalibArgs {
  const uint16_t *k;             // bf16 [layers][rows][d]
  int64_t rows;
  int32_t max_iters;
  float rsqrt_d;                 // fp32(1/sqrt(d))
  double rsqrt_d64;              // fp64(1/sqrt(d))
  uint16_t init_f16[16];         // the table in use
  float *u;                      // workspace [layers][rows * d]: unit coordinates (NaN: row not sampled)
  double *y;                     // workspace [layers][rows * d]: exact rotation
  float *s;                      // workspace [layers][rows]: key scale (fp16 value)
  uint16_t *tables;              // [layers][16]
  double *levels;                // [layers][16] or null
  double *mse;                   // [layers][2] or null
  int32_t *updates;              // [layers] or null
};

// Per-element squared key error of the layer coded with the fp16 table whose
// values (as fp32) and fp32 midpoints sit in LDS.  The code is the coder's
// fp32 rule #{ j : u > t_j }.
__device__ double table_mse(const float *u, const double *y, const float *s, int64_t n, int d,
                            const float *c32, const float *t32, double *s_red) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  double acc = 0.0;
  for (int64_t e = tid; e < n; e += kCalThreads) {
    const float ue = u[e];
    // a row whose scale rounds to 0 decodes to 0 whatever its codes
    int code = 0;
#pragma unroll
    for (int j = 0; j < 15; ++j) code += ue > t32[j] ? 1 : 0;
    const double khat = ue != ue ? 0.0 : (double)c32[code] * (double)s[e / d];
    const double err = khat - y[e];
    acc += err * err;
  }
  acc = wave_sum(acc);
  if (lane == 0) s_red[wv] = acc;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < kCalWaves; ++w) tot += s_red[w];
  __syncthreads();
  return n > 0 ? tot / (double)n : 0.0;
}

__device__ void load_table(const uint16_t *t16, float *c32, float *t32) {
  const int tid = threadIdx.x;
  if (tid < 16) c32[tid] = (float)h_from(t16[tid]);
  __syncthreads();
  if (tid < 15) t32[tid] = (c32[tid] + c32[tid + 1]) * 0.5f;
  __syncthreads();
}

template <int D>
__global__ __launch_bounds__(kCalThreads) void calibrate_kernel(CalibArgs a) {
  __shared__ float s_c32[16], s_t32[16];
  __shared__ double s_c[16], s_t[16], s_red[kCalWaves];
  __shared__ double s_psum[kCalWaves][16];
  __shared__ int s_pcnt[kCalWaves][16];
  __shared__ uint16_t s_t16[16];

  const int layer = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t n = a.rows * D;
  const uint16_t *k = a.k + (int64_t)layer * n;
  float *u = a.u + (int64_t)layer * n;
  double *y = a.y + (int64_t)layer * n;
  float *s = a.s + (int64_t)layer * a.rows;

  // ---- unit coordinates as the key coder computes them, and the exact rotation
  for (int64_t r = wv; r < a.rows; r += kCalWaves) {
    const uint16_t *row = k + r * D;
    const uint32_t w = load_query_word<D>(row, lane);
    double ss;
    if constexpr (D == 128) {
      const double lo = bf16_lo(w), hi = bf16_hi(w);
      ss = lo * lo + hi * hi;            // exact (bf16 squares)
    } else {
      const double lo = as_f(w << 16);
      ss = lo * lo;
    }
    ss = wave_sum(ss);
    const _Float16 s16 = f16_rne_sqrt(ss * (1.0 / D));
    const float sv = (float)s16;
    float x0, x1;
    rotate_row<D>(w, lane, x0, x1);
    double y0, y1;
    rotate_row_f64<D>(w, lane, y0, y1);
    float u0 = __builtin_nanf(""), u1 = u0;
    if (sv > 0.f) {
      const float wsc = (1.0f / sv) * a.rsqrt_d;
      u0 = x0 * wsc;
      u1 = x1 * wsc;
    }
    const int64_t base = r * D;
    if constexpr (D == 128) {
      reinterpret_cast<float2 *>(u + base)[lane] = make_float2(u0, u1);
      reinterpret_cast<double2 *>(y + base)[lane] = make_double2(y0 * a.rsqrt_d64, y1 * a.rsqrt_d64);
    } else {
      u[base + lane] = u0;
      y[base + lane] = y0 * a.rsqrt_d64;
    }
    if (lane == 0) s[r] = sv;
  }
  if (tid < 16) {
    s_t16[tid] = a.init_f16[tid];
    s_c[tid] = (double)(float)h_from(a.init_f16[tid]);
  }
  __syncthreads();

  // ---- MSE under the table in use
  load_table(s_t16, s_c32, s_t32);
  const double mse0 = table_mse(u, y, s, n, D, s_c32, s_t32, s_red);

  // ---- Lloyd's iteration in fp64
  int updates = 0;
  while (updates < a.max_iters) {
    if (tid < 15) s_t[tid] = (s_c[tid] + s_c[tid + 1]) * 0.5;
    __syncthreads();
    double t[15];
#pragma unroll
    for (int j = 0; j < 15; ++j) t[j] = s_t[j];
    double sum[16];
    int cnt[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      sum[j] = 0.0;
      cnt[j] = 0;
    }
    for (int64_t e = tid; e < n; e += kCalThreads) {
      const float uf = u[e];
      if (uf != uf) continue;
      const double ue = uf;
      int cell = 0;
#pragma unroll
      for (int j = 0; j < 15; ++j) cell += ue > t[j] ? 1 : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        sum[j] += cell == j ? ue : 0.0;
        cnt[j] += cell == j ? 1 : 0;
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const double sj = wave_sum(sum[j]);
      const int cj = wave_sum(cnt[j]);
      if (lane == 0) {
        s_psum[wv][j] = sj;
        s_pcnt[wv][j] = cj;
      }
    }
    __syncthreads();
    int changed = 0;
    double nc = 0.0;
    if (tid < 16) {
      double tot = 0.0;
      int64_t cn = 0;
#pragma unroll
      for (int w = 0; w < kCalWaves; ++w) {
        tot += s_psum[w][tid];
        cn += s_pcnt[w][tid];
      }
      nc = cn > 0 ? tot / (double)cn + 0.0 : s_c[tid];  // + 0.0: a zero mean is +0
      changed = __builtin_bit_cast(uint64_t, nc) != __builtin_bit_cast(uint64_t, s_c[tid]);
    }
    if (!__syncthreads_or(changed)) break;
    if (tid < 16) s_c[tid] = nc;
    ++updates;
    __syncthreads();
  }

  // ---- outputs, and the MSE under the fitted fp16 table
  if (tid < 16) {
    s_t16[tid] = f64_to_f16_bits(s_c[tid]);
    a.tables[layer * 16 + tid] = s_t16[tid];
    if (a.levels) a.levels[layer * 16 + tid] = s_c[tid];
  }
  __syncthreads();
  load_table(s_t16, s_c32, s_t32);
  const double mse1 = table_mse(u, y, s, n, D, s_c32, s_t32, s_red);
  if (tid == 0) {
    if (a.mse) {
      a.mse[layer * 2] = mse0;
      a.mse[layer * 2 + 1] = mse1;
    }
    if (a.updates) a.updates[layer] = updates;
  }
}

}  // namespace

size_t calibrate_workspace_bytes(int64_t layers, int64_t rows, int d) {
  const size_t n = (size_t)layers * (size_t)rows * (size_t)d;
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return up(n * 8) + up(n * 4) + up((size_t)layers * (size_t)rows * 4);
}

hipError_t launch_calibrate(int d, int layers, int64_t rows, const uint16_t *k, const uint16_t init_f16[16],
                            int max_iters, float rsqrt_d, void *workspace, uint16_t *tables, double *levels,
                            double *mse, int32_t *updates, hipStream_t stream) {
  CalibArgs a{};
  a.k = k;
  a.rows = rows;
  a.max_iters = max_iters;
  a.rsqrt_d = rsqrt_d;
  a.rsqrt_d64 = 1.0 / __builtin_sqrt((double)d);
  for (int i = 0; i < 16; ++i) a.init_f16[i] = init_f16[i];
  const size_t n = (size_t)layers * (size_t)rows * (size_t)d;
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  a.y = reinterpret_cast<double *>(ws);
  a.u = reinterpret_cast<float *>(ws + up(n * 8));
  a.s = reinterpret_cast<float *>(ws + up(n * 8) + up(n * 4));
  a.tables = tables;
  a.levels = levels;
  a.mse = mse;
  a.updates = updates;
  if (d == 128)
    hipLaunchKernelGGL(calibrate_kernel<128>, dim3(layers), dim3(kCalThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(calibrate_kernel<64>, dim3(layers), dim3(kCalThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
