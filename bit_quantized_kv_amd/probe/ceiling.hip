// Measurement probes for bench.py: how fast this GPU streams plain reads and
// how fast it gathers whole records at random positions (the decode's access
// pattern), with no arithmetic on the data.  Built into libtqprobe.so beside
// the library; no entry point of libtq.so uses it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

// A fold of every 32-bit word of a 16-byte load, so that the loads stay whole.
__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// The folds are stored only when they equal a value that the probes' data
// (equal words, so every fold of an even count is 0) never produces: the
// loads cannot be dropped and the store never happens.
constexpr uint32_t kNever = 0x9E3779B9u;

// Thread t reads 16-byte words t, t + S, t + 2S, ... (S = the grid's
// threads), four loads in flight.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *p, int64_t n, uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; i < n; i += stride) acc ^= fold(p[i]);
  if (acc == kNever) sink[0] = acc;
}

// Wave w reads records ids[w], ids[w + W], ... (W = the grid's waves), four
// records in flight: words (lane, lane + 64, ...) of the first `words`
// 16-byte words of each record, `rec_stride` bytes apart in the pool.
__global__ __launch_bounds__(256) void record_gather_kernel(const uint8_t *pool, const int32_t *ids, int64_t n,
                                                            int64_t rec_stride, int words, uint32_t *sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  uint32_t acc = 0;
  int64_t k = wave;
  for (; k + 3 * nwaves < n; k += 4 * nwaves) {
    const uint4 *r0 = reinterpret_cast<const uint4 *>(pool + (int64_t)ids[k] * rec_stride);
    const uint4 *r1 = reinterpret_cast<const uint4 *>(pool + (int64_t)ids[k + nwaves] * rec_stride);
    const uint4 *r2 = reinterpret_cast<const uint4 *>(pool + (int64_t)ids[k + 2 * nwaves] * rec_stride);
    const uint4 *r3 = reinterpret_cast<const uint4 *>(pool + (int64_t)ids[k + 3 * nwaves] * rec_stride);
    for (int w = lane; w < words; w += 64) acc ^= fold(r0[w]) ^ fold(r1[w]) ^ fold(r2[w]) ^ fold(r3[w]);
  }
  for (; k < n; k += nwaves) {
    const uint4 *r = reinterpret_cast<const uint4 *>(pool + (int64_t)ids[k] * rec_stride);
    for (int w = lane; w < words; w += 64) acc ^= fold(r[w]);
  }
  if (acc == kNever) sink[0] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` bytes (a multiple of 16) of device buffer `buf` once, with
// `grid` work-groups of 256 threads, on `stream`.  `sink`: one device word,
// never written in practice.  Returns 0, or 1 on a bad argument, 2 on a
// launch error.
int tqprobe_stream_read(const void *buf, int64_t bytes, void *sink, int grid, void *stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 || grid < 1) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4 *>(buf), bytes / 16, static_cast<uint32_t *>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Reads the first `rec_bytes` bytes (a multiple of 16, at most rec_stride) of
// records ids[0 .. n) of a pool whose record r starts at byte r * rec_stride
// (16-byte aligned; the caller keeps every id inside the pool), with `grid`
// work-groups of 256 threads, on `stream`.  Returns as tqprobe_stream_read.
int tqprobe_record_gather(const void *pool, const int32_t *ids, int64_t n, int64_t rec_stride, int rec_bytes,
                          void *sink, int grid, void *stream) {
  if (!pool || !ids || !sink || n <= 0 || rec_bytes <= 0 || rec_bytes % 16 || rec_stride % 16 ||
      rec_bytes > rec_stride || grid < 1)
    return 1;
  hipLaunchKernelGGL(record_gather_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t *>(pool), ids, n, rec_stride, rec_bytes / 16,
                     static_cast<uint32_t *>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
