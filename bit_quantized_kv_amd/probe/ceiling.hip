// Measurement probes for bench.py: how fast this GPU streams plain reads, how
// fast it gathers whole records at random positions (the decode's access
// pattern) and how fast it streams the quantize's mix of reads and writes,
// with no arithmetic on the data beyond folding the words read.  Built into libtqprobe.so beside
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

// The quantize's mix of HBM traffic: per item 7 16-byte words read and 2
// written (its 78 : 22 split of read and written bytes).  Wave w takes chunks
// of 64 items: lane l reads words j * 64 + l (j < 7) of the chunk and writes
// the folds of its words 0-3 and 4-6 to words l and 64 + l of the chunk's
// output, so that every load and store is coalesced and every store depends on
// loads.  With `perm`, chunk c's output goes to output chunk perm[c] (a
// permutation): whole 2 KB pieces written at scattered places, as the
// quantize writes its records into the paged pool.
__device__ __forceinline__ uint4 xor4(uint4 a, uint4 b) {
  return make_uint4(a.x ^ b.x, a.y ^ b.y, a.z ^ b.z, a.w ^ b.w);
}
__global__ __launch_bounds__(256) void mixed_stream_kernel(const uint4 *src, uint4 *dst, const int32_t *perm,
                                                           int64_t chunks) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t c = wave; c < chunks; c += nwaves) {
    const uint4 *s = src + c * (7 * 64) + lane;
    uint4 a[7];
#pragma unroll
    for (int j = 0; j < 7; ++j) a[j] = s[j * 64];
    uint4 *d = dst + (perm ? (int64_t)perm[c] : c) * (2 * 64) + lane;
    d[0] = xor4(xor4(a[0], a[1]), xor4(a[2], a[3]));
    d[64] = xor4(xor4(a[4], a[5]), a[6]);
  }
}

}  // namespace

extern "C" {

// Reads 7 * 1024 * chunks bytes of `src` and writes 2 * 1024 * chunks bytes of
// `dst` (chunks of 64 items of 7 read and 2 written 16-byte words), with
// `grid` work-groups of 256 threads, on `stream`.  `perm`: NULL (chunk c
// writes output chunk c), or a device int32 permutation of [0, chunks) (the
// caller's; not checked).  Returns as tqprobe_stream_read.
int tqprobe_mixed_stream(const void *src, void *dst, const int32_t *perm, int64_t chunks, int grid,
                         void *stream) {
  if (!src || !dst || chunks <= 0 || grid < 1) return 1;
  hipLaunchKernelGGL(mixed_stream_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), perm, chunks);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

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
