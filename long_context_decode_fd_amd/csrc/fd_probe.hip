// fd_probe.hip -- measurement helper of the benchmark, not part of the
// decode path: a plain streaming read of one buffer, the practical HBM read
// ceiling that the decode kernel's bandwidth is compared with next to the
// vendor figure.  Built as libfdprobe.so.
//
// Each workgroup of 256 threads reads one contiguous share of the buffer
// (1/grid of it, in whole kilobytes) with 16-byte nontemporal loads, UNR of them in flight per thread,
// consecutive threads on consecutive 16-byte units (every wavefront
// instruction reads 1 KB contiguously).  The loaded words are folded into
// one value that is stored only if it equals a constant, so the loads stay
// live without writing anything in practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 16;
constexpr unsigned kMagic = 0x9E3779B9u;

__global__ __launch_bounds__(kThreads) void stream_read(
    const u32x4 *__restrict__ p, size_t n16, unsigned *__restrict__ sink) {
  // Shares are balanced in whole kilobytes (64 units), so every wavefront
  // instruction reads whole 128-byte lines of an aligned buffer.
  constexpr size_t kStep = (size_t)kUnroll * kThreads;
  const size_t nkb = (n16 + 63) / 64;
  const size_t lo = nkb * blockIdx.x / gridDim.x * 64;
  size_t hi = nkb * (blockIdx.x + 1) / gridDim.x * 64;
  if (hi > n16) hi = n16;
  unsigned acc = 0;
  if (lo < hi) {
    // whole steps of kStep units need no bounds check
    const size_t full = lo + (hi - lo) / kStep * kStep;
    for (size_t i = lo + threadIdx.x; i < full; i += kStep) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        v[u] = __builtin_nontemporal_load(p + i + (size_t)u * kThreads);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (size_t j = full + threadIdx.x; j < hi; j += kThreads) {
      const u32x4 x = __builtin_nontemporal_load(p + j);
      acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
  }
  if (acc == kMagic) *sink = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from device buffer `buf` once on
// `stream` (a hipStream_t); `sink` is a device word the kernel may write.
// grid: workgroups (0 = 256).  Returns 0, or -1 for bad arguments, -4 for a
// HIP launch error.
int fdp_stream_read(const void *buf, size_t bytes, unsigned *sink, int grid,
                    void *stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || grid < 0 ||
      (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return -1;
  if (grid == 0) grid = 256;
  hipLaunchKernelGGL(stream_read, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const u32x4 *>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
