// Streaming HBM read probe, for measurement only (not part of the verify path): every
// workgroup reads a contiguous share of a buffer with 16-byte non-temporal loads, eight per
// thread in flight, and folds them into one word per thread so that no load is dead.  The
// bench divides the bytes read by the time to report the bandwidth this GPU delivers to a plain
// read, next to the 8 TB/s specification.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4* __restrict__ src,
                                                              int64_t n_vec, uint32_t* sink) {
  const int64_t per_wg = (n_vec + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per_wg;
  const int64_t hi = lo + per_wg < n_vec ? lo + per_wg : n_vec;
  uint32_t acc = 0;
  for (int64_t base = lo; base < hi; base += (int64_t)kThreads * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kThreads + threadIdx.x;
      v[u] = i < hi ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

// bytes: a multiple of 16; sink: workgroups * 256 uint32 of device memory.  Returns a
// hipError_t code (0 on success).
extern "C" int rkv_probe_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* sink,
                              void* stream) {
  if (src == nullptr || sink == nullptr || bytes <= 0 || bytes % 16 != 0 || workgroups < 1)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_probe_kernel, dim3(workgroups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     bytes / 16, sink);
  return (int)hipGetLastError();
}
