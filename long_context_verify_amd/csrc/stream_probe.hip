// stream_probe.hip -- plain HBM streaming kernels that measure the device's
// practical read and copy rates, the reference the benchmark divides the
// verification kernels' rates by.  Not part of the verification path; built
// into its own library (libstreamprobe.so).
//
// Each work-group streams one contiguous share of the buffer in steps of
// 256 threads x 16 bytes x UNROLL (all loads of a step issued before any is
// used), so a step is UNROLL x 4 KB of one contiguous run, the access pattern
// of the attention kernels' K/V streams.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <int UNROLL, bool NT>
__global__ __launch_bounds__(kThreads) void stream_read(const f32x4* __restrict__ src,
                                                        size_t n_vec, float* sink) {
  const size_t per = (n_vec + gridDim.x - 1) / gridDim.x;
  const size_t lo = per * blockIdx.x;
  const size_t hi = lo + per < n_vec ? lo + per : n_vec;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (size_t base = lo; base < hi; base += (size_t)kThreads * UNROLL) {
    f32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const size_t i = base + (size_t)u * kThreads + threadIdx.x;
      v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i < hi) v[u] = NT ? __builtin_nontemporal_load(src + i) : src[i];
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc += v[u];
  }
  // Keeps the loads alive; the condition never holds for finite data.
  const float s = acc.x + acc.y + acc.z + acc.w;
  if (s == 1.2345e38f) sink[0] = s;
}

template <int UNROLL>
__global__ __launch_bounds__(kThreads) void stream_copy(const f32x4* __restrict__ src,
                                                        f32x4* __restrict__ dst, size_t n_vec) {
  const size_t per = (n_vec + gridDim.x - 1) / gridDim.x;
  const size_t lo = per * blockIdx.x;
  const size_t hi = lo + per < n_vec ? lo + per : n_vec;
  for (size_t base = lo; base < hi; base += (size_t)kThreads * UNROLL) {
    f32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const size_t i = base + (size_t)u * kThreads + threadIdx.x;
      if (i < hi) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const size_t i = base + (size_t)u * kThreads + threadIdx.x;
      if (i < hi) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16, 16-byte aligned) from src with `grid`
// work-groups; unroll in {4, 8, 16}; nt != 0 uses non-temporal loads.
// Returns 0, or -1 on a bad argument or a failed launch.
int probe_stream_read(const void* src, size_t bytes, float* sink, int grid, int unroll, int nt,
                      hipStream_t stream) {
  if (!src || !sink || bytes % 16 || grid < 1) return -1;
  const size_t n = bytes / 16;
  const f32x4* s = static_cast<const f32x4*>(src);
  dim3 g(grid), b(kThreads);
  if (unroll == 4 && nt)
    hipLaunchKernelGGL((stream_read<4, true>), g, b, 0, stream, s, n, sink);
  else if (unroll == 4)
    hipLaunchKernelGGL((stream_read<4, false>), g, b, 0, stream, s, n, sink);
  else if (unroll == 8 && nt)
    hipLaunchKernelGGL((stream_read<8, true>), g, b, 0, stream, s, n, sink);
  else if (unroll == 8)
    hipLaunchKernelGGL((stream_read<8, false>), g, b, 0, stream, s, n, sink);
  else if (unroll == 16 && nt)
    hipLaunchKernelGGL((stream_read<16, true>), g, b, 0, stream, s, n, sink);
  else if (unroll == 16)
    hipLaunchKernelGGL((stream_read<16, false>), g, b, 0, stream, s, n, sink);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Copy `bytes` (a multiple of 16, both pointers 16-byte aligned, no overlap).
int probe_stream_copy(const void* src, void* dst, size_t bytes, int grid, int unroll,
                      hipStream_t stream) {
  if (!src || !dst || bytes % 16 || grid < 1) return -1;
  const size_t n = bytes / 16;
  const f32x4* s = static_cast<const f32x4*>(src);
  f32x4* d = static_cast<f32x4*>(dst);
  dim3 g(grid), b(kThreads);
  if (unroll == 4)
    hipLaunchKernelGGL((stream_copy<4>), g, b, 0, stream, s, d, n);
  else if (unroll == 8)
    hipLaunchKernelGGL((stream_copy<8>), g, b, 0, stream, s, d, n);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
