// spec_common.hpp -- device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"

namespace specv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Pack two fp32 values into one dword of two bf16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Butterfly max / sum across the lanes whose ids differ only in bits 4 and 5
// (lanes l, l^16, l^32, l^48: the four k-groups of one MFMA 16x16x32 column).
__device__ __forceinline__ float xgroup_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float xgroup_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ void report_error(int32_t* dev_err, int32_t bits) {
  if (dev_err) atomicOr(dev_err, bits);
}

// Split-K partials that another work-group of the same launch reads back
// (possibly on another XCD, whose L2 is not coherent with this one) are
// stored and loaded with device-scope accesses (cache policy sc1): they go to
// the device's coherence point instead of resting in one XCD's L2.  The
// vector forms go through a raw buffer view of a work-group-uniform base.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(double* p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double load_coherent(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr int kBufferWord3 = 0x00020000;   // raw buffer descriptor, word 3 (32-bit data format)
constexpr int kDeviceScope = 16;           // buffer cache policy: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_view(const float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes,
                                           kBufferWord3);
}
__device__ __forceinline__ float load_coherent(__amdgpu_buffer_rsrc_t v, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(v, byte_off, 0,
                                                                        kDeviceScope));
}
__device__ __forceinline__ f32x4 load4_coherent(__amdgpu_buffer_rsrc_t v, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(v, byte_off, 0,
                                                                         kDeviceScope));
}
__device__ __forceinline__ void store4_coherent(__amdgpu_buffer_rsrc_t v, uint32_t byte_off,
                                                f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), v, byte_off, 0,
                                         kDeviceScope);
}

// Split merge (fixed split order, log2-domain running max): the factors that
// rescale the running sums (s_old) and a partial with max ms (s_new) when the
// partial is folded in; mx becomes the new running max.
__device__ __forceinline__ void merge_scales(float& mx, float ms, float& s_old, float& s_new) {
  const float mn = fmaxf(mx, ms);
  const float mu = (mn == -INFINITY) ? 0.f : mn;
  s_old = fast_exp2(mx - mu);
  s_new = fast_exp2(ms - mu);
  mx = mn;
}

// Split-K completion: every work-group of a group of n calls this once, after
// its partials are stored with the coherent stores above; it returns true in
// exactly one of them, the last to arrive, which may then read every member's
// partials with the coherent loads.  Each thread waits for its own stores to complete
// before the work-group barrier, and the counter is incremented after it.
// (An agent-scope release fence would also do, but it writes back the whole
// L2 of the XCD in every work-group, which costs tens of microseconds per
// launch.)  The counter lives in the caller's workspace: zero before the
// group's first use, and the last arrival puts it back to zero.  A count
// found at n or beyond (a workspace that was not zero-filled) sets
// SPEC_DEVERR_WORKSPACE and no member merges.  Every thread of the
// work-group must call it.
__device__ __forceinline__ bool last_arrival(uint32_t* counter, uint32_t n, int32_t* dev_err) {
  __shared__ uint32_t s_last;
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    uint32_t last = old + 1u == n;
    if (old >= n) {
      report_error(dev_err, SPEC_DEVERR_WORKSPACE);
      last = 0u;
    }
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  return s_last != 0u;
}

}  // namespace specv
