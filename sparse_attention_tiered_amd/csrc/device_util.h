// Wave64 / workgroup primitives used by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spin {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
  return v;
}

// Exclusive prefix sum over a workgroup of NT threads (NT a multiple of 64,
// <= 1024), in thread order.  `tmp` is __shared__ int[NT / 64 + 1].  Every
// thread must call it; it contains barriers.  *total receives the sum.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int x = lane < W ? tmp[lane] : 0;
    const int xs = wave_incl_scan(x);
    if (lane < W) tmp[lane] = xs - x;
    if (lane == W - 1) tmp[W] = xs;
  }
  __syncthreads();
  const int res = tmp[w] + inc - v;
  *total = tmp[W];
  __syncthreads();
  return res;
}

// Exclusive prefix sums of counts[0 .. B) into pre (LDS, B <= 1024), in
// request order, by an NT-thread workgroup; returns the total.  tmp is LDS of
// NT / 64 + 1 ints.
template <int NT>
__device__ __forceinline__ int request_offsets(const int* __restrict__ counts, int B, int* pre,
                                               int* tmp) {
  constexpr int per = 1024 / NT;  // max_batch <= 1024
  static_assert(per * NT == 1024, "");
  const int tid = threadIdx.x;
  int loc[per], sum = 0;
#pragma unroll
  for (int u = 0; u < per; ++u) {
    const int b = tid * per + u;
    loc[u] = b < B ? counts[b] : 0;
    sum += loc[u];
  }
  int total;
  int ex = block_excl_scan<NT>(sum, tmp, &total);
#pragma unroll
  for (int u = 0; u < per; ++u) {
    const int b = tid * per + u;
    if (b < B) pre[b] = ex;
    ex += loc[u];
  }
  __syncthreads();
  return total;
}

// Largest b in [0, nb) with prefix[b] <= j (prefix ascending, prefix[0] = 0):
// the request that owns flat index j of a per-request concatenation.
__device__ __forceinline__ int owner_of(const int* prefix, int nb, int j) {
  int lo = 0, hi = nb;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= j) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Relaxed device-scope load that does not use a stale L1 line.
__device__ __forceinline__ int load_device(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace spin
