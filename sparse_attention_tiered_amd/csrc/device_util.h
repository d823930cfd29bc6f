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

// Cross-lane moves on the VALU (DPP), not through the LDS crossbar: a
// wave64 is four rows of 16 lanes; row_shr:n (control 0x110 + n) reads lane
// i - n of the same row, row_bcast:15 / row_bcast:31 (0x142 / 0x143) read
// the last lane of the row before / of row 1.  Lanes whose source lies
// outside the row, or whose row is masked off, receive `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_move(int old, int x) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele inside
// each row (shifts 1, 2, 4, 8), then row 0's total into row 1 and row 2's
// into row 3, then row 1's (now rows 0-1) into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_move<0x111, 0xf>(0, v);
  v += dpp_move<0x112, 0xf>(0, v);
  v += dpp_move<0x114, 0xf>(0, v);
  v += dpp_move<0x118, 0xf>(0, v);
  v += dpp_move<0x142, 0xa>(0, v);
  v += dpp_move<0x143, 0xc>(0, v);
  return v;
}

// Largest / smallest value over the 64 lanes of a wave, in every lane (the
// same steps as wave_incl_scan with max / min; lane 63 ends with the whole
// wave's, read back as a scalar).
__device__ __forceinline__ float wave_max(float v) {
  const int lo = (int)0xFF800000u;  // -inf: neutral for max
  v = fmaxf(v, __int_as_float(dpp_move<0x111, 0xf>(lo, __float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<0x112, 0xf>(lo, __float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<0x114, 0xf>(lo, __float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<0x118, 0xf>(lo, __float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<0x142, 0xa>(lo, __float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<0x143, 0xc>(lo, __float_as_int(v))));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_min(float v) {
  const int hi = (int)0x7F800000u;  // +inf: neutral for min
  v = fminf(v, __int_as_float(dpp_move<0x111, 0xf>(hi, __float_as_int(v))));
  v = fminf(v, __int_as_float(dpp_move<0x112, 0xf>(hi, __float_as_int(v))));
  v = fminf(v, __int_as_float(dpp_move<0x114, 0xf>(hi, __float_as_int(v))));
  v = fminf(v, __int_as_float(dpp_move<0x118, 0xf>(hi, __float_as_int(v))));
  v = fminf(v, __int_as_float(dpp_move<0x142, 0xa>(hi, __float_as_int(v))));
  v = fminf(v, __int_as_float(dpp_move<0x143, 0xc>(hi, __float_as_int(v))));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
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

}  // namespace spin
