// One page-head of attention on MFMA (v_mfma_f32_16x16x32_bf16): operand
// loads of a 32 KiB page (keys token-major, values dim-major), shared by the
// attention kernels and the transfer that attends pages on arrival.
//
// For one KV head the G <= 16 query heads (zero-padded to 16) give
//   logits^T [64 tok x 16 heads] = K [64 x 128] . q^T [128 x 16]
//   out^T    [128 dims x 16]    += V^T [128 x 64] . P^T [64 x 16]
// Lane (r, g) = (lane % 16, lane / 16).  The key rows are read in a permuted
// token order so the logits come out of the first MFMA exactly in the
// register layout the second MFMA needs for P^T.
#pragma once

#include "device_util.h"
#include "spin_internal.h"

namespace spin {

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Key tile tt, row r holds token 32 (tt/2) + 8 (r/4) + 4 (tt%2) + r%4: with
// that order the logits come out of the MFMA in the P^T operand layout.
__device__ __forceinline__ void load_keys(const uint16_t* K, int r, int g, bf16x8 (&ka)[4][4]) {
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int tok = 32 * (tt >> 1) + 8 * (r >> 2) + 4 * (tt & 1) + (r & 3);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      ka[tt][kb] = *reinterpret_cast<const bf16x8*>(K + tok * kHeadDim + 32 * kb + 8 * g);
  }
}

// Value tile dt, row r holds dim 16 dt + r; its k-slots are tokens 32 kt + 8 g + 0..7.
__device__ __forceinline__ void load_values(const uint16_t* Vt, int r, int g, bf16x8 (&va)[8][2]) {
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
      va[dt][kt] = *reinterpret_cast<const bf16x8*>(Vt + (16 * dt + r) * kPageTokens + 32 * kt + 8 * g);
}

}  // namespace spin
