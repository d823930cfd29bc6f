// Attention over the selected pages: paged sparse GQA decode.
//
// The SPIN pages run the algorithm's attention over the selected partitions
// only ([XT] design part 1, Fig. 3).  For query head g of request b (KV head
// h = g / G): out = softmax(q K^T / sqrt(128)) V over the valid tokens of the
// (b, h) block-table pages.
//
// Mapping to gfx950.  One (b, h) has G <= 16 query heads sharing every page,
// so each 64-token page is two small dense contractions done on MFMA
// (v_mfma_f32_16x16x32_bf16):
//   logits^T [64 tok x 16 heads] = K [64 x 128] . q^T [128 x 16]
//   out^T    [128 dims x 16]    += V^T [128 x 64] . P^T [64 x 16]
// Heads past G are zero padding.  The page layout (keys token-major, values
// dim-major) lets every MFMA operand be one contiguous 16-byte load per lane
// straight from HBM; the token order inside the key tiles is permuted so that
// the logits come out of the first MFMA exactly in the register layout the
// second MFMA needs for P^T.  P is split into a bf16 high part and a bf16
// residual so the PV product keeps about 16 mantissa bits of P.
//
// Work split: a workgroup of 4 waves takes a run of `pps` pages of one (b, h)
// (waves interleave pages), keeps an fp32 online softmax per head, merges its
// waves through LDS and writes one partial (max, sum, unnormalised output).
// k_attend_reduce merges the partials of a head (log-sum-exp).
#include "device_util.h"
#include "spin_internal.h"

namespace spin {

constexpr int kAttWG = 256;

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kAttWG) void k_attend_partial(Dev d, const uint16_t* __restrict__ q,
                                                           const int* __restrict__ bt,
                                                           const int* __restrict__ bntok,
                                                           const int* __restrict__ bcount) {
  __shared__ float sm_m[4][16];
  __shared__ float sm_l[4][16];
  __shared__ float sm_o[4][16][132];

  const int split = blockIdx.x % d.splits;
  const int bh = blockIdx.x / d.splits;
  const int b = bh / d.Hkv, h = bh - b * d.Hkv;
  const int G = d.G;
  const int cnt = min(bcount[bh], d.max_blocks);
  const int p_begin = split * d.pps;
  if (p_begin >= cnt) return;  // whole workgroup: nothing to do
  const int p_end = min(cnt, p_begin + d.pps);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;

  // B operand of the logits MFMA: lane (r, g) holds q[head r][32 kb + 8 g + 0..7]
  bf16x8 qb[4];
  if (r < G) {
    const uint16_t* qp = q + ((size_t)b * d.Hq + (size_t)h * G + r) * kHeadDim;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qb[kb] = *reinterpret_cast<const bf16x8*>(qp + 32 * kb + 8 * g);
  } else {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qb[kb] = bf16x8{};
  }

  f32x4 acc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // running max (log2 units) and this lane's partial sum
  const float sl2 = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)
  const int* btr = bt + (size_t)bh * d.max_blocks;
  const int* bnr = bntok + (size_t)bh * d.max_blocks;

  for (int p = p_begin + wave; p < p_end; p += 4) {
    const int slot = btr[p];
    const int nt = bnr[p];
    // a malformed entry (caller-supplied table) is skipped rather than read
    if ((unsigned)slot >= (unsigned)(d.B * d.C) || nt <= 0 || nt > kPageTokens) continue;
    const uint16_t* K = d.pool + (size_t)slot * kPageElems;
    const uint16_t* Vt = K + kPageTokens * kHeadDim;
    // key tile tt, row r holds token 32 (tt/2) + 8 (r/4) + 4 (tt%2) + r%4
    bf16x8 ka[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int tok = 32 * (tt >> 1) + 8 * (r >> 2) + 4 * (tt & 1) + (r & 3);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        ka[tt][kb] = *reinterpret_cast<const bf16x8*>(K + tok * kHeadDim + 32 * kb + 8 * g);
    }
    // value tile dt, row r holds dim 16 dt + r; k-slots are tokens 32 kt + 8 g + 0..7
    bf16x8 va[8][2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        va[dt][kt] = *reinterpret_cast<const bf16x8*>(Vt + (16 * dt + r) * kPageTokens + 32 * kt + 8 * g);

    f32x4 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[tt] = mfma16x16x32(ka[tt][kb], qb[kb], s[tt]);
    }
    // s[tt][i]: head r, token 32 (tt/2) + 8 g + 4 (tt%2) + i
    float pm = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 32 * (tt >> 1) + 8 * g + 4 * (tt & 1) + i;
        const float x = tok < nt ? s[tt][i] * sl2 : -INFINITY;
        s[tt][i] = x;
        pm = fmaxf(pm, x);
      }
    pm = fmaxf(pm, __shfl_xor(pm, 16, 64));
    pm = fmaxf(pm, __shfl_xor(pm, 32, 64));
    const float mn = fmaxf(m, pm);  // finite: every page has a valid token
    const float alpha = exp2f(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] *= alpha;
    bf16x8 phi[2], plo[2];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = exp2f(s[tt][i] - mn);
        l += pv;
        const __bf16 hi = (__bf16)pv;
        phi[tt >> 1][4 * (tt & 1) + i] = hi;
        plo[tt >> 1][4 * (tt & 1) + i] = (__bf16)(pv - (float)hi);
      }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        acc[dt] = mfma16x16x32(va[dt][kt], phi[kt], acc[dt]);
        acc[dt] = mfma16x16x32(va[dt][kt], plo[kt], acc[dt]);
      }
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  // acc[dt][i] = unnormalised out[head r][dim 16 dt + 4 g + i]
  if (g == 0) {
    sm_m[wave][r] = m;
    sm_l[wave][r] = l;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[wave][r][16 * dt + 4 * g + i] = acc[dt][i];
  __syncthreads();
  const int hh = threadIdx.x >> 4, dc = (threadIdx.x & 15) * 8;
  if (hh < G) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][hh]);
    float L = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sm_m[w][hh];
      const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
      L += sm_l[w][hh] * f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += sm_o[w][hh][dc + e] * f;
    }
    const size_t pi = ((size_t)bh * d.splits + split) * G + hh;
    float4* po = reinterpret_cast<float4*>(d.part_o + pi * kHeadDim + dc);
    po[0] = make_float4(o[0], o[1], o[2], o[3]);
    po[1] = make_float4(o[4], o[5], o[6], o[7]);
    if (dc == 0) {
      d.part_ml[2 * pi] = M;
      d.part_ml[2 * pi + 1] = L;
    }
  }
}

// One workgroup of 128 lanes per (request, query head): merge the head's
// split partials and normalise.
__global__ __launch_bounds__(128) void k_attend_reduce(Dev d, const int* __restrict__ bcount,
                                                       float* __restrict__ out) {
  const int bq = blockIdx.x;
  const int b = bq / d.Hq, gq = bq - b * d.Hq;
  const int h = gq / d.G, r = gq - h * d.G;
  const int bh = b * d.Hkv + h;
  const int ns = (min(bcount[bh], d.max_blocks) + d.pps - 1) / d.pps;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, d.part_ml[2 * (((size_t)bh * d.splits + s) * d.G + r)]);
  float L = 0.f, o = 0.f;
  for (int s = 0; s < ns; ++s) {
    const size_t pi = ((size_t)bh * d.splits + s) * d.G + r;
    const float ms = d.part_ml[2 * pi];
    const float f = ms == -INFINITY ? 0.f : exp2f(ms - M);
    L += d.part_ml[2 * pi + 1] * f;
    o += d.part_o[pi * kHeadDim + threadIdx.x] * f;
  }
  out[(size_t)bq * kHeadDim + threadIdx.x] = L > 0.f ? o / L : 0.f;
}

hipError_t launch_attend(const Dev& d, const uint16_t* q, const int* bt, const int* bntok,
                         const int* bcount, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_attend_partial, dim3(d.B * d.Hkv * d.splits), dim3(kAttWG), 0, s, d, q,
                     bt, bntok, bcount);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attend_reduce, dim3(d.B * d.Hq), dim3(kHeadDim), 0, s, d, bcount, out);
  return hipGetLastError();
}

}  // namespace spin
