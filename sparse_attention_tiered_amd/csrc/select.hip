// Select: partition scoring and per-KV-head top-k.
//
// The SPIN pages leave the Select rule to the algorithm ([XT] design part 1,
// Fig. 3); the rule here is fixed: score = (mean of the G queries of the KV
// head's group) . (partition summary) / sqrt(128), and the k highest scores
// per (request, KV head) are kept, the lower partition id winning an exact
// tie, output in ascending id order.
//
// Scoring streams the float32 summaries once (512 B per partition) and is
// HBM-bound: eight lanes cover one 512 B summary row with float4 loads, so a
// wave instruction touches eight whole 128 B lines; the dot product is reduced
// over those eight lanes with three xor shuffles.
#include "device_util.h"
#include "spin_internal.h"

namespace spin {

constexpr int kScoreWG = 256;             // 4 waves
constexpr int kScorePerWave = 64;         // partitions per wave
constexpr int kScorePerWG = 4 * kScorePerWave;

__global__ __launch_bounds__(kScoreWG) void k_score(Dev d, const uint16_t* __restrict__ q,
                                                    float* __restrict__ scores) {
  __shared__ uint4 sq[kMaxGroup * kHeadDim / 8];  // the group's bf16 queries
  __shared__ float sqbar[kHeadDim];               // their sum, times 1 / (G sqrt(128))
  const int bh = blockIdx.y;
  const int b = bh / d.Hkv, h = bh - b * d.Hkv;
  const int n = d.req_parts[b];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 3, r = lane & 7;
  const int p0 = blockIdx.x * kScorePerWG + wave * kScorePerWave;
  const bool active = p0 < n;
  float* srow = scores + (size_t)bh * d.Nmax;

  // 1. the group's queries: one 16-byte load per thread, issued first so that
  //    waiting for it does not wait for the summary loads behind it
  const int nq = d.G * kHeadDim / 8;
  uint4 qc = make_uint4(0u, 0u, 0u, 0u);
  if (tid < nq) qc = reinterpret_cast<const uint4*>(q + ((size_t)b * d.Hq + (size_t)h * d.G) * kHeadDim)[tid];
  // 2. the summaries, branch-free: a row past the request's partitions
  //    re-reads row p0 and its score is replaced below; group `grp` handles
  //    partitions p0 + 8 grp + it
  const float* S = d.summaries + (size_t)bh * d.Nmax * kHeadDim;
  float4 v[8][4];
  if (active) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int p = p0 + 8 * grp + it;
      const float* row = S + (size_t)(p < n ? p : p0) * kHeadDim + 4 * r;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[it][j] = *reinterpret_cast<const float4*>(row + 32 * j);
    }
  }
  // 3. mean query through LDS while the summaries are in flight
  if (tid < nq) sq[tid] = qc;
  __syncthreads();
  if (tid < kHeadDim) {
    const uint16_t* sq16 = reinterpret_cast<const uint16_t*>(sq);
    float sum = 0.f;
    for (int g = 0; g < d.G; ++g) sum += __uint_as_float((uint32_t)sq16[g * kHeadDim + tid] << 16);
    sqbar[tid] = sum * (1.0f / ((float)d.G * sqrtf((float)kHeadDim)));
  }
  __syncthreads();
  if (!active) {
    if (p0 + lane < d.Nmax) srow[p0 + lane] = -INFINITY;
    return;
  }
  float qv[16];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[4 * j + e] = sqbar[32 * j + 4 * r + e];
  float acc[8];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a = fmaf(v[it][j].x, qv[4 * j + 0], a);
      a = fmaf(v[it][j].y, qv[4 * j + 1], a);
      a = fmaf(v[it][j].z, qv[4 * j + 2], a);
      a = fmaf(v[it][j].w, qv[4 * j + 3], a);
    }
    a += __shfl_xor(a, 1, 64);
    a += __shfl_xor(a, 2, 64);
    a += __shfl_xor(a, 4, 64);
    acc[it] = a;
  }
  // lane 8 grp + r takes partition p0 + 8 grp + r, i.e. acc[r]
  float mine = acc[0];
#pragma unroll
  for (int it = 1; it < 8; ++it) mine = (r == it) ? acc[it] : mine;
  const int p = p0 + lane;
  if (p < d.Nmax) srow[p] = (p < n) ? mine : -INFINITY;
}

// Order-preserving map of float32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exact top-k per (request, KV head) by MSB-first radix select over 8-bit
// digits of the order-preserving keys, in LDS.  One workgroup per list.
template <int NT>
__global__ __launch_bounds__(NT) void k_topk(Dev d, const float* __restrict__ scores,
                                             int* __restrict__ sel) {
  __shared__ uint32_t keys[kMaxPartitions];
  __shared__ int hist[256];
  __shared__ int tmp[NT / 64 + 1];
  __shared__ int sh_digit, sh_kk;
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv;
  const int n = d.req_parts[b];
  const int k = d.k;
  const int tid = threadIdx.x;
  int* out = sel + (size_t)bh * k;
  if (n <= k) {
    for (int i = tid; i < k; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  const float* srow = scores + (size_t)bh * d.Nmax;
  for (int i = tid; i < n; i += NT) keys[i] = float_key(srow[i]);
  uint32_t prefix = 0, mask = 0;
  int kk = k;  // how many still to take among keys matching `prefix`
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds digits 255-4l .. 252-4l (descending)
      int c[4], cs = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * tid - j];
        cs += c[j];
      }
      const int inc = wave_incl_scan(cs);
      const unsigned long long hit = __ballot(inc >= kk);
      const int L = __ffsll((long long)hit) - 1;
      if (tid == L) {
        int above = inc - cs;
        int dg = 255 - 4 * tid;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (above + c[j] >= kk) {
            dg = 255 - 4 * tid - j;
            break;
          }
          above += c[j];
        }
        sh_digit = dg;
        sh_kk = kk - above;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh_digit << shift;
    mask |= 0xFFu << shift;
    kk = sh_kk;
    __syncthreads();
  }
  // prefix is the k-th largest key; take every larger key and the kk lowest
  // indices among keys equal to it.
  const uint32_t T = prefix;
  const int E = (n + NT - 1) / NT;
  const int lo = tid * E, hi = min(n, lo + E);
  int n_eq = 0;
  for (int i = lo; i < hi; ++i) n_eq += keys[i] == T;
  int tot;
  int eq_rank = block_excl_scan<NT>(n_eq, tmp, &tot);
  int n_take = 0;
  for (int i = lo, er = eq_rank; i < hi; ++i) {
    const uint32_t key = keys[i];
    if (key > T) ++n_take;
    else if (key == T) n_take += (er++ < kk);
  }
  int pos = block_excl_scan<NT>(n_take, tmp, &tot);
  for (int i = lo, er = eq_rank; i < hi; ++i) {
    const uint32_t key = keys[i];
    bool take = key > T;
    if (key == T) take = er++ < kk;
    if (take && pos < k) out[pos++] = i;
  }
}

hipError_t launch_score(const Dev& d, const uint16_t* q, float* scores, hipStream_t s) {
  dim3 grid((d.Nmax + kScorePerWG - 1) / kScorePerWG, d.B * d.Hkv);
  hipLaunchKernelGGL(k_score, grid, dim3(kScoreWG), 0, s, d, q, scores);
  return hipGetLastError();
}

hipError_t launch_topk(const Dev& d, const float* scores, int* sel, hipStream_t s) {
  // 1024 threads: measured fastest (per-key work dominates, not barriers;
  // 512 and 256 threads were 1.1-1.9x slower on 2048 and 7.7K-key lists)
  hipLaunchKernelGGL(k_topk<1024>, dim3(d.B * d.Hkv), dim3(1024), 0, s, d, scores, sel);
  return hipGetLastError();
}

}  // namespace spin
