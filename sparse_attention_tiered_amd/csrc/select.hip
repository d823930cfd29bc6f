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
  q = step_queries(d, q);
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

// Exact top-k per (request, KV head), one workgroup per list, in LDS.
//
// Scores are spread into 2048 buckets linearly between their minimum and
// maximum.  The map is monotone, so every score in a higher bucket beats every
// score in a lower one: one histogram and one suffix scan find the bucket
// holding the k-th score, everything above it is taken, and only that
// bucket's few candidates are ranked exactly (higher score first, lower id on
// ties).  A crowded boundary bucket (many equal or nearly equal scores) falls
// back to an MSB-first radix select over order-preserving keys of its members.
constexpr int kTopkBins = 2048;
constexpr int kTopkCand = 256;  // largest boundary bucket ranked pairwise

// Clamped in float before the conversion, so any input (an infinite or NaN
// score from corrupt keys) still lands in a valid bucket.
__device__ __forceinline__ int topk_bucket(float v, float mn, float scale) {
  const float f = fminf(fmaxf((v - mn) * scale, 0.f), (float)(kTopkBins - 1));
  return (int)f;
}

// LDS of one top-k workgroup, besides the scores themselves (an array of
// the list's length, reused for radix keys, that each caller provides).
template <int NT>
struct TopkLds {
  int hist[kTopkBins];
  int cand[kTopkCand];
  float candv[kTopkCand];
  uint32_t chosen[kMaxPartitions / 32];
  int tmp[NT / 64 + 1];
  float rmin[NT / 64], rmax[NT / 64];
  int sh[4];  // boundary bucket, count above it, fill counter / radix state
};

// The selection itself, once the n > k scores of the list sit in vals (LDS)
// and each thread holds the min / max of the scores it wrote: writes the k
// chosen ids, ascending, to out.  Every thread of the workgroup calls it.
template <int NT>
__device__ void topk_select(TopkLds<NT>& L, float* vals, int n, int k, float mn, float mx, int* out) {
  static_assert(kTopkBins % NT == 0 && NT >= kTopkCand && NT >= 256, "whole buckets per thread");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < kTopkBins; i += NT) L.hist[i] = 0;
  for (int i = tid; i < (n + 31) / 32; i += NT) L.chosen[i] = 0;
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) {
    L.rmin[wv] = mn;
    L.rmax[wv] = mx;
  }
  if (tid == 0) L.sh[2] = 0;
  __syncthreads();
  mn = L.rmin[0];
  mx = L.rmax[0];
  for (int w = 1; w < NT / 64; ++w) {
    mn = fminf(mn, L.rmin[w]);
    mx = fmaxf(mx, L.rmax[w]);
  }
  // a range too narrow for a finite scale puts everything in bucket 0
  float scale = (float)kTopkBins / (mx - mn);
  if (!(scale < 3.0e38f)) scale = 0.f;
  for (int i = tid; i < n; i += NT) atomicAdd(&L.hist[topk_bucket(vals[i], mn, scale)], 1);
  __syncthreads();
  // counts from the top: thread t holds the PER buckets just below
  // 2047 - PER t, highest first
  {
    constexpr int PER = kTopkBins / NT;
    const int top = kTopkBins - 1 - PER * tid;
    int cnts[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      cnts[i] = L.hist[top - i];
      sum += cnts[i];
    }
    int tot;
    int before = block_excl_scan<NT>(sum, L.tmp, &tot);
    if (before < k && before + sum >= k) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if (before + cnts[i] >= k) {
          L.sh[0] = top - i;
          L.sh[1] = before;
          break;
        }
        before += cnts[i];
      }
    }
  }
  __syncthreads();
  const int cut = L.sh[0];
  const int need = k - L.sh[1];  // >= 1: taken from the boundary bucket
  const int m = L.hist[cut];     // its members
  if (m <= kTopkCand) {
    for (int i = tid; i < n; i += NT) {
      const float v = vals[i];
      const int bk = topk_bucket(v, mn, scale);
      if (bk > cut) atomicOr(&L.chosen[i >> 5], 1u << (i & 31));
      if (bk == cut) {
        const int slot = atomicAdd(&L.sh[2], 1);
        if (slot < kTopkCand) {
          L.cand[slot] = i;
          L.candv[slot] = v;
        }
      }
    }
    __syncthreads();
    if (tid < m) {
      const int me = L.cand[tid];
      const float v = L.candv[tid];
      int rank = 0;
      for (int j = 0; j < m; ++j) {
        const int o = L.cand[j];
        const float w = L.candv[j];
        rank += (w > v || (w == v && o < me)) ? 1 : 0;
      }
      if (rank < need) atomicOr(&L.chosen[me >> 5], 1u << (me & 31));
    }
  } else {
    // radix select among the boundary bucket's members; key 0 marks the rest
    // (no finite score maps to 0)
    uint32_t* keys = reinterpret_cast<uint32_t*>(vals);
    for (int i = tid; i < n; i += NT) {
      const float v = vals[i];
      const int bk = topk_bucket(v, mn, scale);
      if (bk > cut) atomicOr(&L.chosen[i >> 5], 1u << (i & 31));
      keys[i] = bk == cut ? float_key(v + 0.f) : 0u;  // -0 ranks as +0
    }
    uint32_t prefix = 0, mask = 0;
    int kk = need;
    for (int shift = 24; shift >= 0; shift -= 8) {
      __syncthreads();
      for (int i = tid; i < 256; i += NT) L.hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += NT) {
        const uint32_t key = keys[i];
        if (key != 0u && (key & mask) == prefix) atomicAdd(&L.hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        int c4[4], cs = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c4[j] = L.hist[255 - 4 * tid - j];
          cs += c4[j];
        }
        const int inc = wave_incl_scan(cs);
        const unsigned long long hitm = __ballot(inc >= kk);
        const int lead = __ffsll((long long)hitm) - 1;
        if (tid == lead) {
          int ab = inc - cs, dg = 255 - 4 * tid;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (ab + c4[j] >= kk) {
              dg = 255 - 4 * tid - j;
              break;
            }
            ab += c4[j];
          }
          L.sh[3] = dg;
          L.sh[2] = kk - ab;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)L.sh[3] << shift;
      mask |= 0xFFu << shift;
      kk = L.sh[2];
    }
    // members above the k-th key, then the kk lowest ids equal to it
    const int E = (n + NT - 1) / NT;
    const int lo = tid * E, hi = min(n, lo + E);
    int n_eq = 0;
    for (int i = lo; i < hi; ++i) n_eq += keys[i] == prefix;
    int tot;
    int er = block_excl_scan<NT>(n_eq, L.tmp, &tot);
    for (int i = lo; i < hi; ++i) {
      const uint32_t key = keys[i];
      const bool take = key > prefix || (key == prefix && er++ < kk);
      if (take) atomicOr(&L.chosen[i >> 5], 1u << (i & 31));
    }
  }
  __syncthreads();
  // output in ascending partition id
  const int E = (n + NT - 1) / NT;
  const int lo = tid * E, hi = min(n, lo + E);
  int n_take = 0;
  for (int i = lo; i < hi; ++i) n_take += (L.chosen[i >> 5] >> (i & 31)) & 1u;
  int tot;
  int pos = block_excl_scan<NT>(n_take, L.tmp, &tot);
  for (int i = lo; i < hi; ++i)
    if (((L.chosen[i >> 5] >> (i & 31)) & 1u) && pos < k) out[pos++] = i;
}

// The same selection in fewer dependent steps (each step of a 1024-thread
// workgroup is a barrier and an LDS round trip, which is what the top-k's time
// goes into): the scores are spread over 256 value bins linearly between the
// list's minimum and maximum, so one wave finds the boundary bin with a single
// prefix scan; the bins above it are taken, the boundary bin's members
// (usually a handful) are ranked exactly, and the chosen ids are written in
// ascending order from a popcount prefix over the chosen bitmask.  A crowded
// boundary bin (more than kTopkCand members: many equal or nearly equal
// scores) goes to topk_select, which splits it further.
constexpr int kCoarseBins = 256;

struct BinMap {
  float mn, scale;
};

// Monotone map of [mn, mx] onto the coarse bins; a range too narrow for a
// finite scale puts every score into bin 0.  Clamped in float before the
// conversion, so any input lands in a valid bin.
__device__ __forceinline__ BinMap coarse_map(float mn, float mx) {
  float scale = (float)kCoarseBins / (mx - mn);
  if (!(scale < 3.0e38f)) scale = 0.f;
  return BinMap{mn, scale};
}
__device__ __forceinline__ int coarse_bin(float v, BinMap m) {
  return (int)fminf(fmaxf((v - m.mn) * m.scale, 0.f), (float)(kCoarseBins - 1));
}

// Clears what the coarse selection accumulates into: the first kCoarseBins
// histogram entries, the chosen bitmask over n ids and the member counter.
// Must be followed by a barrier before the histogram is filled.
template <int NT>
__device__ __forceinline__ void topk_coarse_clear(TopkLds<NT>& L, int n) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kCoarseBins; i += NT) L.hist[i] = 0;
  for (int i = tid; i < (n + 31) / 32; i += NT) L.chosen[i] = 0;
  if (tid == 0) L.sh[2] = 0;
}

// The selection once the n > k scores sit in vals (LDS) and each is counted
// once in L.hist[coarse_bin(score, m)], with a barrier passed since (and the
// bitmask and member counter cleared before it).  mn, mx: the list's range,
// for the fallback.  Writes the k chosen ids, ascending, to out.  Every
// thread of the workgroup calls it.
template <int NT>
__device__ void topk_coarse(TopkLds<NT>& L, float* vals, int n, int k, BinMap m, float mn, float mx,
                            int* out) {
  static_assert(NT >= kTopkCand && kCoarseBins == 4 * 64, "four bins per lane of one wave");
  const int tid = threadIdx.x, lane = tid & 63;
  // 1. the boundary bin: counts from the top, four bins per lane, found by
  //    every wave on its own (the same scan of the same counts, so the same
  //    answer in each, and no barrier to pass it on)
  int cut, above, mem;
  {
    int c[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = L.hist[kCoarseBins - 1 - 4 * lane - j];
      sum += c[j];
    }
    const int inc = wave_incl_scan(sum);
    const int lead = __ffsll((long long)__ballot(inc >= k)) - 1;  // exists: the total is n > k
    int ab = inc - sum, b = kCoarseBins - 1 - 4 * lane, mb = c[0];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b = kCoarseBins - 1 - 4 * lane - j;
      mb = c[j];
      if (ab + c[j] >= k) break;
      ab += c[j];
    }
    cut = __builtin_amdgcn_readlane(b, lead);
    above = __builtin_amdgcn_readlane(ab, lead);
    mem = __builtin_amdgcn_readlane(mb, lead);
  }
  const int need = k - above;  // >= 1: taken from the boundary bin
  if (mem > kTopkCand) {  // (uniform over the workgroup)
    __syncthreads();       // every wave is done reading the counts it reuses
    topk_select<NT>(L, vals, n, k, mn, mx, out);
    return;
  }
  // 2. every score above the boundary bin is taken; the bin's members listed
  for (int i = tid; i < n; i += NT) {
    const float v = vals[i];
    const int bk = coarse_bin(v, m);
    if (bk > cut) {
      atomicOr(&L.chosen[i >> 5], 1u << (i & 31));
    } else if (bk == cut) {
      const int slot = atomicAdd(&L.sh[2], 1);
      L.cand[slot] = i;
      L.candv[slot] = v;
    }
  }
  __syncthreads();
  // 3. the members ranked exactly: higher score first, the lower id on a tie.
  //    Up to 64 members sit in wave 0's lanes and are compared through
  //    readlane (no LDS round trip per comparison), and the same wave goes on
  //    to step 4 with no barrier between; more members take one thread each.
  if (mem > 64) {
    if (tid < mem) {
      const int me = L.cand[tid];
      const float v = L.candv[tid];
      int rank = 0;
      for (int j = 0; j < mem; ++j) {
        const int o = L.cand[j];
        const float w = L.candv[j];
        rank += (w > v || (w == v && o < me)) ? 1 : 0;
      }
      if (rank < need) atomicOr(&L.chosen[me >> 5], 1u << (me & 31));
    }
    __syncthreads();
  } else if (tid < 64) {
    const int me = lane < mem ? L.cand[lane] : 0;
    const float v = lane < mem ? L.candv[lane] : 0.f;
    int rank = 0;
    for (int j = 0; j < mem; ++j) {
      const int o = __builtin_amdgcn_readlane(me, j);
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
      rank += (w > v || (w == v && o < me)) ? 1 : 0;
    }
    if (lane < mem && rank < need) atomicOr(&L.chosen[me >> 5], 1u << (me & 31));
  }
  // 4. ids ascending, written by wave 0 alone: consecutive bitmask words per
  //    lane, an exclusive prefix of their popcounts, then each lane writes
  //    the ids of its words' set bits (no barrier, no pass over every id by
  //    the whole workgroup).  In the readlane case wave 0 set the members'
  //    bits itself just before: one wave's LDS accesses take effect in
  //    program order.
  if (tid < 64) {
    const int nw = (n + 31) / 32;
    const int W = (nw + 63) / 64;
    const int w0 = lane * W, w1 = min(nw, w0 + W);
    int sum = 0;
    for (int w = w0; w < w1; ++w) sum += __popc(L.chosen[w]);
    int pos = wave_incl_scan(sum) - sum;
    for (int w = w0; w < w1; ++w) {
      uint32_t word = L.chosen[w];
      while (word != 0u) {
        if (pos < k) out[pos] = 32 * w + __builtin_ctz(word);
        ++pos;
        word &= word - 1u;
      }
    }
  }
}

// The coarse selection from scores that each thread wrote to vals itself,
// with each thread's own minimum and maximum of them: the range is combined
// over the workgroup (one barrier), every score binned, then topk_coarse.
// Clears its own accumulators.  Every thread calls it.
template <int NT>
__device__ void topk_from_lds(TopkLds<NT>& L, float* vals, int n, int k, float mn, float mx, int* out) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  topk_coarse_clear<NT>(L, n);
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) {
    L.rmin[wv] = mn;
    L.rmax[wv] = mx;
  }
  __syncthreads();
  mn = L.rmin[0];
  mx = L.rmax[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) {
    mn = fminf(mn, L.rmin[w]);
    mx = fmaxf(mx, L.rmax[w]);
  }
  const BinMap m = coarse_map(mn, mx);
  for (int i = tid; i < n; i += NT) atomicAdd(&L.hist[coarse_bin(vals[i], m)], 1);
  __syncthreads();
  topk_coarse<NT>(L, vals, n, k, m, mn, mx, out);
}

template <int NT>
__global__ __launch_bounds__(NT) void k_topk(Dev d, const float* __restrict__ scores,
                                             int* __restrict__ sel) {
  __shared__ TopkLds<NT> L;
  __shared__ float vals[kMaxPartitions];
  const int bh = blockIdx.x;
  const int n = d.req_parts[bh / d.Hkv];
  const int k = d.k;
  const int tid = threadIdx.x;
  int* out = sel + (size_t)bh * k;
  if (n <= k) {
    for (int i = tid; i < k; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  const float* srow = scores + (size_t)bh * d.Nmax;
  float mn = INFINITY, mx = -INFINITY;
  // eight scores' loads in flight per thread (from clamped indices, so no
  // load sits in a branch of its own), one round trip per 8 NT scores
  constexpr int U = 8;
  for (int i0 = tid; i0 < n; i0 += NT * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = srow[min(i0 + NT * u, n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + NT * u;
      if (i < n) {
        vals[i] = v[u];
        mn = fminf(mn, v[u]);
        mx = fmaxf(mx, v[u]);
      }
    }
  }
  topk_from_lds<NT>(L, vals, n, k, mn, mx, out);
}

// Scoring and top-k of one (request, KV head) in one 1024-thread workgroup,
// for batches with enough heads to occupy the chip: the scores go straight
// into the top-k's LDS (and to `scores`), with no second launch and no
// re-read.  Each row's dot product is computed exactly as in k_score (same
// lanes, same order of operations), so both paths give the same scores.
constexpr int kFusedRows = 4;  // rows in flight per 8-lane group

__global__ __launch_bounds__(1024) void k_select_fused(Dev d, const uint16_t* __restrict__ q,
                                                       float* __restrict__ scores,
                                                       int* __restrict__ sel) {
  q = step_queries(d, q);
  __shared__ TopkLds<1024> L;
  __shared__ float vals[kMaxPartitions];
  __shared__ uint4 sq[kMaxGroup * kHeadDim / 8];
  __shared__ float sqbar[kHeadDim];
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv, h = bh - b * d.Hkv;
  const int n = d.req_parts[b];
  const int k = d.k;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 3, r = lane & 7;
  float* srow = scores + (size_t)bh * d.Nmax;
  int* out = sel + (size_t)bh * k;
  for (int p = n + tid; p < d.Nmax; p += 1024) srow[p] = -INFINITY;

  // wave `wave` of a pass covers rows base + 32 wave + 4 grp + it, it < 4; a
  // row past the list re-reads row 0 and is not used
  const float* S = d.summaries + (size_t)bh * d.Nmax * kHeadDim;
  constexpr int kRowsPerPass = 16 * 8 * kFusedRows;
  float4 v[kFusedRows][4];
  auto load_pass = [&](int base) {
    const int p0 = base + wave * 8 * kFusedRows + kFusedRows * grp;
#pragma unroll
    for (int it = 0; it < kFusedRows; ++it) {
      const int p = p0 + it;
      const float* row = S + (size_t)(p < n ? p : 0) * kHeadDim + 4 * r;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[it][j] = *reinterpret_cast<const float4*>(row + 32 * j);
    }
  };
  // the group's queries, then the first pass's summaries in flight while
  // their mean is formed
  const int nq = d.G * kHeadDim / 8;
  uint4 qc = make_uint4(0u, 0u, 0u, 0u);
  if (tid < nq) qc = reinterpret_cast<const uint4*>(q + ((size_t)b * d.Hq + (size_t)h * d.G) * kHeadDim)[tid];
  load_pass(0);
  if (tid < nq) sq[tid] = qc;
  __syncthreads();
  if (tid < kHeadDim) {
    const uint16_t* sq16 = reinterpret_cast<const uint16_t*>(sq);
    float sum = 0.f;
    for (int g = 0; g < d.G; ++g) sum += __uint_as_float((uint32_t)sq16[g * kHeadDim + tid] << 16);
    sqbar[tid] = sum * (1.0f / ((float)d.G * sqrtf((float)kHeadDim)));
  }
  __syncthreads();
  float qv[16];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[4 * j + e] = sqbar[32 * j + 4 * r + e];

  float mn = INFINITY, mx = -INFINITY;
  for (int base = 0; base < n; base += kRowsPerPass) {
    if (base > 0) load_pass(base);
    const int p0 = base + wave * 8 * kFusedRows + kFusedRows * grp;
    float acc[kFusedRows];
#pragma unroll
    for (int it = 0; it < kFusedRows; ++it) {
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
    // lane r < 4 of the group writes row p0 + r
    if (r < kFusedRows) {
      float mine = acc[0];
#pragma unroll
      for (int it = 1; it < kFusedRows; ++it) mine = (r == it) ? acc[it] : mine;
      const int p = p0 + r;
      if (p < n) {
        vals[p] = mine;
        srow[p] = mine;
        mn = fminf(mn, mine);
        mx = fmaxf(mx, mine);
      }
    }
  }
  if (n <= k) {
    for (int i = tid; i < k; i += 1024) out[i] = i < n ? i : -1;
    return;
  }
  topk_from_lds<1024>(L, vals, n, k, mn, mx, out);
}

// Scoring and top-k in one launch for batches with fewer lists than CUs.
//
// Each (request, KV head) list is spread over several 1024-thread
// workgroups of 256 or 512 partitions (ROWS = two or four rows in flight per
// 8-lane group), so the summaries stream from HBM from as many CUs as
// k_score would use; each row's dot product is the same arithmetic as in
// k_score.  The last workgroup of a list to finish its
// rows runs the top-k over the whole list, which a second launch did before.
//
// The hand-over between workgroups costs no cache write-back: the scores are
// written as agent-scope atomic stores, which write through the XCD's L2, and
// each wave waits for its stores to complete before the workgroup barrier;
// only then does one thread count the workgroup in (relaxed agent-scope
// atomic add on the list's counter).  The workgroup that brings the count to
// the list's number of chunks reads the scores back with agent-scope atomic
// loads, which do not hit stale lines of its own L2, and resets the counter
// for the next launch.  A release fence would instead write back the whole L2
// of every workgroup's XCD, which costs more than the second launch.
template <int ROWS>
struct SplitSelect {
  static constexpr int kRows = 16 * 8 * ROWS;  // partitions per workgroup
};

template <int ROWS>
__global__ __launch_bounds__(1024) void k_select_split(Dev d, const uint16_t* __restrict__ q,
                                                       float* __restrict__ scores,
                                                       int* __restrict__ sel, int* __restrict__ arrive) {
  constexpr int kRows = SplitSelect<ROWS>::kRows;
  extern __shared__ float vals[];  // [Nmax]: the list's scores, last workgroup only
  __shared__ TopkLds<1024> L;
  __shared__ uint4 sq[kMaxGroup * kHeadDim / 8];
  __shared__ float sqbar[kHeadDim];
  __shared__ int s_last;
  q = step_queries(d, q);
  const int bh = blockIdx.y;
  const int b = bh / d.Hkv, h = bh - b * d.Hkv;
  const int n = d.req_parts[b];
  const int k = d.k;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 3, r = lane & 7;
  const int p0 = blockIdx.x * kRows;
  float* srow = scores + (size_t)bh * d.Nmax;
  int* out = sel + (size_t)bh * k;
  // a list of at most k partitions keeps all of them, whatever the scores
  if (blockIdx.x == 0 && n <= k)
    for (int i = tid; i < k; i += 1024) out[i] = i < n ? i : -1;
  if (p0 >= n) {
    for (int p = p0 + tid; p < min(p0 + kRows, d.Nmax); p += 1024) srow[p] = -INFINITY;
    return;
  }

  // the group's queries, then this workgroup's summary rows in flight while
  // their mean is formed; group `grp` of wave `wave` takes rows
  // p0 + wave 8 ROWS + ROWS grp + it (a row past the list re-reads row p0)
  const int nq = d.G * kHeadDim / 8;
  uint4 qc = make_uint4(0u, 0u, 0u, 0u);
  if (tid < nq) qc = reinterpret_cast<const uint4*>(q + ((size_t)b * d.Hq + (size_t)h * d.G) * kHeadDim)[tid];
  const float* S = d.summaries + (size_t)bh * d.Nmax * kHeadDim;
  const int pw = p0 + wave * 8 * ROWS + ROWS * grp;
  float4 v[ROWS][4];
#pragma unroll
  for (int it = 0; it < ROWS; ++it) {
    const int p = pw + it;
    const float* row = S + (size_t)(p < n ? p : p0) * kHeadDim + 4 * r;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[it][j] = *reinterpret_cast<const float4*>(row + 32 * j);
  }
  if (tid < nq) sq[tid] = qc;
  __syncthreads();
  if (tid < kHeadDim) {
    const uint16_t* sq16 = reinterpret_cast<const uint16_t*>(sq);
    float sum = 0.f;
    for (int g = 0; g < d.G; ++g) sum += __uint_as_float((uint32_t)sq16[g * kHeadDim + tid] << 16);
    sqbar[tid] = sum * (1.0f / ((float)d.G * sqrtf((float)kHeadDim)));
  }
  __syncthreads();
  float qv[16];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[4 * j + e] = sqbar[32 * j + 4 * r + e];
  float acc[ROWS];
#pragma unroll
  for (int it = 0; it < ROWS; ++it) {
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
  // lane r < ROWS of the group writes row pw + r
  float smin = INFINITY, smax = -INFINITY;
  if (r < ROWS) {
    float mine = acc[0];
#pragma unroll
    for (int it = 1; it < ROWS; ++it) mine = (r == it) ? acc[it] : mine;
    const int p = pw + r;
    if (p < n) {
      __hip_atomic_store(&srow[p], mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      smin = smax = mine;
    } else if (p < d.Nmax) {
      srow[p] = -INFINITY;
    }
  }
  if (n <= k) return;
  // this wave's score range goes beside the scores, so the last workgroup can
  // bin the list's scores as they arrive, without combining ranges first
  smin = wave_min(smin);
  smax = wave_max(smax);
  const int chunks = (n + kRows - 1) / kRows;
  float* rg = d.srange + (size_t)bh * kSplitRangeSlots * 2;
  if (lane == 0) {
    float* mine = rg + 2 * (blockIdx.x * 16 + wave);
    __hip_atomic_store(mine, smin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(mine + 1, smax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  topk_coarse_clear<1024>(L, n);  // (only the last workgroup of the list uses them)

  // count this workgroup in once every wave's score and range stores have
  // completed
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&arrive[bh], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == chunks - 1;
  __syncthreads();
  if (!s_last) return;
  if (tid == 0) __hip_atomic_store(&arrive[bh], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the list's first kHeld * 1024 scores and every wave's range (one entry
  // per lane) loaded together, so the two wait out one round trip; then the
  // range combined, and each score binned
  constexpr int kHeld = 4;
  float held[kHeld];
#pragma unroll
  for (int j = 0; j < kHeld; ++j) {
    const int i = tid + 1024 * j;
    held[j] = i < n ? __hip_atomic_load(&srow[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
  }
  float mn = INFINITY, mx = -INFINITY;
  for (int e = lane; e < chunks * 16; e += 64) {
    mn = fminf(mn, __hip_atomic_load(rg + 2 * e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    mx = fmaxf(mx, __hip_atomic_load(rg + 2 * e + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  const BinMap m = coarse_map(mn, mx);
#pragma unroll
  for (int j = 0; j < kHeld; ++j) {
    const int i = tid + 1024 * j;
    if (i < n) {
      vals[i] = held[j];
      atomicAdd(&L.hist[coarse_bin(held[j], m)], 1);
    }
  }
  for (int i = tid + 1024 * kHeld; i < n; i += 1024) {
    const float x = __hip_atomic_load(&srow[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    vals[i] = x;
    atomicAdd(&L.hist[coarse_bin(x, m)], 1);
  }
  __syncthreads();
  topk_coarse<1024>(L, vals, n, k, m, mn, mx, out);
}

hipError_t launch_score(const Dev& d, const uint16_t* q, float* scores, hipStream_t s) {
  dim3 grid((d.Nmax + kScorePerWG - 1) / kScorePerWG, d.B * d.Hkv);
  hipLaunchKernelGGL(k_score, grid, dim3(kScoreWG), 0, s, d, q, scores);
  return hipGetLastError();
}

hipError_t launch_select_fused(const Dev& d, const uint16_t* q, float* scores, int* sel,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_select_fused, dim3(d.B * d.Hkv), dim3(1024), 0, s, d, q, scores, sel);
  return hipGetLastError();
}

hipError_t launch_select_split(const Dev& d, const uint16_t* q, float* scores, int* sel,
                               hipStream_t s) {
  // four rows in flight per 8-lane group (512 partitions per workgroup) for
  // lists of 1024+ partitions, two (256) for shorter ones, where four would
  // leave most waves idle (measured: 2048-partition lists 19.2 -> 17.6 us,
  // 64-partition lists 7.4 -> 8.4 us)
  if (d.Nmax >= 1024) {
    constexpr int rows = SplitSelect<4>::kRows;
    dim3 grid((d.Nmax + rows - 1) / rows, d.B * d.Hkv);
    hipLaunchKernelGGL(k_select_split<4>, grid, dim3(1024), d.Nmax * sizeof(float), s, d, q, scores, sel,
                       d.arrive);
  } else {
    constexpr int rows = SplitSelect<2>::kRows;
    dim3 grid((d.Nmax + rows - 1) / rows, d.B * d.Hkv);
    hipLaunchKernelGGL(k_select_split<2>, grid, dim3(1024), d.Nmax * sizeof(float), s, d, q, scores, sel,
                       d.arrive);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const Dev& d, const float* scores, int* sel, hipStream_t s) {
  // 1024 threads: measured fastest (512 and 256 threads took 1.0-1.3x and
  // 1.3-2.0x as long on 2048- and 7.7K-score lists)
  hipLaunchKernelGGL(k_topk<1024>, dim3(d.B * d.Hkv), dim3(1024), 0, s, d, scores, sel);
  return hipGetLastError();
}

}  // namespace spin
