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
// Work split: a workgroup of 4 waves takes a run of `pps` pages of one (b, h);
// each wave takes a contiguous quarter of it, keeps an fp32 online softmax per
// head, and pipelines its page loads (next keys during this page's softmax and
// PV, next values during the next logits), with the block-table entries of
// its pages loaded once up front, beside the head's page count.  The waves
// merge through LDS.  A head whose pages fit in one workgroup is finished
// there; in the whole-table pass the split that finishes last merges the
// head's split partials (log-sum-exp), handed over as agent-scope stores and
// loads within the launch (on the 128K workload with 64-page heads, 4 splits:
// 24 + 4.6 us with a merge launch -> 26.6 us; a device-scope fence per
// workgroup instead, which writes back the whole L2, was far slower).  The
// overlapped passes' partials are merged by k_attend_merge or
// k_attend_merge_arrival after the launch.
// The resident-page pass that runs beside the transfer uses its own, longer
// splits (d.pps_res): it only has to keep pace with the transfer, and fewer
// attention workgroups contend less with the PCIe pulls.
#include "arrival.h"
#include "segments.h"
#include "attend_tile.h"
#include "device_util.h"
#include "spin_internal.h"

namespace spin {

constexpr int kAttWG = 256;

// Two floats as one 64-bit agent-scope (write-through) store, and the 64-bit
// agent-scope load that reads them back with its two halves: the hand-over
// of split partials between workgroups of one launch.
__device__ __forceinline__ void store_pair_agent(float* p, float a, float b) {
  const unsigned long long v = ((unsigned long long)__float_as_uint(b) << 32) | __float_as_uint(a);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long load_u64_agent(const float* p) {
  return __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float lo_float(unsigned long long v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ float hi_float(unsigned long long v) { return __uint_as_float((uint32_t)(v >> 32)); }

// Pages per split of a head with cnt pages: its pages spread evenly over the
// head's `nsp` workgroups (whole pages per wave), so heads with fewer pages
// than the largest possible count still use all their workgroups and the
// slowest workgroup carries no more than it must.  Never above the split
// size the grid was sized with (d.pps for nsp = d.splits, d.pps_res for the
// resident-page pass's d.splits_res).
__device__ __forceinline__ int head_pps(int cnt, int nsp) {
  const int per = (cnt + nsp - 1) / nsp;
  return max(4, (per + 3) & ~3);
}

// Splits per head of an attention pass: the resident-page pass that runs
// beside the transfer uses fewer, longer ones.
__device__ __forceinline__ int pass_splits(const Dev& d, int mode) {
  return mode == kAttendResident ? d.splits_res : d.splits;
}

// Workgroup wg of the attention grid (B * Hkv * nsp, nsp = pass_splits):
// split wg % nsp of (request, KV head) wg / nsp; q already points at this
// step's queries.
__device__ __forceinline__ void attend_wg(const Dev& d, const uint16_t* __restrict__ q,
                                          const int* __restrict__ bt, const int* __restrict__ bntok,
                                          const int* __restrict__ bcount, float* __restrict__ out,
                                          int mode, int wg) {
  __shared__ float sm_m[4][16];
  __shared__ float sm_l[4][16];
  __shared__ float sm_o[4][16][132];

  const int nsp = pass_splits(d, mode);
  const int split = wg % nsp;
  const int bh = wg / nsp;
  const int b = bh / d.Hkv, h = bh - b * d.Hkv;
  const int G = d.G;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  // The block-table entries this wave takes when the head's split size is the
  // grid's (a head with every page it can have: a full selection of
  // one-page partitions), loaded beside the head's page count instead of
  // after it; another split size loads them again below.
  const int pps_g = nsp == d.splits ? d.pps : d.pps_res;
  const int p0_g = split * pps_g + wave * (pps_g / 4);
  int g_slot = 0, g_nt = 0, g_miss = 0;
  if (lane < pps_g / 4 && p0_g + lane < d.max_blocks) {
    const size_t e = (size_t)bh * d.max_blocks + p0_g + lane;
    g_slot = bt[e];
    g_nt = bntok[e];
    if (mode != kAttendAll) g_miss = d.bmiss[e];
  }
  const int cnt = max(0, min(bcount[bh], d.max_blocks));
  const int pps = head_pps(cnt, nsp);
  const int ns = (cnt + pps - 1) / pps;  // splits that hold pages
  const int hh = tid >> 4, dc = (tid & 15) * 8;  // merge layout: head, 8 dims
  float* orow = out + ((size_t)b * d.Hq + (size_t)h * G) * kHeadDim;
  if (cnt == 0) {  // no pages: the head's output is zero
    if (mode == kAttendAll && split == 0 && hh < G) {
      float4* o4 = reinterpret_cast<float4*>(orow + (size_t)hh * kHeadDim + dc);
      o4[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      o4[1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  if (split >= ns) return;
  const int r = lane & 15, g = lane >> 4;
  const int ppw = pps / 4;
  const int p0 = split * pps + wave * ppw;
  const int np = max(0, min(cnt, p0 + ppw) - p0);  // this wave's pages: p0 .. p0+np-1

  // block-table entries of the wave's pages, one per lane; in the two
  // overlapped passes a wave keeps only the resident or only the fetched ones
  int my_slot = 0, my_nt = 0;
  bool keep = false;
  if (lane < np) {
    const size_t e = (size_t)bh * d.max_blocks + p0 + lane;
    const bool same = pps == pps_g;  // (then p0 == p0_g)
    const int s = same ? g_slot : bt[e];
    const int n = same ? g_nt : bntok[e];
    // a malformed entry (caller-supplied table) reads slot 0 with every token masked
    if ((unsigned)s < (unsigned)d.pool_slots && n > 0 && n <= kPageTokens) {
      my_slot = s;
      my_nt = n;
    }
    const int fetched = mode == kAttendAll ? 0 : same ? g_miss : d.bmiss[e];
    keep = mode == kAttendAll || (fetched != 0) == (mode == kAttendFetched);
  }
  unsigned long long pages = __ballot(keep);  // lanes holding this wave's pages, in order

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
  float m = -INFINITY, l = 0.f;  // running max (log2 units), this lane's partial sum
  const float sl2 = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)

  if (pages != 0) {
    // two-stage pipeline: keys of the next page load during softmax/PV of this
    // one, values of the next page load during the next logits
    bf16x8 ka[4][4], va[8][2];
    int cur = __builtin_ctzll(pages);
    pages &= pages - 1;
    {
      const uint16_t* P = d.pool + (size_t)__shfl(my_slot, cur, 64) * kPageElems;
      load_keys(P, r, g, ka);
      load_values(P + kPageTokens * kHeadDim, r, g, va);
    }
    while (true) {
      const int nt = __shfl(my_nt, cur, 64);
      // the next page (the last one reloads itself, an L2 hit, so the buffers
      // stay single registers across the loop)
      const int nxt = pages != 0 ? __builtin_ctzll(pages) : cur;
      f32x4 s[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) s[tt] = mfma16x16x32(ka[tt][kb], qb[kb], s[tt]);
      }
      const uint16_t* Pn = d.pool + (size_t)__shfl(my_slot, nxt, 64) * kPageElems;
      // keep the key buffer single: its refill may not move above the MFMAs reading it
      __builtin_amdgcn_sched_barrier(0);
      load_keys(Pn, r, g, ka);
      // s[tt][j]: head r, token 32 (tt/2) + 8 g + 4 (tt%2) + j
      float pm = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tok = 32 * (tt >> 1) + 8 * g + 4 * (tt & 1) + j;
          const float x = tok < nt ? s[tt][j] * sl2 : -INFINITY;
          s[tt][j] = x;
          pm = fmaxf(pm, x);
        }
      pm = fmaxf(pm, __shfl_xor(pm, 16, 64));
      pm = fmaxf(pm, __shfl_xor(pm, 32, 64));
      const float mn = fmaxf(m, pm);
      const bool none = mn == -INFINITY;  // nothing valid seen yet
      const float alpha = none ? 1.f : exp2f(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[dt] *= alpha;
      bf16x8 phi[2], plo[2];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pv = none ? 0.f : exp2f(s[tt][j] - mn);
          l += pv;
          const __bf16 hi = (__bf16)pv;
          phi[tt >> 1][4 * (tt & 1) + j] = hi;
          plo[tt >> 1][4 * (tt & 1) + j] = (__bf16)(pv - (float)hi);
        }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          acc[dt] = mfma16x16x32(va[dt][kt], phi[kt], acc[dt]);
          acc[dt] = mfma16x16x32(va[dt][kt], plo[kt], acc[dt]);
        }
      __builtin_amdgcn_sched_barrier(0);
      load_values(Pn + kPageTokens * kHeadDim, r, g, va);
      if (pages == 0) break;
      cur = nxt;
      pages &= pages - 1;
    }
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  // acc[dt][j] = unnormalised out[head r][dim 16 dt + 4 g + j]
  if (g == 0) {
    sm_m[wave][r] = m;
    sm_l[wave][r] = l;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) sm_o[wave][r][16 * dt + 4 * g + j] = acc[dt][j];
  __syncthreads();

  // merge the four waves: thread (hh, dc) owns head hh, dims dc .. dc+7
  float M = -INFINITY, L = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  if (hh < G) {
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][hh]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sm_m[w][hh];
      const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
      L += sm_l[w][hh] * f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += sm_o[w][hh][dc + e] * f;
    }
  }
  if (mode == kAttendAll && ns == 1) {  // the whole head in one workgroup: normalise and store
    if (hh < G) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      float4* o4 = reinterpret_cast<float4*>(orow + (size_t)hh * kHeadDim + dc);
      o4[0] = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
      o4[1] = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
    }
    return;
  }
  // publish this split's partial (fetched-page partials sit after the
  // resident-page ones)
  const int slot_s = mode == kAttendFetched ? d.splits + split : split;
  if (hh < G) {
    const size_t pi = ((size_t)bh * 2 * d.splits + slot_s) * G + hh;
    float* po = d.part_o + pi * kHeadDim + dc;
    if (mode == kAttendAll) {
      // read back within this launch by the head's last split, maybe on
      // another XCD: agent-scope stores, which write through its L2
      store_pair_agent(po, o[0], o[1]);
      store_pair_agent(po + 2, o[2], o[3]);
      store_pair_agent(po + 4, o[4], o[5]);
      store_pair_agent(po + 6, o[6], o[7]);
      if (dc == 0) store_pair_agent(d.part_ml + 2 * pi, M, L);
    } else {  // for k_attend_merge / k_attend_merge_arrival, after this launch
      float4* p4 = reinterpret_cast<float4*>(po);
      p4[0] = make_float4(o[0], o[1], o[2], o[3]);
      p4[1] = make_float4(o[4], o[5], o[6], o[7]);
      if (dc == 0) {
        d.part_ml[2 * pi] = M;
        d.part_ml[2 * pi + 1] = L;
      }
    }
  }
  if (mode != kAttendAll) return;
  // The whole-table pass merges its splits in this launch: once every wave's
  // partial stores have completed the workgroup counts itself in on its
  // head; the split that completes the count folds every split's partial
  // (its own from registers, the others with agent-scope loads, which miss
  // stale lines of its own L2) in split order, so the result does not depend
  // on which split finished last, and resets the counter for the next launch.
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&d.att_arrive[bh], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ns - 1;
  __syncthreads();
  if (!s_last) return;
  if (tid == 0) __hip_atomic_store(&d.att_arrive[bh], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (hh >= G) return;
  float Mf = -INFINITY, Lf = 0.f, of[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) of[e] = 0.f;
  constexpr int UX = 8;  // partials' loads in flight at a time
  for (int x0 = 0; x0 < ns; x0 += UX) {
    // each partial as five 64-bit words ((max, sum), then 8 dims), loaded
    // under its condition and passed through an empty asm before anything
    // reads them: otherwise the compiler unpacks each word inside its load's
    // branch and waits for it there, before the next partial's loads
    unsigned long long w[UX][5];
#pragma unroll
    for (int u = 0; u < UX; ++u) {
      const int x = x0 + u;
#pragma unroll
      for (int k = 0; k < 5; ++k) w[u][k] = 0ull;
      if (x < ns && x != split) {
        const size_t pi = ((size_t)bh * 2 * d.splits + x) * G + hh;
        w[u][0] = load_u64_agent(d.part_ml + 2 * pi);
        const float* po = d.part_o + pi * kHeadDim + dc;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[u][1 + k] = load_u64_agent(po + 2 * k);
      }
    }
#pragma unroll
    for (int u = 0; u < UX; ++u)
#pragma unroll
      for (int k = 0; k < 5; ++k) asm volatile("" : "+v"(w[u][k]));
#pragma unroll
    for (int u = 0; u < UX; ++u) {
      const int x = x0 + u;
      float ms = -INFINITY, ls = 0.f, a[8];
      if (x < ns && x != split) {
        ms = lo_float(w[u][0]);
        ls = hi_float(w[u][0]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          a[2 * k] = lo_float(w[u][1 + k]);
          a[2 * k + 1] = hi_float(w[u][1 + k]);
        }
      } else if (x == split) {
        ms = M;
        ls = L;
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = o[e];
      }
      if (ms == -INFINITY) continue;
      const float Mn = fmaxf(Mf, ms);
      const float fo = Mf == -INFINITY ? 0.f : exp2f(Mf - Mn), fn = exp2f(ms - Mn);
      Mf = Mn;
      Lf = Lf * fo + ls * fn;
#pragma unroll
      for (int e = 0; e < 8; ++e) of[e] = of[e] * fo + a[e] * fn;
    }
  }
  const float inv = Lf > 0.f ? 1.f / Lf : 0.f;
  float4* o4 = reinterpret_cast<float4*>(orow + (size_t)hh * kHeadDim + dc);
  o4[0] = make_float4(of[0] * inv, of[1] * inv, of[2] * inv, of[3] * inv);
  o4[1] = make_float4(of[4] * inv, of[5] * inv, of[6] * inv, of[7] * inv);
}

__global__ __launch_bounds__(kAttWG, 2) void k_attend(Dev d, const uint16_t* __restrict__ q,
                                                   const int* __restrict__ bt,
                                                   const int* __restrict__ bntok,
                                                   const int* __restrict__ bcount,
                                                   float* __restrict__ out, int mode) {
  attend_wg(d, step_queries(d, q), bt, bntok, bcount, out, mode, blockIdx.x);
}

// Retrieve and the resident-page attention in one launch on one stream: the
// first kRetrieveGrid workgroups pull the step's missed pages and attend each
// on arrival, the rest attend the resident pages (partials), so the two
// overlap without a second stream or any event between them; the merge
// follows on the same stream.  With segments set, workgroup kRetrieveGrid
// runs the segment-pool pass and the inserts, which nothing else in the
// launch reads, behind the transfer instead of before it: every insert is a
// page this launch pulls (about 0.6 us of the link each), against a few
// hundredths of a microsecond per insert for the one workgroup.
__global__ __launch_bounds__(kAttWG, 2) void k_transfer_attend(Dev d, const uint16_t* __restrict__ q,
                                                            const int* __restrict__ bt,
                                                            const int* __restrict__ bntok,
                                                            const int* __restrict__ bcount,
                                                            int segments) {
  static_assert(kRetrieveWG == kAttWG, "one workgroup size for both roles");
  static_assert(3 * 1025 <= kPageBytes / 4, "the segment pass borrows the page buffer");
  __shared__ int pm[1025];
  __shared__ int tmp[kAttWG / 64 + 1];
  __shared__ u32x4 page[kPageBytes / 16];
  q = step_queries(d, q);
  const int wg = blockIdx.x;
  if (wg < kRetrieveGrid) {
    retrieve_attend_wg(d, q, wg, kRetrieveGrid, pm, tmp, page);
  } else if (segments && wg == kRetrieveGrid) {
    int* lds = reinterpret_cast<int*>(page);
    segments_wg<kAttWG>(d, 1, lds, tmp);
  } else {
    attend_wg(d, q, bt, bntok, bcount, nullptr, kAttendResident, wg - kRetrieveGrid - segments);
  }
}

// Log-sum-exp merge of the n_all partials of one (request, KV head), then
// normalisation into out; part(x, hh, dc, ml, po) points ml at partial x's
// (max, sum) for query head hh and po at its dims dc .. dc+7.  The 256
// threads form 16 groups of 16: nsub = 16 / G subgroups per query head, each
// folding every nsub-th partial (8 dims per thread) with sixteen partials'
// loads in flight at a time, combined through LDS.  Every thread calls it.
template <class Part>
__device__ void merge_head(const Dev& d, int bh, int n_all, Part part, float* __restrict__ out) {
  __shared__ float sm[16][16][10];
  const int b = bh / d.Hkv, h = bh - b * d.Hkv;
  const int G = d.G;
  const int tid = threadIdx.x;
  const int nsub = 16 / G;
  const int grp = tid >> 4, ln = tid & 15, dc = ln * 8;
  const int sg = grp / G, hh = grp - sg * G;
  const bool active = sg < nsub;
  float M = -INFINITY, L = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  auto fold = [&](float ms, float ls, float4 a, float4 c) {
    if (ms == -INFINITY) return;
    const float Mn = fmaxf(M, ms);
    const float fo = M == -INFINITY ? 0.f : exp2f(M - Mn), fn = exp2f(ms - Mn);
    M = Mn;
    L = L * fo + ls * fn;
    o[0] = o[0] * fo + a.x * fn; o[1] = o[1] * fo + a.y * fn;
    o[2] = o[2] * fo + a.z * fn; o[3] = o[3] * fo + a.w * fn;
    o[4] = o[4] * fo + c.x * fn; o[5] = o[5] * fo + c.y * fn;
    o[6] = o[6] * fo + c.z * fn; o[7] = o[7] * fo + c.w * fn;
  };
  if (active) {
    constexpr int U = 16;
    for (int base = sg; base < n_all; base += U * nsub) {
      float ms[U], ls[U];
      float4 a[U], c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int x = base + u * nsub;
        ms[u] = -INFINITY;
        ls[u] = 0.f;
        if (x < n_all) {
          const float* ml;
          const float* po;
          part(x, hh, dc, ml, po);
          ms[u] = ml[0];
          ls[u] = ml[1];
          a[u] = reinterpret_cast<const float4*>(po)[0];
          c[u] = reinterpret_cast<const float4*>(po)[1];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (ms[u] != -INFINITY) fold(ms[u], ls[u], a[u], c[u]);
    }
  }
  sm[grp][ln][0] = M;
  sm[grp][ln][1] = L;
#pragma unroll
  for (int e = 0; e < 8; ++e) sm[grp][ln][2 + e] = o[e];
  __syncthreads();
  if (!active || sg != 0) return;
  for (int t2 = 1; t2 < nsub; ++t2) {
    const float* x = sm[t2 * G + hh][ln];
    fold(x[0], x[1], make_float4(x[2], x[3], x[4], x[5]), make_float4(x[6], x[7], x[8], x[9]));
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float4* o4 = reinterpret_cast<float4*>(out + ((size_t)b * d.Hq + (size_t)h * G + hh) * kHeadDim + dc);
  o4[0] = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
  o4[1] = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
}

// One workgroup per (request, KV head): merge the split partials of the
// resident-page pass and of the fetched-page pass, and normalise.
__global__ __launch_bounds__(kAttWG) void k_attend_merge(Dev d, const int* __restrict__ bcount,
                                                         float* __restrict__ out) {
  const int bh = blockIdx.x;
  const int cnt = max(0, min(bcount[bh], d.max_blocks));
  // splits holding pages: of the resident-page pass, then of the fetched-page pass
  const int ns = (cnt + head_pps(cnt, d.splits) - 1) / head_pps(cnt, d.splits);
  const int ns_res = (cnt + head_pps(cnt, d.splits_res) - 1) / head_pps(cnt, d.splits_res);
  const int G = d.G;
  merge_head(d, bh, ns_res + ns,
             [&](int x, int hh, int dc, const float*& ml, const float*& po) {
               const int slot = x < ns_res ? x : d.splits + (x - ns_res);
               const size_t pi = ((size_t)bh * 2 * d.splits + slot) * G + hh;
               ml = d.part_ml + 2 * pi;
               po = d.part_o + pi * kHeadDim + dc;
             },
             out);
}

// One workgroup per (request, KV head): the resident-page partials of its
// splits and the partials of its pages attended on arrival (a contiguous run
// of the batch's insert lists: this request's offset plus the head's).
__global__ __launch_bounds__(kAttWG) void k_attend_merge_arrival(Dev d, const int* __restrict__ bcount,
                                                                 float* __restrict__ out,
                                                                 int* __restrict__ advance) {
  __shared__ int pm[1025];
  __shared__ int tmp[kAttWG / 64 + 1];
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv, h = bh - b * d.Hkv;
  // the next step's index (an atomic whose result is not read: nothing waits
  // for it here, and the next step's kernels run after this launch)
  if (advance && bh == 0 && threadIdx.x == 0) atomicAdd(advance, 1);
  // the head's own counts first, so their loads overlap the batch's prefix
  const int cnt = max(0, min(bcount[bh], d.max_blocks));
  const int nm = d.nmiss[b];
  const int* mo = d.head_moff + (size_t)b * (d.Hkv + 1);
  const int mo0 = mo[h], mo1 = mo[h + 1];
  request_offsets<kAttWG>(d.nmiss, d.B, pm, tmp);
  const int ns = (cnt + head_pps(cnt, d.splits_res) - 1) / head_pps(cnt, d.splits_res);  // resident-page splits
  const int j0 = pm[b] + min(max(mo0, 0), nm), j1 = pm[b] + min(max(mo1, 0), nm);
  const int G = d.G;
  merge_head(d, bh, ns + (j1 - j0),
             [&](int x, int hh, int dc, const float*& ml, const float*& po) {
               if (x < ns) {
                 const size_t pi = ((size_t)bh * 2 * d.splits + x) * G + hh;
                 ml = d.part_ml + 2 * pi;
                 po = d.part_o + pi * kHeadDim + dc;
               } else {
                 const size_t pi = (size_t)(j0 + x - ns) * G + hh;
                 ml = d.arr_ml + 2 * pi;
                 po = d.arr_o + pi * kHeadDim + dc;
               }
             },
             out);
}

hipError_t launch_transfer_attend(const Dev& d, const uint16_t* q, const int* bt, const int* bntok,
                                  const int* bcount, bool segments, hipStream_t s) {
  const int seg = segments ? 1 : 0;
  hipLaunchKernelGGL(k_transfer_attend, dim3(kRetrieveGrid + seg + d.B * d.Hkv * d.splits_res),
                     dim3(kAttWG), 0, s, d, q, bt, bntok, bcount, seg);
  return hipGetLastError();
}

hipError_t launch_attend(const Dev& d, const uint16_t* q, const int* bt, const int* bntok,
                         const int* bcount, float* out, int mode, hipStream_t s, int* advance) {
  if (mode == kAttendMergeArrival) {
    hipLaunchKernelGGL(k_attend_merge_arrival, dim3(d.B * d.Hkv), dim3(kAttWG), 0, s, d, bcount, out,
                       advance);
    return hipGetLastError();
  }
  const int nsp = mode == kAttendResident ? d.splits_res : d.splits;
  hipLaunchKernelGGL(k_attend, dim3(d.B * d.Hkv * nsp), dim3(kAttWG), 0, s, d, q, bt, bntok,
                     bcount, out, mode);
  hipError_t e = hipGetLastError();
  // the whole-table pass merges its splits itself; the fetched-page pass
  // is merged with the resident-page one by a second launch
  if (e != hipSuccess || mode != kAttendFetched) return e;
  hipLaunchKernelGGL(k_attend_merge, dim3(d.B * d.Hkv), dim3(kAttWG), 0, s, d, bcount, out);
  return hipGetLastError();
}

}  // namespace spin
