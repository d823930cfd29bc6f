// The transfer that attends each fetched page on arrival, as a workgroup
// body shared by the transfer kernel and the one-launch transfer + attention
// kernel.
#pragma once

#include "attend_tile.h"
#include "device_util.h"
#include "spin_internal.h"

namespace spin {

constexpr int kXferPagesPerWG = 4, kXferMinWG = 16;

// A transfer reads the key rows of a page's valid tokens (its partition's
// tokens on that page) and every value row, and leaves zeros in the pool slot
// for every token slot past them, whatever the host buffer holds there
// (attention gives those slots zero weight, and a zero value keeps a product
// with that weight zero, where a NaN in host padding would not).  Keys are
// token-major, 256 contiguous bytes (16 chunks of 16 bytes) per token, so a
// partly filled page skips a contiguous tail; values are dim-major, where the
// valid tokens are a prefix of each 128-byte dimension row: reading only
// those prefixes measured no faster than reading the rows whole (a 1M-token
// workload with variable partitions: 1312 us per step's transfer either way,
// against 1450 us for whole pages), so the value half moves whole and its
// entries past the valid tokens are zeroed in registers.
constexpr int kKeyChunks = kPageTokens * kHeadDim / 8;  // 16-byte chunks of the key half

__device__ __forceinline__ bool chunk_live(int c, int ntok) { return c >= kKeyChunks || (c >> 4) < ntok; }

// chunk c of a page as it goes to the pool: a value chunk (8 consecutive
// tokens of one dimension, two bf16 per word, the lower token in the low
// half) with the entries of tokens at or past ntok set to zero
__device__ __forceinline__ u32x4 pool_chunk(u32x4 v, int c, int ntok) {
  if (c < kKeyChunks) return v;
  const int keep = ntok - ((c & 7) << 3);  // tokens of this chunk below ntok
  if (keep < 8) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const unsigned m = (2 * w < keep ? 0x0000ffffu : 0u) | (2 * w + 1 < keep ? 0xffff0000u : 0u);
      v[w] &= m;
    }
  }
  return v;
}

// the bytes a transfer reads over the link for a page of ntok valid tokens
__device__ __forceinline__ unsigned long long link_bytes(int ntok) {
  return 256ull * (unsigned)ntok + (unsigned long long)kPageTokens * kHeadDim * 2;
}

// The transfer with the fetched pages attended on arrival: each page also
// goes into LDS, and wave 0 runs its attention there for the G query heads of
// its KV head (the same MFMA tiles as the attention kernel, one page at a
// time), writing an unnormalised partial (max, sum, output) under the page's
// insert-list index.  The page is never read back from HBM for attention;
// k_attend_merge_arrival folds these partials into the resident-page ones.
// One page costs the wave about a microsecond, against tens of microseconds
// of its workgroup's share of the link, and the next page's loads are
// already in flight meanwhile.
//
// Workgroup wg of nwg: pages wg, wg + nwg, ... of the batch's insert lists;
// q already points at this step's queries.  LDS from the caller: pm holds
// 1025 ints, tmp kRetrieveWG / 64 + 1, page one 32 KiB page.
__device__ __forceinline__ void retrieve_attend_wg(const Dev& d, const uint16_t* __restrict__ q,
                                                   int wg, int nwg, int* pm, int* tmp,
                                                   u32x4* page) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int G = d.G;
  // where each request's misses start in the batch-wide concatenation of the
  // insert lists k_resolve wrote
  const int M = request_offsets<kRetrieveWG>(d.nmiss, d.B, pm, tmp);
  const float sl2 = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)
  // a page's host address and its checks; its loads are issued one page
  // ahead, so they stay in flight while the wave attends the page before it
  struct Item {
    int b, ntok;
    int4 m;  // (slot, KV head, page)
    bool ok;
  };
  auto item = [&](int j) {
    Item it;
    it.b = owner_of(pm, d.B, j);
    const size_t e = (size_t)it.b * d.max_mand + (j - pm[it.b]);
    it.m = d.ins[e];
    it.ntok = d.miss_tmp[e].w;
    it.ok = (unsigned)it.m.x < (unsigned)d.C && (unsigned)it.m.y < (unsigned)d.Hkv &&
            (unsigned)it.m.z < (unsigned)d.req_pages[it.b];
    return it;
  };
  auto load = [&](const Item& it, u32x4 (&v)[8]) {
    if (!it.ok) return;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        d.host_base[it.b] + ((size_t)it.m.y * d.req_stride[it.b] + it.m.z) * (size_t)kPageBytes);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = u * kRetrieveWG + tid;
      v[u] = chunk_live(c, it.ntok) ? src[c] : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // A step with few misses spreads them over fewer workgroups, about four
  // pages each (at least 16 workgroups), so not every page is requested at
  // once: the link still runs full, and the HBM reads of the attention
  // beside it suffer less from the PCIe requests queued with them (measured
  // on the 128K workload with ~90 misses a step: 0.117 -> 0.113 ms per step
  // at three pages, then 0.1065 -> 0.1057 at four once the resident-page
  // pass took longer splits; one or two pages per workgroup, or six, were
  // slower).  From 256 misses on, every workgroup takes part.
  {
    const int nact = min(nwg, max(kXferMinWG, (M + kXferPagesPerWG - 1) / kXferPagesPerWG));
    if (wg >= nact) return;
    nwg = nact;
  }
  // wave 0's queries for a page's G heads (zeros past G), loaded with the
  // page's own loads, a page ahead, so no round trip of its own stands
  // between a page's arrival and its attention (next to the PCIe pulls an
  // HBM round trip takes many times longer than alone)
  auto load_q = [&](const Item& it, bf16x8 (&qq)[4]) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qq[kb] = bf16x8{};
    if (wave != 0 || !it.ok || r >= G) return;
    const uint16_t* qp = q + ((size_t)it.b * d.Hq + (size_t)it.m.y * G + r) * kHeadDim;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qq[kb] = *reinterpret_cast<const bf16x8*>(qp + 32 * kb + 8 * g);
  };
  int j = wg;
  Item cur;
  u32x4 v[8], vn[8];
  bf16x8 qc[4], qn[4];
  unsigned long long moved = 0;  // bytes this workgroup read over the link
  if (j < M) {
    cur = item(j);
    load(cur, v);
    load_q(cur, qc);
  }
  for (; j < M; j += nwg) {
    float* po = d.arr_o + (size_t)j * G * kHeadDim;
    float* pml = d.arr_ml + (size_t)j * G * 2;
    // the next page's loads go out first: two pages in flight per workgroup,
    // and the next one keeps arriving while this one is stored and attended
    const int jn = j + nwg;
    Item nxt;
    nxt.ok = false;
    if (jn < M) {
      nxt = item(jn);
      load(nxt, vn);
      load_q(nxt, qn);
    }
    if (cur.ok) {
      moved += link_bytes(cur.ntok);
      u32x4* dst = reinterpret_cast<u32x4*>(d.pool + ((size_t)cur.b * d.C + cur.m.x) * kPageElems);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const u32x4 x = pool_chunk(v[u], u * kRetrieveWG + tid, cur.ntok);
        __builtin_nontemporal_store(x, dst + u * kRetrieveWG + tid);
        page[u * kRetrieveWG + tid] = x;
      }
    }
    __syncthreads();
    if (wave == 0 && !cur.ok) {
      // (the same decision in every thread) an empty partial
      if (r < G && g == 0) {
        pml[2 * r] = -INFINITY;
        pml[2 * r + 1] = 0.f;
      }
    } else if (wave == 0) {
      const int ntok = cur.ntok;
      const bf16x8* qb = qc;
      const uint16_t* P = reinterpret_cast<const uint16_t*>(page);
      bf16x8 ka[4][4];
      load_keys(P, r, g, ka);
      f32x4 s[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) s[tt] = mfma16x16x32(ka[tt][kb], qb[kb], s[tt]);
      }
      // s[tt][i]: head r, token 32 (tt/2) + 8 g + 4 (tt%2) + i
      float mx = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 32 * (tt >> 1) + 8 * g + 4 * (tt & 1) + i;
          const float x = tok < ntok ? s[tt][i] * sl2 : -INFINITY;
          s[tt][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const bool none = mx == -INFINITY;
      float l = 0.f;
      bf16x8 phi[2], plo[2];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = none ? 0.f : exp2f(s[tt][i] - mx);
          l += pv;
          const __bf16 hi = (__bf16)pv;
          phi[tt >> 1][4 * (tt & 1) + i] = hi;
          plo[tt >> 1][4 * (tt & 1) + i] = (__bf16)(pv - (float)hi);
        }
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
      bf16x8 va[8][2];
      load_values(P + kPageTokens * kHeadDim, r, g, va);
      f32x4 acc[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          acc[dt] = mfma16x16x32(va[dt][kt], phi[kt], acc[dt]);
          acc[dt] = mfma16x16x32(va[dt][kt], plo[kt], acc[dt]);
        }
      }
      // acc[dt][i] = unnormalised out[head r][dim 16 dt + 4 g + i]
      if (r < G) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<float4*>(po + (size_t)r * kHeadDim + 16 * dt + 4 * g) =
              make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
        if (g == 0) {
          pml[2 * r] = mx;
          pml[2 * r + 1] = l;
        }
      }
    }
    __syncthreads();  // the LDS page is free for the next one
    cur = nxt;
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = vn[u];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qc[kb] = qn[kb];
  }
  if (tid == 0 && moved) atomicAdd(d.h2d, moved);
}

}  // namespace spin
