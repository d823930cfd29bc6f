// The segment-pool pass of the two-level page table ([XT] part 3, Fig. 6;
// [GP] C) as a workgroup body: k_segments runs it on its own, and the
// one-launch transfer + attention kernel runs it in one extra workgroup, where
// it is hidden behind the transfer.
#pragma once

#include "device_util.h"
#include "spin_internal.h"

namespace spin {

// The inserts of the step into their segments (slot entries and live
// counts), once every segment they need is linked: items start, start +
// stride, ... of the batch's insert lists (pm: each request's offset in it,
// M: its length), four items' loads in flight per thread.
__device__ __forceinline__ void insert_segments(const Dev& d, const int* pm, int M, int start, int stride) {
  const int ne = d.Hkv * d.ndir;
  constexpr int U = 4;
  for (int j0 = start; j0 < M; j0 += stride * U) {
    int4 ms[U];
    int bs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + stride * u;
      ms[u] = make_int4(-1, 0, 0, 0);
      bs[u] = 0;
      if (j < M) {
        bs[u] = owner_of(pm, d.B, j);
        ms[u] = d.ins[(size_t)bs[u] * d.max_mand + (j - pm[bs[u]])];  // (slot, h, page)
      }
    }
    int segs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      segs[u] = -1;
      if (j0 + stride * u < M && (unsigned)ms[u].y < (unsigned)d.Hkv && ms[u].z >= 0)
        segs[u] = d.directory[(size_t)bs[u] * ne + ms[u].y * d.ndir + (ms[u].z >> 6)];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int seg = segs[u];
      if (j0 + stride * u < M && seg >= 0 && seg < d.n_seg) {
        d.segments[(size_t)seg * kSegEntries + (ms[u].z & 63)] = ms[u].x;
        atomicAdd(&d.seg_live[seg], 1);
      }
    }
  }
}

// Shared segment pool, one workgroup for the batch: push every request's
// emptied segments (requests ascending), then hand segments to the directory
// ranges that k_resolve listed (requests ascending, canonical order), then
// (with_inserts) write the inserts into their segments, which
// k_segment_inserts does instead for large batches.  Each phase is a flat loop over the
// batch; a request is found from a flat index by binary search over the
// per-request prefix sums kept in LDS.  The retrieve does not wait for this
// pass: it reads the insert lists k_resolve wrote.

// LDS from the caller: lds holds 3 * 1025 ints, tmp NT / 64 + 1.
template <int NT>
__device__ __forceinline__ void segments_wg(const Dev& d, int with_inserts, int* lds, int* tmp) {
  int* pf = lds;
  int* pa = lds + 1025;
  int* pm = lds + 2 * 1025;
  const int tid = threadIdx.x;
  const int ne = d.Hkv * d.ndir;
  const int B = d.B;
  const int F = request_offsets<NT>(d.nfreed, B, pf, tmp);
  const int A = request_offsets<NT>(d.nalloc, B, pa, tmp);
  const int M = request_offsets<NT>(d.nmiss, B, pm, tmp);
  // each loop below issues the loads of U iterations before using any, so a
  // thread waits for one round trip per U items rather than one per item
  constexpr int U = 8;
  const int top0 = d.seg_ctl[0];
  for (int j0 = tid; j0 < F; j0 += NT * U) {
    int fs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + NT * u;
      fs[u] = -1;
      if (j < F) {
        const int b = owner_of(pf, B, j);
        fs[u] = d.freed[(size_t)b * ne + (j - pf[b])];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + NT * u;
      if (j >= F) break;
      const int at = top0 + j;
      if (at < d.n_seg) d.seg_stack[at] = fs[u];
      else atomicOr(d.err, kErrState);
    }
  }
  const int top1 = min(top0 + F, d.n_seg);
  __syncthreads();
  for (int j0 = tid; j0 < A; j0 += NT * U) {
    int es[U], ss[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + NT * u;
      es[u] = -1;
      ss[u] = -1;
      if (j < A) {
        const int b = owner_of(pa, B, j);
        es[u] = b * ne + d.alloc[(size_t)b * ne + (j - pa[b])];
        const int idx = top1 - 1 - j;
        if (idx >= 0) ss[u] = d.seg_stack[idx];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + NT * u;
      if (j >= A) break;
      if (top1 - 1 - j >= 0) d.directory[es[u]] = ss[u];
      else atomicOr(d.err, kErrSegPool);
    }
  }
  if (tid == 0) d.seg_ctl[0] = max(top1 - A, 0);
  if (with_inserts) {
    __syncthreads();
    insert_segments(d, pm, M, tid, NT);
  }
}


}  // namespace spin
