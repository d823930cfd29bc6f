// Retrieve: copy the step's missed pages from pinned host memory into their
// GPU slots ([XT] design part 2, Fig. 5 steps 3-4: the host address comes
// from the CPU page table, then the transfer is issued; [GP] B: pages are per
// KV head, so only the needed head's page, at most 32 KiB, crosses the link).
//
// The GPU pulls the pages itself: each workgroup reads 32 KiB pages through
// the host buffer's device-mapped address with 16-byte loads per lane (two
// pages, sixteen loads, in flight per lane; key rows of valid tokens only)
// and writes them whole to HBM.  The host never reads the miss count: the
// grid is fixed and every workgroup strides over the batch's insert lists,
// which k_resolve writes, so the transfer does not wait for the segment-pool
// pass.
#include "arrival.h"
#include "device_util.h"
#include "spin_internal.h"

namespace spin {

// A few dozen workgroups keep far more than the link's bandwidth-delay product
// in flight (sixteen 16 B loads per lane, 64 KiB per workgroup); measured on
// MI355X, 16-128 workgroups pull 56.5-57.4 GB/s of scattered pages, as fast as
// a bulk DMA copy, while 256+ workgroups drop to 55 GB/s.  A small grid also
// leaves the other CUs to the attention pass that overlaps the transfer.
// (96 and 128 workgroups, and half- or quarter-page work units, measured no
// better for a few misses per step and worse for thousands.)  kRetrieveGrid
// and kRetrieveWG live with the other shared constants.

__global__ __launch_bounds__(kRetrieveWG) void k_retrieve(Dev d) {
  __shared__ int pm[1025];
  __shared__ int tmp[kRetrieveWG / 64 + 1];
  const int tid = threadIdx.x;
  // where each request's misses start in the batch-wide concatenation of the
  // insert lists k_resolve wrote (requests ascending, canonical order)
  const int M = request_offsets<kRetrieveWG>(d.nmiss, d.B, pm, tmp);
  // a page's source, destination and valid tokens, or null when its entry
  // is out of range
  auto page = [&](int j, const u32x4*& src, u32x4*& dst, int& ntok) {
    src = nullptr;
    dst = nullptr;
    ntok = 0;
    if (j >= M) return;
    const int b = owner_of(pm, d.B, j);
    const size_t e = (size_t)b * d.max_mand + (j - pm[b]);
    const int4 m = d.ins[e];  // (slot, KV head, page)
    if ((unsigned)m.x >= (unsigned)d.C || (unsigned)m.y >= (unsigned)d.Hkv ||
        (unsigned)m.z >= (unsigned)d.req_pages[b])
      return;
    ntok = d.miss_tmp[e].w;
    src = reinterpret_cast<const u32x4*>(d.host_base[b] +
                                         ((size_t)m.y * d.req_stride[b] + m.z) * (size_t)kPageBytes);
    dst = reinterpret_cast<u32x4*>(d.pool + ((size_t)b * d.C + m.x) * kPageElems);
  };
  // two pages in flight per workgroup (pages j and j + grid), 64 KiB
  const int nwg = gridDim.x;
  unsigned long long moved = 0;  // bytes this workgroup read over the link
  for (int j = blockIdx.x; j < M; j += 2 * nwg) {
    const u32x4 *s0, *s1;
    u32x4 *d0, *d1;
    int n0, n1;
    page(j, s0, d0, n0);
    page(j + nwg, s1, d1, n1);
    u32x4 v[8], w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = u * kRetrieveWG + tid;
      if (s0) v[u] = chunk_live(c, n0) ? s0[c] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = u * kRetrieveWG + tid;
      if (s1) w[u] = chunk_live(c, n1) ? s1[c] : u32x4{0u, 0u, 0u, 0u};
    }
    if (s0) moved += link_bytes(n0);
    if (s1) moved += link_bytes(n1);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (d0) __builtin_nontemporal_store(pool_chunk(v[u], u * kRetrieveWG + tid, n0), d0 + u * kRetrieveWG + tid);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (d1) __builtin_nontemporal_store(pool_chunk(w[u], u * kRetrieveWG + tid, n1), d1 + u * kRetrieveWG + tid);
  }
  if (tid == 0 && moved) atomicAdd(d.h2d, moved);
}

__global__ __launch_bounds__(kRetrieveWG) void k_retrieve_attend(Dev d, const uint16_t* __restrict__ q) {
  __shared__ int pm[1025];
  __shared__ int tmp[kRetrieveWG / 64 + 1];
  __shared__ u32x4 page[kPageBytes / 16];
  retrieve_attend_wg(d, step_queries(d, q), blockIdx.x, gridDim.x, pm, tmp, page);
}

hipError_t launch_retrieve_attend(const Dev& d, const uint16_t* q, hipStream_t s) {
  hipLaunchKernelGGL(k_retrieve_attend, dim3(kRetrieveGrid), dim3(kRetrieveWG), 0, s, d, q);
  return hipGetLastError();
}

hipError_t launch_retrieve(const Dev& d, hipStream_t s) {
  hipLaunchKernelGGL(k_retrieve, dim3(kRetrieveGrid), dim3(kRetrieveWG), 0, s, d);
  return hipGetLastError();
}

}  // namespace spin
