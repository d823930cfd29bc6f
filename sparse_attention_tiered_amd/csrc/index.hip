// State reset, request release, and Index (partition summaries).
//
// Index follows the partition abstraction of the SPIN pages ([XT] design part
// 1, Fig. 3: Index organises the KV into partitions and summarises them).  The
// summary is the mean key of a partition's valid tokens, read zero-copy from
// the request's pinned host KV through its device-mapped address.  bf16 keys
// are summed in float64, which is exact for up to 256 bf16 terms of the
// magnitudes involved, then divided and rounded once to float32.
#include "device_util.h"
#include "spin_internal.h"

namespace spin {

__global__ void k_init(Dev d) {
  const size_t tid = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t nth = gridDim.x * (size_t)blockDim.x;
  const size_t ndir = (size_t)d.B * d.Hkv * d.ndir;
  for (size_t i = tid; i < ndir; i += nth) d.directory[i] = -1;
  for (size_t i = tid; i < (size_t)d.n_seg * kSegEntries; i += nth) d.segments[i] = -1;
  for (size_t i = tid; i < (size_t)d.n_seg; i += nth) {
    d.seg_live[i] = 0;
    d.seg_stack[i] = d.n_seg - 1 - (int)i;  // top (last) is segment 0
  }
  for (size_t i = tid; i < (size_t)d.B * d.C; i += nth) {
    d.owner[i] = -1;
    d.last_use[i] = -1;
  }
  for (size_t i = tid; i < (size_t)d.B * d.Hkv; i += nth) {
    d.arrive[i] = 0;
    d.att_arrive[i] = 0;
  }
  for (size_t i = tid; i < (size_t)d.B; i += nth) {
    d.free_count[i] = d.C;
    d.budget[i] = d.C;
    d.last_t[i] = -1;
    d.req_parts[i] = 0;
    d.req_pages[i] = 0;
    d.req_stride[i] = 0;
    d.host_base[i] = 0;
    d.nmiss[i] = 0;
    d.nfreed[i] = 0;
    d.nalloc[i] = 0;
    d.stats[4 * i + 0] = 0;
    d.stats[4 * i + 1] = 0;
    d.stats[4 * i + 2] = 0;
    d.stats[4 * i + 3] = -1;
  }
  if (tid == 0) {
    d.seg_ctl[0] = d.n_seg;
    d.err[0] = 0;
    d.h2d[0] = 0;
  }
}

// Release request `req`: its linked segments go back on the free stack in
// (KV head, directory index) order with their entries cleared, and all of its
// slots become free.  One workgroup.
__global__ __launch_bounds__(1024) void k_release(Dev d, int req) {
  __shared__ int tmp[17];
  const int tid = threadIdx.x;
  const int n = d.Hkv * d.ndir;
  int* dir = d.directory + (size_t)req * n;
  const int top = d.seg_ctl[0];
  int carry = 0;
  for (int base = 0; base < n; base += 1024) {
    const int e = base + tid;
    int seg = e < n ? dir[e] : -1;
    if (seg >= d.n_seg) {
      atomicOr(d.err, kErrState);
      seg = -1;
    }
    int tot;
    const int ex = block_excl_scan<1024>(seg >= 0 ? 1 : 0, tmp, &tot);
    if (seg >= 0) {
      for (int j = 0; j < kSegEntries; ++j) d.segments[(size_t)seg * kSegEntries + j] = -1;
      d.seg_live[seg] = 0;
      const int at = top + carry + ex;
      if (at < d.n_seg) d.seg_stack[at] = seg;
      else atomicOr(d.err, kErrState);
      dir[e] = -1;
    }
    carry += tot;
  }
  for (int c = tid; c < d.C; c += 1024) {
    d.owner[(size_t)req * d.C + c] = -1;
    d.last_use[(size_t)req * d.C + c] = -1;
  }
  if (tid == 0) {
    d.seg_ctl[0] = min(top + carry, d.n_seg);
    d.free_count[req] = d.C;
    d.budget[req] = d.C;
    d.req_parts[req] = 0;
    d.req_pages[req] = 0;
    d.req_stride[req] = 0;
    d.host_base[req] = 0;
    d.nmiss[req] = 0;
    d.nfreed[req] = 0;
    d.nalloc[req] = 0;
  }
}

// One workgroup of 64 lanes per (partition, KV head); lane l owns dims 2l, 2l+1.
// `src` holds the request's pages as [Hkv][src_stride][page]: the device-mapped
// host buffer (Index of an offloaded request) or device memory (Index of
// freshly computed KV before it is offloaded).
__global__ __launch_bounds__(64) void k_index(Dev d, int req, const char* __restrict__ src,
                                              int src_stride) {
  const int i = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int len = d.part_len[(size_t)req * d.Nmax + i];
  const int first = d.part_first[(size_t)req * d.Nmax + i];
  const uint32_t* base = reinterpret_cast<const uint32_t*>(
      src + ((size_t)h * src_stride + first) * (size_t)kPageBytes);
  double s0 = 0.0, s1 = 0.0;
#pragma unroll 8
  for (int t = 0; t < len; ++t) {
    const uint32_t u = base[((t >> 6) * kPageElems + (t & 63) * kHeadDim) / 2 + lane];
    s0 += (double)bf16_lo(u);
    s1 += (double)bf16_hi(u);
  }
  float* out = d.summaries + (((size_t)req * d.Hkv + h) * d.Nmax + i) * kHeadDim;
  out[2 * lane] = (float)(s0 / (double)len);
  out[2 * lane + 1] = (float)(s1 / (double)len);
  if (i == gridDim.x - 1) {  // the last partition keeps its exact sum for appends
    double* ts = d.tail_sum + ((size_t)req * d.Hkv + h) * kHeadDim;
    ts[2 * lane] = s0;
    ts[2 * lane + 1] = s1;
  }
}

// Decode-time append of one token per registered request (k, v: [B][Hkv][128]
// bf16).  The token fills the last page of the request's last partition; a
// full page starts a new one-page partition.  The token is written to the
// host copy and, when the page is resident, to its pool slot; the tail
// partition's summary is its exact fp64 key sum over its length.  The host
// has checked that every request has room.
//
// One 1024-lane workgroup per request; lane e owns element e (and e + 1024
// when Hkv > 8) of the token's [Hkv][128] rows.  The kernel is a chain of
// dependent round trips (the request's tail, then the token and its
// directory entry, then the segment entry), so every load a lane needs is
// issued before its first store and loads are never conditional: the
// compiler cannot tell the stores from the loads apart, and would otherwise
// wait for each store before the next load.
constexpr int kAppendLanes = 1024;
constexpr int kAppendPer = kMaxKvHeads * kHeadDim / kAppendLanes;

__global__ __launch_bounds__(kAppendLanes) void k_append(Dev d, const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v) {
  __shared__ int sh[5];  // new partition?, tail index, page, token slot, new length
  const int b = blockIdx.x, tid = threadIdx.x;
  const unsigned long long host = d.host_base[b];
  const int stride = d.req_stride[b];
  if (tid == 0) {
    const int n = d.req_parts[b], pages = d.req_pages[b];
    const size_t last = (size_t)b * d.Nmax + (n > 0 ? n - 1 : 0);
    int L0 = d.part_len[last], F0 = d.part_first[last];
    asm volatile("" : "+s"(L0), "+s"(F0));  // both loads in flight before either is used
    const int L = n > 0 ? L0 : 0;
    const bool fresh = n == 0 || (L % kPageTokens) == 0;
    const int len = fresh ? 1 : L + 1;
    const int first = fresh ? pages : F0;
    sh[0] = fresh;
    sh[1] = fresh ? n : n - 1;
    sh[2] = first + (len - 1) / kPageTokens;
    sh[3] = (len - 1) % kPageTokens;
    sh[4] = len;
  }
  __syncthreads();
  if (host == 0) return;  // no registered KV (uniform over the workgroup)
  const bool fresh = sh[0];
  const int tail = sh[1], page = sh[2], tok = sh[3], len = sh[4];
  const int nel = d.Hkv * kHeadDim;
  uint16_t kb[kAppendPer], vb[kAppendPer];
  int seg[kAppendPer];
  double prev[kAppendPer];
#pragma unroll
  for (int j = 0; j < kAppendPer; ++j) {
    const int e = min(tid + j * kAppendLanes, nel - 1);
    const int h = e / kHeadDim;
    kb[j] = k[(size_t)b * nel + e];
    vb[j] = v[(size_t)b * nel + e];
    seg[j] = d.directory[((size_t)b * d.Hkv + h) * d.ndir + (page >> 6)];
    prev[j] = d.tail_sum[(size_t)b * nel + e];
  }
  int slot[kAppendPer];
#pragma unroll
  for (int j = 0; j < kAppendPer; ++j) {
    const bool ok = seg[j] >= 0 && seg[j] < d.n_seg;
    slot[j] = d.segments[(size_t)(ok ? seg[j] : 0) * kSegEntries + (page & 63)];
    if (!ok) slot[j] = -1;
  }
#pragma unroll
  for (int j = 0; j < kAppendPer; ++j) {
    const int e = tid + j * kAppendLanes;
    if (e >= nel) break;
    const int h = e / kHeadDim, dim = e - h * kHeadDim;
    // a global (not generic) pointer: generic stores may complete out of
    // order with loads, so every later wait would have to drain them
    __attribute__((address_space(1))) uint16_t* hp =
        reinterpret_cast<__attribute__((address_space(1))) uint16_t*>(
            host + ((size_t)h * stride + page) * (size_t)kPageBytes);
    hp[tok * kHeadDim + dim] = kb[j];
    hp[kPageTokens * kHeadDim + dim * kPageTokens + tok] = vb[j];
    if (slot[j] >= 0 && slot[j] < d.C) {
      uint16_t* pp = d.pool + ((size_t)b * d.C + slot[j]) * kPageElems;
      pp[tok * kHeadDim + dim] = kb[j];
      pp[kPageTokens * kHeadDim + dim * kPageTokens + tok] = vb[j];
    }
    const double sum = (fresh ? 0.0 : prev[j]) + (double)__uint_as_float((uint32_t)kb[j] << 16);
    d.tail_sum[(size_t)b * nel + e] = sum;
    d.summaries[(((size_t)b * d.Hkv + h) * d.Nmax + tail) * kHeadDim + dim] = (float)(sum / (double)len);
  }
  if (tid == 0) {  // read only by later launches
    d.part_len[(size_t)b * d.Nmax + tail] = len;
    if (fresh) {
      d.part_first[(size_t)b * d.Nmax + tail] = page;
      d.req_parts[b] = tail + 1;
      d.req_pages[b] = page + 1;
    }
  }
}

hipError_t launch_init(const Dev& d, hipStream_t s) {
  hipLaunchKernelGGL(k_init, dim3(1024), dim3(256), 0, s, d);
  return hipGetLastError();
}

hipError_t launch_release(const Dev& d, int req, hipStream_t s) {
  hipLaunchKernelGGL(k_release, dim3(1), dim3(1024), 0, s, d, req);
  return hipGetLastError();
}

__global__ void k_set_budget(Dev d, int req, int slots) { d.budget[req] = slots; }

hipError_t launch_set_budget(const Dev& d, int req, int slots, hipStream_t s) {
  hipLaunchKernelGGL(k_set_budget, dim3(1), dim3(1), 0, s, d, req, slots);
  return hipGetLastError();
}

hipError_t launch_index(const Dev& d, int req, int n_parts, const void* src, int src_stride,
                        hipStream_t s) {
  if (n_parts == 0) return hipSuccess;
  hipLaunchKernelGGL(k_index, dim3(n_parts, d.Hkv), dim3(64), 0, s, d, req,
                     static_cast<const char*>(src), src_stride);
  return hipGetLastError();
}

hipError_t launch_append(const Dev& d, const uint16_t* k, const uint16_t* v, hipStream_t s) {
  hipLaunchKernelGGL(k_append, dim3(d.B), dim3(kAppendLanes), 0, s, d, k, v);
  return hipGetLastError();
}

}  // namespace spin
