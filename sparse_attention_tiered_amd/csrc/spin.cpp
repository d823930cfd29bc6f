// Host side of libspin.so: configuration checks, workspace layout, the
// per-call launch sequences, stream/event ordering, stats and snapshots.
// All device memory is the caller's; this file only carves it up.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "spin.h"
#include "spin_internal.h"

using spin::Dev;

// Host copy of what decides an append: whether a request has registered KV,
// its partition count, the last partition's length, its pages and the room
// its host buffer has (pages per KV head).
struct ReqMirror {
  bool registered = false;
  int n_parts = 0, last_len = 0, pages = 0, stride = 0;
};

struct spin_ctx {
  spin_config cfg;
  Dev dev;
  std::vector<ReqMirror> req;
  // Cross-stream ordering, recorded lazily: an event record or wait costs the
  // GPU several microseconds even when nothing is pending, so the events are
  // recorded only when another stream has to wait.  ev_resolved marks the
  // latest resolve (enqueued on resolved_on), ev_fetched the latest transfer
  // (fetched_gen counts transfers, 0: none yet; enqueued on fetched_on); each
  // is recorded, behind everything enqueued on its stream by then, the first
  // time another stream needs it.  waited_on already waited for transfer
  // waited_gen and needs no second wait.
  hipEvent_t ev_resolved = nullptr;
  hipEvent_t ev_fetched = nullptr;
  uint64_t fetched_gen = 0, waited_gen = 0;
  hipStream_t fetched_on = nullptr, waited_on = nullptr;
  bool fetched_recorded = false;
  hipStream_t resolved_on = nullptr;
  bool resolved_any = false, resolved_recorded = false;
  int hip_err = 0;
  int last_t = -1;
  size_t ws_bytes = 0;
  int32_t* h_segments = nullptr;  // host address of the segment tables, if in host memory
  bool arrival = false;  // the last transfer attended its pages on arrival
};

namespace {

// Orders stream s after the latest transfer (see spin_ctx).
hipError_t wait_fetched(spin_ctx* ctx, hipStream_t s) {
  if (ctx->fetched_gen == 0 || s == ctx->fetched_on) return hipSuccess;
  if (s == ctx->waited_on && ctx->waited_gen == ctx->fetched_gen) return hipSuccess;
  hipError_t e = hipSuccess;
  if (!ctx->fetched_recorded) {
    e = hipEventRecord(ctx->ev_fetched, ctx->fetched_on);
    if (e != hipSuccess) return e;
    ctx->fetched_recorded = true;
  }
  e = hipStreamWaitEvent(s, ctx->ev_fetched, 0);
  if (e == hipSuccess) {
    ctx->waited_on = s;
    ctx->waited_gen = ctx->fetched_gen;
  }
  return e;
}

// Orders stream s after the latest resolve.
hipError_t wait_resolved(spin_ctx* ctx, hipStream_t s) {
  if (!ctx->resolved_any || s == ctx->resolved_on) return hipSuccess;
  hipError_t e = hipSuccess;
  if (!ctx->resolved_recorded) {
    e = hipEventRecord(ctx->ev_resolved, ctx->resolved_on);
    if (e != hipSuccess) return e;
    ctx->resolved_recorded = true;
  }
  return hipStreamWaitEvent(s, ctx->ev_resolved, 0);
}

// A transfer was just enqueued on s.
void transfer_enqueued(spin_ctx* ctx, hipStream_t s) {
  ++ctx->fetched_gen;
  ctx->fetched_on = s;
  ctx->fetched_recorded = false;
}

struct Derived {
  int G, ndir, max_blocks, max_mand, pps, splits, pps_res, splits_res;
};

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

int check(const spin_config* c) {
  if (!c) return SPIN_EINVAL;
  if (c->head_dim != spin::kHeadDim || c->page_tokens != spin::kPageTokens ||
      c->seg_entries != spin::kSegEntries || c->num_buckets != spin::kBuckets)
    return SPIN_EINVAL;
  if (c->max_batch < 1 || c->max_batch > 1024) return SPIN_EINVAL;
  if (c->num_kv_heads < 1 || c->num_kv_heads > spin::kMaxKvHeads) return SPIN_EINVAL;
  if (c->num_q_heads < c->num_kv_heads || c->num_q_heads % c->num_kv_heads) return SPIN_EINVAL;
  if (c->num_q_heads / c->num_kv_heads > spin::kMaxGroup) return SPIN_EINVAL;
  if (c->max_partitions < 1 || c->max_partitions > spin::kMaxPartitions) return SPIN_EINVAL;
  if (c->max_pages_per_partition < 1 || c->max_pages_per_partition > spin::kMaxPPP) return SPIN_EINVAL;
  if (c->max_pages < 1 || (long long)c->max_pages > (long long)c->max_partitions * c->max_pages_per_partition)
    return SPIN_EINVAL;
  if (c->topk < 1 || c->topk > 1024 || c->num_kv_heads * c->topk > spin::kMaxItems) return SPIN_EINVAL;
  if (c->num_segments < 1 || c->num_segments > (1 << 28)) return SPIN_EINVAL;
  if (c->attend_pages_per_split < 0 || c->attend_pages_per_split > 256) return SPIN_EINVAL;
  if (c->segments_in_host_memory != 0 && c->segments_in_host_memory != 1) return SPIN_EINVAL;
  if (c->slots_per_request < 1 || c->slots_per_request > spin::kMaxSlots) return SPIN_EINVAL;
  if ((long long)c->max_batch * c->slots_per_request > (1LL << 31) / 2) return SPIN_EINVAL;
  // every page one step can need must fit in the request's slots
  if (c->slots_per_request < c->num_kv_heads * c->topk * c->max_pages_per_partition)
    return SPIN_ECAPACITY;
  return SPIN_OK;
}

}  // namespace

int spin::whole_table_pages_per_split(long long work, int pages_per_split) {
  if (pages_per_split > 0) return (pages_per_split + 3) / 4 * 4;  // whole pages per wave
  // about one workgroup per CU over the worst-case page count: long-lived
  // waves keep their page pipeline full (measured best on MI355X)
  const int pps = (int)std::min<long long>(64, std::max<long long>(4, (work + 255) / 256));
  return (pps + 3) / 4 * 4;
}

namespace {

Derived derive(const spin_config* c) {
  Derived d;
  d.G = c->num_q_heads / c->num_kv_heads;
  d.ndir = (c->max_pages + spin::kSegEntries - 1) / spin::kSegEntries;
  d.max_blocks = c->topk * c->max_pages_per_partition;
  d.max_mand = c->num_kv_heads * d.max_blocks;
  const long long work = (long long)c->max_batch * c->num_kv_heads * d.max_blocks;
  const int pps = spin::whole_table_pages_per_split(work, c->attend_pages_per_split);
  int pps_res = pps;
  if (c->attend_pages_per_split == 0) {
    // the resident-page pass runs beside the transfer, which it must only
    // keep up with: about half a workgroup per CU, each streaming pages
    // while the PCIe pulls are in flight, contends less with them (128K
    // workload, ~90 misses a step: 0.1115 -> 0.1070 ms per step), but at
    // least two splits per head (one split per head there, 64 workgroups:
    // 0.117 ms; on the 32K workload one split per head was 0.1-0.4% slower
    // than two)
    const int half = (d.max_blocks + 1) / 2;
    pps_res = (int)std::min<long long>(64, std::max<long long>(pps, (work + 127) / 128));
    pps_res = std::min(pps_res, std::max(pps, half));
    pps_res = (pps_res + 3) / 4 * 4;
  }
  d.pps = pps;
  d.splits = (d.max_blocks + pps - 1) / pps;
  d.pps_res = pps_res;
  d.splits_res = (d.max_blocks + pps_res - 1) / pps_res;
  return d;
}

// Byte offsets of every workspace region (each 256-byte aligned).
struct Layout {
  size_t summaries, part_first, part_len, req_parts, req_pages, req_stride, tail_sum, host_base,
      directory, segments,
      seg_live, seg_stack, seg_ctl, owner, last_use, free_count, budget, last_t, scores, arrive, srange,
      miss_tmp, ins,
      nmiss,
      freed, nfreed, alloc, nalloc, bmiss, att_arrive, part_o, part_ml, arr_o, arr_ml, head_moff, stats, h2d, err,
      total;
};

Layout layout(const spin_config* c, const Derived& d) {
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = up(o + bytes);
    return at;
  };
  const size_t B = c->max_batch, Hkv = c->num_kv_heads, N = c->max_partitions;
  const size_t C = c->slots_per_request, S = c->num_segments;
  L.summaries = take(B * Hkv * N * spin::kHeadDim * sizeof(float));
  L.part_first = take(B * N * sizeof(int));
  L.part_len = take(B * N * sizeof(int));
  L.req_parts = take(B * sizeof(int));
  L.req_pages = take(B * sizeof(int));
  L.req_stride = take(B * sizeof(int));
  L.tail_sum = take(B * Hkv * spin::kHeadDim * sizeof(double));
  L.host_base = take(B * sizeof(unsigned long long));
  L.directory = take(B * Hkv * d.ndir * sizeof(int));
  L.segments = take(c->segments_in_host_memory ? 0 : S * spin::kSegEntries * sizeof(int));
  L.seg_live = take(S * sizeof(int));
  L.seg_stack = take(S * sizeof(int));
  L.seg_ctl = take(4 * sizeof(int));
  L.owner = take(B * C * sizeof(int));
  L.last_use = take(B * C * sizeof(int));
  L.free_count = take(B * sizeof(int));
  L.budget = take(B * sizeof(int));
  L.last_t = take(B * sizeof(int));
  L.scores = take(B * Hkv * N * sizeof(float));
  L.arrive = take(B * Hkv * sizeof(int));
  L.srange = take(B * Hkv * spin::kSplitRangeSlots * 2 * sizeof(float));
  L.miss_tmp = take(B * d.max_mand * sizeof(int4));
  L.ins = take(B * d.max_mand * sizeof(int4));
  L.nmiss = take(B * sizeof(int));
  L.freed = take(B * Hkv * d.ndir * sizeof(int));
  L.nfreed = take(B * sizeof(int));
  L.alloc = take(B * Hkv * d.ndir * sizeof(int));
  L.nalloc = take(B * sizeof(int));
  L.bmiss = take(B * Hkv * d.max_blocks);
  L.att_arrive = take(B * Hkv * sizeof(int));
  L.part_o = take(B * Hkv * 2 * d.splits * d.G * spin::kHeadDim * sizeof(float));
  L.part_ml = take(B * Hkv * 2 * d.splits * d.G * 2 * sizeof(float));
  L.arr_o = take(B * d.max_mand * d.G * spin::kHeadDim * sizeof(float));
  L.arr_ml = take(B * d.max_mand * d.G * 2 * sizeof(float));
  L.head_moff = take(B * (Hkv + 1) * sizeof(int));
  L.stats = take(B * 4 * sizeof(long long));
  L.h2d = take(sizeof(unsigned long long));
  L.err = take(4 * sizeof(int));
  L.total = o;
  return L;
}

#define HIPCHK(ctx, expr)                       \
  do {                                          \
    hipError_t e_ = (expr);                     \
    if (e_ != hipSuccess) {                     \
      if (ctx) (ctx)->hip_err = (int)e_;        \
      return SPIN_EHIP;                         \
    }                                           \
  } while (0)

hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

SPIN_API int spin_config_init(spin_config* cfg) {
  if (!cfg) return SPIN_EINVAL;
  std::memset(cfg, 0, sizeof(*cfg));
  cfg->head_dim = spin::kHeadDim;
  cfg->page_tokens = spin::kPageTokens;
  cfg->seg_entries = spin::kSegEntries;
  cfg->num_buckets = spin::kBuckets;
  cfg->max_pages_per_partition = 1;
  return SPIN_OK;
}

SPIN_API int spin_config_check(const spin_config* cfg) { return check(cfg); }

SPIN_API int spin_workspace_size(const spin_config* cfg, size_t* ws_bytes, size_t* pool_bytes) {
  const int rc = check(cfg);
  if (rc) return rc;
  const Derived d = derive(cfg);
  if (ws_bytes) *ws_bytes = layout(cfg, d).total;
  if (pool_bytes) *pool_bytes = (size_t)cfg->max_batch * cfg->slots_per_request * spin::kPageBytes;
  return SPIN_OK;
}

SPIN_API int spin_host_segment_bytes(const spin_config* cfg, size_t* bytes) {
  const int rc = check(cfg);
  if (rc) return rc;
  if (bytes)
    *bytes = cfg->segments_in_host_memory
                 ? (size_t)cfg->num_segments * spin::kSegEntries * sizeof(int32_t)
                 : 0;
  return SPIN_OK;
}

SPIN_API int spin_derived(const spin_config* cfg, int32_t* ndir, int32_t* max_blocks,
                          int32_t* attend_splits) {
  const int rc = check(cfg);
  if (rc) return rc;
  const Derived d = derive(cfg);
  if (ndir) *ndir = d.ndir;
  if (max_blocks) *max_blocks = d.max_blocks;
  if (attend_splits) *attend_splits = d.splits;
  return SPIN_OK;
}

SPIN_API int spin_create(const spin_config* cfg, void* d_ws, size_t ws_bytes, void* d_pool,
                         size_t pool_bytes, void* stream, spin_ctx** out) {
  return spin_create_ex(cfg, d_ws, ws_bytes, d_pool, pool_bytes, nullptr, 0, stream, out);
}

SPIN_API int spin_create_ex(const spin_config* cfg, void* d_ws, size_t ws_bytes, void* d_pool,
                            size_t pool_bytes, void* h_seg, size_t h_seg_bytes, void* stream,
                            spin_ctx** out) {
  if (!out) return SPIN_EINVAL;
  *out = nullptr;
  int rc = check(cfg);
  if (rc) return rc;
  // the segment tables: in the workspace, or in the caller's pinned host memory
  int32_t* seg_dev = nullptr;
  if (cfg->segments_in_host_memory) {
    const size_t need_seg = (size_t)cfg->num_segments * spin::kSegEntries * sizeof(int32_t);
    if (!h_seg || h_seg_bytes < need_seg) return SPIN_EINVAL;
    void* p = nullptr;
    if (hipHostGetDevicePointer(&p, h_seg, 0) != hipSuccess || !aligned(p, 16)) return SPIN_EINVAL;
    seg_dev = static_cast<int32_t*>(p);
  } else if (h_seg) {
    return SPIN_EINVAL;
  }
  const Derived d = derive(cfg);
  const Layout L = layout(cfg, d);
  const size_t need_pool = (size_t)cfg->max_batch * cfg->slots_per_request * spin::kPageBytes;
  if (!d_ws || !d_pool || ws_bytes < L.total || pool_bytes < need_pool) return SPIN_EINVAL;
  if (!aligned(d_ws, kAlign) || !aligned(d_pool, kAlign)) return SPIN_EINVAL;
  spin_ctx* ctx = new (std::nothrow) spin_ctx();
  if (!ctx) return SPIN_EINVAL;
  ctx->cfg = *cfg;
  ctx->ws_bytes = ws_bytes;
  ctx->req.assign(cfg->max_batch, ReqMirror());
  char* w = static_cast<char*>(d_ws);
  Dev& v = ctx->dev;
  v.B = cfg->max_batch;
  v.Hq = cfg->num_q_heads;
  v.Hkv = cfg->num_kv_heads;
  v.G = d.G;
  v.k = cfg->topk;
  v.Nmax = cfg->max_partitions;
  v.max_pages = cfg->max_pages;
  v.max_ppp = cfg->max_pages_per_partition;
  v.C = cfg->slots_per_request;
  v.n_seg = cfg->num_segments;
  v.ndir = d.ndir;
  v.max_blocks = d.max_blocks;
  v.max_mand = d.max_mand;
  v.splits = d.splits;
  v.pps = d.pps;
  v.splits_res = d.splits_res;
  v.pps_res = d.pps_res;
  v.pool_slots = cfg->max_batch * cfg->slots_per_request;
  v.summaries = reinterpret_cast<float*>(w + L.summaries);
  v.part_first = reinterpret_cast<int*>(w + L.part_first);
  v.part_len = reinterpret_cast<int*>(w + L.part_len);
  v.req_parts = reinterpret_cast<int*>(w + L.req_parts);
  v.req_pages = reinterpret_cast<int*>(w + L.req_pages);
  v.req_stride = reinterpret_cast<int*>(w + L.req_stride);
  v.tail_sum = reinterpret_cast<double*>(w + L.tail_sum);
  v.host_base = reinterpret_cast<unsigned long long*>(w + L.host_base);
  v.directory = reinterpret_cast<int*>(w + L.directory);
  v.segments = seg_dev ? seg_dev : reinterpret_cast<int*>(w + L.segments);
  ctx->h_segments = seg_dev ? static_cast<int32_t*>(h_seg) : nullptr;
  v.seg_live = reinterpret_cast<int*>(w + L.seg_live);
  v.seg_stack = reinterpret_cast<int*>(w + L.seg_stack);
  v.seg_ctl = reinterpret_cast<int*>(w + L.seg_ctl);
  v.owner = reinterpret_cast<int*>(w + L.owner);
  v.last_use = reinterpret_cast<int*>(w + L.last_use);
  v.free_count = reinterpret_cast<int*>(w + L.free_count);
  v.budget = reinterpret_cast<int*>(w + L.budget);
  v.last_t = reinterpret_cast<int*>(w + L.last_t);
  v.scores = reinterpret_cast<float*>(w + L.scores);
  v.arrive = reinterpret_cast<int*>(w + L.arrive);
  v.srange = reinterpret_cast<float*>(w + L.srange);
  v.miss_tmp = reinterpret_cast<int4*>(w + L.miss_tmp);
  v.ins = reinterpret_cast<int4*>(w + L.ins);
  v.nmiss = reinterpret_cast<int*>(w + L.nmiss);
  v.freed = reinterpret_cast<int*>(w + L.freed);
  v.nfreed = reinterpret_cast<int*>(w + L.nfreed);
  v.alloc = reinterpret_cast<int*>(w + L.alloc);
  v.nalloc = reinterpret_cast<int*>(w + L.nalloc);
  v.bmiss = reinterpret_cast<unsigned char*>(w + L.bmiss);
  v.att_arrive = reinterpret_cast<int*>(w + L.att_arrive);
  v.part_o = reinterpret_cast<float*>(w + L.part_o);
  v.part_ml = reinterpret_cast<float*>(w + L.part_ml);
  v.arr_o = reinterpret_cast<float*>(w + L.arr_o);
  v.arr_ml = reinterpret_cast<float*>(w + L.arr_ml);
  v.head_moff = reinterpret_cast<int*>(w + L.head_moff);
  v.stats = reinterpret_cast<long long*>(w + L.stats);
  v.h2d = reinterpret_cast<unsigned long long*>(w + L.h2d);
  v.err = reinterpret_cast<int*>(w + L.err);
  v.pool = static_cast<uint16_t*>(d_pool);
  v.step_t = nullptr;
  v.q_step = 0;
  hipError_t e = hipEventCreateWithFlags(&ctx->ev_resolved, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ctx->ev_fetched, hipEventDisableTiming);
  if (e == hipSuccess) e = spin::launch_init(v, S(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(S(stream));
  if (e != hipSuccess) {
    spin_destroy(ctx);
    return SPIN_EHIP;
  }
  *out = ctx;
  return SPIN_OK;
}

SPIN_API int spin_destroy(spin_ctx* ctx) {
  if (!ctx) return SPIN_EINVAL;
  if (ctx->fetched_gen) {
    if (!ctx->fetched_recorded) (void)hipStreamSynchronize(ctx->fetched_on);
    else (void)hipEventSynchronize(ctx->ev_fetched);
  }
  if (ctx->ev_resolved) (void)hipEventDestroy(ctx->ev_resolved);
  if (ctx->ev_fetched) (void)hipEventDestroy(ctx->ev_fetched);
  delete ctx;
  return SPIN_OK;
}

SPIN_API int spin_release(spin_ctx* ctx, int32_t req, void* stream) {
  if (!ctx || req < 0 || req >= ctx->cfg.max_batch) return SPIN_EINVAL;
  HIPCHK(ctx, wait_fetched(ctx, S(stream)));
  HIPCHK(ctx, spin::launch_release(ctx->dev, req, S(stream)));
  HIPCHK(ctx, hipStreamSynchronize(S(stream)));
  ctx->req[req] = ReqMirror();
  return SPIN_OK;
}

SPIN_API int spin_set_budget(spin_ctx* ctx, int32_t req, int32_t slots, void* stream) {
  if (!ctx || req < 0 || req >= ctx->cfg.max_batch) return SPIN_EINVAL;
  const spin_config& c = ctx->cfg;
  if (slots > c.slots_per_request) return SPIN_EINVAL;
  if (slots < c.num_kv_heads * c.topk * c.max_pages_per_partition) return SPIN_ECAPACITY;
  HIPCHK(ctx, spin::launch_set_budget(ctx->dev, req, slots, S(stream)));
  return SPIN_OK;
}

namespace {

// Partition lengths of a request: part_lens, or fixed 64-token partitions
// covering n_tokens.  Returns SPIN_OK and fills lens/first/pages.
int partition_table(const spin_config& c, int64_t n_tokens, const int32_t* part_lens,
                    int32_t n_parts, std::vector<int32_t>& lens, std::vector<int32_t>& first,
                    int64_t& pages) {
  if (n_tokens < 0) return SPIN_EINVAL;
  lens.clear();
  if (part_lens) {
    if (n_parts < 0) return SPIN_EINVAL;
    lens.assign(part_lens, part_lens + n_parts);
    int64_t sum = 0;
    for (int32_t L : lens) {
      if (L < 1 || L > spin::kPageTokens * c.max_pages_per_partition) return SPIN_EINVAL;
      sum += L;
    }
    if (sum != n_tokens) return SPIN_EINVAL;
  } else {
    const int64_t full = n_tokens / spin::kPageTokens, tail = n_tokens % spin::kPageTokens;
    if (full + (tail ? 1 : 0) > c.max_partitions) return SPIN_EINVAL;
    lens.assign((size_t)full, spin::kPageTokens);
    if (tail) lens.push_back((int32_t)tail);
  }
  if ((int64_t)lens.size() > c.max_partitions) return SPIN_EINVAL;
  first.resize(lens.size());
  pages = 0;
  for (size_t i = 0; i < lens.size(); ++i) {
    first[i] = (int32_t)pages;
    pages += (lens[i] + spin::kPageTokens - 1) / spin::kPageTokens;
  }
  if (pages > c.max_pages) return SPIN_EINVAL;
  return SPIN_OK;
}

// Register request `req`: release it, write its partition table, host base
// and host stride, then build the summaries from `src` ([Hkv][src_stride]
// pages; device-mapped host or device memory).  Leaves the stream busy.
int register_request(spin_ctx* ctx, int32_t req, unsigned long long host_base, int stride,
                     const std::vector<int32_t>& lens, const std::vector<int32_t>& first,
                     int pages, const void* src, int src_stride, hipStream_t s) {
  Dev& v = ctx->dev;
  const int np = (int)lens.size();
  HIPCHK(ctx, wait_fetched(ctx, s));
  HIPCHK(ctx, spin::launch_release(v, req, s));
  if (np) {
    HIPCHK(ctx, hipMemcpyAsync(v.part_first + (size_t)req * v.Nmax, first.data(), np * sizeof(int),
                               hipMemcpyHostToDevice, s));
    HIPCHK(ctx, hipMemcpyAsync(v.part_len + (size_t)req * v.Nmax, lens.data(), np * sizeof(int),
                               hipMemcpyHostToDevice, s));
  }
  HIPCHK(ctx, hipMemcpyAsync(v.req_pages + req, &pages, sizeof(int), hipMemcpyHostToDevice, s));
  HIPCHK(ctx, hipMemcpyAsync(v.req_stride + req, &stride, sizeof(int), hipMemcpyHostToDevice, s));
  HIPCHK(ctx, hipMemcpyAsync(v.host_base + req, &host_base, sizeof(host_base), hipMemcpyHostToDevice, s));
  HIPCHK(ctx, spin::launch_index(v, req, np, src, src_stride, s));
  // partitions become visible to select/resolve only once the summaries exist
  HIPCHK(ctx, hipMemcpyAsync(v.req_parts + req, &np, sizeof(int), hipMemcpyHostToDevice, s));
  HIPCHK(ctx, hipStreamSynchronize(s));
  ReqMirror& m = ctx->req[req];
  m.registered = host_base != 0;
  m.n_parts = np;
  m.last_len = np ? lens.back() : 0;
  m.pages = pages;
  m.stride = stride;
  return SPIN_OK;
}

}  // namespace

SPIN_API int spin_index(spin_ctx* ctx, int32_t req, const void* h_kv, int64_t n_tokens,
                        const int32_t* part_lens, int32_t n_parts, void* stream) {
  if (!ctx || req < 0 || req >= ctx->cfg.max_batch) return SPIN_EINVAL;
  std::vector<int32_t> lens, first;
  int64_t pages = 0;
  int rc = partition_table(ctx->cfg, n_tokens, part_lens, n_parts, lens, first, pages);
  if (rc) return rc;
  unsigned long long base = 0;
  if (!lens.empty()) {
    if (!h_kv) return SPIN_EINVAL;
    void* dptr = nullptr;
    HIPCHK(ctx, hipHostGetDevicePointer(&dptr, const_cast<void*>(h_kv), 0));
    if (!aligned(dptr, 16)) return SPIN_EINVAL;
    base = reinterpret_cast<unsigned long long>(dptr);
  }
  return register_request(ctx, req, base, (int)pages, lens, first, (int)pages,
                          reinterpret_cast<const void*>(base), (int)pages, S(stream));
}

SPIN_API int spin_offload(spin_ctx* ctx, int32_t req, const void* d_kv, void* h_kv,
                          size_t h_kv_bytes, int64_t n_tokens, const int32_t* part_lens,
                          int32_t n_parts, void* stream) {
  if (!ctx || req < 0 || req >= ctx->cfg.max_batch || !h_kv) return SPIN_EINVAL;
  const spin_config& c = ctx->cfg;
  std::vector<int32_t> lens, first;
  int64_t pages = 0;
  int rc = partition_table(c, n_tokens, part_lens, n_parts, lens, first, pages);
  if (rc) return rc;
  const size_t head_bytes = (size_t)c.num_kv_heads * spin::kPageBytes;
  const int64_t capacity = (int64_t)(h_kv_bytes / head_bytes);
  if (capacity < pages || capacity < 1 || capacity > (1 << 30)) return SPIN_ECAPACITY;
  if (pages > 0 && (!d_kv || !aligned(d_kv, 16))) return SPIN_EINVAL;
  void* dptr = nullptr;
  HIPCHK(ctx, hipHostGetDevicePointer(&dptr, h_kv, 0));
  if (!aligned(dptr, 16)) return SPIN_EINVAL;
  hipStream_t s = S(stream);
  if (pages > 0)  // Offload: each head's pages to its reserved run in host memory
    HIPCHK(ctx, hipMemcpy2DAsync(h_kv, (size_t)capacity * spin::kPageBytes, d_kv,
                                 (size_t)pages * spin::kPageBytes, (size_t)pages * spin::kPageBytes,
                                 c.num_kv_heads, hipMemcpyDeviceToHost, s));
  // Index from the device copy (HBM), after the copy in stream order
  return register_request(ctx, req, reinterpret_cast<unsigned long long>(dptr), (int)capacity, lens,
                          first, (int)pages, d_kv, (int)pages, s);
}

SPIN_API int spin_append(spin_ctx* ctx, const void* d_k, const void* d_v, void* stream) {
  if (!ctx || !d_k || !d_v) return SPIN_EINVAL;
  const spin_config& c = ctx->cfg;
  // every registered request must have room for the token before anything runs
  for (const ReqMirror& m : ctx->req) {
    if (!m.registered) continue;
    const bool fresh = m.n_parts == 0 || m.last_len % spin::kPageTokens == 0;
    if (fresh && (m.n_parts >= c.max_partitions || m.pages >= std::min(m.stride, c.max_pages)))
      return SPIN_ECAPACITY;
    if (!fresh && m.last_len >= spin::kPageTokens * c.max_pages_per_partition) return SPIN_ECAPACITY;
  }
  HIPCHK(ctx, wait_fetched(ctx, S(stream)));
  HIPCHK(ctx, spin::launch_append(ctx->dev, static_cast<const uint16_t*>(d_k),
                                  static_cast<const uint16_t*>(d_v), S(stream)));
  for (ReqMirror& m : ctx->req) {
    if (!m.registered) continue;
    const bool fresh = m.n_parts == 0 || m.last_len % spin::kPageTokens == 0;
    if (fresh) {
      ++m.n_parts;
      ++m.pages;
      m.last_len = 1;
    } else {
      ++m.last_len;
    }
  }
  return SPIN_OK;
}

SPIN_API int spin_select(spin_ctx* ctx, const void* d_q, int32_t* d_sel, float* d_scores,
                         void* stream) {
  if (!ctx || !d_q || !d_sel || !aligned(d_q, 16)) return SPIN_EINVAL;
  float* sc = d_scores ? d_scores : ctx->dev.scores;
  const uint16_t* q = static_cast<const uint16_t*>(d_q);
  if (ctx->dev.B * ctx->dev.Hkv >= spin::kFusedSelectMinLists) {
    HIPCHK(ctx, spin::launch_select_fused(ctx->dev, q, sc, d_sel, S(stream)));
  } else if (ctx->dev.Nmax <= spin::kSplitSelectMaxParts) {
    HIPCHK(ctx, spin::launch_select_split(ctx->dev, q, sc, d_sel, S(stream)));
  } else {
    HIPCHK(ctx, spin::launch_score(ctx->dev, q, sc, S(stream)));
    HIPCHK(ctx, spin::launch_topk(ctx->dev, sc, d_sel, S(stream)));
  }
  return SPIN_OK;
}

namespace {

// Resolve/evict; segments false leaves the segment-pool pass to the
// transfer launch that follows on the same stream (the one-launch step).
int resolve_impl(spin_ctx* ctx, const int32_t* d_sel, int32_t t, int32_t* d_block_table,
                 int32_t* d_block_ntok, int32_t* d_block_count, void* stream, bool segments) {
  if (!ctx || !d_sel || !d_block_table || !d_block_ntok || !d_block_count || t < 0) return SPIN_EINVAL;
  if (!ctx->dev.step_t) {  // a device-side step index is checked by nobody but its owner
    if (t < ctx->last_t) return SPIN_EINVAL;
    ctx->last_t = t;
  }
  // the previous step's transfer reads the insert lists this call rewrites
  HIPCHK(ctx, wait_fetched(ctx, S(stream)));
  HIPCHK(ctx, spin::launch_resolve(ctx->dev, d_sel, t, d_block_table, d_block_ntok, d_block_count,
                                   S(stream)));
  // The transfer needs only k_resolve's insert lists, but the segment-pool
  // pass is latency-bound and runs several times slower next to the PCIe
  // pulls (measured), so on its own stream it finishes before the transfer
  // starts; inside the one-launch transfer it runs in a workgroup of its own,
  // where its time is hidden.
  if (segments) HIPCHK(ctx, spin::launch_segments(ctx->dev, S(stream)));
  ctx->resolved_on = S(stream);
  ctx->resolved_any = true;
  ctx->resolved_recorded = false;
  return SPIN_OK;
}

int transfer_attend_impl(spin_ctx* ctx, const void* d_q, const int32_t* d_block_table,
                         const int32_t* d_block_ntok, const int32_t* d_block_count, void* stream,
                         bool segments) {
  if (!ctx || !d_q || !d_block_table || !d_block_ntok || !d_block_count) return SPIN_EINVAL;
  if (!aligned(d_q, 16)) return SPIN_EINVAL;
  HIPCHK(ctx, wait_resolved(ctx, S(stream)));
  const uint16_t* q = static_cast<const uint16_t*>(d_q);
  HIPCHK(ctx, spin::launch_transfer_attend(ctx->dev, q, d_block_table, d_block_ntok, d_block_count,
                                           segments, S(stream)));
  ctx->arrival = true;
  transfer_enqueued(ctx, S(stream));
  return SPIN_OK;
}

int attend_finish_impl(spin_ctx* ctx, const void* d_q, const int32_t* d_block_table,
                       const int32_t* d_block_ntok, const int32_t* d_block_count, float* d_out,
                       void* stream, int32_t* advance) {
  if (!ctx || !d_q || !d_block_table || !d_block_ntok || !d_block_count || !d_out) return SPIN_EINVAL;
  if (!aligned(d_q, 16) || !aligned(d_out, 16)) return SPIN_EINVAL;
  HIPCHK(ctx, wait_fetched(ctx, S(stream)));
  // pages attended on arrival need only the merge; otherwise attend them now
  HIPCHK(ctx, spin::launch_attend(ctx->dev, static_cast<const uint16_t*>(d_q), d_block_table,
                                  d_block_ntok, d_block_count, d_out,
                                  ctx->arrival ? spin::kAttendMergeArrival : spin::kAttendFetched,
                                  S(stream), ctx->arrival ? advance : nullptr));
  return SPIN_OK;
}

}  // namespace

SPIN_API int spin_resolve_evict(spin_ctx* ctx, const int32_t* d_sel, int32_t t,
                                int32_t* d_block_table, int32_t* d_block_ntok,
                                int32_t* d_block_count, void* stream) {
  return resolve_impl(ctx, d_sel, t, d_block_table, d_block_ntok, d_block_count, stream, true);
}

SPIN_API int spin_retrieve(spin_ctx* ctx, void* copy_stream) {
  if (!ctx) return SPIN_EINVAL;
  HIPCHK(ctx, wait_resolved(ctx, S(copy_stream)));
  HIPCHK(ctx, spin::launch_retrieve(ctx->dev, S(copy_stream)));
  ctx->arrival = false;
  transfer_enqueued(ctx, S(copy_stream));
  return SPIN_OK;
}

SPIN_API int spin_retrieve_attend(spin_ctx* ctx, const void* d_q, void* copy_stream) {
  if (!ctx || !d_q || !aligned(d_q, 16)) return SPIN_EINVAL;
  HIPCHK(ctx, wait_resolved(ctx, S(copy_stream)));
  HIPCHK(ctx, spin::launch_retrieve_attend(ctx->dev, static_cast<const uint16_t*>(d_q),
                                           S(copy_stream)));
  ctx->arrival = true;
  transfer_enqueued(ctx, S(copy_stream));
  return SPIN_OK;
}

SPIN_API int spin_transfer_attend(spin_ctx* ctx, const void* d_q, const int32_t* d_block_table,
                                  const int32_t* d_block_ntok, const int32_t* d_block_count,
                                  void* stream) {
  return transfer_attend_impl(ctx, d_q, d_block_table, d_block_ntok, d_block_count, stream, false);
}

SPIN_API int spin_attend(spin_ctx* ctx, const void* d_q, const int32_t* d_block_table,
                         const int32_t* d_block_ntok, const int32_t* d_block_count, float* d_out,
                         void* stream) {
  if (!ctx || !d_q || !d_block_table || !d_block_ntok || !d_block_count || !d_out) return SPIN_EINVAL;
  if (!aligned(d_q, 16) || !aligned(d_out, 16)) return SPIN_EINVAL;
  HIPCHK(ctx, wait_fetched(ctx, S(stream)));
  HIPCHK(ctx, spin::launch_attend(ctx->dev, static_cast<const uint16_t*>(d_q), d_block_table,
                                  d_block_ntok, d_block_count, d_out, spin::kAttendAll, S(stream)));
  return SPIN_OK;
}

SPIN_API int spin_attend_begin(spin_ctx* ctx, const void* d_q, const int32_t* d_block_table,
                               const int32_t* d_block_ntok, const int32_t* d_block_count,
                               void* stream) {
  if (!ctx || !d_q || !d_block_table || !d_block_ntok || !d_block_count) return SPIN_EINVAL;
  if (!aligned(d_q, 16)) return SPIN_EINVAL;
  HIPCHK(ctx, spin::launch_attend(ctx->dev, static_cast<const uint16_t*>(d_q), d_block_table,
                                  d_block_ntok, d_block_count, nullptr, spin::kAttendResident,
                                  S(stream)));
  return SPIN_OK;
}

SPIN_API int spin_attend_finish(spin_ctx* ctx, const void* d_q, const int32_t* d_block_table,
                                const int32_t* d_block_ntok, const int32_t* d_block_count,
                                float* d_out, void* stream) {
  return attend_finish_impl(ctx, d_q, d_block_table, d_block_ntok, d_block_count, d_out, stream,
                            nullptr);
}

namespace {

// One decode step.  Overlapped (copy_stream != stream), the transfer, with
// each fetched page attended on arrival, and the resident-page attention run
// in one launch on `stream`, which also takes the segment-pool pass; then the
// merge, which increments a non-null advance (the device-side step index),
// *advanced telling the caller so.  No second stream and no event inside the
// step: measured faster than the transfer on copy_stream beside the
// resident-page pass on `stream`, both with eager launches and as replays of
// a captured graph.  Otherwise retrieve, then attention, on `stream`.
int step_impl(spin_ctx* ctx, const void* d_q, int32_t t, int32_t* d_sel, int32_t* d_block_table,
              int32_t* d_block_ntok, int32_t* d_block_count, float* d_out, void* stream,
              void* copy_stream, int32_t* advance = nullptr, bool* advanced = nullptr) {
  const bool overlap = copy_stream != stream;
  int rc = spin_select(ctx, d_q, d_sel, nullptr, stream);
  if (!rc)
    rc = resolve_impl(ctx, d_sel, t, d_block_table, d_block_ntok, d_block_count, stream, !overlap);
  if (!overlap) {
    if (!rc) rc = spin_retrieve(ctx, stream);
    if (!rc) rc = spin_attend(ctx, d_q, d_block_table, d_block_ntok, d_block_count, d_out, stream);
    return rc;
  }
  // the arguments were all checked by the calls above, so the deferred
  // segment pass cannot be skipped by an argument error here
  if (!rc)
    rc = transfer_attend_impl(ctx, d_q, d_block_table, d_block_ntok, d_block_count, stream, true);
  if (!rc) {
    rc = attend_finish_impl(ctx, d_q, d_block_table, d_block_ntok, d_block_count, d_out, stream,
                            advance);
    if (!rc && advanced) *advanced = advance != nullptr;
  }
  return rc;
}

}  // namespace

SPIN_API int spin_step(spin_ctx* ctx, const void* d_q, int32_t t, int32_t* d_sel,
                       int32_t* d_block_table, int32_t* d_block_ntok, int32_t* d_block_count,
                       float* d_out, void* stream, void* copy_stream) {
  return step_impl(ctx, d_q, t, d_sel, d_block_table, d_block_ntok, d_block_count, d_out, stream,
                   copy_stream);
}

SPIN_API int spin_step_at(spin_ctx* ctx, const void* d_q_steps, int64_t q_step_elems,
                          int32_t* d_t, int32_t* d_sel, int32_t* d_block_table,
                          int32_t* d_block_ntok, int32_t* d_block_count, float* d_out,
                          void* stream, void* copy_stream) {
  if (!ctx || !d_q_steps || !d_t || q_step_elems < 0 || (q_step_elems * 2) % 16 != 0)
    return SPIN_EINVAL;
  if (!aligned(d_t, 4)) return SPIN_EINVAL;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  HIPCHK(ctx, hipStreamIsCapturing(S(stream), &cap));
  // a capture starts from an idle context: no transfer recorded before it is
  // waited for inside the graph (stream order between replays covers it), so
  // `stream` counts as having waited for the latest one
  if (cap == hipStreamCaptureStatusActive) {
    ctx->waited_on = S(stream);
    ctx->waited_gen = ctx->fetched_gen;
  }
  ctx->dev.step_t = d_t;
  ctx->dev.q_step = q_step_elems;
  bool advanced = false;
  int rc = step_impl(ctx, d_q_steps, 0, d_sel, d_block_table, d_block_ntok, d_block_count, d_out,
                     stream, copy_stream, d_t, &advanced);
  ctx->dev.step_t = nullptr;
  ctx->dev.q_step = 0;
  if (rc) return rc;
  if (!advanced) HIPCHK(ctx, spin::launch_step_advance(d_t, S(stream)));
  return SPIN_OK;
}

SPIN_API int spin_get_stats(spin_ctx* ctx, spin_stats* st, int64_t* per_request) {
  if (!ctx) return SPIN_EINVAL;
  const Dev& v = ctx->dev;
  HIPCHK(ctx, hipDeviceSynchronize());
  std::vector<long long> s(4 * (size_t)v.B);
  int top = 0, err = 0;
  unsigned long long h2d = 0;
  HIPCHK(ctx, hipMemcpy(s.data(), v.stats, s.size() * sizeof(long long), hipMemcpyDeviceToHost));
  HIPCHK(ctx, hipMemcpy(&h2d, v.h2d, sizeof(h2d), hipMemcpyDeviceToHost));
  HIPCHK(ctx, hipMemcpy(&top, v.seg_ctl, sizeof(int), hipMemcpyDeviceToHost));
  HIPCHK(ctx, hipMemcpy(&err, v.err, sizeof(int), hipMemcpyDeviceToHost));
  if (st) {
    std::memset(st, 0, sizeof(*st));
    for (int b = 0; b < v.B; ++b) {
      st->hits += s[4 * b];
      st->misses += s[4 * b + 1];
      st->evictions += s[4 * b + 2];
    }
    st->h2d_bytes = h2d;
    st->live_segments = v.n_seg - top;
    st->error_word = err;
  }
  if (per_request) std::memcpy(per_request, s.data(), s.size() * sizeof(long long));
  return SPIN_OK;
}

SPIN_API int spin_snapshot(spin_ctx* ctx, int32_t* directory, int32_t* segments, int32_t* seg_live,
                           int32_t* seg_stack, int32_t* seg_top, int32_t* owner, int32_t* last_use,
                           int32_t* free_count) {
  if (!ctx) return SPIN_EINVAL;
  const Dev& v = ctx->dev;
  HIPCHK(ctx, hipDeviceSynchronize());
  auto cp = [&](void* dst, const void* src, size_t n) -> hipError_t {
    return dst ? hipMemcpy(dst, src, n, hipMemcpyDeviceToHost) : hipSuccess;
  };
  HIPCHK(ctx, cp(directory, v.directory, (size_t)v.B * v.Hkv * v.ndir * sizeof(int)));
  const size_t seg_n = (size_t)v.n_seg * spin::kSegEntries * sizeof(int);
  if (ctx->h_segments && segments)
    std::memcpy(segments, ctx->h_segments, seg_n);
  else
    HIPCHK(ctx, cp(segments, v.segments, seg_n));
  HIPCHK(ctx, cp(seg_live, v.seg_live, (size_t)v.n_seg * sizeof(int)));
  HIPCHK(ctx, cp(seg_stack, v.seg_stack, (size_t)v.n_seg * sizeof(int)));
  HIPCHK(ctx, cp(seg_top, v.seg_ctl, sizeof(int)));
  HIPCHK(ctx, cp(owner, v.owner, (size_t)v.B * v.C * sizeof(int)));
  HIPCHK(ctx, cp(last_use, v.last_use, (size_t)v.B * v.C * sizeof(int)));
  HIPCHK(ctx, cp(free_count, v.free_count, (size_t)v.B * sizeof(int)));
  return SPIN_OK;
}

SPIN_API int spin_metadata_footprint(spin_ctx* ctx, spin_metadata* out) {
  if (!ctx || !out) return SPIN_EINVAL;
  const Dev& v = ctx->dev;
  HIPCHK(ctx, hipDeviceSynchronize());
  int top = 0;
  HIPCHK(ctx, hipMemcpy(&top, v.seg_ctl, sizeof(int), hipMemcpyDeviceToHost));
  const uint64_t seg_bytes = spin::kSegEntries * 4 + 4 + 4;
  std::memset(out, 0, sizeof(*out));
  out->directory_bytes = (uint64_t)v.B * v.Hkv * v.ndir * 4;
  if (ctx->h_segments) {
    out->host_segment_bytes = (uint64_t)v.n_seg * spin::kSegEntries * 4;
    out->segment_pool_bytes = (uint64_t)v.n_seg * 8;
  } else {
    out->segment_pool_bytes = (uint64_t)v.n_seg * seg_bytes;
  }
  out->live_segments = v.n_seg - top;
  out->num_segments = v.n_seg;
  out->live_segment_bytes = (uint64_t)out->live_segments * seg_bytes;
  out->reverse_map_bytes = (uint64_t)v.B * v.C * 8;
  out->flat_table_bytes = (uint64_t)v.B * v.Hkv * v.max_pages * 4;
  return SPIN_OK;
}

SPIN_API int spin_read_summaries(spin_ctx* ctx, int32_t req, float* host_out) {
  if (!ctx || !host_out || req < 0 || req >= ctx->cfg.max_batch) return SPIN_EINVAL;
  const Dev& v = ctx->dev;
  HIPCHK(ctx, hipDeviceSynchronize());
  int np = 0;
  HIPCHK(ctx, hipMemcpy(&np, v.req_parts + req, sizeof(int), hipMemcpyDeviceToHost));
  for (int h = 0; h < v.Hkv; ++h)
    HIPCHK(ctx, hipMemcpy(host_out + (size_t)h * np * spin::kHeadDim,
                          v.summaries + ((size_t)req * v.Hkv + h) * v.Nmax * spin::kHeadDim,
                          (size_t)np * spin::kHeadDim * sizeof(float), hipMemcpyDeviceToHost));
  return SPIN_OK;
}

SPIN_API int spin_sync_status(spin_ctx* ctx) {
  if (!ctx) return SPIN_EINVAL;
  HIPCHK(ctx, hipDeviceSynchronize());
  int err = 0;
  HIPCHK(ctx, hipMemcpy(&err, ctx->dev.err, sizeof(int), hipMemcpyDeviceToHost));
  if (err & SPIN_DEVERR_SEGPOOL) return SPIN_ESEGPOOL;
  if (err) return SPIN_EDEVICE;
  return SPIN_OK;
}

SPIN_API int spin_read_stream(const void* d_buf, size_t bytes, void* d_sink, void* stream) {
  if (!d_buf || !d_sink || bytes < 16 || !aligned(d_buf, 16)) return SPIN_EINVAL;
  if (spin::launch_read_stream(d_buf, bytes, static_cast<unsigned*>(d_sink), S(stream)) != hipSuccess)
    return SPIN_EHIP;
  return SPIN_OK;
}

SPIN_API const char* spin_strerror(int code) {
  switch (code) {
    case SPIN_OK: return "ok";
    case SPIN_EINVAL: return "invalid argument or configuration";
    case SPIN_ECAPACITY: return "slots per request below the pages one step can need";
    case SPIN_ESEGPOOL: return "second-level segment pool exhausted";
    case SPIN_EHIP: return "HIP runtime error";
    case SPIN_EDEVICE: return "device error word set";
    case SPIN_ESTATE: return "call made in the wrong state";
    case SPIN_ESCRATCH: return "input too large for the static scratch of spin_attend_noalloc";
    default: return "unknown error";
  }
}

SPIN_API int spin_last_hip_error(spin_ctx* ctx) { return ctx ? ctx->hip_err : 0; }

}  // extern "C"
