// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer over the library's host code (spin.cpp) and run
// on the CPU: every entry point that needs no GPU, with null and malformed
// arguments, the configurations of the five workloads, the edges of every
// field's range and seeded random configurations.  A context is created on
// host memory standing in for the workspace and the pool; the first kernel
// launch (or, with no GPU, the first HIP call) fails, and the failure path
// must free what it allocated.  Exit status 0 when every expectation holds
// and the sanitizers reported nothing (they abort the process otherwise).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "spin.h"

namespace {

int g_fail = 0;

void expect(bool ok, const char* what, long long detail = 0) {
  if (!ok) {
    std::fprintf(stderr, "FAIL: %s (%lld)\n", what, detail);
    ++g_fail;
  }
}

// splitmix64: the seeded stream of the random configurations
uint64_t g_state = 0x5EED5EED5EED5EEDull;
uint64_t next_u64() {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// A field value near one of the interesting points: small, the limits the
// header documents and one past them, the extremes of int32.
int32_t pick(int32_t lo, int32_t hi) {
  const uint64_t r = next_u64();
  switch (r % 8) {
    case 0: return lo;
    case 1: return hi;
    case 2: return lo - 1;
    case 3: return hi + 1;
    case 4: return (r >> 8) & 1 ? INT32_MAX : INT32_MIN;
    default: return lo + (int32_t)((r >> 16) % (uint64_t)((int64_t)hi - lo + 1));
  }
}

// a product of two fields, saturated to the int32 range
int32_t mul_sat(int32_t a, int32_t b) {
  const int64_t v = (int64_t)a * b;
  return v > INT32_MAX ? INT32_MAX : v < INT32_MIN ? INT32_MIN : (int32_t)v;
}

spin_config workload(int B, int Hq, int Hkv, int N, int pages, int ppp, int k, int C) {
  spin_config c;
  spin_config_init(&c);
  c.max_batch = B;
  c.num_q_heads = Hq;
  c.num_kv_heads = Hkv;
  c.max_partitions = N;
  c.max_pages = pages;
  c.max_pages_per_partition = ppp;
  c.topk = k;
  c.slots_per_request = C;
  const int ndir = (pages + 63) / 64;
  const long long a = (long long)B * C, b = (long long)B * Hkv * ndir;
  c.num_segments = (int32_t)(a < b ? a : b);
  return c;
}

// What a valid configuration must give: sizes that cover its arrays.
void check_sizes(const spin_config& c) {
  size_t ws = 0, pool = 0, hseg = 0;
  expect(spin_workspace_size(&c, &ws, &pool) == SPIN_OK, "workspace size of a valid config");
  expect(spin_host_segment_bytes(&c, &hseg) == SPIN_OK, "host segment bytes of a valid config");
  int32_t ndir = 0, mb = 0, splits = 0;
  expect(spin_derived(&c, &ndir, &mb, &splits) == SPIN_OK, "derived values of a valid config");
  expect(ndir == (c.max_pages + 63) / 64, "directory entries per head", ndir);
  expect(mb == c.topk * c.max_pages_per_partition, "block-table length", mb);
  expect(splits >= 1 && splits <= mb, "attention splits", splits);
  expect(pool == (size_t)c.max_batch * c.slots_per_request * 32768u, "pool bytes", (long long)pool);
  const size_t summaries = (size_t)c.max_batch * c.num_kv_heads * c.max_partitions * 128 * 4;
  expect(ws >= summaries, "workspace holds the summaries", (long long)ws);
  expect(hseg == (c.segments_in_host_memory ? (size_t)c.num_segments * 64 * 4 : 0), "host segment bytes",
         (long long)hseg);
}

void* aligned_block(size_t bytes) {
  void* p = std::aligned_alloc(256, (bytes + 255) / 256 * 256);
  if (p) std::memset(p, 0, bytes);
  return p;
}

// A context on host memory: rejected arguments first, then the real call,
// which fails at its first HIP call or kernel launch and must clean up.
void try_create(const spin_config& c) {
  size_t ws = 0, pool = 0, hseg = 0;
  if (spin_workspace_size(&c, &ws, &pool) != SPIN_OK) return;
  spin_host_segment_bytes(&c, &hseg);
  if (ws > ((size_t)64 << 20) || pool > ((size_t)256 << 20)) return;  // keep host memory small
  void* w = aligned_block(ws);
  void* p = aligned_block(pool);
  void* h = hseg ? aligned_block(hseg) : nullptr;
  expect(w && p && (!hseg || h), "host stand-in buffers");
  spin_ctx* ctx = reinterpret_cast<spin_ctx*>(0x1);
  expect(spin_create(&c, w, ws, p, pool, nullptr, nullptr) == SPIN_EINVAL, "create without out");
  expect(spin_create(&c, w, ws - 1, p, pool, nullptr, &ctx) == SPIN_EINVAL && ctx == nullptr,
         "workspace one byte short");
  expect(spin_create(&c, w, ws, p, pool - 1, nullptr, &ctx) == SPIN_EINVAL, "pool one byte short");
  expect(spin_create(&c, static_cast<char*>(w) + 16, ws, p, pool, nullptr, &ctx) == SPIN_EINVAL,
         "unaligned workspace");
  expect(spin_create(&c, nullptr, ws, p, pool, nullptr, &ctx) == SPIN_EINVAL, "null workspace");
  if (!c.segments_in_host_memory) {
    int32_t dummy[64];
    expect(spin_create_ex(&c, w, ws, p, pool, dummy, sizeof dummy, nullptr, &ctx) == SPIN_EINVAL,
           "host segments passed without the flag");
    const int rc = spin_create(&c, w, ws, p, pool, nullptr, &ctx);
    expect(rc == SPIN_EHIP && ctx == nullptr, "create fails at its first HIP call, nothing returned", rc);
  } else {
    expect(spin_create_ex(&c, w, ws, p, pool, h, hseg - 1, nullptr, &ctx) == SPIN_EINVAL,
           "host segment buffer one byte short");
    const int rc = spin_create_ex(&c, w, ws, p, pool, h, hseg, nullptr, &ctx);
    // host memory that was not allocated pinned has no device address
    expect((rc == SPIN_EINVAL || rc == SPIN_EHIP) && ctx == nullptr, "host-segment create fails", rc);
  }
  std::free(h);
  std::free(p);
  std::free(w);
}

void null_context_calls() {
  spin_stats st;
  spin_metadata md;
  int32_t i32[4] = {0, 0, 0, 0};
  float f32[4] = {0, 0, 0, 0};
  expect(spin_destroy(nullptr) == SPIN_EINVAL, "destroy(null)");
  expect(spin_release(nullptr, 0, nullptr) == SPIN_EINVAL, "release(null)");
  expect(spin_set_budget(nullptr, 0, 1, nullptr) == SPIN_EINVAL, "set_budget(null)");
  expect(spin_index(nullptr, 0, i32, 64, nullptr, 0, nullptr) == SPIN_EINVAL, "index(null)");
  expect(spin_offload(nullptr, 0, i32, i32, 16, 64, nullptr, 0, nullptr) == SPIN_EINVAL, "offload(null)");
  expect(spin_append(nullptr, i32, i32, nullptr) == SPIN_EINVAL, "append(null)");
  expect(spin_select(nullptr, i32, i32, f32, nullptr) == SPIN_EINVAL, "select(null)");
  expect(spin_resolve_evict(nullptr, i32, 0, i32, i32, i32, nullptr) == SPIN_EINVAL, "resolve(null)");
  expect(spin_retrieve(nullptr, nullptr) == SPIN_EINVAL, "retrieve(null)");
  expect(spin_retrieve_attend(nullptr, i32, nullptr) == SPIN_EINVAL, "retrieve_attend(null)");
  expect(spin_transfer_attend(nullptr, i32, i32, i32, i32, nullptr) == SPIN_EINVAL, "transfer_attend(null)");
  expect(spin_attend(nullptr, i32, i32, i32, i32, f32, nullptr) == SPIN_EINVAL, "attend(null)");
  expect(spin_attend_begin(nullptr, i32, i32, i32, i32, nullptr) == SPIN_EINVAL, "attend_begin(null)");
  expect(spin_attend_finish(nullptr, i32, i32, i32, i32, f32, nullptr) == SPIN_EINVAL, "attend_finish(null)");
  expect(spin_step(nullptr, i32, 0, i32, i32, i32, i32, f32, nullptr, nullptr) == SPIN_EINVAL, "step(null)");
  expect(spin_step_at(nullptr, i32, 128, i32, i32, i32, i32, i32, f32, nullptr, nullptr) == SPIN_EINVAL,
         "step_at(null)");
  expect(spin_get_stats(nullptr, &st, nullptr) == SPIN_EINVAL, "get_stats(null)");
  expect(spin_snapshot(nullptr, i32, i32, i32, i32, i32, i32, i32, i32) == SPIN_EINVAL, "snapshot(null)");
  expect(spin_metadata_footprint(nullptr, &md) == SPIN_EINVAL, "metadata_footprint(null)");
  expect(spin_read_summaries(nullptr, 0, f32) == SPIN_EINVAL, "read_summaries(null)");
  expect(spin_sync_status(nullptr) == SPIN_EINVAL, "sync_status(null)");
  expect(spin_last_hip_error(nullptr) == 0, "last_hip_error(null)");
  expect(spin_read_stream(nullptr, 16, nullptr, nullptr) == SPIN_EINVAL, "read_stream(null)");
}

}  // namespace

int main() {
  // every code has a message
  for (int c = -64; c <= 64; ++c) {
    const char* s = spin_strerror(c);
    expect(s != nullptr && std::strlen(s) > 0, "strerror", c);
  }
  expect(spin_config_init(nullptr) == SPIN_EINVAL, "config_init(null)");
  expect(spin_config_check(nullptr) == SPIN_EINVAL, "config_check(null)");
  expect(spin_workspace_size(nullptr, nullptr, nullptr) == SPIN_EINVAL, "workspace_size(null)");
  null_context_calls();

  // the five workloads' shapes (1M context: 7.7K variable partitions of up to
  // four pages), their host-segment forms, and automatic and fixed splits
  std::vector<spin_config> valid = {
      workload(1, 8, 2, 64, 64, 1, 8, 96),
      workload(16, 40, 8, 512, 512, 1, 32, 1536),
      workload(8, 64, 8, 2048, 2048, 1, 64, 3072),
      workload(32, 64, 8, 2048, 2048, 1, 64, 768),
      workload(4, 32, 8, 8192, 16384, 4, 128, 24576),
  };
  for (size_t i = 0, n = valid.size(); i < n; ++i) {
    spin_config h = valid[i];
    h.segments_in_host_memory = 1;
    valid.push_back(h);
    spin_config s = valid[i];
    s.attend_pages_per_split = 256;
    valid.push_back(s);
  }
  for (const spin_config& c : valid) {
    expect(spin_config_check(&c) == SPIN_OK, "workload config is valid", c.max_batch);
    check_sizes(c);
  }
  for (const spin_config& c : valid) try_create(c);

  // seeded random configurations around every field's limits: whatever the
  // check says, the sizes of an accepted one must hold and nothing may
  // overflow on the way
  int accepted = 0;
  for (int it = 0; it < 200000; ++it) {
    spin_config c;
    spin_config_init(&c);
    c.max_batch = pick(1, 1024);
    c.num_kv_heads = pick(1, 16);
    c.num_q_heads = (next_u64() & 3) ? mul_sat(c.num_kv_heads, pick(1, 16)) : pick(1, 256);
    c.head_dim = (next_u64() % 16) ? 128 : pick(64, 256);
    c.page_tokens = (next_u64() % 16) ? 64 : pick(32, 128);
    c.max_partitions = pick(1, 16384);
    c.max_pages_per_partition = pick(1, 4);
    c.max_pages = (next_u64() & 1) ? mul_sat(c.max_partitions, c.max_pages_per_partition) : pick(1, 65536);
    c.topk = pick(1, 1024);
    c.slots_per_request = pick(1, 65536);
    c.num_segments = pick(1, 1 << 28);
    c.seg_entries = (next_u64() % 16) ? 64 : pick(32, 128);
    c.num_buckets = (next_u64() % 16) ? 64 : pick(32, 128);
    c.attend_pages_per_split = pick(0, 256);
    c.segments_in_host_memory = pick(0, 1);
    const int rc = spin_config_check(&c);
    expect(rc == SPIN_OK || rc == SPIN_EINVAL || rc == SPIN_ECAPACITY, "check returns a known code", rc);
    size_t ws = 0, pool = 0;
    const int rw = spin_workspace_size(&c, &ws, &pool);
    expect(rw == rc, "workspace_size agrees with check", rw);
    if (rc == SPIN_OK) {
      ++accepted;
      check_sizes(c);
      if (accepted % 4000 == 1) try_create(c);
    }
  }
  expect(accepted > 100, "some random configurations are accepted", accepted);
  std::printf("host ABI checks: %d failures, %d random configurations accepted\n", g_fail, accepted);
  return g_fail ? 1 : 0;
}
