// Attention with no context and no workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that
// forbid hipMalloc): the paged sparse GQA decode of spin_attend, whose split
// partials (the only scratch its kernels use) live in a static device array
// instead of a caller-provided workspace.
//
// The array is one per GPU, held until the process ends.  Its device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) on the entry point's first call there and kept; the array's name
// itself is only a host-side stand-in and is never passed to a kernel.  Every
// call on a GPU shares that GPU's array: calls that overlap in time on one
// GPU race on it.  The per-head counters of the split merge start at zero
// (cleared on the first call) and every call leaves them at zero; the
// partials are written before the same call reads them.
#include <hip/hip_runtime.h>

#include <mutex>

#include "spin.h"
#include "spin_internal.h"

// spin_attend_noalloc's scratch: the per-head counters of the split merge
// (kCounterBytes: one int per (request, KV head) of the largest batch), then
// the split partials (part_o, then part_ml)
static __device__ __align__(256) unsigned char scratch[SPIN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kCounterBytes = 1024 * spin::kMaxKvHeads * sizeof(int);
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device

// The counters start at zero, and every launch leaves them at zero (the
// head's last split resets its own); they are cleared once, by a kernel on
// the first call's stream, before the first attention that counts on them.
__global__ void k_clear_counters(int* c, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) c[i] = 0;
}

// The current device's copy of the array (looked up, and its counters
// cleared on `s`, on first use there).
hipError_t scratch_on_current_device(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    const int n = (int)(kCounterBytes / sizeof(int));
    hipLaunchKernelGGL(k_clear_counters, dim3(16), dim3(256), 0, s, static_cast<int*>(p), n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" SPIN_API int spin_attend_noalloc(const void* d_q, const void* d_pool, int64_t pool_pages,
                                            const int32_t* d_block_table, const int32_t* d_block_ntok,
                                            const int32_t* d_block_count, float* d_out,
                                            int32_t batch, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t max_blocks,
                                            int32_t pages_per_split, void* stream) {
  if (!d_q || !d_pool || !d_block_table || !d_block_ntok || !d_block_count || !d_out)
    return SPIN_EINVAL;
  if (!aligned16(d_q) || !aligned16(d_out) || !aligned16(d_pool)) return SPIN_EINVAL;
  if (batch < 1 || batch > 1024 || num_kv_heads < 1 || num_kv_heads > spin::kMaxKvHeads)
    return SPIN_EINVAL;
  if (num_q_heads < num_kv_heads || num_q_heads % num_kv_heads ||
      num_q_heads / num_kv_heads > spin::kMaxGroup)
    return SPIN_EINVAL;
  if (max_blocks < 1 || max_blocks > 1024 * spin::kMaxPPP) return SPIN_EINVAL;
  if (pages_per_split < 0 || pages_per_split > 256) return SPIN_EINVAL;
  if (pool_pages < 1 || pool_pages > 0x7fffffffLL) return SPIN_EINVAL;
  const int G = num_q_heads / num_kv_heads;
  const int pps = spin::whole_table_pages_per_split(
      (long long)batch * num_kv_heads * max_blocks, pages_per_split);
  const int splits = (max_blocks + pps - 1) / pps;
  // the partials, laid out as in a context's workspace: [B * Hkv][2 * splits][G]
  // rows of 128 floats, then their (max, sum) pairs, after the counters; a
  // single split per head needs none
  const size_t rows = (size_t)batch * num_kv_heads * 2 * splits * G;
  const size_t o_bytes = rows * spin::kHeadDim * sizeof(float);
  const size_t need = splits > 1 ? kCounterBytes + o_bytes + rows * 2 * sizeof(float) : 0;
  if (need > SPIN_NOALLOC_SCRATCH_BYTES) return SPIN_ESCRATCH;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* base = nullptr;
  if (scratch_on_current_device(s, &base) != hipSuccess) return SPIN_EHIP;
  spin::Dev d{};
  d.B = batch;
  d.Hq = num_q_heads;
  d.Hkv = num_kv_heads;
  d.G = G;
  d.max_blocks = max_blocks;
  d.pps = pps;
  d.splits = splits;
  d.pps_res = pps;
  d.splits_res = splits;
  d.pool_slots = (int)pool_pages;
  d.pool = static_cast<uint16_t*>(const_cast<void*>(d_pool));
  d.att_arrive = static_cast<int*>(base);
  d.part_o = reinterpret_cast<float*>(static_cast<char*>(base) + kCounterBytes);
  d.part_ml = reinterpret_cast<float*>(static_cast<char*>(base) + kCounterBytes + o_bytes);
  d.step_t = nullptr;
  d.q_step = 0;
  if (spin::launch_attend(d, static_cast<const uint16_t*>(d_q), d_block_table, d_block_ntok,
                          d_block_count, d_out, spin::kAttendAll, s) != hipSuccess)
    return SPIN_EHIP;
  return SPIN_OK;
}
