// Internal declarations shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spin {

constexpr int kHeadDim = 128;
constexpr int kPageTokens = 64;
constexpr int kPageElems = 2 * kPageTokens * kHeadDim;  // bf16 elements per page
constexpr int kPageBytes = kPageElems * 2;               // 32 KiB
constexpr int kSegEntries = 64;
constexpr int kBuckets = 64;
constexpr int kMaxPartitions = 16384;
constexpr int kMaxSlots = 65536;
constexpr int kMaxItems = 4096;        // Hkv * topk, mandatory partitions of one request
constexpr int kMaxPPP = 4;             // pages per partition
constexpr int kMaxGroup = 16;          // query heads per KV head
constexpr int kMaxKvHeads = 16;
constexpr int kRetrieveWG = 256;       // threads of a transfer workgroup
constexpr int kRetrieveGrid = 64;      // transfer workgroups (see retrieve.hip)

// device error-word bits (kept equal to the SPIN_DEVERR_* values of spin.h)
constexpr int kErrPartition = 1;       // selected partition id out of range
constexpr int kErrSegPool = 2;         // no free second-level segment
constexpr int kErrState = 4;           // residency state inconsistent
constexpr int kErrStep = 8;            // decode step below the last resolved one

// Device-visible view of the workspace, passed by value to kernels.
struct Dev {
  // geometry
  int B, Hq, Hkv, G, k, Nmax, max_pages, max_ppp, C, n_seg, ndir, max_blocks, max_mand;
  int splits, pps;             // attention over the whole block table: splits per head, pages per split
  int splits_res, pps_res;     // the resident-page pass beside the transfer (fewer, longer splits)
  int pool_slots;              // pages the pool holds (B * C)
  // index tables (written by spin_index)
  float* summaries;            // [B][Hkv][Nmax][128]
  int* part_first;             // [B][Nmax] first page of partition
  int* part_len;               // [B][Nmax] tokens
  int* req_parts;              // [B]
  int* req_pages;              // [B] pages per KV head
  int* req_stride;             // [B] pages reserved per KV head in the host buffer
  double* tail_sum;            // [B][Hkv][128] key sum of each request's last partition
  unsigned long long* host_base;  // [B] device-mapped address of the host KV
  // residency state
  int* directory;              // [B][Hkv][ndir] segment id or -1
  int* segments;               // [n_seg][64] request-local slot or -1
  int* seg_live;               // [n_seg]
  int* seg_stack;              // [n_seg]
  int* seg_ctl;                // [0] = stack top
  int* owner;                  // [B][C] h * max_pages + page, or -1
  int* last_use;               // [B][C]
  int* free_count;             // [B]
  int* budget;                 // [B] cap on resident pages (<= C)
  int* last_t;                 // [B] step of the request's last resolve (-1: none)
  // per-step scratch
  float* scores;               // [B][Hkv][Nmax]
  int* arrive;                 // [B][Hkv] workgroups of the list done scoring (0 between launches)
  float* srange;               // [B][Hkv][kSplitRangeSlots][2] each scoring wave's (min, max) score
  int4* miss_tmp;              // [B][max_mand] (h, page, block position, valid tokens)
  int4* ins;                   // [B][max_mand] (slot, h, page, 0)
  int* nmiss;                  // [B]
  int* freed;                  // [B][Hkv * ndir]
  int* nfreed;                 // [B]
  int* alloc;                  // [B][Hkv * ndir] directory entries that need a segment
  int* nalloc;                 // [B]
  unsigned char* bmiss;        // [B][Hkv][max_blocks] 1 = block fetched by this step's retrieve
  int* att_arrive;             // [B][Hkv] splits of the whole-table pass done (0 between launches)
  float* part_o;               // [B * Hkv][2 * splits][G][128]
  float* part_ml;              // [B * Hkv][2 * splits][G][2] (max in log2 units, sum)
  // attention of each fetched page on arrival, indexed by its place in the
  // batch's insert lists (requests ascending, canonical order)
  float* arr_o;                // [B * max_mand][G][128] unnormalised
  float* arr_ml;               // [B * max_mand][G][2]
  int* head_moff;              // [B][Hkv + 1] first insert-list index of each head; [Hkv] = count
  long long* stats;            // [B][4] hits, misses, evictions, last cutoff
  unsigned long long* h2d;     // [1] bytes the transfers read over the link, cumulative
  int* err;                    // [1] error bits
  uint16_t* pool;              // [B * C][kPageElems]
  // Device-side step index (spin_step_at): when set, kernels take the step t
  // from *step_t and the step's queries at q + t * q_step instead of their
  // host arguments, so one captured step replays for consecutive steps.
  const int* step_t;
  long long q_step;            // elements between consecutive steps' queries
};

// Pages per split of the whole-table attention pass: pages_per_split rounded
// up to whole pages per wave, or (0) about one workgroup per CU over `work`,
// the worst-case page count of the batch (B * Hkv * max_blocks).
int whole_table_pages_per_split(long long work, int pages_per_split);

// launchers (each returns the hipError_t of its launch)
// The queries of this step: q itself, or q + t * q_step with a device-side step index.
__device__ __forceinline__ const uint16_t* step_queries(const Dev& d, const uint16_t* q) {
  return d.step_t ? q + (long long)(*d.step_t) * d.q_step : q;
}

hipError_t launch_init(const Dev& d, hipStream_t s);
hipError_t launch_release(const Dev& d, int req, hipStream_t s);
hipError_t launch_set_budget(const Dev& d, int req, int slots, hipStream_t s);
hipError_t launch_index(const Dev& d, int req, int n_parts, const void* src, int src_stride,
                        hipStream_t s);
hipError_t launch_append(const Dev& d, const uint16_t* k, const uint16_t* v, hipStream_t s);
hipError_t launch_score(const Dev& d, const uint16_t* q, float* scores, hipStream_t s);
hipError_t launch_topk(const Dev& d, const float* scores, int* sel, hipStream_t s);
// smaller batches with lists of at most this many partitions score and
// select in one launch, several workgroups per list (measured: faster up to
// 2048-partition lists, slower at 7.7K, where the last workgroup's top-k
// tail outweighs the launch it saves)
constexpr int kSplitSelectMaxParts = 4096;
// one (min, max) per wave of every workgroup of a list: 512-partition
// workgroups of 16 waves over at most kSplitSelectMaxParts partitions
constexpr int kSplitRangeSlots = kSplitSelectMaxParts / 512 * 16;
hipError_t launch_select_split(const Dev& d, const uint16_t* q, float* scores, int* sel,
                               hipStream_t s);
hipError_t launch_select_fused(const Dev& d, const uint16_t* q, float* scores, int* sel,
                               hipStream_t s);
// batches of at least this many (request, KV head) lists score and select in
// one kernel, one workgroup per list (enough workgroups to stream HBM)
constexpr int kFusedSelectMinLists = 128;
hipError_t launch_resolve(const Dev& d, const int* sel, int t, int* bt, int* bntok, int* bcount,
                          hipStream_t s);
// the segment-pool pass; large batches write the inserts in a second launch
hipError_t launch_segments(const Dev& d, hipStream_t s);
hipError_t launch_step_advance(int* t, hipStream_t s);
hipError_t launch_retrieve(const Dev& d, hipStream_t s);
hipError_t launch_retrieve_attend(const Dev& d, const uint16_t* q, hipStream_t s);
// the transfer with attention on arrival and the resident-page attention pass
// in one launch (kRetrieveGrid transfer workgroups, then the attention grid);
// with segments, one more workgroup runs the segment-pool pass and the
// inserts
hipError_t launch_transfer_attend(const Dev& d, const uint16_t* q, const int* bt, const int* bntok,
                                  const int* bcount, bool segments, hipStream_t s);
hipError_t launch_read_stream(const void* buf, size_t bytes, unsigned* sink, hipStream_t s);
// mode 0: every block, finished output; 1: resident blocks only, partials;
// 2: fetched blocks only, partials, then the merge of both passes;
// 3: no attention, only the merge of the resident-block partials with the
// fetched pages attended on arrival (launch_retrieve_attend); in that mode a
// non-null advance is incremented once the kernel is done with the step
// (nothing in it reads the device-side step index)
enum AttendMode { kAttendAll = 0, kAttendResident = 1, kAttendFetched = 2, kAttendMergeArrival = 3 };
hipError_t launch_attend(const Dev& d, const uint16_t* q, const int* bt, const int* bntok,
                         const int* bcount, float* out, int mode, hipStream_t s,
                         int* advance = nullptr);

}  // namespace spin
