/*
 * spin.h -- C ABI of the MI355X sparse-decode library (libspin.so).
 *
 * One decode step of one attention layer over a KV cache split into
 * partitions, following the five-operation pipeline of "Unifying Sparse
 * Attention with Hierarchical Memory for Scalable Long-Context LLM Serving"
 * (SPIN).  Page citations below:
 *   [XT] the m.x-techcon.com article on the paper ("吞吐量提升5.66倍！…Spin框架…"),
 *        design section "Spin的核心设计：从抽象到高效管理", parts 1 (partition
 *        abstraction, Fig. 3), 2 (locality-aware KV management, Fig. 5) and
 *        3 (hierarchical metadata, Fig. 6);
 *   [GP] the gist.science/pt summary, "2. Metodologia" parts A, B, C.
 *
 * Index, Select and Attention are the algorithm's operations; Offload and
 * Retrieve move data between host memory and the GPU ([XT] part 1, Fig. 3;
 * [GP] A).  Here the full KV of a request stays in pinned host memory (the
 * offloaded copy); the GPU holds a per-request pool of page slots.
 *
 * ---------------------------------------------------------------- layouts
 * bf16 values are passed as their 16-bit patterns.
 *   page     64 token slots of one KV head, 32768 bytes:
 *            keys   [64 tokens][128 dims] bf16, token-major, then
 *            values [128 dims][64 tokens] bf16, dim-major (transposed).
 *            Slots past a partition's last token are ignored and may hold
 *            anything in host memory: a transfer reads the key rows of the
 *            valid tokens and the whole value half, and the pool slot gets
 *            zeros in every key and value entry of the other token slots.
 *   host KV  one pinned, device-mapped buffer per request:
 *            [Hkv][pages][page]; partition i of every head starts on page
 *            sum_{j<i} ceil(len_j / 64) ([GP] B: physical pages per head).
 *   pool     device, [max_batch * slots_per_request][page]; request b owns
 *            global slots b*C .. b*C + C - 1 (C = slots_per_request).
 *   q        device, [max_batch][Hq][128] bf16; query head g uses KV head
 *            g / (Hq / Hkv).
 *   sel      device, [max_batch][Hkv][topk] int32, ascending partition ids,
 *            -1 padding when a head has fewer than topk partitions.
 *   block    device tables written by spin_resolve_evict:
 *            table [max_batch][Hkv][max_blocks] int32 global pool slot,
 *            ntok  [max_batch][Hkv][max_blocks] int32 valid tokens of the page,
 *            count [max_batch][Hkv] int32 pages of the head.  Entries are in
 *            canonical order (partition ascending, page ascending); entries
 *            past count hold -1 / 0.  max_blocks = topk * max_pages_per_partition.
 *   out      device, [max_batch][Hq][128] float32.
 *
 * ---------------------------------------------------------------- contract
 * Every call returns SPIN_OK (0) or a negative code.  Device pointers must be
 * 256-byte aligned (workspace, pool) or 16-byte aligned (q, out), and must
 * outlive the context.  The caller owns all device memory (workspace, pool,
 * inputs, outputs) and the pinned host KV; the library allocates no device
 * memory.  Enqueue calls (select / resolve_evict / retrieve / attend / step)
 * are asynchronous and stream-ordered; spin_index, spin_release, spin_create,
 * spin_get_stats, spin_snapshot, spin_read_summaries and spin_sync_status
 * synchronise.  Errors a kernel detects (a partition id out of range, an
 * exhausted segment pool) set a device error word that the next synchronising
 * call reports as SPIN_EDEVICE (SPIN_ESEGPOOL for an exhausted pool); the
 * residency state is then undefined until the requests are indexed again,
 * except after SPIN_DEVERR_STEP alone (see spin_resolve_evict).  A context
 * is not thread-safe; use one per (compute stream, copy stream) pair.
 * Streams are hipStream_t values passed as void* (NULL = the null stream).
 * resolve_evict, attention and every call that changes a request (index,
 * offload, append, release) wait for the latest transfer (spin_retrieve,
 * spin_retrieve_attend or spin_transfer_attend); the context records an
 * event only when another stream has to wait, remembers which stream already
 * waited for that transfer and does not wait there twice, so a stream given
 * to a context must not be destroyed (and its handle reused) before the
 * context is.
 */
#ifndef SPIN_H
#define SPIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPIN_API __attribute__((visibility("default")))

#define SPIN_OK 0
#define SPIN_EINVAL (-1)     /* bad argument or configuration */
#define SPIN_ECAPACITY (-2)  /* budget smaller than one step's mandatory pages */
#define SPIN_ESEGPOOL (-3)   /* device reported an exhausted segment pool */
#define SPIN_EHIP (-4)       /* a HIP runtime call failed; see spin_last_hip_error */
#define SPIN_EDEVICE (-5)    /* device error word set (see spin_get_stats) */
#define SPIN_ESTATE (-6)     /* call made in the wrong state (e.g. unindexed request) */
#define SPIN_ESCRATCH (-7)   /* input too large for spin_attend_noalloc's static scratch */

/* Size of the static device array that holds spin_attend_noalloc's scratch
 * (one per GPU the library runs on, held until the process ends). */
#define SPIN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* device error-word bits */
#define SPIN_DEVERR_PARTITION 1   /* a selected partition id is out of range */
#define SPIN_DEVERR_SEGPOOL 2     /* no free second-level segment for an insert */
#define SPIN_DEVERR_STATE 4       /* residency state found inconsistent */
#define SPIN_DEVERR_STEP 8        /* a resolve's step index was below the last resolved
                                     step; that resolve changed nothing */

typedef struct spin_ctx spin_ctx;

typedef struct spin_config {
  int32_t max_batch;               /* requests (B), >= 1 */
  int32_t num_q_heads;             /* Hq, a multiple of Hkv, Hq / Hkv <= 16 */
  int32_t num_kv_heads;            /* Hkv, 1..16 */
  int32_t head_dim;                /* must be 128 */
  int32_t page_tokens;             /* must be 64 */
  int32_t max_partitions;          /* per (request, KV head), 1..16384 */
  int32_t max_pages;               /* per (request, KV head) */
  int32_t max_pages_per_partition; /* 1..4 (a partition is at most 256 tokens) */
  int32_t topk;                    /* partitions selected per KV head, 1..1024 */
  int32_t slots_per_request;       /* C: GPU page slots of one request, <= 65536 */
  int32_t num_segments;            /* second-level segments in the shared pool */
  int32_t seg_entries;             /* must be 64 */
  int32_t num_buckets;             /* must be 64 */
  int32_t attend_pages_per_split;  /* attention split size in pages; 0 = automatic */
  int32_t segments_in_host_memory; /* 0: segments in the GPU workspace; 1: the segment
                                      tables in caller-provided pinned host memory
                                      (spin_create_ex) */
} spin_config;

typedef struct spin_stats {
  uint64_t hits;           /* mandatory pages found resident, summed over steps */
  uint64_t misses;         /* mandatory pages fetched from host memory */
  uint64_t evictions;      /* pages reclaimed by the bucketed LRU */
  uint64_t h2d_bytes;      /* bytes the transfers read from host memory: per fetched
                              page 256 per valid token's key row + 16384 of values
                              (32768 for a full page); replays count again */
  int32_t live_segments;   /* segments linked into the directory now */
  int32_t error_word;      /* SPIN_DEVERR_* bits */
} spin_stats;

typedef struct spin_metadata {
  uint64_t directory_bytes;     /* static top-level directory, GPU */
  uint64_t segment_pool_bytes;  /* pre-allocated shared pool of second-level segments, GPU */
  uint64_t live_segment_bytes;  /* the segments linked into the directory now */
  uint64_t reverse_map_bytes;   /* owner + last_use per slot: scales with the GPU buffer */
  uint64_t flat_table_bytes;    /* one flat entry per (request, KV head, page) instead */
  int32_t live_segments;
  int32_t num_segments;
  uint64_t host_segment_bytes;  /* segment tables held in host memory (0 unless
                                   segments_in_host_memory); segment_pool_bytes
                                   then counts only the GPU part (live counts, stack) */
} spin_metadata;

/* Fill *cfg with the fixed geometry (head_dim 128, page_tokens 64,
 * seg_entries 64, num_buckets 64) and zeros elsewhere. */
SPIN_API int spin_config_init(spin_config* cfg);

/* Check a configuration.  SPIN_ECAPACITY when slots_per_request is below
 * Hkv * topk * max_pages_per_partition, the most pages one step can need
 * ([XT] part 2: the mandatory pages of a step must fit in the request's GPU
 * area), SPIN_EINVAL for other violations. */
SPIN_API int spin_config_check(const spin_config* cfg);

/* Bytes of device workspace and of the page pool the caller must provide. */
SPIN_API int spin_workspace_size(const spin_config* cfg, size_t* ws_bytes, size_t* pool_bytes);

/* Bytes of pinned host memory spin_create_ex needs for the segment tables
 * (num_segments * 64 * 4 when segments_in_host_memory, else 0). */
SPIN_API int spin_host_segment_bytes(const spin_config* cfg, size_t* bytes);

/* Derived sizes: directory entries per (request, head) = ceil(max_pages/64),
 * max_blocks = topk * max_pages_per_partition, and attention splits per head
 * of the whole-table pass (spin_attend).  When attend_pages_per_split is 0,
 * the resident-page pass of the overlapped forms (spin_attend_begin,
 * spin_transfer_attend, spin_step) may take fewer, longer splits; the
 * partial buffers are sized for the whole-table count, never exceeded. */
SPIN_API int spin_derived(const spin_config* cfg, int32_t* ndir, int32_t* max_blocks,
                          int32_t* attend_splits);

/* Create a context over caller-owned device memory and reset all state
 * (every slot free, every directory entry empty, all segments on the free
 * stack).  Synchronises `stream`. */
SPIN_API int spin_create(const spin_config* cfg, void* d_workspace, size_t ws_bytes,
                         void* d_pool, size_t pool_bytes, void* stream, spin_ctx** out);

/* spin_create with the second-level segment tables in host memory (the tier
 * split of the hierarchical metadata in [GP] C, where the second level sits
 * in host memory; [XT] part 3 keeps it on the GPU, which spin_create does).
 * h_segments: pinned host memory (hipHostMalloc or a pinned torch tensor) of
 * at least spin_host_segment_bytes() bytes, owned by the caller, outliving
 * the context; the kernels read and write it through its device-mapped
 * address.  The directory, the segments' live counts and the free stack stay
 * in the workspace.  cfg->segments_in_host_memory must be 1 (and h_segments
 * NULL when it is 0, which makes this spin_create).  Same results as
 * spin_create, bit for bit. */
SPIN_API int spin_create_ex(const spin_config* cfg, void* d_workspace, size_t ws_bytes,
                            void* d_pool, size_t pool_bytes, void* h_segments,
                            size_t h_segment_bytes, void* stream, spin_ctx** out);

/* Waits for the latest transfer, then frees the context (not the caller's
 * memory). */
SPIN_API int spin_destroy(spin_ctx* ctx);

/* Index + Offload registration of request `req` ([XT] part 1, Fig. 3; [GP] A).
 * h_kv: the request's pinned host KV in the host layout above (it must come
 * from hipHostMalloc / a pinned torch tensor; its device-mapped address is
 * taken with hipHostGetDevicePointer).  part_lens: host array of n_parts
 * partition lengths in tokens (1..64*max_pages_per_partition), or NULL for
 * fixed 64-token partitions covering n_tokens (the last one may be shorter).
 * Releases whatever the request held, records its CPU page table (host base
 * address, partition -> first page, lengths) and writes its partition
 * summaries: the mean key over each partition's tokens, accumulated in
 * float64 and rounded to float32.  Synchronises `stream`. */
SPIN_API int spin_index(spin_ctx* ctx, int32_t req, const void* h_kv, int64_t n_tokens,
                        const int32_t* part_lens, int32_t n_parts, void* stream);

/* Buffer elasticity ([XT] part 2; [GP] B): set request `req`'s budget, the
 * most pages it may keep resident, between Hkv * topk *
 * max_pages_per_partition (SPIN_ECAPACITY below) and slots_per_request
 * (SPIN_EINVAL above).  Stream-ordered; nothing is evicted at once: the next
 * spin_resolve_evict reclaims the excess with the bucketed LRU (its shortfall
 * is resident + misses - budget).  spin_index / spin_release reset the budget
 * to slots_per_request. */
SPIN_API int spin_set_budget(spin_ctx* ctx, int32_t req, int32_t slots, void* stream);

/* Prefill side ([XT] part 1, Fig. 3: Index, then Offload of the KV to CPU
 * memory).  d_kv: the request's freshly computed KV in device memory,
 * [Hkv][pages][page] (pages from n_tokens / part_lens as in spin_index).
 * h_kv: a pinned host buffer of h_kv_bytes; it reserves h_kv_bytes / (Hkv *
 * 32768) pages per KV head (room for spin_append; SPIN_ECAPACITY if that is
 * below the request's pages), laid out [Hkv][reserved][page].  Copies each
 * head's pages to its run in h_kv and builds the summaries from the device
 * copy, then registers the request as spin_index does.  Synchronises. */
SPIN_API int spin_offload(spin_ctx* ctx, int32_t req, const void* d_kv, void* h_kv,
                          size_t h_kv_bytes, int64_t n_tokens, const int32_t* part_lens,
                          int32_t n_parts, void* stream);

/* Decode-time append of one token to every request with registered KV.
 * d_k, d_v: device [max_batch][Hkv][128] bf16 (rows of requests without KV
 * are ignored).  Reading (the pages do not say): the token fills the last
 * page of the request's last partition; a full page starts a new one-page
 * partition.  The token is written to the host copy and, if that page is
 * resident, to its pool slot; the tail partition's summary is updated
 * exactly (fp64 key sum / length).  SPIN_ECAPACITY, before anything runs, if
 * some request has no room (partition table, max_pages or its reserved host
 * pages).  Stream-ordered. */
SPIN_API int spin_append(spin_ctx* ctx, const void* d_k, const void* d_v, void* stream);

/* Return request `req`'s slots and second-level segments to the free state;
 * the request then has no partitions.  Synchronises `stream`. */
SPIN_API int spin_release(spin_ctx* ctx, int32_t req, void* stream);

/* Select ([XT] part 1, Fig. 3): score every partition of every (request, KV
 * head), score = (mean of the group's G queries) . summary / sqrt(128), in
 * float32, and keep the topk highest per KV head (ties: lower partition id).
 * d_scores may be NULL ([max_batch][Hkv][max_partitions] float32, -inf past a
 * request's partitions).  Two selects of one context must not overlap in time
 * (on different streams): they share the workspace's scores and the per-list
 * counters that hand each list to its top-k. */
SPIN_API int spin_select(spin_ctx* ctx, const void* d_q, int32_t* d_sel, float* d_scores,
                         void* stream);

/* Residency check and eviction for decode step t ([XT] part 2 / Fig. 5 steps
 * 1-2, part 3 / Fig. 6; [GP] B, C).  The mandatory pages are every page of
 * every selected partition of the request.  Each is translated through the
 * two-level page table (directory -> segment -> slot); hits get last_use = t.
 * When a request's misses exceed its free slots, exactly the shortfall is
 * reclaimed by bucketed LRU: bucket = 63 - min(63, t - last_use) over the
 * resident, non-mandatory slots; whole buckets from 0 upward, lower slot
 * first in the last bucket.  Misses take the free slots in ascending order.
 * Emptied segments return to the shared pool; first inserts into an empty
 * directory range take one.  Writes the block tables and the insert lists
 * spin_retrieve reads (so it waits for the previous spin_retrieve).
 * t must not decrease between calls: the ages t - last_use are never
 * negative.  A host-side t below the last one this call was given returns
 * SPIN_EINVAL; a step index below the last resolved step that the host
 * cannot see (the device-side index of spin_step_at, or a mix of both
 * forms) sets SPIN_DEVERR_STEP, and that resolve changes no residency state
 * and no counter: it leaves the step's block tables empty (its heads attend
 * no pages) and its insert lists empty (nothing is transferred). */
SPIN_API int spin_resolve_evict(spin_ctx* ctx, const int32_t* d_sel, int32_t t,
                                int32_t* d_block_table, int32_t* d_block_ntok,
                                int32_t* d_block_count, void* stream);

/* Retrieve ([XT] part 2 / Fig. 5 steps 3-4): copy every page listed by the
 * last spin_resolve_evict from its host address into its pool slot, on
 * `copy_stream` (it waits for that resolve; spin_attend waits for this). */
SPIN_API int spin_retrieve(spin_ctx* ctx, void* copy_stream);

/* spin_retrieve that also attends each fetched page as it arrives ([XT]
 * part 1 attention, done where the page already sits in the transfer's
 * registers): for the G query heads of the page's KV head, d_q as for
 * spin_attend, it keeps an unnormalised partial per fetched page, so
 * spin_attend_finish after it only merges (no fetched page is read back from
 * HBM).  The next spin_attend_finish must be given the same d_q.  spin_attend
 * after it attends every page as usual. */
SPIN_API int spin_retrieve_attend(spin_ctx* ctx, const void* d_q, void* copy_stream);

/* Attention ([XT] part 1, Fig. 3) over the block-table pages:
 * out[b][g] = softmax(q[b][g] . K^T / sqrt(128)) V over the valid tokens of
 * the pages of KV head g / G, bf16 inputs, float32 accumulation.  A head with
 * no pages yields zeros.  Waits for the latest transfer. */
SPIN_API int spin_attend(spin_ctx* ctx, const void* d_q, const int32_t* d_block_table,
                         const int32_t* d_block_ntok, const int32_t* d_block_count,
                         float* d_out, void* stream);

/* spin_attend for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops or harnesses that forbid hipMalloc): no
 * context and no workspace.  The same attention kernels as spin_attend; the
 * split partials, their only scratch, live in a static device array of
 * SPIN_NOALLOC_SCRATCH_BYTES per GPU instead of a caller's workspace.
 * Allocates nothing: the array's address on the current device is looked up
 * once (hipGetSymbolAddress) on the first call there, which must therefore
 * run with the stream's device current.
 *   d_q          device [batch][num_q_heads][128] bf16, 16-byte aligned
 *   d_pool       device page pool, [pool_pages][page] (layout above)
 *   d_block_*    device block tables as spin_resolve_evict writes them,
 *                [batch][num_kv_heads][max_blocks] global pool slots / valid
 *                tokens, [batch][num_kv_heads] page counts; entries naming a
 *                slot outside the pool or 0 / >64 tokens are masked out
 *   d_out        device [batch][num_q_heads][128] float32, 16-byte aligned
 *   pages_per_split  as spin_config.attend_pages_per_split (0 = automatic);
 *                with the same batch, heads, max_blocks and split size the
 *                results equal spin_attend's bit for bit.
 * SPIN_EINVAL for bad arguments (batch 1..1024, Hkv 1..16, Hq / Hkv <= 16,
 * max_blocks 1..4096); SPIN_ESCRATCH, before anything is enqueued, when the
 * partials (batch * num_q_heads * 2 * splits * 520 bytes, none for a single
 * split per head) exceed the array.  Stream-ordered, waits for nothing else.
 * Every call on one GPU shares that GPU's array and leaves its partials
 * there: calls that overlap in time on one GPU (on different streams or
 * threads) race and must not be issued. */
SPIN_API int spin_attend_noalloc(const void* d_q, const void* d_pool, int64_t pool_pages,
                                 const int32_t* d_block_table, const int32_t* d_block_ntok,
                                 const int32_t* d_block_count, float* d_out, int32_t batch,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t max_blocks,
                                 int32_t pages_per_split, void* stream);

/* Retrieve overlapped with attention (the pages' ideal serving envelope
 * hides the transfer; [XT] problem section, Fig. 1).  spin_attend_begin runs
 * attention over the pages of the last spin_resolve_evict that were already
 * resident, without waiting for spin_retrieve, and keeps per-head partials;
 * spin_attend_finish waits for spin_retrieve, attends the pages it fetched and
 * merges both passes (log-sum-exp) into d_out (after spin_retrieve_attend it
 * only merges).  Both must be given the block
 * tables written by the last spin_resolve_evict; the result equals spin_attend
 * up to float32 rounding of the merge. */
SPIN_API int spin_attend_begin(spin_ctx* ctx, const void* d_q, const int32_t* d_block_table,
                               const int32_t* d_block_ntok, const int32_t* d_block_count,
                               void* stream);
SPIN_API int spin_attend_finish(spin_ctx* ctx, const void* d_q, const int32_t* d_block_table,
                                const int32_t* d_block_ntok, const int32_t* d_block_count,
                                float* d_out, void* stream);

/* Retrieve and Attention overlapped in one launch on `stream`: some
 * workgroups pull the pages the last spin_resolve_evict listed and attend
 * each on arrival (as spin_retrieve_attend), the others attend the resident
 * pages (as spin_attend_begin); spin_attend_finish then merges into d_out.
 * No second stream and no event between the two.  The block tables are
 * those of the last spin_resolve_evict; the same d_q goes to
 * spin_attend_finish. */
SPIN_API int spin_transfer_attend(spin_ctx* ctx, const void* d_q, const int32_t* d_block_table,
                                  const int32_t* d_block_ntok, const int32_t* d_block_count,
                                  void* stream);

/* One whole decode step: select, resolve_evict, then Retrieve and
 * Attention.  When copy_stream differs from stream the two overlap in one
 * launch on `stream` (spin_transfer_attend, which here also runs the
 * segment-pool pass of resolve_evict in a workgroup of its own), then
 * spin_attend_finish merges; nothing is enqueued on copy_stream (the staged
 * calls spin_retrieve_attend + spin_attend_begin / _finish put the transfer
 * on a stream of its own, with the same results bit for bit).  When the two
 * streams are equal it is spin_retrieve, then spin_attend. */
SPIN_API int spin_step(spin_ctx* ctx, const void* d_q, int32_t t, int32_t* d_sel,
                       int32_t* d_block_table, int32_t* d_block_ntok, int32_t* d_block_count,
                       float* d_out, void* stream, void* copy_stream);

/* spin_step with the step index on the device, for HIP graph capture: the
 * kernels read t from *d_t (device int32) and the step's queries at
 * d_q_steps + t * q_step_elems (bf16 elements; q_step_elems * 2 a multiple
 * of 16), and the step's last kernel on `stream` increments *d_t, so one
 * captured call replays as consecutive steps.  Overlapped (copy_stream !=
 * stream) nothing runs on copy_stream and the graph holds no event; the
 * results (outputs, selections, the whole residency state) equal
 * spin_step's bit for bit.  t is the caller's to keep non-decreasing.
 * Captured (stream capture active on `stream`), the call waits for no
 * transfer enqueued before the capture: the context must be idle when the
 * capture begins (synchronise the streams it used).  The captured graph holds
 * kernel launches and event record / wait dependencies only (no memset or
 * copy nodes). */
SPIN_API int spin_step_at(spin_ctx* ctx, const void* d_q_steps, int64_t q_step_elems,
                          int32_t* d_t, int32_t* d_sel, int32_t* d_block_table,
                          int32_t* d_block_ntok, int32_t* d_block_count, float* d_out,
                          void* stream, void* copy_stream);

/* Totals since create.  per_request may be NULL, else [max_batch][4] int64:
 * hits, misses, evictions, cutoff bucket of the last step (-1 = none).
 * Synchronises the device. */
SPIN_API int spin_get_stats(spin_ctx* ctx, spin_stats* stats, int64_t* per_request);

/* Copy the residency state to host arrays (any may be NULL):
 * directory [max_batch][Hkv][ndir], segments [num_segments][64],
 * seg_live [num_segments], seg_stack [num_segments] (entries below *seg_top
 * are the free segments, top last), owner [max_batch][C] (h * max_pages +
 * page, or -1), last_use [max_batch][C] (-1 when free), free_count
 * [max_batch].  Synchronises the device. */
SPIN_API int spin_snapshot(spin_ctx* ctx, int32_t* directory, int32_t* segments,
                           int32_t* seg_live, int32_t* seg_stack, int32_t* seg_top,
                           int32_t* owner, int32_t* last_use, int32_t* free_count);

/* Metadata footprint ([XT] part 3, Fig. 6; [GP] C): bytes of the two-level
 * page table as provisioned and as live now, next to a flat table for the
 * same configuration.  A segment counts 64 entries + its live count + its
 * stack slot (264 B).  Synchronises the device. */
SPIN_API int spin_metadata_footprint(spin_ctx* ctx, spin_metadata* out);

/* Copy request req's summaries ([Hkv][n_parts][128] float32) to host memory. */
SPIN_API int spin_read_summaries(spin_ctx* ctx, int32_t req, float* host_out);

/* Synchronise the device and report the device error word: SPIN_OK,
 * SPIN_ESEGPOOL (segment pool exhausted) or SPIN_EDEVICE (other bits). */
SPIN_API int spin_sync_status(spin_ctx* ctx);

/* Diagnostic, not part of the decode step: read `bytes` (a multiple of 16)
 * of the device buffer d_buf with a plain streaming kernel on `stream`;
 * d_sink is a 4-byte device word that keeps the loads alive.  Timing it gives
 * the practical HBM read ceiling next to the decode kernels. */
SPIN_API int spin_read_stream(const void* d_buf, size_t bytes, void* d_sink, void* stream);

SPIN_API const char* spin_strerror(int code);
/* The hipError_t of the last failed HIP call in this context (0 if none). */
SPIN_API int spin_last_hip_error(spin_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif /* SPIN_H */
