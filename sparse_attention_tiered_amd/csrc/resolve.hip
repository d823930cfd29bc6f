// Residency check, bucketed-LRU eviction and the two-level page table.
//
// Follows the SPIN pages' KV manager ([XT] design part 2, Fig. 5 steps 1-2;
// [GP] B) and hierarchical metadata ([XT] part 3, Fig. 6; [GP] C):
//   * a request's GPU area holds the pages the step needs (mandatory) plus a
//     buffer of earlier pages;
//   * the lookup is two-level: a small static directory per (request, KV
//     head) on the GPU points at 64-entry segments that come from one shared
//     pool only while they hold resident pages;
//   * eviction is a bucketed LRU: one pass over the request's slots builds a
//     64-bin histogram of recency buckets, and whole buckets are reclaimed
//     from the oldest until the shortfall is covered, mandatory pages never
//     being candidates.
// Readings where the pages are silent: bucket = 63 - min(63, t - last_use),
// the step index never decreasing (a resolve below the last resolved step is
// refused with the error word, nothing changed);
// exactly the shortfall is evicted, lower slot first inside the cutoff
// bucket; misses take free slots in ascending order; emptied segments return
// to the pool in (KV head, directory index) order per request, requests in
// ascending order, and all returns happen before any segment is handed out.
//
// k_resolve runs one 1024-thread workgroup per request: every ordering
// decision is a workgroup prefix scan in canonical order, so results are
// deterministic and match a sequential walk.  k_segments is one workgroup for
// the whole batch because the segment pool is shared.
#include "device_util.h"
#include "segments.h"
#include "spin_internal.h"

namespace spin {

// the emptied-segment flags of a request's whole directory fit the slot bitmask
static_assert(kMaxKvHeads * (kMaxPartitions * kMaxPPP / kSegEntries) <= kMaxSlots, "");

// slot codes besides the recency buckets 0..63 of eviction candidates
constexpr uint8_t kCodeVictim = 0xFD, kCodeFree = 0xFE, kCodePinned = 0xFF;

// misses of a request's step kept in LDS besides the workspace list (which
// the transfer reads), with the directory entry translation read for each:
// steps 4 and 5 read them back without a global round trip
constexpr int kLdsMisses = 2048;

// a request's directory (Hkv * ndir entries) is copied to LDS when it fits:
// every lookup of the launch (the misses' translation, the victims' ranges,
// the ranges step 5 checks) is then an LDS read
constexpr int kLdsDir = 4096;

__global__ __launch_bounds__(1024) void k_resolve(Dev d, const int* __restrict__ sel, int t,
                                                  int* __restrict__ bt, int* __restrict__ bntok,
                                                  int* __restrict__ bcount) {
  __shared__ uint32_t mand[kMaxSlots / 32];
  __shared__ uint8_t code[kMaxSlots];  // per slot: recency bucket, or a kCode* mark
  __shared__ int item_off[kMaxItems + 1];
  __shared__ int hist[kBuckets];
  __shared__ int tmp[17];
  __shared__ int sh_cut, sh_below;
  __shared__ int4 lmiss[kLdsMisses];  // (h, page, block position, valid tokens)
  __shared__ int ldir[kLdsMisses];    // the miss's directory entry before step 3
  __shared__ int sdir[kLdsDir];       // the request's directory, when it fits

  if (d.step_t) t = *d.step_t;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int C = d.C, Hkv = d.Hkv, k = d.k, MB = d.max_blocks;
  const int n_parts = d.req_parts[b];
  const int n_items = Hkv * k;
  const int* selb = sel + (size_t)b * n_items;
  const int* pfirst = d.part_first + (size_t)b * d.Nmax;
  const int* plen = d.part_len + (size_t)b * d.Nmax;
  int* owner = d.owner + (size_t)b * C;
  int* last = d.last_use + (size_t)b * C;
  int* dir = d.directory + (size_t)b * Hkv * d.ndir;
  int4* misses = d.miss_tmp + (size_t)b * d.max_mand;
  int* btb = bt + (size_t)b * Hkv * MB;
  int* bnb = bntok + (size_t)b * Hkv * MB;

  // loads that depend on nothing before them are issued first, so their
  // round trips overlap the translation instead of following it: the free
  // count and budget, and the first batch of the slot sweep of step 3 (the
  // sweep reads owner, which nothing changes before it, and last_use, which
  // step 2 changes only for mandatory slots, whose value the sweep ignores)
  constexpr int U = 8;  // slots per thread whose loads are in flight together
  const int freec = d.free_count[b];
  const int budget = d.budget[b];
  const int t_prev = d.last_t[b];
  // (every load is issued, from a clamped index, and its value dropped
  // afterwards if out of range: loads under a condition each sit in their own
  // branch, where the compiler waits for each before the next is issued)
  int ow0[U], lu0[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = tid + 1024 * u, cc = min(c, C - 1);
    const int o = owner[cc], lv = last[cc];
    ow0[u] = c < C ? o : -1;
    lu0[u] = c < C ? lv : 0;
  }
  // the directory, stored to LDS at the end of step 1
  const int ne = Hkv * d.ndir;
  const bool dir_lds = ne <= kLdsDir;
  int dv0[kLdsDir / 1024];
#pragma unroll
  for (int u = 0; u < kLdsDir / 1024; ++u) {
    const int e = tid + 1024 * u;
    const int v = dir[min(e, ne - 1)];
    dv0[u] = e < ne ? v : -1;
  }
  auto dir_at = [&](int e) { return dir_lds ? sdir[e] : dir[e]; };
  for (int i = tid; i < (C + 31) / 32; i += 1024) mand[i] = 0;

  // 1. position of every selected partition in the canonical page list (the
  //    first 1024 items' ids, lengths and first pages stay in registers for 2)
  int carry = 0;
  int p_keep = -1, len_keep = 0, first_keep = 0;
  bool bad_part = false;  // reported once the step is known not to go back
  for (int base = 0; base < n_items; base += 1024) {
    const int i = base + tid;
    int np = 0;
    if (i < n_items) {
      const int p = selb[i];
      if (base == 0) p_keep = p;
      if (p >= 0) {
        if (p < n_parts) {
          const int pl = plen[p];
          const int pf = pfirst[p];
          np = (pl + kPageTokens - 1) / kPageTokens;
          if (base == 0) {
            len_keep = pl;
            first_keep = pf;
          }
        } else {
          bad_part = true;
        }
      }
    }
    int tot;
    const int ex = block_excl_scan<1024>(np, tmp, &tot);
    if (i < n_items) item_off[i] = carry + ex;
    carry += tot;
  }
  if (tid == 0) item_off[n_items] = carry;
  const int M = carry;
  if (dir_lds) {
#pragma unroll
    for (int u = 0; u < kLdsDir / 1024; ++u) {
      const int e = tid + 1024 * u;
      if (e < ne) sdir[e] = dv0[u];
    }
  }
  __syncthreads();
  if (t < t_prev) {
    // Steps never go back: below the last resolved step some ages t -
    // last_use would be negative.  Refused before anything in global memory
    // changes (step 1 above only read it; the error word reports the
    // rewind); the step's lists are left empty, so the kernels after this
    // one do nothing for the request and its heads attend no pages.  Checked
    // here rather than first so that step 1's loads do not wait for the two
    // step indices.  (t_prev is one load of one address: the branch is
    // uniform over the workgroup.)
    for (int i = tid; i < Hkv * MB; i += 1024) {
      btb[i] = -1;
      bnb[i] = 0;
    }
    if (tid < Hkv) bcount[(size_t)b * Hkv + tid] = 0;
    if (tid <= Hkv) d.head_moff[(size_t)b * (Hkv + 1) + tid] = 0;
    if (tid == 0) {
      atomicOr(d.err, kErrStep);
      d.nmiss[b] = 0;
      d.nfreed[b] = 0;
      d.nalloc[b] = 0;
    }
    return;
  }
  if (bad_part) atomicOr(d.err, kErrPartition);

  // block counts per head; clear the unused tail of the block table
  for (int i = tid; i < Hkv * MB; i += 1024) {
    const int h = i / MB, pos = i - h * MB;
    const int cnt = item_off[(h + 1) * k] - item_off[h * k];
    if (pos >= cnt) {
      btb[i] = -1;
      bnb[i] = 0;
    }
  }
  if (tid < Hkv) bcount[(size_t)b * Hkv + tid] = item_off[(tid + 1) * k] - item_off[tid * k];

  // 2. translate every mandatory page through directory -> segment
  int mcarry = 0;
  for (int base = 0; base < n_items; base += 1024) {
    const int i = base + tid;
    int nm = 0, p = -1, h = 0, np = 0, pos0 = 0, pf0 = 0, pl = 0;
    int segv[kMaxPPP];  // directory entry of each page's range
    unsigned missmask = 0;
    if (i < n_items) {
      p = base == 0 ? p_keep : selb[i];
      h = i / k;
      if (p >= 0 && p < n_parts) {
        pf0 = base == 0 ? first_keep : pfirst[p];
        pl = base == 0 ? len_keep : plen[p];
        np = (pl + kPageTokens - 1) / kPageTokens;
        pos0 = item_off[i] - item_off[h * k];
        // every page's segment entry loaded before any is tested (a page
        // past the partition, or in a range without a valid segment, loads
        // the first page's entry again and drops it; with one page per
        // partition, a uniform case, only that page is loaded)
        int slots[kMaxPPP];
        bool ok[kMaxPPP];
        size_t at[kMaxPPP];
#pragma unroll
        for (int j = 0; j < kMaxPPP; ++j) {
          const int page = pf0 + j;
          const int seg = j < np ? dir_at(h * d.ndir + (page >> 6)) : -1;
          segv[j] = seg;
          ok[j] = seg >= 0 && seg < d.n_seg;
          at[j] = ok[j] ? (size_t)seg * kSegEntries + (page & 63) : 0;
        }
        if (!ok[0]) at[0] = 0;
        if (d.max_ppp == 1) {
          slots[0] = d.segments[at[0]];
#pragma unroll
          for (int j = 1; j < kMaxPPP; ++j) slots[j] = -1;
        } else {
#pragma unroll
          for (int j = 0; j < kMaxPPP; ++j) slots[j] = d.segments[ok[j] ? at[j] : at[0]];
        }
#pragma unroll
        for (int j = 0; j < kMaxPPP; ++j) {
          asm volatile("" : "+v"(slots[j]));
          if (!ok[j]) slots[j] = -1;
        }
#pragma unroll
        for (int j = 0; j < kMaxPPP; ++j) {
          if (j >= np) break;
          const int ntok = min(kPageTokens, pl - kPageTokens * j);
          int slot = slots[j];
          if (slot >= C) {
            atomicOr(d.err, kErrState);
            slot = -1;
          }
          if (slot >= 0) {
            last[slot] = t;
            atomicOr(&mand[slot >> 5], 1u << (slot & 31));
            btb[h * MB + pos0 + j] = b * C + slot;
            bnb[h * MB + pos0 + j] = ntok;
            d.bmiss[((size_t)b * Hkv + h) * MB + pos0 + j] = 0;
          } else {
            missmask |= 1u << j;
            ++nm;
          }
        }
      }
    }
    int tot;
    const int ex = block_excl_scan<1024>(nm, tmp, &tot);
    // insert-list index of each head's first miss (items are head-major)
    if (i < n_items && i % k == 0) d.head_moff[(size_t)b * (Hkv + 1) + i / k] = mcarry + ex;
    if (nm) {
      int rnk = mcarry + ex;
      for (int j = 0; j < np; ++j)
        if (missmask & (1u << j)) {
          const int4 mv = make_int4(h, pf0 + j, pos0 + j, min(kPageTokens, pl - kPageTokens * j));
          misses[rnk] = mv;
          if (rnk < kLdsMisses) {
            lmiss[rnk] = mv;
            ldir[rnk] = segv[j];
          }
          ++rnk;
        }
    }
    mcarry += tot;
  }
  const int nmiss = mcarry;
  if (tid == 0) d.head_moff[(size_t)b * (Hkv + 1) + Hkv] = nmiss;
  __syncthreads();
  // the first 1024 misses, the one before each, and each one's directory
  // entry as it stands before step 3 (as step 2 read it), for steps 4 and 5
  // (step 3 can only clear directory entries, and it flags each one it
  // clears)
  auto miss_at = [&](int j) { return j < kLdsMisses ? lmiss[j] : misses[j]; };
  int4 m_pre = make_int4(0, 0, 0, 0), m_prev = make_int4(-1, 0, 0, 0);
  int dir_pre = -1;
  if (tid < nmiss) {
    m_pre = lmiss[tid];
    if (tid > 0) m_prev = lmiss[tid - 1];
    dir_pre = ldir[tid];
  }

  // 3. bucketed LRU, only when the resident pages plus the misses exceed the
  //    request's budget (with the budget at the whole area: when the misses
  //    outnumber the free slots); a shrunk budget is enforced here, lazily.
  //
  //    One coalesced sweep turns the request's slots into one-byte codes in
  //    LDS (recency bucket of an eviction candidate, or free / pinned) and
  //    builds the histogram; every ordered decision after it (the victims of
  //    the cutoff bucket, the free slots the misses take) is one workgroup
  //    scan over contiguous per-thread slot ranges of those codes, and the
  //    global updates run afterwards, one slot or one miss per thread.
  const int need = (C - freec) + nmiss - budget;
  int nfreed = 0, cut = -1;
  if (tid < kBuckets) hist[tid] = 0;
  __syncthreads();
  if (need > 0 || nmiss > 0) {
    for (int c0 = tid; c0 < C; c0 += 1024 * U) {
      int ow[U], lu[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 1024 * u;
        if (c0 == tid) {
          ow[u] = ow0[u];
          lu[u] = lu0[u];
        } else {
          const int cc = min(c, C - 1);
          const int o = owner[cc], lv = last[cc];
          ow[u] = c < C ? o : -1;
          lu[u] = c < C ? lv : 0;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 1024 * u;
        if (c >= C) break;
        uint8_t v;
        if (ow[u] < 0) {
          v = kCodeFree;
        } else if ((mand[c >> 5] >> (c & 31)) & 1u) {
          v = kCodePinned;
        } else if (need > 0) {
          // (t >= the last resolved step >= last_use: the age is never
          // negative; clamped all the same, so a code is always a bucket)
          v = (uint8_t)((kBuckets - 1) - min(kBuckets - 1, max(0, t - lu[u])));
          atomicAdd(&hist[v], 1);
        } else {
          v = kCodePinned;  // nothing is evicted this step
        }
        code[c] = v;
      }
    }
  }
  __syncthreads();
  // from here on the bitmask flags the directory ranges whose segment this
  // step empties (set by the victims' loop, listed in step 3's last scan)
  if (need > 0)
    for (int i = tid; i < (ne + 31) / 32; i += 1024) mand[i] = 0;
  const int E = (C + 1023) / 1024;  // contiguous slots per thread
  const int lo = min(C, tid * E), hi = min(C, lo + E);
  if (need > 0) {
    // the cutoff: the first bucket whose inclusive count reaches `need`, or
    // the newest one (one wave, one bucket per lane)
    static_assert(kBuckets == 64, "one bucket per lane");
    if (tid < 64) {
      const int hv = hist[tid];
      const int inc = wave_incl_scan(hv);
      const unsigned long long hit = __ballot(inc >= need) | (1ull << (kBuckets - 1));
      const int cv = __ffsll((long long)hit) - 1;
      if (tid == cv) {
        sh_cut = cv;
        sh_below = inc - hv;
      }
    }
    __syncthreads();
    cut = sh_cut;
    const int rem = need - sh_below;  // taken from the cutoff bucket, lowest slots first
    int nv = 0;  // victims in this thread's slot range
    {
      int at = 0;
      for (int c = lo; c < hi; ++c) at += code[c] == cut;
      int tot;
      int rank = block_excl_scan<1024>(at, tmp, &tot);
      for (int c = lo; c < hi; ++c) {
        const int v = code[c];
        if (v < cut || (v == cut && rank++ < rem)) {
          code[c] = kCodeVictim;
          ++nv;
        }
      }
    }
    // the victims listed in LDS (the item offsets are no longer read), so the
    // loop below runs over the victims rather than over every slot; a list
    // longer than that buffer falls back to the sweep over all slots
    int nvict;
    const int voff = block_excl_scan<1024>(nv, tmp, &nvict);
    int* vlist = item_off;
    const bool listed = nvict <= kMaxItems + 1;
    if (listed && nv) {
      int o = voff;
      for (int c = lo; c < hi; ++c)
        if (code[c] == kCodeVictim) vlist[o++] = c;
    }
    __syncthreads();
    // the victims' owners, then their directory entries, eight victims'
    // loads in flight at a time, then the table updates
    constexpr int UV = 8;
    const int nloop = listed ? nvict : C;
    for (int j0 = tid; j0 < nloop; j0 += 1024 * UV) {
      int own[UV], seg[UV], cs[UV];
#pragma unroll
      for (int u = 0; u < UV; ++u) {
        const int j = j0 + 1024 * u;
        cs[u] = -1;
        own[u] = -1;
        if (j < nloop) {
          const int c = listed ? vlist[j] : j;
          if (code[c] == kCodeVictim) {
            cs[u] = c;
            own[u] = owner[c];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < UV; ++u) {
        seg[u] = -2;  // not a victim
        if (own[u] >= 0) {
          const int h = own[u] / d.max_pages, page = own[u] - h * d.max_pages;
          seg[u] = h < Hkv ? dir_at(h * d.ndir + (page >> 6)) : -1;
        }
      }
      // the live-count decrements of all eight issued before any result is
      // read; the victim that takes its segment's count to zero flags the
      // range: every linked segment holds at least one resident page, so
      // these are exactly the segments this step empties
      int before[UV];
#pragma unroll
      for (int u = 0; u < UV; ++u) {
        before[u] = 0;
        if (seg[u] == -2) continue;
        const int c = cs[u];
        const int page = own[u] % d.max_pages;
        if (seg[u] >= 0 && seg[u] < d.n_seg) {
          d.segments[(size_t)seg[u] * kSegEntries + (page & 63)] = -1;
          before[u] = atomicSub(&d.seg_live[seg[u]], 1);
        } else {
          atomicOr(d.err, kErrState);
        }
        owner[c] = -1;
        last[c] = -1;
        code[c] = kCodeFree;
      }
      // (an empty asm that takes each result as a register keeps the
      // compiler from testing it inside its own branch, which would wait for
      // every decrement before issuing the next)
#pragma unroll
      for (int u = 0; u < UV; ++u) asm volatile("" : "+v"(before[u]));
#pragma unroll
      for (int u = 0; u < UV; ++u)
        if (before[u] == 1) {
          const int h = own[u] / d.max_pages, page = own[u] - h * d.max_pages;
          const int e = h * d.ndir + (page >> 6);
          atomicOr(&mand[e >> 5], 1u << (e & 31));
        }
    }
    __syncthreads();
    // emptied segments leave the directory, in (head, directory index) order:
    // one ordered scan over the flags the victims set
    const int Ed = (ne + 1023) / 1024;
    const int elo = min(ne, tid * Ed), ehi = min(ne, elo + Ed);
    int nf = 0;
    for (int e = elo; e < ehi; ++e) nf += (mand[e >> 5] >> (e & 31)) & 1u;
    int r = block_excl_scan<1024>(nf, tmp, &nfreed);
    for (int e = elo; e < ehi; ++e)
      if ((mand[e >> 5] >> (e & 31)) & 1u) {
        d.freed[(size_t)b * ne + r++] = dir_at(e);
        dir[e] = -1;
        if (dir_lds) sdir[e] = -1;
      }
  }

  // 4. misses take the free slots in ascending slot order: the rank of each
  //    free slot goes to an LDS list (the item offsets' space, free again
  //    since step 2; the insert list itself when there are more misses), then
  //    one thread per miss fills it
  int assigned = 0;
  int4* insb = d.ins + (size_t)b * d.max_mand;
  if (nmiss > 0) {
    const bool lds_slots = nmiss <= kMaxItems + 1;
    int* slot_of = item_off;
    int fr = 0;
    for (int c = lo; c < hi; ++c) fr += code[c] == kCodeFree;
    int tot;
    int r = block_excl_scan<1024>(fr, tmp, &tot);
    for (int c = lo; c < hi && r < nmiss; ++c)
      if (code[c] == kCodeFree) {
        if (lds_slots) slot_of[r] = c;
        else insb[r].x = c;
        ++r;
      }
    assigned = min(tot, nmiss);
    __syncthreads();
    for (int j = tid; j < assigned; j += 1024) {
      const int c = lds_slots ? slot_of[j] : insb[j].x;
      const int4 m = j == tid ? m_pre : miss_at(j);  // (h, page, block position, valid tokens)
      owner[c] = m.x * d.max_pages + m.y;
      last[c] = t;
      btb[m.x * MB + m.z] = b * C + c;
      bnb[m.x * MB + m.z] = m.w;
      d.bmiss[((size_t)b * Hkv + m.x) * MB + m.z] = 1;
      insb[j] = make_int4(c, m.x, m.y, 0);
    }
  }
  __syncthreads();

  // 5. directory ranges that need a segment from the shared pool: the first
  //    insert of each range whose entry is empty after this request's frees
  //    (canonical order; inserts of one range are consecutive)
  int nalloc = 0;
  {
    int ccarry = 0;
    for (int base = 0; base < assigned; base += 1024) {
      const int r = base + tid;
      int fl = 0, e = 0;
      if (r < assigned) {
        const int4 m = base == 0 ? m_pre : miss_at(r);
        e = m.x * d.ndir + (m.y >> 6);
        bool first = true;
        if (r > 0) {
          const int4 pm = base == 0 ? m_prev : miss_at(r - 1);
          first = (pm.x * d.ndir + (pm.y >> 6)) != e;
        }
        // the entry now: step 3 emptied it (and flagged it) or left it as it was
        int dv;
        if (base == 0) dv = (need > 0 && ((mand[e >> 5] >> (e & 31)) & 1u)) ? -1 : dir_pre;
        else dv = dir_at(e);
        fl = (first && dv < 0) ? 1 : 0;
      }
      int tot;
      const int ex = block_excl_scan<1024>(fl, tmp, &tot);
      if (fl) d.alloc[(size_t)b * ne + ccarry + ex] = e;
      ccarry += tot;
    }
    nalloc = ccarry;
  }
  if (tid == 0) {
    d.last_t[b] = t;
    d.nalloc[b] = nalloc;
    const int ev = need > 0 ? need : 0;
    if (assigned < nmiss) atomicOr(d.err, kErrState);
    d.free_count[b] = freec + ev - assigned;
    d.nmiss[b] = assigned;
    d.nfreed[b] = nfreed;
    long long* st = d.stats + 4 * (size_t)b;
    st[0] += M - nmiss;
    st[1] += nmiss;
    st[2] += ev;
    st[3] = cut;
  }
}

__global__ __launch_bounds__(1024) void k_segments(Dev d, int with_inserts) {
  __shared__ int lds[3 * 1025];
  __shared__ int tmp[1024 / 64 + 1];
  segments_wg<1024>(d, with_inserts, lds, tmp);
}

hipError_t launch_resolve(const Dev& d, const int* sel, int t, int* bt, int* bntok, int* bcount,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_resolve, dim3(d.B), dim3(1024), 0, s, d, sel, t, bt, bntok, bcount);
  return hipGetLastError();
}

__global__ void k_step_advance(int* t) {
  if (threadIdx.x == 0) *t += 1;
}

hipError_t launch_step_advance(int* t, hipStream_t s) {
  hipLaunchKernelGGL(k_step_advance, dim3(1), dim3(64), 0, s, t);
  return hipGetLastError();
}

// Large batches write the inserts with many workgroups (one workgroup would
// be bound by its own CU's scattered accesses: 23 -> 12 us for 4.7K inserts),
// small ones inside the segment-pool pass (a second launch would cost more).
constexpr int kInsertWG = 256, kInsertGrid = 64;
constexpr long long kInsertSplitMin = 8192;  // B * max pages per step above which

__global__ __launch_bounds__(kInsertWG) void k_segment_inserts(Dev d) {
  __shared__ int pm[1025];
  __shared__ int tmp[kInsertWG / 64 + 1];
  const int M = request_offsets<kInsertWG>(d.nmiss, d.B, pm, tmp);
  insert_segments(d, pm, M, blockIdx.x * kInsertWG + threadIdx.x, kInsertGrid * kInsertWG);
}

hipError_t launch_segments(const Dev& d, hipStream_t s) {
  const bool split = (long long)d.B * d.max_mand > kInsertSplitMin;
  hipLaunchKernelGGL(k_segments, dim3(1), dim3(1024), 0, s, d, split ? 0 : 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  hipLaunchKernelGGL(k_segment_inserts, dim3(kInsertGrid), dim3(kInsertWG), 0, s, d);
  return hipGetLastError();
}

}  // namespace spin
