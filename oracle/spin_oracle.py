"""CPU oracle for one SPIN decode step -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It is a plain, slow, step-by-step restatement of what the method
computes, in float64 with Python control flow, and shares no code with the HIP
library.  The product path never calls it.

Sources (web pages about "Unifying Sparse Attention with Hierarchical Memory
for Scalable Long-Context LLM Serving", the SPIN framework):

  [XT] m.x-techcon.com article "吞吐量提升5.66倍！微软、港中大等Spin框架如何统一
       稀疏注意力与分级内存，让稀疏注意力算法真正高效落地"; its design section
       "Spin的核心设计：从抽象到高效管理" has three parts: (1) the unified
       partition abstraction (Fig. 3 pipeline), (2) locality-aware KV management
       (buffer elasticity, bucketed LRU, Fig. 5), (3) hierarchical metadata
       (two-level page table, Fig. 6).
  [GP] gist.science/pt summary of the same paper, "2. Metodologia", parts A
       (partition abstraction), B (KV management, per-head physical pages) and
       C (hierarchical metadata).
  [PM] publish-md.pages.dev digest "今日 Attention 论文：SPIN 统一稀疏注意力与分层
       KV 存储", section "方法拆解".

Where the pages leave a step open, the reading taken is stated at that step
(R-numbers match the readings table of the design notes).

What each part follows:
  index()          [XT] part 1 / Fig. 3: Index groups KV into partitions
                   (contiguous token runs) and summarises them.  Summary =
                   mean key of the partition's valid tokens (fixed rule, R1).
  select()         [XT] part 1 / Fig. 3: Select scores partitions against the
                   query; rule R1/R2: score = mean-over-group query . summary
                   / sqrt(D); per-KV-head top-k, lower index wins ties (R4).
  resolve_evict()  [XT] part 2 / Fig. 5 steps 1-2 and part 3 / Fig. 6:
                   residency check through the two-level table, mandatory vs
                   buffer pages, 64-bucket LRU reclaim oldest bucket first
                   until the demand is met; [GP] B: pages are per KV head.
  set_budget()     [XT] part 2 buffer elasticity: per-request budget.
  offload()        [XT] part 1 / Fig. 3: prefill KV copied to host, indexed.
  append()         decode-time append of a token (reading stated there).
  retrieve()       [XT] part 2 / Fig. 5 steps 3-4: host address from the CPU
                   page table, copy of the missed pages' valid tokens (the
                   token slots past them arrive as zeros, reading R25).
  attend()         [XT] part 1 / Fig. 3: attention over the selected
                   partitions only (softmax(q K^T / sqrt(D)) V).

Pins: every function here is pinned by tests/test_oracle_pins.py to closed
forms, brute force, library special cases (dense attention) and structural
invariants; see that file.  Nothing is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

PAGE_TOKENS = 64          # tokens per physical page
SEG_ENTRIES = 64          # page-table entries per second-level segment
NUM_BUCKETS = 64          # recency buckets of the bucketed LRU ([XT] part 2)
FREE = -1                 # owner / page-table value of an empty slot / entry
PAGE_ELEMS = 2 * PAGE_TOKENS * 128


# --------------------------------------------------------------------------- decoding of inputs
def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values (bf16 is the top half of fp32)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def page_keys(page: np.ndarray, D: int = 128) -> np.ndarray:
    """Keys of one stored page as float64 [64 tokens][D] (token-major half)."""
    return bf16_bits_to_f64(page[: PAGE_TOKENS * D]).reshape(PAGE_TOKENS, D)


def page_values(page: np.ndarray, D: int = 128) -> np.ndarray:
    """Values of one stored page as float64 [64 tokens][D] (stored dim-major)."""
    return bf16_bits_to_f64(page[PAGE_TOKENS * D: 2 * PAGE_TOKENS * D]).reshape(D, PAGE_TOKENS).T


def pages_of_partition(length: int) -> int:
    """Physical pages a partition of ``length`` tokens occupies (it starts on a fresh page)."""
    return (length + PAGE_TOKENS - 1) // PAGE_TOKENS


def bucket_of(t: int, last_use: int) -> int:
    """Recency bucket of a resident page, reading R6: 63 = used this step, one
    bucket per step of age, 0 = 63 or more steps old (the oldest)."""
    return (NUM_BUCKETS - 1) - min(NUM_BUCKETS - 1, t - last_use)


class Request:
    """CPU page table of one request: where its pages live in host memory, and
    how partitions map onto pages ([XT] part 1: partitions are contiguous token
    runs mapped onto the shared paged substrate; [GP] A)."""

    def __init__(self, host_pages: np.ndarray, lens: np.ndarray, Hkv: int, stride: int | None = None):
        self.lens = np.asarray(lens, dtype=np.int64)
        self.n_parts = len(self.lens)
        npg = [pages_of_partition(int(L)) for L in self.lens]
        self.first_page = np.zeros(self.n_parts, np.int64)
        acc = 0
        for i, n in enumerate(npg):
            self.first_page[i] = acc
            acc += n
        self.n_pages = np.asarray(npg, np.int64)
        self.pages = acc
        # pages reserved per KV head in the host buffer (room to append)
        self.stride = acc if stride is None else stride
        # [Hkv][stride][PAGE_ELEMS] uint16, the request's full KV in host memory
        self.host = host_pages[: Hkv * self.stride * PAGE_ELEMS].reshape(Hkv, self.stride, PAGE_ELEMS) \
            if self.stride > 0 else np.zeros((Hkv, 0, PAGE_ELEMS), np.uint16)
        self.summaries = None  # [Hkv][n_parts][D] float32

    def page_tokens(self, part: int, j: int) -> int:
        """Valid tokens on the j-th page of partition ``part``."""
        L = int(self.lens[part])
        return min(PAGE_TOKENS, L - j * PAGE_TOKENS)


class SpinOracle:
    """State and per-step operations of the sparse decode layer.

    Residency state (compared bit-exactly with the GPU):
      directory[b][h][e]  segment id holding pages e*64 .. e*64+63, or FREE
      segments[s][i]      slot (local to the request) of a page, or FREE
      seg_live[s]         number of non-FREE entries of segment s
      free_stack          unused segment ids; the top is the last element
      owner[b][c]         h * max_pages + page held by slot c, or FREE
      last_use[b][c]      decode step of the slot's last use, FREE if empty
    """

    def __init__(self, B, Hq, Hkv, k, slots_per_request, max_pages, num_segments, D=128):
        assert Hq % Hkv == 0
        self.B, self.Hq, self.Hkv, self.G, self.k, self.D = B, Hq, Hkv, Hq // Hkv, k, D
        self.C = slots_per_request
        self.max_pages = max_pages
        self.ndir = (max_pages + SEG_ENTRIES - 1) // SEG_ENTRIES
        self.n_seg = num_segments
        self.directory = np.full((B, Hkv, self.ndir), FREE, np.int64)
        self.segments = np.full((num_segments, SEG_ENTRIES), FREE, np.int64)
        self.seg_live = np.zeros(num_segments, np.int64)
        # LIFO of unused segments; it starts as [n_seg-1, ..., 1, 0] so the
        # first segment handed out is 0
        self.free_stack = list(range(num_segments - 1, -1, -1))
        self.owner = np.full((B, self.C), FREE, np.int64)
        self.last_use = np.full((B, self.C), FREE, np.int64)
        self.pool = np.zeros((B * self.C, PAGE_ELEMS), np.uint16)
        self.requests = [None] * B
        # per-request cap on resident pages ([XT] part 2, buffer elasticity);
        # it starts at the request's full area
        self.budget = [slots_per_request] * B
        self.error = None
        self.stats = [dict(hits=0, misses=0, evictions=0, cutoff=-1) for _ in range(B)]
        self._pending = []   # (global slot, b, h, page, valid tokens) copies for retrieve()
        # decode step of the last resolve: steps never go back, so every age
        # t - last_use is at least 0 (reading R23)
        self.last_t = -1

    # ------------------------------------------------------------------ Index (+ Offload registration)
    def release(self, b: int):
        """Request turnover ([XT] part 2: each request owns a GPU area; part 3:
        second-level segments come from, and go back to, one shared pool).
        Every segment linked in request b's directory is cleared and pushed
        back on the pool's stack, in (KV head, directory index) order (R18);
        every slot of the request becomes free; its budget returns to the
        whole area.  Other requests keep their state.  Counters (stats) are
        per request position and are kept."""
        for h in range(self.Hkv):
            for e in range(self.ndir):
                s = self.directory[b, h, e]
                if s != FREE:
                    self.segments[s, :] = FREE
                    self.seg_live[s] = 0
                    self.free_stack.append(int(s))
                    self.directory[b, h, e] = FREE
        self.owner[b, :] = FREE
        self.last_use[b, :] = FREE
        self.budget[b] = self.C
        self.requests[b] = None

    def summary(self, req: Request, h: int, i: int) -> np.ndarray:
        """Mean key of partition i of head h over its valid tokens, in float64,
        stored as float32 (reading R1)."""
        rows = []
        for j in range(int(req.n_pages[i])):
            K = page_keys(req.host[h, req.first_page[i] + j], self.D)
            rows.append(K[: req.page_tokens(i, j)])
        keys = np.concatenate(rows, axis=0)
        return (keys.sum(axis=0) / keys.shape[0]).astype(np.float32)

    def index(self, b: int, host_pages: np.ndarray, lens: np.ndarray, stride: int | None = None):
        """Index: register request b's host KV (the CPU page table) and build its
        partition summaries ([XT] part 1, Fig. 3)."""
        self.release(b)
        req = Request(host_pages, lens, self.Hkv, stride)
        assert req.pages <= self.max_pages and req.pages <= req.stride
        summ = np.zeros((self.Hkv, req.n_parts, self.D), np.float32)
        for h in range(self.Hkv):
            for i in range(req.n_parts):
                summ[h, i] = self.summary(req, h, i)
        req.summaries = summ
        self.requests[b] = req

    def offload(self, b: int, kv_pages: np.ndarray, lens: np.ndarray, capacity_pages: int):
        """Prefill side ([XT] part 1, Fig. 3: Index then Offload): the request's
        freshly computed KV ([Hkv][pages][page]) is copied to host memory, into
        a buffer that reserves capacity_pages per KV head, and indexed."""
        pages = sum(pages_of_partition(int(L)) for L in lens)
        host = np.zeros((self.Hkv, capacity_pages, PAGE_ELEMS), np.uint16)
        host[:, :pages] = np.asarray(kv_pages).reshape(self.Hkv, pages, PAGE_ELEMS)
        self.index(b, host.reshape(-1), lens, capacity_pages)

    def append(self, k_bits: np.ndarray, v_bits: np.ndarray):
        """Decode-time append of one token per registered request (k_bits,
        v_bits: [B][Hkv][D] bf16).  Reading (not on the pages): the token fills
        the last page of the request's last partition; when that page is full,
        it starts a new one-page partition.  The token is written to the host
        copy and, if its page is resident, to the GPU-side copy too; the tail
        partition's summary is recomputed."""
        for b in range(self.B):
            req = self.requests[b]
            if req is None:
                continue
            tail = req.n_parts - 1
            if req.n_parts == 0 or req.lens[tail] % PAGE_TOKENS == 0:
                assert req.pages < min(req.stride, self.max_pages), "no room to append"
                req.lens = np.append(req.lens, 1)
                req.first_page = np.append(req.first_page, req.pages)
                req.n_pages = np.append(req.n_pages, 1)
                req.n_parts += 1
                req.pages += 1
                tail = req.n_parts - 1
                req.summaries = np.concatenate(
                    [req.summaries, np.zeros((self.Hkv, 1, self.D), np.float32)], axis=1)
            else:
                req.lens[tail] += 1
            page = int(req.first_page[tail] + req.n_pages[tail] - 1)
            slot_tok = (int(req.lens[tail]) - 1) % PAGE_TOKENS
            for h in range(self.Hkv):
                dst = [req.host[h, page]]
                c = self.translate(b, h, page)
                if c != FREE:
                    dst.append(self.pool[b * self.C + c])
                for pg in dst:
                    pg[slot_tok * self.D:(slot_tok + 1) * self.D] = k_bits[b, h]
                    vt = pg[PAGE_TOKENS * self.D:].reshape(self.D, PAGE_TOKENS)
                    vt[:, slot_tok] = v_bits[b, h]
                req.summaries[h, tail] = self.summary(req, h, tail)

    # ------------------------------------------------------------------ Select
    def scores(self, q_bits: np.ndarray) -> list:
        """score[b][h][i] = (qbar_bh . s_bhi) / sqrt(D), qbar = mean of the group's
        queries (readings R2, R3: query head g belongs to KV head g // G)."""
        q = bf16_bits_to_f64(q_bits).reshape(self.B, self.Hq, self.D)
        out = []
        for b in range(self.B):
            req = self.requests[b]
            row = []
            for h in range(self.Hkv):
                if req is None or req.n_parts == 0:
                    row.append(np.zeros(0))
                    continue
                qbar = q[b, h * self.G:(h + 1) * self.G].sum(axis=0) / self.G
                s = req.summaries[h].astype(np.float64)
                row.append((s @ qbar) / math.sqrt(self.D))
            out.append(row)
        return out

    def select(self, q_bits: np.ndarray):
        """Per-KV-head top-k: highest scores first, the lower partition index on an
        exact tie (R4); the chosen ids are returned sorted ascending, padded
        with FREE when a head has fewer than k partitions."""
        sc = self.scores(q_bits)
        sel = np.full((self.B, self.Hkv, self.k), FREE, np.int64)
        for b in range(self.B):
            for h in range(self.Hkv):
                s = sc[b][h]
                if len(s) == 0:
                    continue
                order = np.lexsort((np.arange(len(s)), -s))  # primary -score, then index
                chosen = np.sort(order[: self.k])
                sel[b, h, : len(chosen)] = chosen
        return sel, sc

    # ------------------------------------------------------------------ Retrieve: residency + eviction
    def set_budget(self, b: int, slots: int):
        """Buffer elasticity ([XT] part 2; [GP] B): the scheduler resizes a
        request's GPU buffer with load.  Reading: the budget caps the number of
        resident pages of the request (at least the pages one step can need,
        at most its slot area); shrinking evicts nothing at once, the next
        resolve reclaims the excess through the same bucketed LRU."""
        assert 1 <= slots <= self.C
        self.budget[b] = int(slots)

    def translate(self, b: int, h: int, page: int) -> int:
        """Two-level lookup ([XT] part 3 / Fig. 6): directory entry -> segment ->
        slot.  FREE when the page is not resident."""
        s = self.directory[b, h, page // SEG_ENTRIES]
        if s == FREE:
            return FREE
        return int(self.segments[s, page % SEG_ENTRIES])

    def mandatory_pages(self, b: int, sel_b: np.ndarray):
        """Pages the step needs ([XT] part 2, mandatory pages; R9), in canonical
        order: KV head ascending, partition ascending, page ascending.  Each
        entry is (h, page, valid tokens)."""
        req = self.requests[b]
        out = []
        if req is None:
            return out
        for h in range(self.Hkv):
            for p in sel_b[h]:
                if p == FREE:
                    continue
                if not (0 <= p < req.n_parts):
                    raise IndexError(f"partition {p} out of range for request {b}")
                for j in range(int(req.n_pages[p])):
                    out.append((h, int(req.first_page[p] + j), req.page_tokens(int(p), j)))
        return out

    def choose_victims(self, b: int, need: int, mandatory_slots: set, t: int):
        """Bucketed LRU ([XT] part 2; [GP] B): one pass over the request's slots
        builds a 64-bin histogram of recency buckets of the resident pages that
        are not mandatory; reclaim whole buckets from the oldest (bucket 0) up,
        until ``need`` pages are freed.  Within the last bucket, lower slot
        index goes first (R8).  Returns (victims ascending, cutoff bucket)."""
        cands = [c for c in range(self.C)
                 if self.owner[b, c] != FREE and c not in mandatory_slots]
        hist = [0] * NUM_BUCKETS
        for c in cands:
            hist[bucket_of(t, int(self.last_use[b, c]))] += 1
        below, cut = 0, 0
        while below + hist[cut] < need:
            below += hist[cut]
            cut += 1
        take_at_cut = need - below
        victims = []
        for c in cands:  # ascending slot order
            bk = bucket_of(t, int(self.last_use[b, c]))
            if bk < cut:
                victims.append(c)
            elif bk == cut and take_at_cut > 0:
                victims.append(c)
                take_at_cut -= 1
        return sorted(victims), cut

    def evict(self, b: int, victims):
        """Drop the victims from the page table.  A segment whose live count
        reaches zero leaves the directory; the request's emptied segments go
        back on the shared pool's stack in (KV head, directory index) order."""
        for c in victims:
            own = int(self.owner[b, c])
            h, page = divmod(own, self.max_pages)
            s = self.directory[b, h, page // SEG_ENTRIES]
            self.segments[s, page % SEG_ENTRIES] = FREE
            self.seg_live[s] -= 1
            self.owner[b, c] = FREE
            self.last_use[b, c] = FREE
        for h in range(self.Hkv):
            for e in range(self.ndir):
                s = self.directory[b, h, e]
                if s != FREE and self.seg_live[s] == 0:
                    self.directory[b, h, e] = FREE
                    self.free_stack.append(int(s))

    def insert(self, b: int, h: int, page: int, slot: int):
        """Page-table insert; the directory range gets a segment from the shared
        pool on its first resident page ([XT] part 3 / Fig. 6)."""
        e = page // SEG_ENTRIES
        if self.directory[b, h, e] == FREE:
            if not self.free_stack:
                raise MemoryError("segment pool exhausted")
            s = self.free_stack.pop()
            self.segments[s, :] = FREE
            self.directory[b, h, e] = s
        s = self.directory[b, h, e]
        self.segments[s, page % SEG_ENTRIES] = slot
        self.seg_live[s] += 1

    def resolve_evict(self, sel: np.ndarray, t: int):
        """Fig. 5 steps 1-2 for every request, then the page-table inserts.

        Phase 1 (requests in ascending order): translate the mandatory pages,
        refresh hits (last_use = t), list misses in canonical order; if the
        misses outnumber the free slots evict exactly the shortfall (R7); give
        the misses the free slots in ascending slot order (R10).
        Phase 2 (requests in ascending order, after every request's frees):
        insert the misses into the two-level table.

        Returns block tables: per (b, h) a list of (global slot, valid tokens)
        in canonical order."""
        if t < self.last_t:
            # a rewound step index would give negative ages; refused before
            # anything changes (R23)
            raise ValueError(f"decode step {t} is below the last resolved step {self.last_t}")
        self.last_t = t
        blocks = [[[] for _ in range(self.Hkv)] for _ in range(self.B)]
        inserts = []
        self._pending = []
        for b in range(self.B):
            M = self.mandatory_pages(b, sel[b])
            mand = set()
            misses = []
            for pos, (h, page, ntok) in enumerate(M):
                c = self.translate(b, h, page)
                if c != FREE:
                    self.last_use[b, c] = t
                    mand.add(c)
                    blocks[b][h].append([b * self.C + c, ntok])
                else:
                    blocks[b][h].append([None, ntok])
                    misses.append((h, page, len(blocks[b][h]) - 1))
            # the shortfall against the request's budget: resident pages plus
            # the misses, minus what the budget allows (with the budget equal
            # to the whole area this is misses minus free slots)
            n_resident = int(np.sum(self.owner[b] != FREE))
            need = max(0, n_resident + len(misses) - self.budget[b])
            st = self.stats[b]
            st["hits"] += len(M) - len(misses)
            st["misses"] += len(misses)
            st["cutoff"] = -1
            if need > 0:
                victims, cut = self.choose_victims(b, need, mand, t)
                self.evict(b, victims)
                st["evictions"] += len(victims)
                st["cutoff"] = cut
            free_slots = [c for c in range(self.C) if self.owner[b, c] == FREE]
            for (h, page, bi), c in zip(misses, free_slots):
                self.owner[b, c] = h * self.max_pages + page
                self.last_use[b, c] = t
                blocks[b][h][bi][0] = b * self.C + c
                inserts.append((b, h, page, c, blocks[b][h][bi][1]))
        for (b, h, page, c, ntok) in inserts:
            self.insert(b, h, page, c)
            self._pending.append((b * self.C + c, b, h, page, ntok))
        return blocks

    def retrieve(self):
        """Fig. 5 steps 3-4: copy each missed page from its host address into
        its GPU slot: the keys and values of its valid tokens verbatim, and
        zeros in every other token slot of the page, whatever the host holds
        there (reading R25: token slots past a partition's last token carry
        nothing the method uses).  Returns the bytes that land in the pool."""
        D = self.D
        for gslot, b, h, page, ntok in self._pending:
            src = self.requests[b].host[h, page]
            dst = np.zeros(PAGE_ELEMS, np.uint16)
            dst[: ntok * D] = src[: ntok * D]                        # key rows, token-major
            vs = src[PAGE_TOKENS * D:].reshape(D, PAGE_TOKENS)       # values, dim-major
            dst[PAGE_TOKENS * D:].reshape(D, PAGE_TOKENS)[:, :ntok] = vs[:, :ntok]
            self.pool[gslot] = dst
        return len(self._pending) * PAGE_ELEMS * 2

    # ------------------------------------------------------------------ Attention
    def attend_group(self, q_bits: np.ndarray, b: int, h: int, blocks) -> np.ndarray:
        """Outputs of the G query heads of KV head h of request b:
        softmax(q K^T / sqrt(D)) V over the valid tokens of the (b, h)
        block-table pages, read from the GPU-side pool copy (GQA: query head g
        uses KV head g // G).  float64, returned as float32 [G][D]."""
        Ks, Vs = [], []
        for gslot, ntok in blocks[b][h]:
            Ks.append(page_keys(self.pool[gslot], self.D)[:ntok])
            Vs.append(page_values(self.pool[gslot], self.D)[:ntok])
        out = np.zeros((self.G, self.D), np.float32)
        if not Ks:
            return out
        K = np.concatenate(Ks, axis=0)
        V = np.concatenate(Vs, axis=0)
        q = bf16_bits_to_f64(q_bits.reshape(self.B, self.Hq, self.D)[b])
        for j in range(self.G):
            logits = (K @ q[h * self.G + j]) / math.sqrt(self.D)
            w = np.exp(logits - logits.max())
            out[j] = ((w @ V) / w.sum()).astype(np.float32)
        return out

    def attend_one(self, q_bits: np.ndarray, b: int, g: int, blocks) -> np.ndarray:
        return self.attend_group(q_bits, b, g // self.G, blocks)[g % self.G]

    def attend(self, q_bits: np.ndarray, blocks) -> np.ndarray:
        out = np.zeros((self.B, self.Hq, self.D), np.float32)
        for b in range(self.B):
            for h in range(self.Hkv):
                out[b, h * self.G:(h + 1) * self.G] = self.attend_group(q_bits, b, h, blocks)
        return out

    # ------------------------------------------------------------------ one full step
    def step(self, q_bits: np.ndarray, t: int):
        sel, sc = self.select(q_bits)
        blocks = self.resolve_evict(sel, t)
        self.retrieve()
        out = self.attend(q_bits, blocks)
        return sel, blocks, out

    # ------------------------------------------------------------------ flat views for comparison
    def flat_page_table(self, b: int, h: int, n_pages: int) -> np.ndarray:
        return np.array([self.translate(b, h, p) for p in range(n_pages)], np.int64)

    def block_arrays(self, blocks, max_blocks: int):
        """Block tables as dense arrays: slots [B][Hkv][max_blocks] (FREE past
        the count), valid tokens (0 past the count), counts [B][Hkv]."""
        slots = np.full((self.B, self.Hkv, max_blocks), FREE, np.int64)
        ntok = np.zeros((self.B, self.Hkv, max_blocks), np.int64)
        cnt = np.zeros((self.B, self.Hkv), np.int64)
        for b in range(self.B):
            for h in range(self.Hkv):
                lst = blocks[b][h]
                cnt[b, h] = len(lst)
                for i, (s, n) in enumerate(lst):
                    slots[b, h, i] = s
                    ntok[b, h, i] = n
        return slots, ntok, cnt
