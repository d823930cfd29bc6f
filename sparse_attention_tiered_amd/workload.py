"""Seeded synthetic inputs for the sparse-decode step.

This module only *draws* inputs: paged bf16 K/V in the host layout the library
reads, per-step bf16 queries, and (for the variable-partition workload) the
partition lengths.  It holds none of the method's arithmetic (no summaries, no
scores, no selection, no residency policy, no attention), so both the HIP path
and the CPU oracle can be fed from it without sharing any code with each other.

Workload shapes follow the five decode-layer workloads the method is measured
on: the Qwen3-14B / Qwen3-32B / Llama-3.1-70B attention shapes (grouped-query
heads, head_dim 128) at 32K, 128K and 1M-token contexts.  The pages evaluate on
LongBench-v2 and LongGenBench with real models; neither the datasets nor the
weights are used here, only these shapes, with random data whose structure
(hot partitions, drifting hot sets, clustered keys, AR(1) query streams) gives
the selection step something non-trivial to find.

Host KV layout (one request): ``[Hkv][pages][16384]`` uint16 (bf16 bits).  A
page holds 64 token slots of one KV head: the 64x128 keys row-major
(token-major), then the values *transposed*, 128x64 (dim-major).  Token slots
past a partition's length on its last page are zero.  A partition always starts
on a fresh page.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

PAGE_TOKENS = 64
HEAD_DIM = 128
PAGE_ELEMS = 2 * PAGE_TOKENS * HEAD_DIM      # uint16 elements per page (K + V^T)
PAGE_BYTES = PAGE_ELEMS * 2                  # 32 KiB

# substream tags for SeedSequence([seed, cfg_id, b, x, tag])
_Q_INIT, _Q_INNOV, _K_NOISE, _V_NOISE, _HOT, _DRIFT_DIR, _CENTROID, _ASSIGN, _LENS = range(9)


@dataclass(frozen=True)
class Workload:
    """One synthetic decode-layer workload.

    ``ctx`` is the context length of each request (a tuple, so requests may be
    ragged).  ``part_len`` is 64 for fixed one-page partitions; ``var_len`` =
    (lo, hi) instead draws per-request partition lengths uniformly in [lo, hi].
    ``kv_kind`` picks the key structure: "hot" (a few partitions per head pushed
    toward the group's initial query direction), "drift" (a hot set that
    changes over time and pulls the queries with it), "cluster" (keys scattered
    around seeded centroids), "ties" (every key of a head is one seeded vector,
    the hot partitions shifted as in "hot", so scores tie exactly within the
    two groups), or "plain".
    """

    name: str
    cfg_id: int
    B: int
    Hq: int
    Hkv: int
    ctx: tuple
    k: int
    slots_per_request: int
    steps: int
    kv_kind: str = "hot"
    hot_count: int = 0
    hot_shift: float = 2.0
    drift_every: int = 16
    drift_replace: int = 0
    n_centroids: int = 4096
    cluster_std: float = 0.5
    var_len: tuple | None = None
    ar_coef: float = 0.9
    seed: int = 0
    D: int = HEAD_DIM
    layers: int = 1          # attention layers of the model whose shape this is

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


def _std(name, cfg_id, B, Hq, Hkv, ctx, k, steps, **kw):
    max_ppp = 1 if kw.get("var_len") is None else -(-kw["var_len"][1] // PAGE_TOKENS)
    slots = kw.pop("slots", None)
    if slots is None:
        # per request: every KV head keeps its k mandatory partitions plus a
        # buffer five times that size
        slots = Hkv * 6 * k * max_ppp
    return Workload(name=name, cfg_id=cfg_id, B=B, Hq=Hq, Hkv=Hkv, ctx=tuple([ctx] * B),
                    k=k, slots_per_request=slots, steps=steps, **kw)


# The five workloads, sized as stated for the method's decode layer.
C1 = _std("c1_tiny", 1, 1, 8, 2, 4096, 8, 16, kv_kind="hot", hot_count=4)
C2 = _std("c2_qwen3_14b_32k", 2, 16, 40, 8, 32768, 32, 64, kv_kind="hot", hot_count=5, layers=40)
C3 = _std("c3_qwen3_32b_128k", 3, 8, 64, 8, 131072, 64, 128, kv_kind="drift", hot_count=20,
          drift_every=16, drift_replace=2, layers=64)
# pool capped at a quarter of the summed per-request budget: 768 slots each
C4 = _std("c4_llama70b_128k_pressure", 4, 32, 64, 8, 131072, 64, 128, kv_kind="hot",
          hot_count=20, slots=(8 * 6 * 64) // 4, layers=80)
C5 = _std("c5_cluster_1m", 5, 4, 32, 8, 1 << 20, 128, 64, kv_kind="cluster",
          var_len=(16, 256), layers=64)

WORKLOADS = {w.name: w for w in (C1, C2, C3, C4, C5)}
ALIASES = {"c1": C1.name, "c2": C2.name, "c3": C3.name, "c4": C4.name, "c5": C5.name}


def get(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


def variant(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields changed (``ctx`` may be an int or a tuple)."""
    if "ctx" in changes and isinstance(changes["ctx"], int):
        changes["ctx"] = tuple([changes["ctx"]] * changes.get("B", w.B))
    elif "B" in changes and "ctx" not in changes:
        changes["ctx"] = tuple([w.ctx[0]] * changes["B"])
    return dataclasses.replace(w, **changes)


def _rng(w: Workload, b: int, x: int, tag: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([w.seed, w.cfg_id, b, x, tag]))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


# ----------------------------------------------------------------------------- geometry
def partition_lengths(w: Workload, b: int) -> np.ndarray:
    """Token length of every partition of request ``b`` (int32)."""
    n = w.ctx[b]
    if n == 0:
        return np.zeros(0, np.int32)
    if w.var_len is None:
        full, tail = divmod(n, PAGE_TOKENS)
        lens = [PAGE_TOKENS] * full + ([tail] if tail else [])
        return np.asarray(lens, np.int32)
    lo, hi = w.var_len
    rng = _rng(w, b, 0, _LENS)
    out, total = [], 0
    while total < n:
        draw = rng.integers(lo, hi + 1, size=4096)
        for L in draw:
            L = int(min(L, n - total))
            out.append(L)
            total += L
            if total >= n:
                break
    return np.asarray(out, np.int32)


def pages_for(lens: np.ndarray) -> int:
    """Pages per KV head of a request whose partitions have lengths ``lens``."""
    return int(np.sum((lens.astype(np.int64) + PAGE_TOKENS - 1) // PAGE_TOKENS))


def max_pages_per_partition(w: Workload) -> int:
    return 1 if w.var_len is None else -(-w.var_len[1] // PAGE_TOKENS)


@dataclass
class Geometry:
    lens: list            # per request: int32 partition lengths
    pages: list           # per request: pages per KV head
    max_parts: int
    max_pages: int
    max_ppp: int


def geometry(w: Workload) -> Geometry:
    lens = [partition_lengths(w, b) for b in range(w.B)]
    pages = [pages_for(l) for l in lens]
    return Geometry(lens=lens, pages=pages, max_parts=max([len(l) for l in lens] + [1]),
                    max_pages=max(pages + [1]), max_ppp=max_pages_per_partition(w))


# ----------------------------------------------------------------------------- structure draws
def _hot_sets(w: Workload, b: int, h: int, n_parts: int, n_epochs: int):
    """Per epoch, the set of hot partition ids of one (request, KV head)."""
    if w.hot_count == 0 or n_parts == 0:
        return [np.zeros(0, np.int64)] * n_epochs
    rng = _rng(w, b, h, _HOT)
    cnt = min(w.hot_count, n_parts)
    cur = np.sort(rng.choice(n_parts, size=cnt, replace=False))
    sets = [cur]
    for _ in range(1, n_epochs):
        if w.kv_kind != "drift" or w.drift_replace == 0:
            sets.append(cur)
            continue
        r = min(w.drift_replace, cnt, n_parts - cnt)
        drop = rng.choice(cnt, size=r, replace=False)
        outside = np.setdiff1d(np.arange(n_parts), cur)
        add = rng.choice(outside, size=r, replace=False)
        cur = np.sort(np.concatenate([np.delete(cur, drop), add]))
        sets.append(cur)
    return sets


def _unit(v):
    n = np.linalg.norm(v)
    return v / n if n > 0 else v


@dataclass
class Draws:
    """Everything random that is not the bulk K/V noise."""
    q_bits: np.ndarray                 # [steps][B][Hq][D] uint16
    hot: dict = field(default_factory=dict)         # (b,h) -> list of per-epoch hot id arrays
    hot_dir: dict = field(default_factory=dict)     # (b,h) -> [D] fp32 shift direction (hot)
    drift_dirs: dict = field(default_factory=dict)  # (b,h) -> {pid: [D] unit vector}


def draw_queries(w: Workload, geo: Geometry, n_steps: int | None = None) -> Draws:
    """AR(1) query streams q_t = a*q_{t-1} + (1-a)*xi_t per query head, with
    q_0 ~ N(0, I).  For the drifting workload the innovations have mean
    mu_e = sum of the unit directions of the epoch's hot partitions."""
    T = w.steps if n_steps is None else n_steps
    D, G = w.D, w.G
    n_epochs = max(1, -(-T // w.drift_every))
    d = Draws(q_bits=np.zeros((T, w.B, w.Hq, D), np.uint16))
    state = np.zeros((w.B, w.Hq, D), np.float32)
    innov = np.zeros((w.B, w.Hq, T, D), np.float32)
    for b in range(w.B):
        for g in range(w.Hq):
            rq = _rng(w, b, g, _Q_INIT)
            state[b, g] = rq.standard_normal(D, dtype=np.float32)
            innov[b, g] = _rng(w, b, g, _Q_INNOV).standard_normal((T, D), dtype=np.float32)
    for b in range(w.B):
        n_parts = len(geo.lens[b])
        for h in range(w.Hkv):
            sets = _hot_sets(w, b, h, n_parts, n_epochs)
            d.hot[(b, h)] = sets
            if w.kv_kind in ("hot", "ties"):
                d.hot_dir[(b, h)] = _unit(state[b, h * G:(h + 1) * G].sum(0)).astype(np.float32)
            elif w.kv_kind == "drift":
                ever = np.unique(np.concatenate(sets)) if sets else np.zeros(0, np.int64)
                rd = _rng(w, b, h, _DRIFT_DIR)
                dirs = {int(p): _unit(rd.standard_normal(D)).astype(np.float32) for p in ever}
                d.drift_dirs[(b, h)] = dirs
                for t in range(T):
                    e = t // w.drift_every
                    mu = np.zeros(D, np.float32)
                    for p in sets[e]:
                        mu += dirs[int(p)]
                    innov[b, h * G:(h + 1) * G, t] += mu
    a = np.float32(w.ar_coef)
    for t in range(T):
        if t > 0:
            state = a * state + (np.float32(1) - a) * innov[:, :, t]
        d.q_bits[t] = to_bf16_bits(state)
    return d


# ----------------------------------------------------------------------------- bulk K/V
def _fill_head(w: Workload, b: int, h: int, lens: np.ndarray, out: np.ndarray, draws: Draws):
    """Write the pages of one (request, KV head) into ``out`` ([pages][16384] uint16)."""
    D = w.D
    n_tok = int(lens.sum())
    if n_tok == 0:
        return
    K = _rng(w, b, h, _K_NOISE).standard_normal((n_tok, D), dtype=np.float32)
    V = _rng(w, b, h, _V_NOISE).standard_normal((n_tok, D), dtype=np.float32)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    if w.kv_kind == "cluster":
        rc = _rng(w, b, h, _CENTROID)
        cent = rc.standard_normal((w.n_centroids, D), dtype=np.float32)
        assign = _rng(w, b, h, _ASSIGN).integers(0, w.n_centroids, size=len(lens))
        K *= np.float32(w.cluster_std)
        K += np.repeat(cent[assign], lens, axis=0)
    elif w.kv_kind == "ties":
        K[:] = K[0]
        for p in draws.hot[(b, h)][0]:
            K[starts[p]:starts[p] + lens[p]] += np.float32(w.hot_shift) * draws.hot_dir[(b, h)]
    elif w.kv_kind in ("hot", "drift"):
        sets = draws.hot[(b, h)]
        if w.kv_kind == "hot":
            for p in sets[0]:
                K[starts[p]:starts[p] + lens[p]] += np.float32(w.hot_shift) * draws.hot_dir[(b, h)]
        else:
            for p, e in draws.drift_dirs[(b, h)].items():
                K[starts[p]:starts[p] + lens[p]] += np.float32(w.hot_shift) * e
    pages = out.shape[0]
    kb, vb = to_bf16_bits(K), to_bf16_bits(V)
    del K, V
    if w.var_len is None and n_tok == pages * PAGE_TOKENS:
        Kp = kb.reshape(pages, PAGE_TOKENS, D)
        Vp = vb.reshape(pages, PAGE_TOKENS, D)
    else:
        npg = (lens.astype(np.int64) + PAGE_TOKENS - 1) // PAGE_TOKENS
        first = np.concatenate([[0], np.cumsum(npg)[:-1]])
        # destination token slot of every token: partition start page * 64 + offset
        dest = np.repeat(first * PAGE_TOKENS - starts, lens) + np.arange(n_tok)
        Kp = np.zeros((pages * PAGE_TOKENS, D), np.uint16)
        Vp = np.zeros((pages * PAGE_TOKENS, D), np.uint16)
        Kp[dest] = kb
        Vp[dest] = vb
        Kp = Kp.reshape(pages, PAGE_TOKENS, D)
        Vp = Vp.reshape(pages, PAGE_TOKENS, D)
    half = PAGE_TOKENS * D
    out[:, :half] = Kp.reshape(pages, half)
    out[:, half:] = Vp.transpose(0, 2, 1).reshape(pages, half)


def fill_request(w: Workload, b: int, geo: Geometry, draws: Draws, out: np.ndarray,
                 threads: int | None = None):
    """Fill ``out`` (uint16, at least Hkv*pages*16384 elements) with request b's paged KV."""
    pages = geo.pages[b]
    view = out[: w.Hkv * pages * PAGE_ELEMS].reshape(w.Hkv, pages, PAGE_ELEMS)
    nthr = threads or min(16, os.cpu_count() or 1)
    if nthr <= 1 or w.Hkv == 1:
        for h in range(w.Hkv):
            _fill_head(w, b, h, geo.lens[b], view[h], draws)
        return view
    with ThreadPoolExecutor(min(nthr, w.Hkv)) as ex:
        list(ex.map(lambda h: _fill_head(w, b, h, geo.lens[b], view[h], draws), range(w.Hkv)))
    return view


def fill_all(w: Workload, geo: Geometry, draws: Draws, outs: list, threads: int | None = None):
    """Fill every request's buffer; jobs are (request, head) pairs spread over threads."""
    nthr = threads or min(16, os.cpu_count() or 1)
    views = []
    for b in range(w.B):
        pages = geo.pages[b]
        views.append(outs[b][: w.Hkv * pages * PAGE_ELEMS].reshape(w.Hkv, pages, PAGE_ELEMS))
    jobs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    if nthr <= 1:
        for b, h in jobs:
            _fill_head(w, b, h, geo.lens[b], views[b][h], draws)
    else:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(lambda j: _fill_head(w, j[0], j[1], geo.lens[j[0]], views[j[0]][j[1]], draws),
                        jobs))
    return views


def host_kv_numpy(w: Workload, geo: Geometry, draws: Draws, threads: int | None = None):
    """Plain numpy buffers (one per request) for CPU-only use."""
    outs = [np.zeros(w.Hkv * max(geo.pages[b], 1) * PAGE_ELEMS, np.uint16) for b in range(w.B)]
    fill_all(w, geo, draws, outs, threads)
    return outs
