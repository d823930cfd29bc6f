"""Drive the HIP library and the CPU oracle side by side on the same seeded inputs.

Stage parity (Pair.run): at every step the GPU's selection is checked against
the oracle's (exact, except members whose oracle scores are within 1e-5 of the
oracle's k-th score); then the GPU's resolve is fed the *oracle's* selection,
so a legitimate near-tie cannot cascade into a state mismatch, and the whole
residency state is compared bit for bit; every pool slot the step filled is
compared byte for byte with the oracle's copy of the host page (its valid
tokens, zeros in the other token slots), and the
device's count of bytes read over the link must have grown by exactly the
valid key rows and the value halves of those pages; attention outputs are
compared within max-abs 2e-3.  Nothing the GPU produces is fed to the oracle.

Whole-step parity (Pair.run_graph, the benchmark's captured one-launch step):
the GPU selects for itself, so once its selection is shown valid (equal to the
oracle's, or differing only by near-ties within the window) the oracle resolves
that selection: the one place where a GPU result enters the oracle, and only
after it has been checked.  The number of lists where the two selections
differ (tie flips) is counted and must not exceed the run's `max_flips`
(0 unless a workload is declared to have near-ties).
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

from oracle.spin_oracle import SpinOracle
from sparse_attention_tiered_amd import binding as bd
from sparse_attention_tiered_amd import workload as W

TIE_WINDOW = 1e-5
OUT_TOL = 2e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Pair:
    """The GPU context and the oracle, indexed with the same host KV."""

    def __init__(self, w: W.Workload, n_steps=None, attend_pps=0, num_segments=None,
                 slots=None, oracle=True, threads=None, offload_extra_pages=None,
                 host_segments=False, max_pages=None, pad_fill=None):
        t0 = time.time()
        self.w = w
        self.geo = geo = W.geometry(w)
        self.draws = W.draw_queries(w, geo, n_steps)
        self.T = self.draws.q_bits.shape[0]
        C = w.slots_per_request if slots is None else slots
        extra = offload_extra_pages or 0
        sized_pages = max_pages
        max_parts, max_pages = geo.max_parts + extra, geo.max_pages + extra
        if sized_pages is not None:
            # a context sized for longer requests than it holds: a larger
            # directory (and partition table) than the data needs
            max_pages = max(sized_pages, max_pages)
            max_parts = max(max_parts, -(-max_pages // geo.max_ppp))
        self.cfg = bd.make_config(w.B, w.Hq, w.Hkv, max_parts, max_pages, w.k, C,
                                  num_segments=num_segments, max_pages_per_partition=geo.max_ppp,
                                  attend_pages_per_split=attend_pps, host_segments=host_segments)
        self.spin = bd.Spin(self.cfg)
        self.oracle = None
        if oracle:
            self.oracle = SpinOracle(w.B, w.Hq, w.Hkv, w.k, C, max_pages, self.cfg.num_segments)
        if offload_extra_pages is None:
            # the full KV starts in pinned host memory and is indexed there
            self.host = [bd.pinned_u16(w.Hkv * max(geo.pages[b], 1) * W.PAGE_ELEMS) for b in range(w.B)]
            W.fill_all(w, geo, self.draws, [h[1] for h in self.host], threads)
            if pad_fill is not None:
                self._fill_padding(pad_fill)
            for b in range(w.B):
                lens = geo.lens[b] if w.var_len is not None else None
                self.spin.index(b, self.host[b][0], w.ctx[b], lens)
                if oracle:
                    self.oracle.index(b, self.host[b][1], geo.lens[b])
        else:
            # prefill side: the KV starts in device memory and is offloaded
            kv = W.host_kv_numpy(w, geo, self.draws, threads)
            self.host = []
            for b in range(w.B):
                cap = geo.pages[b] + extra
                t = torch.zeros(w.Hkv * cap * W.PAGE_ELEMS, dtype=torch.int16, pin_memory=True)
                self.host.append((t, t.numpy().view(np.uint16)))
                pages = kv[b][: w.Hkv * geo.pages[b] * W.PAGE_ELEMS]
                d_kv = torch.from_numpy(pages.view(np.int16)).to("cuda")
                lens = geo.lens[b] if w.var_len is not None else None
                self.spin.offload(b, d_kv, t, w.ctx[b], lens)
                if oracle:
                    self.oracle.offload(b, pages.reshape(w.Hkv, geo.pages[b], W.PAGE_ELEMS), geo.lens[b], cap)
        self.q_dev = torch.from_numpy(self.draws.q_bits.view(np.int16)).to("cuda")
        self.scores = torch.empty((w.B, w.Hkv, max_parts), dtype=torch.float32, device="cuda")
        log(f"[setup] {w.name} B={w.B} ctx={w.ctx[0]} C={C} segs={self.cfg.num_segments} "
            f"splits={self.spin.splits} in {time.time() - t0:.1f}s")

    def _fill_padding(self, value):
        """Write `value` into every key and value entry of every token slot
        past a page's valid tokens, in the host copy (which the library is
        told to ignore, and the oracle's transfer leaves as zeros)."""
        D, T = W.HEAD_DIM, W.PAGE_TOKENS
        for b in range(self.w.B):
            ntok = []
            for L in self.geo.lens[b]:
                L = int(L)
                ntok += [min(T, L - T * j) for j in range(-(-L // T))]
            pages = self.host[b][1][: self.w.Hkv * len(ntok) * W.PAGE_ELEMS].reshape(
                self.w.Hkv, len(ntok), W.PAGE_ELEMS)
            for p, n in enumerate(ntok):
                if n < T:
                    for h in range(self.w.Hkv):
                        pages[h, p, n * D:T * D] = value
                        pages[h, p, T * D:].reshape(D, T)[:, n:] = value  # (a view: rows are contiguous)

    # ------------------------------------------------------------------ checks
    def n_parts(self, b):
        """Partitions of request b now (appends add some; a released request
        has none)."""
        if self.oracle is None:
            return len(self.geo.lens[b])
        r = self.oracle.requests[b]
        return r.n_parts if r is not None else 0

    def check_summaries(self):
        for b in range(self.w.B):
            n = self.n_parts(b)
            if n == 0:
                continue
            got = self.spin.summaries(b, n)
            want = self.oracle.requests[b].summaries
            # within 2 float32 ulp (the accumulation is exact, so normally equal)
            np.testing.assert_array_almost_equal_nulp(got, want, nulp=2)

    def check_select(self, t, sel_gpu, scores_gpu):
        sel_o, sc_o = self.oracle.select(self.draws.q_bits[t])
        k = self.w.k
        flips = 0
        for b in range(self.w.B):
            n = self.n_parts(b)
            for h in range(self.w.Hkv):
                g = sel_gpu[b, h]
                o = sel_o[b, h]
                m = min(k, n)
                assert np.all(g[m:] == -1) and np.all(o[m:] == -1)
                assert np.all(np.diff(g[:m]) > 0), ("GPU selection not ascending", b, h)
                if n:
                    s = sc_o[b][h]
                    # float32 dot products of 128 terms against the float64 oracle
                    tol = 1e-6 + 4e-6 * float(np.max(np.abs(s)))
                    assert np.max(np.abs(scores_gpu[b, h, :n] - s)) < tol, ("score", b, h)
                    assert np.all(np.isneginf(scores_gpu[b, h, n:]))
                if set(g[:m]) != set(o[:m]):
                    kth = np.sort(sc_o[b][h])[::-1][k - 1]
                    for p in set(g[:m]) ^ set(o[:m]):
                        assert abs(sc_o[b][h][p] - kth) <= TIE_WINDOW, (
                            f"step {t} b{b} h{h}: partition {p} score {sc_o[b][h][p]} vs k-th {kth}")
                    flips += 1
        return sel_o, flips

    def check_state(self, t):
        snap = self.spin.snapshot()
        o = self.oracle
        top = int(snap["seg_top"][0])
        assert top == len(o.free_stack), (t, top, len(o.free_stack))
        assert np.array_equal(snap["seg_stack"][:top], np.asarray(o.free_stack, np.int32)), t
        for name in ("directory", "segments", "seg_live", "owner", "last_use"):
            a, b = snap[name], getattr(o, name).astype(np.int32)
            if not np.array_equal(a, b):
                idx = np.argwhere(a != b)[:5]
                raise AssertionError(f"step {t}: {name} differs at {idx.tolist()}: "
                                     f"gpu {a[tuple(idx.T)]} oracle {b[tuple(idx.T)]}")
        free_o = np.sum(o.owner == -1, axis=1).astype(np.int32)
        assert np.array_equal(snap["free_count"], free_o), t

    def check_blocks(self, t, blocks):
        slots, ntok, cnt = self.oracle.block_arrays(blocks, self.spin.max_blocks)
        assert np.array_equal(self.spin.block_count.cpu().numpy(), cnt), t
        assert np.array_equal(self.spin.block_table.cpu().numpy(), slots), t
        assert np.array_equal(self.spin.block_ntok.cpu().numpy(), ntok), t

    def _pool_rows(self, gslots):
        pool = self.spin.pool.view(torch.int16).view(-1, W.PAGE_ELEMS)
        idx = torch.as_tensor(np.asarray(gslots, np.int64), device=pool.device)
        return pool.index_select(0, idx).cpu().numpy().view(np.uint16)

    def check_pool(self, gslots, what="step"):
        """The GPU pool rows of `gslots` (global slots) equal the oracle's,
        byte for byte (the retrieved K and V bytes are the host page's)."""
        gslots = np.asarray(gslots, np.int64)
        for a in range(0, len(gslots), 4096):   # at most 128 MiB at a time
            part = gslots[a:a + 4096]
            got = self._pool_rows(part)
            want = self.oracle.pool[part]
            if not np.array_equal(got, want):
                bad = [int(s) for s, g, o in zip(part, got, want) if not np.array_equal(g, o)]
                raise AssertionError(f"{what}: pool slots {bad[:8]} ({len(bad)} of {len(part)}) "
                                     "differ from the host pages they hold")
        return len(gslots)

    def check_inserted(self, t):
        """Every slot this step's retrieve filled."""
        return self.check_pool([g for g, *_ in self.oracle._pending], f"step {t} inserts")

    def check_link_bytes(self, t, blocks):
        """The step's transfer read over the link exactly the key rows of each
        inserted page's valid tokens (256 bytes each) and its whole value half
        (16 KiB): the device's byte counter moved by that much since the last
        check."""
        ntok = {}
        for b in range(self.w.B):
            for h in range(self.w.Hkv):
                for g, n in blocks[b][h]:
                    ntok[g] = n
        want = sum(256 * ntok[g] + 16384 for g, *_ in self.oracle._pending)
        now = self.spin.stats()[0].h2d_bytes
        assert now - self._h2d == want, (t, now - self._h2d, want)
        self._h2d = now

    def check_resident(self):
        """Every resident slot of every request."""
        o = self.oracle
        b_idx, c_idx = np.nonzero(o.owner != -1)
        return self.check_pool(b_idx * o.C + c_idx, "resident pages")

    def check_stats(self):
        st, per = self.spin.stats()
        assert st.error_word == 0, st.error_word
        for b in range(self.w.B):
            so = self.oracle.stats[b]
            assert (per[b, 0], per[b, 1], per[b, 2], per[b, 3]) == \
                (so["hits"], so["misses"], so["evictions"], so["cutoff"]), (b, per[b], so)
        return st

    # ------------------------------------------------------------------ request turnover
    def release_request(self, b):
        """Release request b on both sides."""
        self.spin.release(b)
        self.oracle.release(b)

    def reindex_request(self, b, n_tokens, seed):
        """Index request b again, on both sides, with fresh KV of n_tokens tokens
        in one-page partitions (N(0,1) bf16, zero padding on a partial last
        page), whatever it held before."""
        Hkv = self.w.Hkv
        lens = [64] * (n_tokens // 64) + ([n_tokens % 64] if n_tokens % 64 else [])
        pages = len(lens)
        rng = np.random.default_rng([4242, seed, b])
        bits = W.to_bf16_bits(rng.standard_normal((Hkv, pages, W.PAGE_ELEMS), dtype=np.float32))
        if n_tokens % 64:
            tail = n_tokens % 64
            bits[:, -1, tail * 128: 64 * 128] = 0
            bits[:, -1, 64 * 128:].reshape(Hkv, 128, 64)[:, :, tail:] = 0
        t, u16 = bd.pinned_u16(Hkv * max(pages, 1) * W.PAGE_ELEMS)
        u16[: bits.size] = bits.reshape(-1)
        self.spin.index(b, t, n_tokens)
        self.oracle.index(b, u16, np.asarray(lens, np.int64))
        self.host[b] = (t, u16)

    # ------------------------------------------------------------------ stepping
    def append_token(self, t):
        """One seeded token per request, appended on both sides."""
        rng = np.random.default_rng([777, t])
        kv = rng.standard_normal((2, self.w.B, self.w.Hkv, 128), dtype=np.float32)
        bits = W.to_bf16_bits(kv)
        dk = torch.from_numpy(bits[0].view(np.int16)).to("cuda")
        dv = torch.from_numpy(bits[1].view(np.int16)).to("cuda")
        self.spin.append(dk, dv)
        self.oracle.append(bits[0], bits[1])

    def check_host(self):
        """The pinned host buffers (written by the offload copy and the append
        kernel) equal the oracle's own host copies byte for byte."""
        for b in range(self.w.B):
            req = self.oracle.requests[b]
            gpu = self.host[b][1][: req.host.size].reshape(req.host.shape)
            assert np.array_equal(gpu, req.host), b

    def run(self, steps=None, out_sample=None, check_every=1, seed=0, on_step=None, append=False,
            max_flips=0):
        """Full stage parity for `steps` steps.  out_sample=None compares every
        output; an int compares that many (b, g) pairs per step, chosen with a
        seeded generator, computed one by one by the oracle.  on_step(t) runs
        before step t (budget changes, releases, re-indexing on both sides)."""
        steps = self.T if steps is None else steps
        rng = np.random.default_rng(seed)
        total_flips = 0
        checked = 0
        worst = 0.0
        self._h2d = self.spin.stats()[0].h2d_bytes
        for t in range(steps):
            if on_step is not None:
                on_step(t)
            if append:
                self.append_token(t)
            q = self.q_dev[t]
            self.spin.select(q, scores=self.scores)
            sel_gpu = self.spin.sel.cpu().numpy()
            sel_o, flips = self.check_select(t, sel_gpu, self.scores.cpu().numpy())
            total_flips += flips
            self.spin.sel.copy_(torch.from_numpy(sel_o.astype(np.int32)))
            self.spin.resolve_evict(t)
            blocks = self.oracle.resolve_evict(sel_o, t)
            if t % check_every == 0 or t == steps - 1:
                self.check_state(t)
                self.check_blocks(t, blocks)
            self.spin.retrieve()
            self.oracle.retrieve()
            self.check_link_bytes(t, blocks)
            self.last_blocks = blocks
            out = self.spin.attend(q).cpu().numpy()
            qb = self.draws.q_bits[t]
            if out_sample is None:
                want = self.oracle.attend(qb, blocks)
                err = float(np.max(np.abs(out - want)))
            else:
                err = 0.0
                for _ in range(out_sample):
                    b = int(rng.integers(self.w.B))
                    g = int(rng.integers(self.w.Hq))
                    want = self.oracle.attend_one(qb, b, g, blocks)
                    err = max(err, float(np.max(np.abs(out[b, g] - want))))
            worst = max(worst, err)
            assert err <= OUT_TOL, (t, err)
            checked += self.check_inserted(t)
        st = self.check_stats()
        resident = self.check_resident()
        self.flips = total_flips
        log(f"[parity] {self.w.name}: {steps} steps, hits={st.hits} misses={st.misses} "
            f"evictions={st.evictions} tie-flips={total_flips} max|out-oracle|={worst:.2e} "
            f"pool bytes checked: {checked} inserts, {resident} resident")
        assert total_flips <= max_flips, f"{total_flips} lists selected differently within the tie window"
        return st, worst

    def valid_selection(self, t, sel_gpu):
        """The GPU's selection, checked against the oracle's: the same sets
        except partitions whose scores tie the k-th within TIE_WINDOW, ascending,
        -1 padded.  Returns the number of (request, head) lists that differ."""
        sel_o, sc_o = self.oracle.select(self.draws.q_bits[t])
        k = self.w.k
        flips = 0
        for b in range(self.w.B):
            n = self.n_parts(b)
            for h in range(self.w.Hkv):
                g, o = sel_gpu[b, h], sel_o[b, h]
                m = min(k, n)
                assert np.all(g[m:] == -1) and np.all(o[m:] == -1)
                assert np.all(np.diff(g[:m]) > 0), ("GPU selection not ascending", b, h)
                if set(g[:m]) != set(o[:m]):
                    kth = np.sort(sc_o[b][h])[::-1][k - 1]
                    for p in set(g[:m]) ^ set(o[:m]):
                        assert 0 <= p < n and abs(sc_o[b][h][p] - kth) <= TIE_WINDOW, (
                            f"step {t} b{b} h{h}: partition {p} vs k-th {kth}")
                    flips += 1
        return flips

    def run_graph(self, steps=None, out_sample=None, seed=0, on_step=None, max_flips=0):
        """The benchmark's timed configuration: one spin_step_at call (the
        transfer and the resident-page attention in one launch, the step index
        on the device) captured in a HIP graph and replayed once per step.
        Each step the oracle takes the GPU's selection once it is shown valid,
        then the whole residency state, the block tables, the pool slots the
        step filled and sampled outputs are compared.  on_step(t) runs before
        step t's replay (eager library calls between replays)."""
        steps = self.T if steps is None else steps
        rng = np.random.default_rng(seed)
        checked = 0
        S, C = torch.cuda.Stream(), torch.cuda.Stream()
        t_dev = torch.zeros(1, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        graph = None
        flips_total, worst = 0, 0.0
        self._h2d = self.spin.stats()[0].h2d_bytes
        for t in range(steps):
            if on_step is not None:
                on_step(t)
                torch.cuda.synchronize()
            if t == 0:  # eagerly, then capture the step once
                self.spin.step_at(self.q_dev, t_dev, stream=S, copy_stream=C)
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=S):
                    self.spin.step_at(self.q_dev, t_dev, stream=S, copy_stream=C)
                torch.cuda.synchronize()
                assert int(t_dev.item()) == 1
            else:
                with torch.cuda.stream(S):
                    graph.replay()
                torch.cuda.synchronize()
                assert int(t_dev.item()) == t + 1
            sel_gpu = self.spin.sel.cpu().numpy()
            flips_total += self.valid_selection(t, sel_gpu)
            blocks = self.oracle.resolve_evict(sel_gpu.astype(np.int64), t)
            self.check_state(t)
            self.check_blocks(t, blocks)
            self.oracle.retrieve()
            self.check_link_bytes(t, blocks)
            out = self.spin.out.cpu().numpy()
            qb = self.draws.q_bits[t]
            if out_sample is None:
                err = float(np.max(np.abs(out - self.oracle.attend(qb, blocks))))
            else:
                err = 0.0
                for _ in range(out_sample):
                    b = int(rng.integers(self.w.B))
                    g = int(rng.integers(self.w.Hq))
                    want = self.oracle.attend_one(qb, b, g, blocks)
                    err = max(err, float(np.max(np.abs(out[b, g] - want))))
            worst = max(worst, err)
            assert err <= OUT_TOL, (t, err)
            checked += self.check_inserted(t)
        st = self.check_stats()
        resident = self.check_resident()
        self.flips = flips_total
        log(f"[parity] {self.w.name} graph: {steps} steps, hits={st.hits} misses={st.misses} "
            f"evictions={st.evictions} tie-flips={flips_total} max|out-oracle|={worst:.2e} "
            f"pool bytes checked: {checked} inserts, {resident} resident")
        assert flips_total <= max_flips, f"{flips_total} lists selected differently within the tie window"
        return st, worst

    def close(self):
        self.spin.close()
