"""Pins of the CPU oracle against things other than itself.

Each ``pin_*`` function takes the oracle module and raises AssertionError when
the oracle disagrees with a closed form, a brute-force enumeration, a library
special case or a structural invariant.  tests/test_oracle_pins.py runs them on
the real oracle; tests/test_oracle_mutations.py runs them on copies of the
oracle with planted mistakes and requires that some pin fails for each.

Nothing here calls the HIP library, and no expected value comes from it.
"""
from __future__ import annotations

import math

import numpy as np
import torch

PT = 64
D = 128


# ----------------------------------------------------------------------------- test-local helpers
def bf16_exact(x: np.ndarray) -> np.ndarray:
    """Truncate fp32 values to ones bf16 represents exactly (test data only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def bits(x: np.ndarray) -> np.ndarray:
    """bf16-exact fp32 -> its bf16 bit pattern."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def pack_request(K_parts, V_parts, Hkv, pad_value=0.0):
    """Pack logical per-head partitions into the documented host page layout.

    K_parts[h][i] / V_parts[h][i]: [len_i][D] bf16-exact fp32.  A page is the
    64x128 keys token-major followed by the 128x64 values dim-major; a
    partition starts on a fresh page; unused token slots hold ``pad_value``."""
    lens = [k.shape[0] for k in K_parts[0]]
    npg = [(L + PT - 1) // PT for L in lens]
    pages = sum(npg)
    buf = np.zeros((Hkv, pages, 2 * PT * D), np.uint16)
    for h in range(Hkv):
        p = 0
        for i, L in enumerate(lens):
            for j in range(npg[i]):
                Kpg = np.full((PT, D), pad_value, np.float32)
                Vpg = np.full((PT, D), pad_value, np.float32)
                n = min(PT, L - j * PT)
                Kpg[:n] = K_parts[h][i][j * PT: j * PT + n]
                Vpg[:n] = V_parts[h][i][j * PT: j * PT + n]
                buf[h, p, : PT * D] = bits(Kpg).reshape(-1)
                buf[h, p, PT * D:] = bits(Vpg.T.copy()).reshape(-1)
                p += 1
    return buf.reshape(-1), np.asarray(lens, np.int32)


def random_parts(rng, Hkv, lens, scale=1.0):
    K = [[bf16_exact(rng.standard_normal((L, D)).astype(np.float32) * scale) for L in lens]
         for _ in range(Hkv)]
    V = [[bf16_exact(rng.standard_normal((L, D)).astype(np.float32)) for L in lens]
         for _ in range(Hkv)]
    return K, V


def dense_attention(q, K, V):
    """Library special case: torch's scaled_dot_product_attention in float64."""
    qt = torch.from_numpy(np.asarray(q, np.float64)).view(1, 1, 1, -1)
    Kt = torch.from_numpy(np.asarray(K, np.float64)).view(1, 1, K.shape[0], -1)
    Vt = torch.from_numpy(np.asarray(V, np.float64)).view(1, 1, V.shape[0], -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt).view(-1).numpy()


def make(om, B, Hq, Hkv, k, C, max_pages, n_seg=None):
    ndir = (max_pages + 63) // 64
    if n_seg is None:
        n_seg = min(B * C, B * Hkv * ndir)
    return om.SpinOracle(B, Hq, Hkv, k, C, max_pages, n_seg)


# ----------------------------------------------------------------------------- decoding
def pin_bf16_decode(om):
    # bf16 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E00 = 0.125, 0x4049 = 3.140625, 0x0000 = 0
    got = om.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x3E00, 0x4049, 0x0000], np.uint16))
    assert np.array_equal(got, [1.0, -2.0, 0.125, 3.140625, 0.0]), got


def pin_page_layout(om):
    # key (t, d) = t + d/128 ; value (t, d) = -(t + d/128): both bf16-exact up to t < 64
    t = np.arange(PT)[:, None].astype(np.float32)
    d = np.arange(D)[None, :].astype(np.float32)
    K = bf16_exact(t * 4 + d / 64)
    V = bf16_exact(-(t * 2) - d / 32)
    page = np.concatenate([bits(K).reshape(-1), bits(V.T.copy()).reshape(-1)])
    assert np.array_equal(om.page_keys(page), K.astype(np.float64))
    assert np.array_equal(om.page_values(page), V.astype(np.float64))


# ----------------------------------------------------------------------------- Index
def pin_summary_closed_form(om):
    """Keys of a partition are c + e_j and c - e_j in pairs (plus c itself for
    odd lengths), so the mean is exactly c; padding slots hold 1000.0 so
    counting them would move the mean."""
    rng = np.random.default_rng(5)
    Hkv = 2
    lens = [64, 1, 130, 255, 17, 64, 256, 3]
    cents = bf16_exact(rng.integers(-8, 8, size=(Hkv, len(lens), D)).astype(np.float32) / 4)
    Kp, Vp = [], []
    for h in range(Hkv):
        kh, vh = [], []
        for i, L in enumerate(lens):
            e = bf16_exact(rng.integers(-4, 5, size=(L // 2, D)).astype(np.float32) / 8)
            rows = [cents[h, i] + e, cents[h, i] - e]
            if L % 2:
                rows.append(cents[h, i][None, :])
            kk = bf16_exact(np.concatenate(rows, axis=0))
            assert kk.shape[0] == L
            kh.append(kk)
            vh.append(np.zeros((L, D), np.float32))
        Kp.append(kh)
        Vp.append(vh)
    buf, lens_a = pack_request(Kp, Vp, Hkv, pad_value=1000.0)
    pages = sum((L + 63) // 64 for L in lens)
    o = make(om, 1, 2 * Hkv, Hkv, 2, 64, pages)
    o.index(0, buf, lens_a)
    assert np.array_equal(o.requests[0].summaries, cents.astype(np.float32)), "summary != centroid"


# ----------------------------------------------------------------------------- Select
def pin_score_closed_form(om):
    """Summaries are scaled basis vectors a_i e_{i mod D}; the group of KV head h
    has queries whose mean is v_h.  Then score = a_i * v_h[i mod D] / sqrt(D).
    Groups get different queries so a wrong head->group map changes scores."""
    Hkv, G = 3, 4
    N = 40
    a = np.arange(1, N + 1, dtype=np.float64) / 8
    Kp, Vp = [], []
    for h in range(Hkv):
        kh = []
        for i in range(N):
            row = np.zeros((64, D), np.float32)
            row[:, i % D] = a[i] * (h + 1)
            kh.append(row)
        Kp.append(kh)
        Vp.append([np.zeros((64, D), np.float32)] * N)
    buf, lens = pack_request(Kp, Vp, Hkv)
    o = make(om, 1, Hkv * G, Hkv, 5, 64, N)
    o.index(0, buf, lens)
    q = np.zeros((1, Hkv * G, D), np.float32)
    rng = np.random.default_rng(3)
    expect_v = np.zeros((Hkv, D))
    for h in range(Hkv):
        base = rng.integers(-6, 7, size=D).astype(np.float32) / 4
        # queries of the group: base + offsets that sum to zero over the group
        offs = rng.integers(-3, 4, size=(G - 1, D)).astype(np.float32) / 4
        offs = np.concatenate([offs, -offs.sum(0, keepdims=True)], axis=0)
        q[0, h * G:(h + 1) * G] = base + offs
        expect_v[h] = base
    sc = o.scores(bits(bf16_exact(q)))
    for h in range(Hkv):
        want = np.array([a[i] * (h + 1) * expect_v[h][i % D] for i in range(N)]) / math.sqrt(D)
        assert np.allclose(sc[0][h], want, rtol=0, atol=1e-12), (h, sc[0][h][:6], want[:6])


def pin_topk_bruteforce(om):
    """Top-k equals a brute-force stable sort of the oracle's own scores with
    key (-score, index); many exact ties are forced by repeated summaries."""
    rng = np.random.default_rng(11)
    for trial in range(6):
        Hkv, G, N = 2, 2, int(rng.integers(3, 60))
        k = int(rng.integers(1, N + 4))
        levels = rng.integers(0, 4, size=(Hkv, N))  # only 4 distinct summaries -> ties
        Kp, Vp = [], []
        for h in range(Hkv):
            kh = []
            for i in range(N):
                row = np.zeros((64, D), np.float32)
                row[:, :4] = levels[h, i] - 1.5
                kh.append(row)
            Kp.append(kh)
            Vp.append([np.zeros((64, D), np.float32)] * N)
        buf, lens = pack_request(Kp, Vp, Hkv)
        o = make(om, 1, Hkv * G, Hkv, k, Hkv * 6 * max(k, 1), N)
        o.index(0, buf, lens)
        q = bf16_exact(rng.standard_normal((1, Hkv * G, D)).astype(np.float32))
        sel, sc = o.select(bits(q))
        for h in range(Hkv):
            s = sc[0][h]
            brute = sorted(sorted(range(N), key=lambda i: (-s[i], i))[:k])
            want = brute + [-1] * (k - len(brute))
            assert list(sel[0, h]) == want, (trial, h, list(sel[0, h]), want)


# ----------------------------------------------------------------------------- bucketed LRU
def _lru_state(om, C, owners, last_use):
    o = make(om, 1, 1, 1, 1, C, 4096, n_seg=64)
    for c, (own, lu) in enumerate(zip(owners, last_use)):
        o.owner[0, c] = own
        o.last_use[0, c] = lu
    return o


def pin_lru_hand_example(om):
    """Worked by hand from the rule (bucket = 63 - min(63, t - last_use); take
    whole buckets oldest first, lower slot first inside the cutoff bucket).

    t = 100, 10 slots, slot 9 free, slots 2 and 5 mandatory:
      slot : 0   1   2*  3   4   5*  6   7   8
      last : 99  30  97  98  37  99  97  10  98
      age  : 1   70  3   2   63  1   3   90  2
      bucket 62  0   -   61  0   -   60  0   61
    need = 4: bucket 0 holds {1, 4, 7} (3 < 4), bucket 60 holds {6}: 3+1 = 4,
    so cutoff = 60 and the victims are {1, 4, 6, 7}."""
    owners = [0, 1, 2, 3, 4, 5, 6, 7, 8, -1]
    last = [99, 30, 97, 98, 37, 99, 97, 10, 98, -1]
    o = _lru_state(om, 10, owners, last)
    victims, cut = o.choose_victims(0, 4, {2, 5}, 100)
    assert (victims, cut) == ([1, 4, 6, 7], 60), (victims, cut)
    # need = 5: bucket 61 holds {3, 8}; one more is needed, the lower slot (3)
    victims, cut = o.choose_victims(0, 5, {2, 5}, 100)
    assert (victims, cut) == ([1, 3, 4, 6, 7], 61), (victims, cut)
    # need = 2 inside bucket 0: lowest slots {1, 4}
    victims, cut = o.choose_victims(0, 2, {2, 5}, 100)
    assert (victims, cut) == ([1, 4], 0), (victims, cut)


def pin_lru_properties(om):
    """Random states: exactly ``need`` victims; none mandatory or free; every
    victim's bucket <= cutoff; every candidate below the cutoff is a victim;
    when all candidate buckets are distinct, victims == exact LRU (the need
    oldest last_use values, by brute force)."""
    rng = np.random.default_rng(7)
    for trial in range(300):
        C = int(rng.integers(2, 40))
        t = int(rng.integers(0, 200))
        distinct = trial % 2 == 0
        if distinct:
            ages = rng.choice(np.arange(1, 64), size=C, replace=False) if C <= 63 else None
            if ages is None:
                continue
            last = t - ages
        else:
            last = t - rng.integers(1, 120, size=C)
        owners = list(range(C))
        free = set(rng.choice(C, size=int(rng.integers(0, C // 3 + 1)), replace=False).tolist())
        for c in free:
            owners[c] = -1
        resident = [c for c in range(C) if owners[c] != -1]
        mand = set(c for c in resident if rng.random() < 0.3)
        cands = [c for c in resident if c not in mand]
        if not cands:
            continue
        need = int(rng.integers(1, len(cands) + 1))
        o = _lru_state(om, C, owners, [l if owners[c] != -1 else -1 for c, l in enumerate(last)])
        victims, cut = o.choose_victims(0, need, mand, t)
        bk = {c: 63 - min(63, t - int(last[c])) for c in cands}
        assert len(victims) == need, (trial, victims, need)
        assert len(set(victims)) == need and all(v in bk for v in victims), trial
        assert all(bk[v] <= cut for v in victims), trial
        assert all(c in victims for c in cands if bk[c] < cut), trial
        at_cut = sorted(c for c in cands if bk[c] == cut)
        assert sorted(v for v in victims if bk[v] == cut) == at_cut[: len([v for v in victims if bk[v] == cut])], trial
        if distinct:
            exact = sorted(sorted(cands, key=lambda c: int(last[c]))[:need])
            assert victims == exact, (trial, victims, exact)


# ----------------------------------------------------------------------------- two-level table
def check_structure(o, pages_per_req):
    """Structural pins of the residency state, from plain definitions:
    the two-level map and the owner map are mutual inverses, live counts equal
    non-empty entries, the directory uses distinct segments, and the stack of
    unused segments is exactly the rest (each of them empty)."""
    used = []
    for b in range(o.B):
        flat = {}
        for h in range(o.Hkv):
            for p in range(pages_per_req[b] if b < len(pages_per_req) else 0):
                c = o.translate(b, h, p)
                if c != -1:
                    flat[(h, p)] = c
        inv = {}
        for c in range(o.C):
            own = int(o.owner[b, c])
            if own != -1:
                inv[divmod(own, o.max_pages)] = c
                assert o.last_use[b, c] >= 0
            else:
                assert o.last_use[b, c] == -1
        assert flat == inv, f"request {b}: two-level map != inverse of owner map"
        for h in range(o.Hkv):
            for e in range(o.ndir):
                s = int(o.directory[b, h, e])
                if s != -1:
                    used.append(s)
                    assert o.seg_live[s] == np.sum(o.segments[s] != -1) > 0
    assert len(used) == len(set(used)), "segment linked twice"
    assert sorted(used + list(o.free_stack)) == list(range(o.n_seg)), "segment lost or duplicated"
    for s in o.free_stack:
        assert o.seg_live[s] == 0 and np.all(o.segments[s] == -1)


def _run_small(om, B=3, Hq=8, Hkv=2, k=4, C=None, lens_fn=None, steps=24, seed=1, n_seg=None):
    rng = np.random.default_rng(seed)
    lens_all = [lens_fn(rng, b) for b in range(B)]
    pages = [sum((L + 63) // 64 for L in lens) for lens in lens_all]
    max_ppp = max(max((L + 63) // 64 for L in lens) for lens in lens_all)
    if C is None:
        C = Hkv * k * max_ppp + 3
    o = make(om, B, Hq, Hkv, k, C, max(pages), n_seg)
    bufs = []
    for b in range(B):
        Kp, Vp = random_parts(rng, Hkv, lens_all[b])
        buf, lens = pack_request(Kp, Vp, Hkv)
        o.index(b, buf, lens)
        bufs.append(buf)
    q = bf16_exact(rng.standard_normal((B, Hq, D)).astype(np.float32))
    return o, pages, rng, q, bufs


def pin_two_level_table(om):
    """Tight pools so eviction fires most steps; structure checked every step,
    and mandatory pages are resident with the step's last_use after it."""
    for seed, lens_fn in [
        (1, lambda r, b: [64] * int(r.integers(150, 300))),
        (2, lambda r, b: list(r.integers(16, 257, size=int(r.integers(40, 90))))),
    ]:
        o, pages, rng, q, _ = _run_small(om, lens_fn=lens_fn, seed=seed)
        for t in range(24):
            q = bf16_exact(0.6 * q + rng.standard_normal(q.shape).astype(np.float32))
            sel, _ = o.select(bits(q))
            ev0 = [st["evictions"] for st in o.stats]
            blocks = o.resolve_evict(sel, t)
            check_structure(o, pages)
            for b in range(o.B):
                # eviction frees exactly the shortfall, so a step that evicted
                # leaves no free slot behind (R7)
                if o.stats[b]["evictions"] > ev0[b]:
                    assert int(np.sum(o.owner[b] == -1)) == 0, (t, b)
            for b in range(o.B):
                M = o.mandatory_pages(b, sel[b])
                assert sum(len(x) for x in blocks[b]) == len(M)
                for (h, p, n) in M:
                    c = o.translate(b, h, p)
                    assert c != -1 and o.last_use[b, c] == t
                resident = int(np.sum(o.owner[b] != -1))
                assert resident <= o.C


def pin_retrieve_bytes(om):
    """After each step, every resident slot of the pool holds exactly the host
    bytes of the page that owns it, and bytes moved = misses x 32 KiB."""
    o, pages, rng, q, bufs = _run_small(om, lens_fn=lambda r, b: [64] * 120, seed=4)
    prev_miss = 0
    for t in range(12):
        q = bf16_exact(0.5 * q + rng.standard_normal(q.shape).astype(np.float32))
        sel, _ = o.select(bits(q))
        o.resolve_evict(sel, t)
        moved = o.retrieve()
        miss = sum(s["misses"] for s in o.stats)
        assert moved == (miss - prev_miss) * 32768
        prev_miss = miss
        for b in range(o.B):
            host = bufs[b].reshape(o.Hkv, pages[b], -1)
            for c in range(o.C):
                own = int(o.owner[b, c])
                if own != -1:
                    h, p = divmod(own, o.max_pages)
                    assert np.array_equal(o.pool[b * o.C + c], host[h, p])


def pin_retrieve_padding(om):
    """Reading R25: token slots past a partition's last token carry nothing
    the method uses.  Two oracles get the same partitions, one with zeros and
    one with NaN in every padding slot of the host pages: summaries,
    selections, residency and outputs agree exactly (and stay finite), and
    every resident slot holds its page's valid keys and values (token counts
    taken from the partition lengths here) and zeros in all other token
    slots."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, k = 2, 8, 2, 4
    lens_all = [list(rng.integers(16, 200, size=int(rng.integers(30, 60)))) for _ in range(B)]
    pages = [sum((L + 63) // 64 for L in lens) for lens in lens_all]
    C = Hkv * k * 4 + 5
    oz, on = make(om, B, Hq, Hkv, k, C, max(pages)), make(om, B, Hq, Hkv, k, C, max(pages))
    hosts, ntoks = [], []
    for b in range(B):
        Kp, Vp = random_parts(rng, Hkv, lens_all[b])
        bz, lens = pack_request(Kp, Vp, Hkv, pad_value=0.0)
        bn, _ = pack_request(Kp, Vp, Hkv, pad_value=float("nan"))
        oz.index(b, bz, lens)
        on.index(b, bn, lens)
        hosts.append(bn.reshape(Hkv, pages[b], -1))
        ntoks.append([min(64, L - 64 * j) for L in lens for j in range((L + 63) // 64)])
        assert np.array_equal(oz.requests[b].summaries, on.requests[b].summaries)
    q = bf16_exact(rng.standard_normal((B, Hq, D)).astype(np.float32))
    partial = 0
    for t in range(16):
        q = bf16_exact(0.5 * q + rng.standard_normal(q.shape).astype(np.float32))
        outs = []
        for o in (oz, on):
            sel, _ = o.select(bits(q))
            blocks = o.resolve_evict(sel, t)
            o.retrieve()
            outs.append(o.attend(bits(q), blocks))
        assert np.array_equal(oz.owner, on.owner) and np.all(np.isfinite(outs[1]))
        assert np.array_equal(outs[0], outs[1])
        assert np.array_equal(oz.pool, on.pool)
        for b in range(B):
            for c in range(C):
                own = int(on.owner[b, c])
                if own == -1:
                    continue
                h, p = divmod(own, on.max_pages)
                n = ntoks[b][p]
                partial += n < 64
                got = on.pool[b * C + c]
                host = hosts[b][h, p]
                assert np.array_equal(got[: n * D], host[: n * D]) and not np.any(got[n * D: 64 * D])
                gv, hv = got[64 * D:].reshape(D, 64), host[64 * D:].reshape(D, 64)
                assert np.array_equal(gv[:, :n], hv[:, :n]) and not np.any(gv[:, n:])
    assert partial > 0


# ----------------------------------------------------------------------------- attention
def pin_attend_dense(om):
    """k = all partitions and an ample pool: the sparse paged output equals dense
    softmax attention (torch SDPA, float64) over the request's logical K/V.
    Ragged tails, variable partitions and non-zero padding are included."""
    rng = np.random.default_rng(21)
    cases = [
        (2, 8, 2, [[64] * 5 + [37], [64] * 3]),
        (1, 10, 2, [[16, 200, 64, 1, 129]]),
        (2, 16, 2, [[256, 100, 33], [70, 70]]),
    ]
    for B, Hq, Hkv, lens_req in cases:
        G = Hq // Hkv
        kmax = max(len(l) for l in lens_req)
        max_ppp = max((L + 63) // 64 for l in lens_req for L in l)
        pages = [sum((L + 63) // 64 for L in l) for l in lens_req]
        o = make(om, B, Hq, Hkv, kmax, Hkv * kmax * max_ppp, max(pages))
        logical = []
        for b in range(B):
            Kp, Vp = random_parts(rng, Hkv, lens_req[b], scale=2.0)
            buf, lens = pack_request(Kp, Vp, Hkv, pad_value=-77.0)
            o.index(b, buf, lens)
            logical.append((Kp, Vp))
        q = bf16_exact(rng.standard_normal((B, Hq, D)).astype(np.float32))
        sel, _ = o.select(bits(q))
        blocks = o.resolve_evict(sel, 0)
        o.retrieve()
        out = o.attend(bits(q), blocks)
        for b in range(B):
            for g in range(Hq):
                h = g // G
                K = np.concatenate(logical[b][0][h], axis=0)
                V = np.concatenate(logical[b][1][h], axis=0)
                want = dense_attention(q[b, g], K, V)
                assert np.allclose(out[b, g], want, rtol=0, atol=2e-6), (b, g, np.abs(out[b, g] - want).max())


def pin_attend_closed_forms(om):
    """Equal keys -> output = mean of the values; one key far above the rest ->
    output = that token's value; shuffling the block order changes nothing."""
    rng = np.random.default_rng(8)
    Hkv, Hq = 1, 2
    lens = [64, 64, 20]
    K = [[np.ones((L, D), np.float32) * 0.5 for L in lens]]
    V = [[bf16_exact(rng.standard_normal((L, D)).astype(np.float32)) for L in lens]]
    buf, la = pack_request(K, V, Hkv, pad_value=9.0)
    o = make(om, 1, Hq, Hkv, 3, 16, 3)
    o.index(0, buf, la)
    q = bf16_exact(rng.standard_normal((1, Hq, D)).astype(np.float32))
    sel, _ = o.select(bits(q))
    blocks = o.resolve_evict(sel, 0)
    o.retrieve()
    out = o.attend(bits(q), blocks)
    mean_v = np.concatenate(V[0], axis=0).astype(np.float64).mean(0)
    assert np.allclose(out[0, 0], mean_v, atol=1e-6) and np.allclose(out[0, 1], mean_v, atol=1e-6)
    # one dominant key: token 70 (partition 1, row 6) aligned with the query
    K2 = [[np.zeros((L, D), np.float32) for L in lens]]
    qv = np.zeros(D, np.float32)
    qv[:8] = 4.0
    K2[0][1][6, :8] = 4.0          # logit = 8*16/sqrt(128) ~ 11.3 vs 0 elsewhere
    K2[0][1][6, 8:16] = 4.0        # 8 more dims (query is zero there): no effect
    buf2, la2 = pack_request(K2, V, Hkv)
    o2 = make(om, 1, Hq, Hkv, 3, 16, 3)
    o2.index(0, buf2, la2)
    qq = np.stack([qv, qv])[None]
    sel2, _ = o2.select(bits(qq))
    blocks2 = o2.resolve_evict(sel2, 0)
    o2.retrieve()
    out2 = o2.attend(bits(qq), blocks2)
    logit = 8 * 16 / math.sqrt(D)
    wdom = math.exp(logit) / (math.exp(logit) + (sum(lens) - 1))
    want = wdom * V[0][1][6] + (1 - wdom) * (np.concatenate(V[0], 0).astype(np.float64).sum(0) - V[0][1][6]) / (sum(lens) - 1)
    assert np.allclose(out2[0, 0], want, atol=1e-6), np.abs(out2[0, 0] - want).max()
    # permutation of block order
    perm = [list(reversed(blocks[0][0]))]
    out3 = o.attend(bits(q), [perm])
    assert np.allclose(out3, out, rtol=0, atol=1e-7)


# ----------------------------------------------------------------------------- whole-step invariants
def pin_step_invariants(om):
    """Step 0 is all misses; hits + misses = |mandatory|; zero evictions while
    the budget holds every page ever selected; errors for bad ids / pool."""
    o, pages, rng, q, _ = _run_small(om, B=2, lens_fn=lambda r, b: [64] * 40, C=2 * 4 * 12, seed=9)
    seen = [set() for _ in range(o.B)]
    for t in range(10):
        q = bf16_exact(0.9 * q + 0.3 * rng.standard_normal(q.shape).astype(np.float32))
        sel, _ = o.select(bits(q))
        before = [dict(s) for s in o.stats]
        o.resolve_evict(sel, t)
        for b in range(o.B):
            M = o.mandatory_pages(b, sel[b])
            d_h = o.stats[b]["hits"] - before[b]["hits"]
            d_m = o.stats[b]["misses"] - before[b]["misses"]
            assert d_h + d_m == len(M)
            if t == 0:
                assert d_h == 0
            seen[b] |= {(h, p) for h, p, _ in M}
            if len(seen[b]) <= o.C:
                assert o.stats[b]["evictions"] == 0
    bad = np.zeros((o.B, o.Hkv, o.k), np.int64)
    bad[0, 0, 0] = 10 ** 6
    try:
        o.resolve_evict(bad, 99)
        raise AssertionError("out-of-range partition accepted")
    except IndexError:
        pass
    # a pool of one segment cannot hold two KV heads' pages
    o2, _, _, q2, _ = _run_small(om, B=1, lens_fn=lambda r, b: [64] * 300, n_seg=1, seed=3)
    sel2, _ = o2.select(bits(q2))
    try:
        o2.resolve_evict(sel2, 0)
        raise AssertionError("exhausted segment pool not reported")
    except MemoryError:
        pass


def pin_first_step_slots(om):
    """On a fresh request every mandatory page misses, and misses take the free
    slots in ascending order (R10): the block table, read in canonical order
    (head, partition, page ascending), is slots 0, 1, 2, ... of the request."""
    rng = np.random.default_rng(12)
    lens = [64, 130, 20, 256, 64, 64, 99]
    Hkv, Hq, k = 2, 4, 3
    o = make(om, 2, Hq, Hkv, k, 2 * k * 4 + 5, 13)
    for b in range(2):
        Kp, Vp = random_parts(rng, Hkv, lens)
        buf, la = pack_request(Kp, Vp, Hkv)
        o.index(b, buf, la)
    q = bf16_exact(rng.standard_normal((2, Hq, D)).astype(np.float32))
    sel, _ = o.select(bits(q))
    blocks = o.resolve_evict(sel, 0)
    for b in range(2):
        flat = [s for h in range(Hkv) for s, _ in blocks[b][h]]
        assert flat == [b * o.C + i for i in range(len(flat))], (b, flat)
        pages = [(h, int(p)) for h in range(Hkv) for part in sorted(sel[b, h])
                 for p in range(sum((L + 63) // 64 for L in lens[:part]),
                                sum((L + 63) // 64 for L in lens[:part + 1]))]
        assert [divmod(int(o.owner[b, i]), o.max_pages) for i in range(len(flat))] == pages
        ntok = [n for h in range(Hkv) for _, n in blocks[b][h]]
        want = [min(64, lens[part] - 64 * j) for h in range(Hkv) for part in sorted(sel[b, h])
                for j in range((lens[part] + 63) // 64)]
        assert ntok == want


def pin_budget_shrink(om):
    """Worked by hand.  One request, one KV head, k = 2 fixed partitions, 8
    slots.  Steps 0-3 select {0,1}, {2,3}, {4,5}, {6,7}: eight misses fill slots
    0..7 (last_use 0,0,1,1,2,2,3,3).  The budget then drops to 4.  Step 4
    selects {6, 8}: page 6 hits (slot 6), page 8 misses; resident 8 + 1 miss -
    budget 4 = 5 pages must go.  Candidates (all but slot 6): ages at t = 4 are
    4,4,3,3,2,2,-,1 -> buckets 59,59,60,60,61,61,-,62.  Taking whole buckets
    from the oldest: {0,1} (59), {2,3} (60) = 4, then one more from bucket 61:
    slot 4.  Page 8 goes to the lowest free slot, 0.  Growing the budget back
    to 8 evicts nothing more."""
    Kp = [[np.full((64, D), 0.0, np.float32) for _ in range(10)]]
    Vp = [[np.zeros((64, D), np.float32) for _ in range(10)]]
    buf, lens = pack_request(Kp, Vp, 1)
    o = make(om, 1, 1, 1, 2, 8, 10)
    o.index(0, buf, lens)
    for t, pair in enumerate([(0, 1), (2, 3), (4, 5), (6, 7)]):
        o.resolve_evict(np.array([[pair]]), t)
    assert list(o.owner[0]) == [0, 1, 2, 3, 4, 5, 6, 7]
    o.set_budget(0, 4)
    blocks = o.resolve_evict(np.array([[(6, 8)]]), 4)
    assert o.stats[0]["evictions"] == 5 and o.stats[0]["cutoff"] == 61, o.stats[0]
    assert list(o.owner[0]) == [8, -1, -1, -1, -1, 5, 6, 7], list(o.owner[0])
    assert [s for s, _ in blocks[0][0]] == [6, 0]
    o.set_budget(0, 8)
    o.resolve_evict(np.array([[(5, 9)]]), 5)
    assert o.stats[0]["evictions"] == 5 and int(np.sum(o.owner[0] != -1)) == 5


def pin_offload_append(om):
    """Offload a request of 94 tokens (partitions 64 + 30) into a host buffer
    with room for 6 pages per head, make every page resident, then append 40
    tokens: 34 fill partition 1 to 64 tokens, the next 6 start partition 2.
    Lengths, host bytes, exact summaries (means of the known keys), and
    attention over all 134 tokens equal to dense SDPA: the last holds only if
    the append also updated the resident GPU-side copy of the tail page."""
    rng = np.random.default_rng(31)
    Hkv, Hq, lens = 2, 4, [64, 30]
    Kp, Vp = random_parts(rng, Hkv, lens)
    buf, la = pack_request(Kp, Vp, Hkv, pad_value=0.0)
    o = make(om, 1, Hq, Hkv, 4, Hkv * 4 + 2, 6)
    o.offload(0, buf.reshape(Hkv, 2, -1), la, 6)
    q = bf16_exact(rng.standard_normal((1, Hq, D)).astype(np.float32))
    sel, _ = o.select(bits(q))
    o.resolve_evict(sel, 0)
    o.retrieve()
    Klog = [np.concatenate(Kp[h], 0) for h in range(Hkv)]
    Vlog = [np.concatenate(Vp[h], 0) for h in range(Hkv)]
    for i in range(40):
        kn = bf16_exact(rng.standard_normal((1, Hkv, D)).astype(np.float32))
        vn = bf16_exact(rng.standard_normal((1, Hkv, D)).astype(np.float32))
        o.append(bits(kn), bits(vn))
        for h in range(Hkv):
            Klog[h] = np.concatenate([Klog[h], kn[0, h][None]], 0)
            Vlog[h] = np.concatenate([Vlog[h], vn[0, h][None]], 0)
    req = o.requests[0]
    assert list(req.lens) == [64, 64, 6] and list(req.first_page) == [0, 1, 2] and req.pages == 3
    bounds = [(0, 64), (64, 128), (128, 134)]
    for h in range(Hkv):
        for i, (a, e) in enumerate(bounds):
            want = (Klog[h][a:e].astype(np.float64).sum(0) / (e - a)).astype(np.float32)
            assert np.array_equal(req.summaries[h, i], want), (h, i)
        # the last appended token sits in slot 5 of page 2: key row 5, value column 5
        pg = req.host[h, 2]
        assert np.array_equal(pg[5 * D:6 * D], bits(Klog[h][133:134]).reshape(-1))
        assert np.array_equal(pg[64 * D:].reshape(D, 64)[:, 5], bits(Vlog[h][133:134]).reshape(-1))
    sel, _ = o.select(bits(q))
    blocks = o.resolve_evict(sel, 1)
    o.retrieve()
    out = o.attend(bits(q), blocks)
    for g in range(Hq):
        h = g // (Hq // Hkv)
        want = dense_attention(q[0, g], Klog[h], Vlog[h])
        assert np.allclose(out[0, g], want, rtol=0, atol=2e-6), (g, np.abs(out[0, g] - want).max())


def _tagged_host(om, Hkv, pages, b, version):
    """Host KV whose every page is filled with one tag, unique per (request,
    version, head, page): the bytes of a retrieved page say which it is."""
    buf = np.zeros((Hkv, pages, om.PAGE_ELEMS), np.uint16)
    for h in range(Hkv):
        for p in range(pages):
            buf[h, p, :] = _tag(b, version, h, p)
    return buf.reshape(-1)


def _tag(b, version, h, p):
    return 1 + p + 192 * (h + 2 * (b + 2 * version))


def pin_release_reindex(om):
    """Worked by hand: request turnover.  Two requests, two KV heads, top-2,
    8 slots each, 192 one-page partitions (3 directory ranges of 64 pages),
    a shared pool of 6 segments (stack [5 4 3 2 1 0], top last).

    Step 0, hand-picked selections: request 0 head 0 {5, 130}, head 1
    {70, 71}; request 1 head 0 {0, 1}, head 1 {64, 190}.  Every page misses
    and takes the free slots in canonical order (slots 0..3 of each request).
    Inserts, request 0 first, pop a segment on a range's first page:
    (r0,h0,e0) <- 0, (r0,h0,e2) <- 1, (r0,h1,e1) <- 2 (pages 70 and 71),
    (r1,h0,e0) <- 3 (pages 0 and 1), (r1,h1,e1) <- 4, (r1,h1,e2) <- 5.

    release(0), after its budget was cut to 5: segments 0, 1, 2 are cleared
    and pushed in (head, directory index) order, so the stack is [0 1 2];
    request 0's slots are free, its budget is 8 again; request 1 is as it was.

    Re-index request 0 with new KV of 100 pages; step 1 selects head 0
    {64, 99}, head 1 {0, 3} for it (request 1 keeps its selection: four
    hits).  Misses take slots 0..3; (r0,h0,e1) pops 2 (pages 64 and 99 ->
    entries 0 and 35), (r0,h1,e0) pops 1 (pages 0 and 3 -> entries 0 and 3);
    the stack is [0].  The pool rows now hold the new KV's pages.

    Re-indexing request 1, which holds segments 3, 4, 5, releases it first:
    the stack becomes [0 3 4 5] and request 0 is untouched."""
    F = om.FREE
    Hkv, C, P0 = 2, 8, 192
    o = make(om, 2, 2, Hkv, 2, C, P0, n_seg=6)
    for b in range(2):
        o.index(b, _tagged_host(om, Hkv, P0, b, 0), np.full(P0, 64))
    sel = np.array([[[5, 130], [70, 71]], [[0, 1], [64, 190]]])
    o.resolve_evict(sel, 0)
    o.retrieve()
    assert o.directory.tolist() == [[[0, F, 1], [F, 2, F]], [[3, F, F], [F, 4, 5]]], o.directory
    assert o.free_stack == []
    assert list(o.seg_live) == [1, 1, 2, 2, 1, 1]
    assert o.owner[0].tolist() == [5, 130, P0 + 70, P0 + 71, F, F, F, F]
    assert o.owner[1].tolist() == [0, 1, P0 + 64, P0 + 190, F, F, F, F]
    want_entries = {(0, 5): 0, (1, 2): 1, (2, 6): 2, (2, 7): 3, (3, 0): 0, (3, 1): 1, (4, 0): 2, (5, 62): 3}
    for s in range(6):
        for e in range(64):
            assert o.segments[s, e] == want_entries.get((s, e), F), (s, e)

    o.set_budget(0, 5)
    seg_r1 = o.segments[3:].copy()
    own1, lu1 = o.owner[1].copy(), o.last_use[1].copy()
    o.release(0)
    assert o.free_stack == [0, 1, 2], o.free_stack
    assert np.all(o.segments[:3] == F) and list(o.seg_live) == [0, 0, 0, 2, 1, 1]
    assert np.array_equal(o.segments[3:], seg_r1)
    assert o.directory[0].tolist() == [[F, F, F], [F, F, F]]
    assert o.directory[1].tolist() == [[3, F, F], [F, 4, 5]]
    assert np.all(o.owner[0] == F) and np.all(o.last_use[0] == F)
    assert o.budget[0] == C and o.requests[0] is None
    assert np.array_equal(o.owner[1], own1) and np.array_equal(o.last_use[1], lu1)

    o.index(0, _tagged_host(om, Hkv, 100, 0, 1), np.full(100, 64))
    sel = np.array([[[64, 99], [0, 3]], [[0, 1], [64, 190]]])
    blocks = o.resolve_evict(sel, 1)
    o.retrieve()
    assert o.free_stack == [0], o.free_stack
    assert o.directory[0].tolist() == [[F, 2, F], [1, F, F]], o.directory[0]
    assert o.segments[2, 0] == 0 and o.segments[2, 35] == 1
    assert o.segments[1, 0] == 2 and o.segments[1, 3] == 3
    assert list(o.seg_live) == [0, 2, 2, 2, 1, 1]
    assert o.owner[0].tolist() == [64, 99, P0 + 0, P0 + 3, F, F, F, F]
    assert o.last_use[0].tolist() == [1, 1, 1, 1, F, F, F, F]
    assert o.last_use[1].tolist() == [1, 1, 1, 1, F, F, F, F]
    assert [[s for s, _ in blocks[0][h]] for h in range(2)] == [[0, 1], [2, 3]]
    assert [[s for s, _ in blocks[1][h]] for h in range(2)] == [[C + 0, C + 1], [C + 2, C + 3]]
    for slot, (h, p) in enumerate([(0, 64), (0, 99), (1, 0), (1, 3)]):
        assert np.all(o.pool[slot] == _tag(0, 1, h, p)), slot
    assert o.stats[0]["misses"] == 8 and o.stats[1]["hits"] == 4 and o.stats[1]["misses"] == 4

    own0, lu0, seg_r0 = o.owner[0].copy(), o.last_use[0].copy(), o.segments[1:3].copy()
    o.index(1, _tagged_host(om, Hkv, P0, 1, 1), np.full(P0, 64))
    assert o.free_stack == [0, 3, 4, 5], o.free_stack
    assert np.all(o.owner[1] == F) and np.all(o.last_use[1] == F)
    assert np.all(o.segments[3:] == F) and o.directory[1].tolist() == [[F, F, F], [F, F, F]]
    assert np.array_equal(o.owner[0], own0) and np.array_equal(o.last_use[0], lu0)
    assert np.array_equal(o.segments[1:3], seg_r0)


def pin_step_order(om):
    """Decode steps never go back (R23): with t below the last resolved step
    some ages t - last_use would be negative.  Such a resolve is refused with
    ValueError before anything changes; the same step index again is
    accepted."""
    Hkv, C, P0 = 2, 8, 192
    o = make(om, 2, 2, Hkv, 2, C, P0, n_seg=6)
    for b in range(2):
        o.index(b, _tagged_host(om, Hkv, P0, b, 0), np.full(P0, 64))
    sels = [np.array([[[5, 130], [70, 71]], [[0, 1], [64, 190]]]),
            np.array([[[6, 130], [70, 72]], [[0, 2], [64, 190]]]),
            np.array([[[7, 131], [73, 71]], [[3, 1], [65, 190]]])]
    for t, s in enumerate(sels):
        o.resolve_evict(s, t)
    names = ("directory", "segments", "seg_live", "owner", "last_use")
    before = {n: getattr(o, n).copy() for n in names}
    stack, stats = list(o.free_stack), [dict(x) for x in o.stats]
    try:
        o.resolve_evict(sels[0], 1)
        raise AssertionError("a rewound step index was accepted")
    except ValueError:
        pass
    for n in names:
        assert np.array_equal(getattr(o, n), before[n]), n
    assert o.free_stack == stack and o.stats == stats
    o.resolve_evict(sels[2], 2)
    assert o.stats[0]["hits"] == stats[0]["hits"] + 4


ALL_PINS = [
    pin_bf16_decode, pin_page_layout, pin_summary_closed_form, pin_score_closed_form,
    pin_topk_bruteforce, pin_lru_hand_example, pin_lru_properties, pin_two_level_table,
    pin_retrieve_bytes, pin_retrieve_padding, pin_attend_dense, pin_attend_closed_forms, pin_step_invariants,
    pin_first_step_slots, pin_budget_shrink, pin_offload_append, pin_release_reindex,
    pin_step_order,
]
