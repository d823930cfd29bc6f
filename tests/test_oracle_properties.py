"""Randomised small cases for the oracle (hypothesis, CPU).

Any mix of shapes, partition lengths, budgets and query streams must keep
the residency state's structural invariants (two-level map = inverse of the
owner map, live counts, segment conservation), make every mandatory page
resident with this step's timestamp, count hits + misses = mandatory pages,
evict exactly the shortfall (a step that evicts leaves exactly the budget
resident), keep the resident pages within a budget that shrinks and grows
between steps, move misses x 32 KiB, and leave every resident slot holding
its page's host bytes.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle.spin_oracle as om
from tests import oracle_pins as P


@settings(max_examples=30, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(B=st.integers(1, 3), Hkv=st.sampled_from([1, 2]), G=st.sampled_from([1, 2, 4]),
       k=st.integers(1, 6), extra=st.integers(0, 10), variable=st.booleans(),
       steps=st.integers(1, 10), ar=st.floats(0.0, 0.9), seed=st.integers(0, 2**31 - 1),
       budgets=st.lists(st.tuples(st.integers(0, 9), st.integers(0, 2), st.floats(0.0, 1.0)),
                        max_size=4))
def test_residency_invariants(B, Hkv, G, k, extra, variable, steps, ar, seed, budgets):
    rng = np.random.default_rng(seed)
    if variable:
        lens_all = [list(rng.integers(16, 257, size=int(rng.integers(1, 25)))) for _ in range(B)]
    else:
        lens_all = [[64] * int(rng.integers(1, 40)) for _ in range(B)]
    pages = [sum((L + 63) // 64 for L in lens) for lens in lens_all]
    max_ppp = max(max((L + 63) // 64 for L in lens) for lens in lens_all)
    C = Hkv * k * max_ppp + extra
    o = P.make(om, B, Hkv * G, Hkv, k, C, max(pages))
    hosts = []
    for b in range(B):
        Kp, Vp = P.random_parts(rng, Hkv, lens_all[b])
        buf, lens = P.pack_request(Kp, Vp, Hkv)
        o.index(b, buf, lens)
        hosts.append(buf.reshape(Hkv, pages[b], -1))
    q = P.bf16_exact(rng.standard_normal((B, Hkv * G, P.D)).astype(np.float32))
    mand_max = Hkv * k * max_ppp
    for t in range(steps):
        for (ts, b, frac) in budgets:
            if ts == t and b < B:  # anywhere between one step's pages and the slot area
                o.set_budget(b, mand_max + int(round(frac * (C - mand_max))))
        q = P.bf16_exact(np.float32(ar) * q + rng.standard_normal(q.shape).astype(np.float32))
        sel, _ = o.select(P.bits(q))
        before = [dict(s) for s in o.stats]
        o.resolve_evict(sel, t)
        moved = o.retrieve()
        P.check_structure(o, pages)
        n_miss = 0
        for b in range(B):
            M = o.mandatory_pages(b, sel[b])
            d = {key: o.stats[b][key] - before[b][key] for key in ("hits", "misses", "evictions")}
            assert d["hits"] + d["misses"] == len(M)
            n_miss += d["misses"]
            for (h, p, _) in M:
                c = o.translate(b, h, p)
                assert c != -1 and o.last_use[b, c] == t
            resident = int(np.sum(o.owner[b] != -1))
            assert resident <= o.budget[b]
            if d["evictions"]:
                assert resident == o.budget[b]
            for c in range(C):
                own = int(o.owner[b, c])
                if own != -1:
                    h, p = divmod(own, o.max_pages)
                    assert np.array_equal(o.pool[b * C + c], hosts[b][h, p])
        assert moved == n_miss * 32768
