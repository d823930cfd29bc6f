"""GPU parity on seeded random shapes (needs MI355X).

Each case draws its own shape from a fixed seed: batch, KV heads, group size,
ragged context lengths (an empty request now and then), fixed or variable
partition lengths, top-k, a budget anywhere between the mandatory pages alone
and six times them, the key structure and how fast the queries drift.  The
shapes are small enough for the oracle to compute every output of every step,
and together they reach corners the named cases do not combine: a tight
budget with variable partitions, G = 1 or 16 with eviction, k above the
partition count of some requests but not others.  The first half of the
cases run stage by stage (the oracle's selection fed to the GPU's resolve,
every state compared bit for bit), the second half run the benchmark's
launch form: one captured spin_step_at graph, replayed once per step.
"""
import numpy as np
import pytest

from sparse_attention_tiered_amd import workload as W
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

N_CASES = 96


def random_case(i: int):
    """Workload and slot count of random case i (a pure function of i)."""
    rng = np.random.default_rng([4242, i])
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 5, 8, 16]))
    while Hkv * G > 64:
        G //= 2
    B = int(rng.integers(1, 5))
    var = bool(rng.random() < 0.4)
    var_len = None
    if var:
        lo = int(rng.integers(8, 96))
        var_len = (lo, int(rng.integers(lo, 257)))
    ctx = []
    for _ in range(B):
        ctx.append(0 if rng.random() < 0.08 else int(rng.integers(1, 14000)))
    k = int(rng.integers(1, 33))
    kind = str(rng.choice(["hot", "plain", "cluster"]))
    ppp = 1 if var_len is None else -(-var_len[1] // W.PAGE_TOKENS)
    mand = Hkv * k * ppp
    # most budgets tight (eviction fires within a few steps), some ample
    slots = mand + int(mand * (rng.uniform(0.0, 0.5) if rng.random() < 0.7 else rng.uniform(0.5, 5.0)))
    w = W.variant(W.C1, name=f"rand{i}", cfg_id=100 + i, seed=i, B=B, Hq=Hkv * G, Hkv=Hkv,
                  ctx=tuple(ctx), k=k, slots_per_request=slots, steps=int(rng.integers(4, 11)),
                  kv_kind=kind, hot_count=int(rng.integers(0, 5)), n_centroids=64,
                  var_len=var_len, ar_coef=float(rng.uniform(0.2, 0.95)))
    return w, slots


CASES = [random_case(i) for i in range(N_CASES)]


def _ids():
    out = []
    for w, slots in CASES:
        parts = "var" if w.var_len is not None else "fixed"
        out.append(f"{w.name}-B{w.B}-{w.Hq}x{w.Hkv}-k{w.k}-{parts}-C{slots}")
    return out


@pytest.mark.parametrize("i", range(N_CASES), ids=_ids())
def test_random_shape_parity(spin_lib, i):
    from tests.gpu_harness import Pair, log
    w, slots = CASES[i]
    log(f"[case] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} ctx={w.ctx} k={w.k} var_len={w.var_len} "
        f"kind={w.kv_kind} C={slots} steps={w.steps} ar={w.ar_coef:.2f}")
    p = Pair(w, slots=slots)
    p.check_summaries()
    if i < N_CASES // 2:
        st, worst = p.run()
    else:
        st, worst = p.run_graph()
    assert st.error_word == 0
    assert st.hits + st.misses > 0 or max(w.ctx) == 0
    p.close()


N_VARIANTS = 48


def variant_case(i: int):
    """Random case i, with the segment tables in host memory or not, and the
    KV offloaded from the device with a token appended per request per step
    or not (each drawn from its own fixed seed)."""
    w, slots = random_case(1000 + i)
    rng = np.random.default_rng([4343, i])
    host_segments = bool(rng.random() < 0.5)
    append = bool(rng.random() < 0.5)
    return w, slots, host_segments, append


VARIANTS = [variant_case(i) for i in range(N_VARIANTS)]


@pytest.mark.parametrize("i", range(N_VARIANTS),
                         ids=[f"{w.name}-{'hostseg' if hs else 'gpuseg'}-{'append' if ap else 'fixed'}"
                              for w, _, hs, ap in VARIANTS])
def test_random_shape_variants(spin_lib, i):
    """Stage parity on random shapes with the second-level tables in pinned
    host memory and/or the prefill-side offload followed by decode-time
    appends (host bytes and summaries compared too)."""
    from tests.gpu_harness import Pair, log
    w, slots, host_segments, append = VARIANTS[i]
    log(f"[case] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} ctx={w.ctx} k={w.k} var_len={w.var_len} "
        f"C={slots} steps={w.steps} host_segments={host_segments} append={append}")
    extra = (w.steps + W.PAGE_TOKENS - 1) // W.PAGE_TOKENS + 2 if append else None
    p = Pair(w, slots=slots, host_segments=host_segments, offload_extra_pages=extra)
    if append:
        p.check_host()
    p.check_summaries()
    st, _ = p.run(append=append)
    if append:
        p.check_host()
        p.check_summaries()
    assert st.error_word == 0
    p.close()


N_KV16 = 8


def kv16_case(i: int):
    """Random offload + append case i with 16 KV heads, where each lane of the
    append kernel owns two elements of the token (a pure function of i)."""
    rng = np.random.default_rng([5151, i])
    G = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 4))
    var_len = None
    if rng.random() < 0.5:
        lo = int(rng.integers(8, 96))
        var_len = (lo, int(rng.integers(lo, 257)))
    ctx = tuple(int(rng.integers(1, 9000)) for _ in range(B))
    k = int(rng.integers(1, 17))
    ppp = 1 if var_len is None else -(-var_len[1] // W.PAGE_TOKENS)
    mand = 16 * k * ppp
    slots = mand + int(mand * rng.uniform(0.0, 0.6))
    w = W.variant(W.C1, name=f"kv16_{i}", cfg_id=300 + i, seed=i, B=B, Hq=16 * G, Hkv=16, ctx=ctx, k=k,
                  slots_per_request=slots, steps=int(rng.integers(20, 80)),
                  kv_kind=str(rng.choice(["hot", "plain", "cluster"])), hot_count=int(rng.integers(0, 5)),
                  n_centroids=64, var_len=var_len, ar_coef=float(rng.uniform(0.2, 0.95)))
    host_segments = bool(rng.random() < 0.5)
    return w, slots, host_segments


KV16 = [kv16_case(i) for i in range(N_KV16)]


@pytest.mark.parametrize("i", range(N_KV16),
                         ids=[f"{w.name}-B{w.B}-{w.Hq}x16-k{w.k}-{'var' if w.var_len else 'fixed'}-"
                              f"{'hostseg' if hs else 'gpuseg'}" for w, _, hs in KV16])
def test_random_append_kv16(spin_lib, i):
    """Offload, then a token appended per request per step, with 16 KV heads
    (pages crossed, new partitions started, resident tail pages written):
    host bytes, summaries and every stage against the oracle."""
    from tests.gpu_harness import Pair, log
    w, slots, host_segments = KV16[i]
    log(f"[case] {w.name} B={w.B} Hq={w.Hq} ctx={w.ctx} k={w.k} var_len={w.var_len} C={slots} "
        f"steps={w.steps} host_segments={host_segments}")
    extra = (w.steps + W.PAGE_TOKENS - 1) // W.PAGE_TOKENS + 2
    p = Pair(w, slots=slots, host_segments=host_segments, offload_extra_pages=extra)
    p.check_host()
    p.check_summaries()
    st, _ = p.run(append=True)
    p.check_host()
    p.check_summaries()
    assert st.error_word == 0 and st.misses > 0
    p.close()
