"""GPU parity: the HIP path against the CPU oracle, stage by stage (needs MI355X)."""
import numpy as np
import pytest

from sparse_attention_tiered_amd import workload as W
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _pair(w, **kw):
    from tests.gpu_harness import Pair, log
    log(f"[case] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} ctx={w.ctx} k={w.k} "
        f"C={kw.get('slots', w.slots_per_request)} steps={w.steps}")
    return Pair(w, **kw)


def test_c1_tiny_full_parity(spin_lib):
    p = _pair(W.C1)
    p.check_summaries()
    st, _ = p.run()
    assert st.misses > 0
    p.close()


# small versions of the larger shapes: every stage, every output, every step;
# tight budgets so the bucketed LRU fires
SMALL = {
    "c2_ragged": (W.variant(W.C2, B=3, ctx=(5000, 8192, 3001), steps=12), dict(slots=8 * 32 + 40)),
    "c4_pressure": (W.variant(W.C4, B=4, ctx=16384, k=16, steps=20), dict(slots=8 * 16 + 4)),
    "c3_drift": (W.variant(W.C3, B=2, ctx=32768, k=32, steps=40, hot_count=10), dict(slots=8 * 32 * 2)),
    "c5_variable": (W.variant(W.C5, B=2, ctx=(40000, 23456), k=24, steps=10, n_centroids=256),
                    dict(slots=8 * 24 * 4 + 2)),
    "g16_single_kv": (W.variant(W.C1, name="g16", Hq=16, Hkv=1, ctx=(9000,), k=12, steps=8),
                      dict(slots=12 + 1)),
    "g1_mha": (W.variant(W.C1, name="g1", Hq=4, Hkv=4, ctx=(3000,), k=6, steps=8), dict(slots=4 * 6 + 3)),
    # fast-changing queries: misses and evictions every step, buckets crowd
    "churn": (W.variant(W.C4, B=3, ctx=8192, k=16, steps=30, ar_coef=0.2), dict(slots=8 * 16 + 40)),
    # longer than the 64-step bucket range: ages saturate in bucket 0
    "long_saturating": (W.variant(W.C1, name="long", ctx=(6000,), steps=90, ar_coef=0.6),
                        dict(slots=2 * 8 + 12)),
    "fewer_parts_than_k": (W.variant(W.C2, B=3, Hq=8, Hkv=2, ctx=(300, 0, 64 * 40), k=8, steps=6),
                           dict(slots=2 * 8 * 2)),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_shapes_full_parity(spin_lib, name):
    w, kw = SMALL[name]
    p = _pair(w, **kw)
    p.check_summaries()
    st, _ = p.run()
    if name in ("c4_pressure", "c5_variable", "g16_single_kv", "churn", "long_saturating"):
        assert st.evictions > 0
    p.close()


def test_split_sizes_agree(spin_lib):
    """The attention split size changes the reduction tree, not the result."""
    w = W.variant(W.C4, B=2, ctx=8192, k=32, steps=3)
    outs = []
    for pps in (4, 12, 64):
        p = _pair(w, attend_pps=pps, slots=8 * 32 * 2)
        p.run()
        outs.append(p.spin.out.cpu().numpy().copy())
        p.close()
    assert np.max(np.abs(outs[0] - outs[1])) < 1e-5 and np.max(np.abs(outs[0] - outs[2])) < 1e-5


def test_whole_step_call_matches_stages(spin_lib):
    """spin_step (one call, retrieve on a second stream) gives the same state and
    outputs as the stage-by-stage calls."""
    import torch
    w = W.variant(W.C4, B=3, ctx=12000, k=16, steps=8)
    a = _pair(w, slots=8 * 16 + 16, oracle=False)
    b = _pair(w, slots=8 * 16 + 16, oracle=False)
    side = torch.cuda.Stream()
    for t in range(w.steps):
        a.spin.step(a.q_dev[t], t, copy_stream=side)
        b.spin.select(b.q_dev[t])
        b.spin.resolve_evict(t)
        b.spin.retrieve()
        b.spin.attend(b.q_dev[t])
        torch.cuda.synchronize()
        assert torch.equal(a.spin.out, b.spin.out), t
    sa, sb = a.spin.snapshot(), b.spin.snapshot()
    for k in sa:
        assert np.array_equal(sa[k], sb[k]), k
    a.close()
    b.close()


def test_bad_partition_id_sets_error_word(spin_lib):
    import torch
    from sparse_attention_tiered_amd import binding as bd
    p = _pair(W.variant(W.C1, steps=1), oracle=False)
    bad = torch.zeros_like(p.spin.sel)
    bad[0, 0, 0] = 10 ** 6   # out of range: flagged, skipped
    p.spin.sel.copy_(bad)
    p.spin.resolve_evict(0)
    assert p.spin.sync_status() == bd.SPIN_EDEVICE
    st, _ = p.spin.stats()
    assert st.error_word & bd.DEVERR_PARTITION
    p.close()


def test_exhausted_segment_pool_is_reported(spin_lib):
    from sparse_attention_tiered_amd import binding as bd
    p = _pair(W.variant(W.C1, steps=1), num_segments=1, oracle=False)
    p.spin.select(p.q_dev[0])
    p.spin.resolve_evict(0)
    p.spin.retrieve()
    assert p.spin.sync_status() == bd.SPIN_ESEGPOOL
    p.close()
