"""The seeded input generator: determinism, geometry and the stated structure (CPU)."""
import numpy as np

import oracle.spin_oracle as om
from sparse_attention_tiered_amd import workload as W


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 1 + 2 ** -9], np.float32)
    assert W.to_bf16_bits(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F80]


def test_named_workload_shapes():
    assert (W.C1.B, W.C1.Hq, W.C1.Hkv, W.C1.k, W.C1.slots_per_request) == (1, 8, 2, 8, 96)
    assert (W.C2.B, W.C2.G, W.C2.slots_per_request) == (16, 5, 1536)
    assert (W.C3.B, W.C3.G, W.C3.slots_per_request, W.C3.ctx[0]) == (8, 8, 3072, 131072)
    assert (W.C4.B, W.C4.slots_per_request, W.C4.steps) == (32, 768, 128)
    assert (W.C5.B, W.C5.k, W.C5.slots_per_request, W.C5.ctx[0]) == (4, 128, 24576, 1 << 20)


def test_variable_partitions_cover_context():
    w = W.variant(W.C5, B=2, ctx=(20000, 777))
    for b in range(2):
        lens = W.partition_lengths(w, b)
        assert lens.sum() == w.ctx[b]
        assert lens[:-1].min() >= 16 and lens.max() <= 256
    full = W.partition_lengths(W.C5, 0)
    assert full.sum() == 1 << 20 and 7000 < len(full) < 8500


def test_deterministic_and_layout():
    w = W.variant(W.C1, ctx=1000, steps=3)
    geo = W.geometry(w)
    a = W.host_kv_numpy(w, geo, W.draw_queries(w, geo), threads=1)
    b = W.host_kv_numpy(w, geo, W.draw_queries(w, geo), threads=4)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    pages = a[0].reshape(w.Hkv, geo.pages[0], -1)
    # 1000 tokens = 15 full pages + 40 tokens: slots 40..63 of the last page are zero
    K = om.page_keys(pages[0, -1])
    V = om.page_values(pages[0, -1])
    assert np.all(K[40:] == 0) and np.all(V[40:] == 0) and np.all(K[:40] != 0)


def test_hot_partitions_are_pushed_toward_group_query():
    w = W.variant(W.C2, B=1, ctx=8192, steps=2)
    geo = W.geometry(w)
    d = W.draw_queries(w, geo)
    kv = W.host_kv_numpy(w, geo, d)[0].reshape(w.Hkv, geo.pages[0], -1)
    for h in range(w.Hkv):
        hot = set(d.hot[(0, h)][0].tolist())
        assert len(hot) == w.hot_count
        proj = [om.page_keys(kv[h, p]).mean(0) @ d.hot_dir[(0, h)] for p in range(geo.pages[0])]
        hot_proj = [proj[p] for p in hot]
        cold_proj = [proj[p] for p in range(geo.pages[0]) if p not in hot]
        assert min(hot_proj) > 1.5 and max(abs(x) for x in cold_proj) < 0.7


def test_queries_follow_ar1():
    w = W.variant(W.C1, steps=40)
    geo = W.geometry(w)
    q = om.bf16_bits_to_f64(W.draw_queries(w, geo).q_bits)
    # the initial draw has unit variance; the stationary law has std sqrt(0.01/0.19)
    assert 0.8 < q[0].std() < 1.2
    assert 0.15 < q[-1].std() < 0.32
