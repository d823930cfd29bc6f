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
    # 128 (request, KV head) lists: scoring and top-k in one kernel
    "fused_select": (W.variant(W.C4, B=16, ctx=tuple(2000 + 300 * b for b in range(16)), k=8, steps=10,
                               ar_coef=0.3), dict(slots=8 * 8 + 16)),
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


@pytest.mark.parametrize("pps", [0, 4])
def test_whole_step_call_matches_stages(spin_lib, pps):
    """spin_step with a second stream (retrieve overlapped with attention over
    the resident pages) gives the same state as the stage-by-stage calls and
    the same outputs up to the rounding of the two-pass merge; both match the
    oracle."""
    import torch
    # with the split size left to the library, 8 x 8 lists of 16 pages get
    # 4-page splits for the whole table and 8-page ones for the resident pass
    w = W.variant(W.C4, B=3 if pps else 8, ctx=12000, k=16, steps=8, ar_coef=0.5)
    a = _pair(w, slots=8 * 16 + 16, attend_pps=pps)
    b = _pair(w, slots=8 * 16 + 16, attend_pps=pps, oracle=False)
    side = torch.cuda.Stream()
    for t in range(w.steps):
        a.spin.step(a.q_dev[t], t, copy_stream=side)
        b.spin.select(b.q_dev[t])
        b.spin.resolve_evict(t)
        b.spin.retrieve()
        b.spin.attend(b.q_dev[t])
        torch.cuda.synchronize()
        assert torch.equal(a.spin.sel, b.spin.sel), t
        assert torch.max(torch.abs(a.spin.out - b.spin.out)).item() < 1e-5, t
        sel_o, blocks, out_o = a.oracle.step(a.draws.q_bits[t], t)
        assert np.array_equal(a.spin.sel.cpu().numpy(), sel_o), t
        assert np.max(np.abs(a.spin.out.cpu().numpy() - out_o)) < 2e-3, t
    st, _ = a.spin.stats()
    assert st.misses > 0 and st.hits > 0
    sa, sb = a.spin.snapshot(), b.spin.snapshot()
    for k in sa:
        assert np.array_equal(sa[k], sb[k]), k
    a.close()
    b.close()


@pytest.mark.parametrize("pps", [8, 0])
@pytest.mark.parametrize("mode", ["fetched_pass", "on_arrival", "one_launch"])
def test_overlapped_attention_calls(spin_lib, mode, pps):
    """attend_begin / attend_finish on one stream equal spin_attend (every
    block a hit, every block a miss, and mixed steps), with the fetched pages
    attended after the transfer, by the transfer itself on arrival, or by
    spin_transfer_attend (the transfer and the resident-page attention in one
    launch, then attend_finish); the last two give the same bits.  With the
    split size left to the library (pps 0) the resident-page pass takes
    longer splits than the whole-table and fetched-page passes (8 x 8 lists
    of 16 pages: 8 pages against 4), so the merges combine differently
    split passes."""
    import torch
    if pps:
        w = W.variant(W.C2, B=2, ctx=(9000, 5000), k=8, steps=6, ar_coef=0.3)
        slots = 8 * 8 + 8
    else:
        w = W.variant(W.C2, B=8, ctx=tuple(5000 + 700 * b for b in range(8)), k=16, steps=6, ar_coef=0.3)
        slots = 8 * 16 + 8
    p = _pair(w, slots=slots, oracle=False, attend_pps=pps)
    ref = torch.empty_like(p.spin.out)
    arr = torch.empty_like(p.spin.out)
    for t in range(w.steps):
        q = p.q_dev[t]
        p.spin.select(q)
        p.spin.resolve_evict(t)
        if mode == "fetched_pass":
            p.spin.retrieve()
        else:
            p.spin.retrieve_attend(q)
        p.spin.attend(q, out=ref)
        if mode == "one_launch":
            # the staged two-stream form's bits, then the one launch over
            # the same state (re-pulling the same pages is idempotent)
            p.spin.attend_begin(q)
            p.spin.attend_finish(q, out=arr)
            p.spin.transfer_attend(q)
        else:
            p.spin.attend_begin(q)
        p.spin.attend_finish(q)
        torch.cuda.synchronize()
        assert torch.max(torch.abs(ref - p.spin.out)).item() < 1e-5, t
        if mode == "one_launch":
            assert torch.equal(arr, p.spin.out), t
    p.close()


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


def test_budget_elasticity(spin_lib):
    """Shrinking a request's budget makes the next resolve reclaim the excess
    with the bucketed LRU; growing it back stops eviction.  Bit-exact state
    against the oracle every step."""
    from sparse_attention_tiered_amd import binding as bd
    w = W.variant(W.C4, B=3, ctx=16384, k=16, steps=24, ar_coef=0.5)
    mand = 8 * 16
    p = _pair(w, slots=mand * 4)

    def hook(t):
        plan = {6: [(0, mand), (1, mand + 40)], 12: [(2, mand + 1)], 16: [(0, mand * 4)]}
        for b, slots in plan.get(t, []):
            p.spin.set_budget(b, slots)
            p.oracle.set_budget(b, slots)

    st, _ = p.run(on_step=hook)
    assert st.evictions > 0
    with pytest.raises(bd.SpinError) as e:
        p.spin.set_budget(0, mand - 1)
    assert e.value.code == bd.SPIN_ECAPACITY
    with pytest.raises(bd.SpinError) as e:
        p.spin.set_budget(0, mand * 4 + 1)
    assert e.value.code == bd.SPIN_EINVAL
    p.close()


def test_metadata_footprint(spin_lib):
    """Two-level metadata accounting: live segments equal the oracle's linked
    segments; static sizes follow the configuration."""
    w = W.variant(W.C4, B=3, ctx=20000, k=16, steps=10, ar_coef=0.5)
    p = _pair(w, slots=8 * 16 * 2)
    p.run()
    md = p.spin.metadata()
    o = p.oracle
    live = o.n_seg - len(o.free_stack)
    assert md["live_segments"] == live > 0
    assert md["num_segments"] == o.n_seg
    assert md["live_segment_bytes"] == live * 264
    assert md["directory_bytes"] == w.B * w.Hkv * o.ndir * 4
    assert md["flat_table_bytes"] == w.B * w.Hkv * o.max_pages * 4
    assert md["reverse_map_bytes"] == w.B * o.C * 8
    p.close()


@pytest.mark.parametrize("name", ["fixed", "variable", "kv16"])
def test_offload_and_append(spin_lib, name):
    """Prefill-side Offload + Index from device KV, then one appended token per
    request per step: host bytes, summaries, selection, residency state and
    outputs match the oracle every step (ragged requests, a partial tail;
    with 16 KV heads each lane of the append kernel owns two elements)."""
    if name == "fixed":
        w = W.variant(W.C4, B=3, ctx=(5000, 3000, 64 * 20), k=8, steps=40, ar_coef=0.5)
        slots = 8 * 8 + 24
    elif name == "kv16":
        w = W.variant(W.C5, name="kv16", B=2, Hq=32, Hkv=16, ctx=(7000, 3333), k=6, steps=30,
                      n_centroids=64)
        slots = 16 * 6 * 4 + 24
    else:
        w = W.variant(W.C5, B=2, ctx=(9000, 4321), k=8, steps=30, n_centroids=64)
        slots = 8 * 8 * 4 + 24
    p = _pair(w, slots=slots, offload_extra_pages=3)
    p.check_host()
    p.check_summaries()
    st, _ = p.run(append=True)
    p.check_host()
    p.check_summaries()
    assert st.misses > 0
    p.close()


@pytest.mark.parametrize("name", ["c4_pressure", "churn", "c5_variable"])
def test_host_segment_tables(spin_lib, name):
    """Second-level segment tables in pinned host memory (the kernels reach
    them through the device-mapped address): the same residency state bit for
    bit, the same outputs, every step."""
    w, kw = SMALL[name]
    p = _pair(w, host_segments=True, **kw)
    st, _ = p.run()
    assert st.evictions > 0
    md = p.spin.metadata()
    assert md["host_segment_bytes"] == p.cfg.num_segments * 64 * 4
    assert md["segment_pool_bytes"] == p.cfg.num_segments * 8
    p.close()


def test_host_segment_tables_with_append(spin_lib):
    """Offload, then a token appended per step, with the segment tables in
    host memory (the append kernel reads them to find a resident tail page)."""
    w = W.variant(W.C4, B=3, ctx=(5000, 3000, 64 * 20), k=8, steps=20, ar_coef=0.5)
    p = _pair(w, slots=8 * 8 + 24, offload_extra_pages=3, host_segments=True)
    st, _ = p.run(append=True)
    p.check_host()
    p.check_summaries()
    assert st.misses > 0
    p.close()


def test_append_capacity_is_checked(spin_lib):
    import torch
    from sparse_attention_tiered_amd import binding as bd
    w = W.variant(W.C1, ctx=(64 * 3,), steps=1)
    p = _pair(w, slots=2 * 8 + 4, offload_extra_pages=1, oracle=False)
    dk = torch.zeros((1, 2, 128), dtype=torch.int16, device="cuda")
    for _ in range(64):      # fills the one reserved page
        p.spin.append(dk, dk)
    with pytest.raises(bd.SpinError) as e:
        p.spin.append(dk, dk)
    assert e.value.code == bd.SPIN_ECAPACITY
    p.close()


def test_size_limits(spin_lib):
    """The kernels' size limits at once: 16384 partitions per head (top-k keys
    fill 64 KiB of LDS), top-k 1024, 65536 slots per request (the resolve
    kernel's LDS bitmask), 16 query heads per KV head."""
    w = W.variant(W.C1, name="limits", Hq=16, Hkv=1, ctx=(16384 * 64,), k=1024, steps=3, hot_count=8)
    p = _pair(w, slots=65536)
    p.check_summaries()
    st, _ = p.run(out_sample=16)
    assert st.misses > 0
    p.close()


def test_split_select_at_its_limit(spin_lib):
    """The several-workgroups-per-list select at the longest lists it takes:
    4096 partitions (eight 512-row workgroups, 128 score ranges handed over)
    and a ragged 4001 (a last workgroup with one row)."""
    w = W.variant(W.C3, name="split_limit", B=2, Hq=16, Hkv=2, ctx=(4096 * 64, 4000 * 64 + 17), k=64,
                  steps=6, hot_count=8)
    p = _pair(w, slots=2 * 64 * 3)
    assert p.geo.max_parts == 4096
    st, _ = p.run()
    assert st.misses > 0
    p.close()


# (partitions per list, k): lists one past k, and lists that end on, one past
# and one short of a workgroup's rows (256-row workgroups below 1024
# partitions, 512-row ones from there), in both split-select row layouts
SPLIT_EDGES = [(9, 8), (65, 64), (255, 8), (256, 8), (257, 64), (511, 64), (512, 8), (513, 64),
               (1023, 64), (1024, 8), (1025, 64), (1537, 64)]


@pytest.mark.parametrize("n,k", SPLIT_EDGES, ids=[f"n{n}-k{k}" for n, k in SPLIT_EDGES])
def test_split_select_chunk_edges(spin_lib, n, k):
    """The several-workgroups-per-list select at the list lengths where its
    work split changes (the second request one partition shorter, its last
    page ragged): the selections and scores of every step against the
    oracle's, with the rest of the step checked as usual."""
    w = W.variant(W.C3, name=f"split_edge_{n}_{k}", B=2, Hq=8, Hkv=2, ctx=(n * 64, (n - 1) * 64 - 37),
                  k=k, steps=4, hot_count=3)
    p = _pair(w, slots=2 * k * 3)
    assert p.geo.max_parts == n
    st, _ = p.run()
    assert st.misses > 0
    p.close()


@pytest.mark.parametrize("form", ["staged", "graph"])
def test_step_lists_beyond_lds(spin_lib, form):
    """One request's step past every list the resolve kernel keeps in LDS:
    8192 misses at step 0 (the slot assignment goes through the insert list
    itself, the misses past 2048 are read back from global memory) and about
    5000 victims a step after it (the victim list no longer fits, so the
    eviction pass walks every slot), with k = 1024 over 4 KV heads and
    two-page partitions."""
    w = W.variant(W.C5, name="big_lists", B=1, Hq=8, Hkv=4, ctx=(300000,), k=1024, steps=4,
                  var_len=(65, 128), n_centroids=64, ar_coef=0.1)
    p = _pair(w, slots=8192 + 64)
    st, _ = p.run(out_sample=16) if form == "staged" else p.run_graph(out_sample=16)
    assert st.misses > 8192 and st.evictions > 3 * 4097
    p.close()


def test_directory_beyond_lds(spin_lib):
    """A request directory larger than the resolve kernel keeps in LDS (16 KV
    heads x 313 ranges of 64 pages = 5008 entries > 4096): every lookup and
    the emptied-range returns go through global memory, under a tight budget
    so the bucketed LRU empties segments every step."""
    w = W.variant(W.C5, name="dir_global", B=2, Hq=16, Hkv=16, ctx=(40000, 23000), k=12, steps=10,
                  n_centroids=64, ar_coef=0.3)
    p = _pair(w, slots=16 * 12 * 4 + 24, max_pages=20000)
    assert p.cfg.num_kv_heads * ((p.cfg.max_pages + 63) // 64) > 4096
    p.check_summaries()
    st, _ = p.run()
    assert st.evictions > 0
    p.close()


def test_tight_budget_with_limits(spin_lib):
    """Eviction at k = 1024 with variable partitions of up to 4 pages."""
    w = W.variant(W.C5, name="limits_var", B=1, Hq=16, Hkv=1, ctx=(300000,), k=1024, steps=4,
                  n_centroids=32, ar_coef=0.2)
    p = _pair(w, slots=1024 * 4 + 16)
    st, _ = p.run(out_sample=16)
    assert st.evictions > 0
    p.close()


@pytest.mark.parametrize("form", ["staged", "graph"])
def test_host_padding_is_never_used(spin_lib, form):
    """Token slots past a partition's last token may hold anything in host
    memory: here bf16 NaN in every key and value entry of every partly filled
    page.  The transfer leaves zeros there in the pool (every filled and every
    resident slot equals its host page with that padding zeroed), so the
    outputs stay those of the valid tokens alone, within the usual tolerance
    of the oracle (which reads only those), with eviction and re-fetches."""
    w = W.variant(W.C5, name="nan_padding", cfg_id=77, B=2, Hq=8, Hkv=2, ctx=(6000, 4000), k=8,
                  steps=16, n_centroids=16, var_len=(16, 200), ar_coef=0.5)
    p = _pair(w, slots=2 * 8 * 4 + 2, pad_fill=0x7FC0)
    st, worst = p.run() if form == "staged" else p.run_graph()
    assert st.evictions > 0 and np.isfinite(worst)
    p.close()


# every key of a head is one vector (hot partitions shifted): scores tie
# exactly inside each group, so the lower-id rule alone decides the selection
TIES = {
    # the boundary falls among ~500 equal scores (the crowded-bucket path)
    "ties_crowded": W.variant(W.C2, name="ties_crowded", B=2, Hq=8, Hkv=2, ctx=(32768, 20000),
                              k=8, steps=4, kv_kind="ties", hot_count=5),
    # the boundary falls among the 40 equal hot scores
    "ties_in_hot": W.variant(W.C2, name="ties_in_hot", B=2, Hq=8, Hkv=2, ctx=(32768, 9000),
                             k=8, steps=4, kv_kind="ties", hot_count=40),
    # ... among 120 equal hot scores: more boundary-bin members than one
    # wave's lanes, ranked one per thread
    "ties_in_hot_120": W.variant(W.C2, name="ties_in_hot_120", B=2, Hq=8, Hkv=2, ctx=(32768, 20000),
                                 k=50, steps=4, kv_kind="ties", hot_count=120),
    # every score of a head equal (a zero-width score range)
    "ties_flat": W.variant(W.C2, name="ties_flat", B=1, Hq=8, Hkv=2, ctx=(20000,),
                           k=16, steps=3, kv_kind="ties", hot_count=0),
    # lists past the split select's 4096 partitions (scoring and top-k as two
    # launches), ties inside the hot group at the boundary
    "ties_two_launch": W.variant(W.C2, name="ties_two_launch", B=1, Hq=8, Hkv=2, ctx=(300000,),
                                 k=16, steps=3, kv_kind="ties", hot_count=40),
    # 128 lists (the fused score + top-k kernel), ties inside the hot group
    "ties_fused": W.variant(W.C2, name="ties_fused", B=32, Hq=16, Hkv=4, ctx=(4096,) * 32,
                            k=8, steps=3, kv_kind="ties", hot_count=20),
}


@pytest.mark.parametrize("name", sorted(TIES))
def test_exact_ties_take_lower_ids(spin_lib, name):
    w = TIES[name]
    p = _pair(w, slots=w.Hkv * w.k * 2)
    for t in range(p.T):
        p.spin.select(p.q_dev[t], scores=p.scores)
        sel_o, _ = p.oracle.select(p.draws.q_bits[t])
        assert np.array_equal(p.spin.sel.cpu().numpy(), sel_o.astype(np.int32)), t
    st, _ = p.run()
    assert st.misses > 0
    p.close()


def test_max_batch(spin_lib):
    """1024 requests (the batch limit) of ragged, tiny contexts under a budget
    of mandatory + 1 page: the batch-wide prefix sums of the transfer and of
    the shared segment pool at their largest."""
    ctx = tuple(64 * 3 - (b % 7) * 20 for b in range(1024))
    w = W.variant(W.C1, name="max_batch", B=1024, Hq=4, Hkv=2, ctx=ctx, k=2, steps=4, ar_coef=0.2)
    p = _pair(w, slots=2 * 2 + 1)
    st, _ = p.run()
    assert st.misses > 0 and st.evictions > 0
    p.close()


@pytest.mark.parametrize("name,host", [("c4_pressure", False), ("c4_pressure", True),
                                       ("churn", False), ("c5_variable", True)],
                         ids=["c4_pressure", "c4_pressure-host_segments", "churn",
                              "c5_variable-host_segments"])
def test_graph_replays_match_oracle(spin_lib, name, host):
    """Graph replays of the device-indexed step (transfer, resident-page
    attention and the segment-pool pass in one launch; the merge advances
    the step index) against the oracle every step: selection, the whole
    residency state, block tables, every output; with the segment tables in
    GPU or in host memory."""
    w, kw = SMALL[name]
    p = _pair(w, host_segments=host, **kw)
    st, _ = p.run_graph()
    assert st.evictions > 0
    p.close()


def test_max_batch_graph_replays(spin_lib):
    """The batch limit through the one-launch step: the segment-pool pass in a
    256-thread workgroup takes the per-request prefix sums of 1024 requests."""
    ctx = tuple(64 * 3 - (b % 7) * 20 for b in range(1024))
    w = W.variant(W.C1, name="max_batch_graph", B=1024, Hq=4, Hkv=2, ctx=ctx, k=2, steps=4,
                  ar_coef=0.2)
    p = _pair(w, slots=2 * 2 + 1)
    st, _ = p.run_graph()
    assert st.misses > 0 and st.evictions > 0
    p.close()


def test_streams_change_between_steps(spin_lib):
    """The staged calls with the transfer on a second stream
    (spin_retrieve_attend on the copy stream beside spin_attend_begin, then
    spin_attend_finish) and the stream roles moving every step (this step's
    copy stream computes the next one) match the oracle, and are
    bit-identical to the whole-step call (transfer and attention in one
    launch) on one fixed stream pair: every cross-stream wait for a transfer
    or a resolve lands where it must."""
    import torch

    w = W.variant(W.C1, name="rotating", steps=12, ar_coef=0.2)
    streams = [torch.cuda.Stream() for _ in range(3)]
    fixed = (torch.cuda.Stream(), torch.cuda.Stream())
    a = _pair(w, slots=2 * 8 + 4)
    b = _pair(w, slots=2 * 8 + 4, oracle=False)
    torch.cuda.synchronize()
    for t in range(w.steps):
        s, c = streams[t % 3], streams[(t + 1) % 3]
        q = a.q_dev[t]
        a.spin.select(q, stream=s)
        a.spin.resolve_evict(t, stream=s)
        a.spin.retrieve_attend(q, copy_stream=c)
        a.spin.attend_begin(q, stream=s)
        a.spin.attend_finish(q, stream=s)
        b.spin.step(b.q_dev[t], t, stream=fixed[0], copy_stream=fixed[1])
        torch.cuda.synchronize()
        sel_o, blocks, out_o = a.oracle.step(a.draws.q_bits[t], t)
        assert np.array_equal(a.spin.sel.cpu().numpy(), sel_o.astype(np.int32)), t
        out = a.spin.out.cpu().numpy()
        assert np.max(np.abs(out - out_o)) <= 2e-3, t
        assert np.array_equal(out.view(np.uint32), b.spin.out.cpu().numpy().view(np.uint32)), t
        a.check_state(t)
        sa, sb = a.spin.snapshot(), b.spin.snapshot()
        for key in sa:
            assert np.array_equal(sa[key], sb[key]), (t, key)
    st, _ = a.spin.stats()
    assert st.error_word == 0 and st.evictions > 0
    a.close()
    b.close()


def test_graph_replayed_steps(spin_lib):
    """One spin_step_at call (device-side step index) captured in a HIP graph
    and replayed for consecutive steps, with eager work and synchronisations
    between the replays, equals the eager whole-step calls bit for bit
    (outputs, selections, the whole residency state) and the oracle."""
    import torch

    w = W.variant(W.C1, name="graph", steps=10, ar_coef=0.2)
    a = _pair(w, slots=2 * 8 + 4)                # eager, checked against the oracle
    b = _pair(w, slots=2 * 8 + 4, oracle=False)  # the graph
    Sa, Ca = torch.cuda.Stream(), torch.cuda.Stream()
    Sb, Cb = torch.cuda.Stream(), torch.cuda.Stream()
    t_dev = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def compare(t):
        sel_o, _, out_o = a.oracle.step(a.draws.q_bits[t], t)
        out = a.spin.out.cpu().numpy()
        assert np.array_equal(a.spin.sel.cpu().numpy(), sel_o.astype(np.int32)), t
        assert np.max(np.abs(out - out_o)) <= 2e-3, t
        assert np.array_equal(out.view(np.uint32), b.spin.out.cpu().numpy().view(np.uint32)), t
        assert torch.equal(a.spin.sel, b.spin.sel), t
        sa, sb = a.spin.snapshot(), b.spin.snapshot()
        for key in sa:
            assert np.array_equal(sa[key], sb[key]), (t, key)
        assert int(t_dev.item()) == t + 1

    # step 0 eagerly through the device-index call, then capture one step
    a.spin.step(a.q_dev[0], 0, stream=Sa, copy_stream=Ca)
    b.spin.step_at(b.q_dev, t_dev, stream=Sb, copy_stream=Cb)
    torch.cuda.synchronize()
    compare(0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=Sb):
        b.spin.step_at(b.q_dev, t_dev, stream=Sb, copy_stream=Cb)
    torch.cuda.synchronize()
    assert int(t_dev.item()) == 1  # capturing ran nothing
    for t in range(1, w.steps):
        with torch.cuda.stream(Sb):
            g.replay()
        a.spin.step(a.q_dev[t], t, stream=Sa, copy_stream=Ca)
        torch.cuda.synchronize()
        compare(t)
        b.spin.stats()  # eager library work between replays
    st, _ = b.spin.stats()
    assert st.error_word == 0 and st.evictions > 0
    a.close()
    b.close()


@pytest.mark.parametrize("name", ["split_select", "fused_select", "long_lists"])
def test_runs_are_deterministic(spin_lib, name):
    """Two contexts driven through the same whole-step calls give the same
    bits every step: selections, block tables, outputs, and the whole
    residency state at the end.  Covers the hand-overs between workgroups of
    one launch (the select's scores to the last workgroup of each list, the
    transfer's arrival partials, the resident-page partials) on all three
    select forms."""
    import torch
    if name == "split_select":      # few lists, 2 048 partitions each: several workgroups per list
        w = W.variant(W.C3, B=2, ctx=131072, k=32, steps=48, hot_count=10)
        slots = 8 * 32 * 2
    elif name == "fused_select":    # 128 lists: one workgroup per list
        w = W.variant(W.C4, B=16, ctx=16384, k=16, steps=24, ar_coef=0.4)
        slots = 8 * 16 + 24
    else:                           # lists longer than 4096 partitions: scoring and top-k as two kernels
        w = W.variant(W.C4, B=1, ctx=300000, k=64, steps=16, ar_coef=0.4)
        slots = 8 * 64 + 64
    a = _pair(w, slots=slots, oracle=False)
    b = _pair(w, slots=slots, oracle=False)
    side_a, side_b = torch.cuda.Stream(), torch.cuda.Stream()
    for t in range(w.steps):
        a.spin.step(a.q_dev[t], t, copy_stream=side_a)
        b.spin.step(b.q_dev[t], t, copy_stream=side_b)
        torch.cuda.synchronize()
        assert torch.equal(a.spin.sel, b.spin.sel), t
        assert torch.equal(a.spin.block_table, b.spin.block_table), t
        assert torch.equal(a.spin.out, b.spin.out), t
    st_a, _ = a.spin.stats()
    st_b, _ = b.spin.stats()
    assert (st_a.hits, st_a.misses, st_a.evictions) == (st_b.hits, st_b.misses, st_b.evictions)
    assert st_a.misses > 0
    sa, sb = a.spin.snapshot(), b.spin.snapshot()
    for k in sa:
        assert np.array_equal(sa[k], sb[k]), k
    a.close()
    b.close()


def _turnover_plan(p):
    """Mid-run request turnover: a request released (its area and segments go
    back; it selects and attends nothing meanwhile), later indexed again with
    new, shorter KV; a request re-indexed in place while it holds pages in
    several directory ranges; another released near the end."""
    def hook(t):
        if t == 5:
            p.release_request(1)
        elif t == 9:
            p.reindex_request(1, 9000, seed=1)
        elif t == 13:
            p.reindex_request(2, 12345, seed=2)
        elif t == 17:
            p.release_request(0)
    return hook


@pytest.mark.parametrize("form", ["staged", "graph"])
def test_request_turnover(spin_lib, form):
    """Request turnover ([XT] part 2: each request's GPU area; part 3: segments
    taken from and returned to one shared pool): releases and re-indexing
    between steps, with eviction firing, staged or between replays of the
    captured one-launch step.  Every step: selection, the whole residency
    state (directory, segments, live counts, free stack, owner, last_use,
    free counts) bit for bit, block tables, the pool bytes of every insert,
    every output; the resident pool at the end."""
    w = W.variant(W.C4, B=4, ctx=16384, k=16, steps=22, ar_coef=0.5)
    p = _pair(w, slots=8 * 16 + 40)
    hook = _turnover_plan(p)
    if form == "staged":
        st, _ = p.run(on_step=hook)
    else:
        st, _ = p.run_graph(on_step=hook)
    assert st.evictions > 0
    per = p.spin.stats()[1]
    assert per[0, 1] > 0 and per[1, 1] > 0
    p.close()


def test_rewound_step_is_refused(spin_lib):
    """A step index below the last resolved step would make ages negative.
    Host-side t: spin_resolve_evict refuses it (SPIN_EINVAL).  A device-side
    index the host cannot see (spin_step_at after host-indexed steps): the
    resolve sets SPIN_DEVERR_STEP and changes nothing (residency state,
    counters), the step attends no pages (zero outputs) and moves no bytes;
    the oracle refuses the same step before changing anything."""
    import torch
    from sparse_attention_tiered_amd import binding as bd
    w = W.variant(W.C1, name="rewind", steps=8, ar_coef=0.2)
    p = _pair(w, slots=2 * 8 + 4)
    p.run(steps=5)
    before = p.spin.snapshot()
    st0, per0 = p.spin.stats()
    with pytest.raises(bd.SpinError) as e:
        p.spin.resolve_evict(3)
    assert e.value.code == bd.SPIN_EINVAL
    S, Cs = torch.cuda.Stream(), torch.cuda.Stream()
    t_dev = torch.full((1,), 2, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    p.spin.out.fill_(1.0)
    p.spin.step_at(p.q_dev, t_dev, stream=S, copy_stream=Cs)
    torch.cuda.synchronize()
    assert p.spin.sync_status() == bd.SPIN_EDEVICE
    st1, per1 = p.spin.stats()
    assert st1.error_word == bd.DEVERR_STEP
    assert (st1.hits, st1.misses, st1.evictions) == (st0.hits, st0.misses, st0.evictions)
    assert np.array_equal(per0, per1)
    after = p.spin.snapshot()
    for key in before:
        assert np.array_equal(before[key], after[key]), key
    assert int(p.spin.block_count.sum().item()) == 0
    assert torch.count_nonzero(p.spin.out).item() == 0
    assert int(t_dev.item()) == 3
    sel_o, _ = p.oracle.select(p.draws.q_bits[2])
    with pytest.raises(ValueError):
        p.oracle.resolve_evict(sel_o, 2)
    p.check_state(2)
    p.close()
