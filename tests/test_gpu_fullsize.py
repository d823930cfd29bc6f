"""GPU parity at the workloads' full sizes, in the benchmark's launch
configuration: selection and the whole residency state every step, attention
on sampled (request, query head) outputs computed one by one by the oracle."""
import pytest

from sparse_attention_tiered_amd import workload as W
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

FULL = {"c2": 10, "c3": 10, "c4": 10, "c5": 5}


@pytest.mark.parametrize("name", sorted(FULL))
def test_full_size(spin_lib, name):
    from tests.gpu_harness import Pair, log
    w = W.get(name)
    steps = FULL[name]
    log(f"[case] full-size {w.name}: {steps} steps")
    p = Pair(w, n_steps=steps)
    st, worst = p.run(steps=steps, out_sample=24)
    assert st.misses > 0
    p.close()


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_full_size_graph_replays(spin_lib, name):
    """The timed configuration of the benchmark (graph replays of the
    device-indexed step, transfer and attention in one launch, the segment
    pass and the inserts inside it in one workgroup: 4.7K inserts a step on
    c4) against the oracle at full size, for every workload: each of the
    three select forms (one launch with several workgroups per list on c1
    and c3, one workgroup per list on c2 and c4, two kernels on c5's
    7.7K-partition lists) and c5's variable partitions."""
    from tests.gpu_harness import Pair, log
    w = W.get(name)
    # c4's pool (25% of demand) fills over its first steps; 24 take it well
    # into eviction every step.  c3's hot set drifts every 16 steps; 40
    # cross two of those boundaries
    steps = {"c3": 40, "c4": 24, "c5": 12}.get(name, 6)
    log(f"[case] full-size graph replays {w.name}: {steps} steps")
    p = Pair(w, n_steps=steps)
    st, worst = p.run_graph(steps=steps, out_sample=24)
    assert st.misses > 0
    if name == "c4":
        assert st.evictions > 0
    p.close()
