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


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_full_size_graph_replays(spin_lib, name):
    """The timed configuration of the benchmark (graph replays of the
    device-indexed step, transfer and attention in one launch, the segment
    pass and the inserts inside it in one workgroup: 4.7K inserts a step on
    c4) against the oracle at full size, every step of every workload (16,
    64, 128, 128 and 64 steps): each of the three select forms (one launch
    with several workgroups per list on c1 and c3, one workgroup per list on
    c2 and c4, two kernels on c5's 7.7K-partition lists) and c5's variable
    partitions.  Every step: selection, the whole residency state, block
    tables, the bytes of every page the step retrieved, sampled outputs; the
    resident pool at the end.  c4 (a pool of 25% of demand) evicts every
    step once it has filled, c2 and c5 once their 5x buffers have, and c3's
    hot set drifts every 16 steps."""
    from tests.gpu_harness import Pair, log
    w = W.get(name)
    steps = w.steps
    log(f"[case] full-size graph replays {w.name}: {steps} steps")
    p = Pair(w, n_steps=steps)
    st, worst = p.run_graph(steps=steps, out_sample=32)
    assert st.misses > 0
    if name in ("c2", "c4", "c5"):
        assert st.evictions > 0
    log(f"[done] {w.name}: evictions={st.evictions}")
    p.close()
