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
