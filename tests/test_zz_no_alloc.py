"""spin_attend_noalloc, the attention entry point that allocates nothing (no
context, no workspace; its split partials live in a static device array),
against spin_attend through the C ABI: two calls in a row, the second on a
smaller batch, each bit for bit equal to spin_attend over the same block
tables and within 2e-3 of the oracle."""
import numpy as np
import pytest

from sparse_attention_tiered_amd import workload as W
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def test_noalloc_attention_matches_spin_attend(spin_lib):
    import torch

    from sparse_attention_tiered_amd import binding as bd
    from tests.gpu_harness import Pair, log

    w = W.variant(W.C4, name="noalloc", B=4, ctx=(16384, 9000, 16384, 5000), k=16, steps=4,
                  ar_coef=0.5)
    log(f"[case] spin_attend_noalloc vs spin_attend, {w.name} B={w.B}")
    p = Pair(w, slots=8 * 16 + 8)
    assert p.spin.splits > 1  # the partials go through the static array
    p.run(steps=w.steps)
    t = w.steps - 1
    q = p.q_dev[t]
    ref = p.spin.attend(q, out=torch.empty_like(p.spin.out))
    torch.cuda.synchronize()
    want = p.oracle.attend(p.draws.q_bits[t], p.last_blocks)
    assert np.max(np.abs(ref.cpu().numpy() - want)) <= 2e-3

    # first call: the whole batch
    out1 = torch.full_like(p.spin.out, float("nan"))
    bd.attend_noalloc(q, p.spin.pool, p.spin.block_table, p.spin.block_ntok, p.spin.block_count, out1)
    torch.cuda.synchronize()
    assert torch.equal(out1, ref)
    assert np.max(np.abs(out1.cpu().numpy() - want)) <= 2e-3

    # second call: a smaller input (the first two requests), over the partials
    # the first call left in the array
    out2 = torch.full((2, w.Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    bd.attend_noalloc(q, p.spin.pool, p.spin.block_table, p.spin.block_ntok, p.spin.block_count, out2,
                      batch=2)
    torch.cuda.synchronize()
    assert torch.equal(out2, ref[:2])
    assert np.max(np.abs(out2.cpu().numpy() - want[:2])) <= 2e-3
    p.close()


def test_noalloc_rejects_sizes_beyond_its_array(spin_lib):
    """Partials larger than the static array are refused before any launch."""
    import ctypes

    import torch

    from sparse_attention_tiered_amd import binding as bd
    lib = bd.load()
    dev = torch.zeros(64, dtype=torch.float32, device="cuda")
    p = ctypes.c_void_p(dev.data_ptr())
    # 1024 requests x 256 query heads x 1024 splits of 4 pages: far beyond 32 MiB
    rc = lib.spin_attend_noalloc(p, p, 1, p, p, p, p, 1024, 256, 16, 4096, 4, None)
    assert rc == bd.SPIN_ESCRATCH
    assert lib.spin_strerror(rc).decode().startswith("input too large")
    # within every limit but the array's: 64 requests x 64 query heads x 16 splits
    rc = lib.spin_attend_noalloc(p, p, 1, p, p, p, p, 64, 64, 8, 1024, 64, None)
    assert rc == bd.SPIN_ESCRATCH
    torch.cuda.synchronize()
