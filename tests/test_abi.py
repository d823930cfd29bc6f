"""The C-ABI library loads, exports every declared symbol, and validates
configurations on the host (no GPU needed: nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest

from sparse_attention_tiered_amd import binding as bd

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "spin.h")


def declared_symbols():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"SPIN_API\s+[\w\s\*]+?\b(spin_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported(spin_lib):
    names = declared_symbols()
    assert len(names) >= 18
    missing = [n for n in names if not hasattr(spin_lib, n)]
    assert not missing, missing
    # and the binding describes exactly the declared calls
    assert sorted(bd.SIGNATURES) == names


def test_config_checks(spin_lib):
    c = bd.make_config(B=4, Hq=32, Hkv=8, max_partitions=2048, max_pages=2048, topk=64,
                       slots_per_request=8 * 6 * 64)
    assert spin_lib.spin_config_check(ctypes.byref(c)) == bd.SPIN_OK
    ws, pool = ctypes.c_size_t(), ctypes.c_size_t()
    assert spin_lib.spin_workspace_size(ctypes.byref(c), ctypes.byref(ws), ctypes.byref(pool)) == 0
    assert pool.value == 4 * 8 * 6 * 64 * 32768
    assert ws.value >= 4 * 8 * 2048 * 128 * 4  # at least the summaries
    nd, mb, sp = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    assert spin_lib.spin_derived(ctypes.byref(c), ctypes.byref(nd), ctypes.byref(mb), ctypes.byref(sp)) == 0
    assert (nd.value, mb.value) == (32, 64) and sp.value >= 1
    # budget below one step's mandatory pages
    c.slots_per_request = 8 * 64 - 1
    assert spin_lib.spin_config_check(ctypes.byref(c)) == bd.SPIN_ECAPACITY
    c.slots_per_request = 8 * 64
    assert spin_lib.spin_config_check(ctypes.byref(c)) == bd.SPIN_OK


@pytest.mark.parametrize("field,value", [
    ("head_dim", 64), ("page_tokens", 32), ("num_q_heads", 14), ("num_kv_heads", 0),
    ("max_partitions", 0), ("max_partitions", 20000), ("topk", 0), ("max_pages_per_partition", 5),
    ("num_segments", 0), ("seg_entries", 32), ("num_buckets", 32), ("max_batch", 0),
    ("segments_in_host_memory", 2),
])
def test_config_rejects(spin_lib, field, value):
    c = bd.make_config(B=2, Hq=16, Hkv=4, max_partitions=128, max_pages=128, topk=8, slots_per_request=4 * 8 * 6)
    setattr(c, field, value)
    assert spin_lib.spin_config_check(ctypes.byref(c)) != bd.SPIN_OK


def test_host_segment_sizes(spin_lib):
    """Segment tables in host memory: their host bytes, and a workspace
    smaller by exactly those bytes (rounded to the 256-byte region alignment)."""
    kw = dict(B=4, Hq=32, Hkv=8, max_partitions=2048, max_pages=2048, topk=64,
              slots_per_request=8 * 6 * 64)
    dev, host = bd.make_config(**kw), bd.make_config(**kw, host_segments=True)
    hb = ctypes.c_size_t()
    assert spin_lib.spin_host_segment_bytes(ctypes.byref(dev), ctypes.byref(hb)) == 0 and hb.value == 0
    assert spin_lib.spin_host_segment_bytes(ctypes.byref(host), ctypes.byref(hb)) == 0
    assert hb.value == host.num_segments * 64 * 4
    ws_d, ws_h, pool = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    spin_lib.spin_workspace_size(ctypes.byref(dev), ctypes.byref(ws_d), ctypes.byref(pool))
    spin_lib.spin_workspace_size(ctypes.byref(host), ctypes.byref(ws_h), ctypes.byref(pool))
    assert ws_d.value - ws_h.value == (hb.value + 255) // 256 * 256
    # spin_create_ex rejects a missing host buffer before touching any device
    out = ctypes.c_void_p()
    assert spin_lib.spin_create_ex(ctypes.byref(host), None, 0, None, 0, None, 0, None,
                                   ctypes.byref(out)) == bd.SPIN_EINVAL


def test_null_arguments_are_rejected(spin_lib):
    assert spin_lib.spin_config_check(None) == bd.SPIN_EINVAL
    assert spin_lib.spin_select(None, None, None, None, None) == bd.SPIN_EINVAL
    assert spin_lib.spin_destroy(None) == bd.SPIN_EINVAL
    assert spin_lib.spin_strerror(bd.SPIN_ECAPACITY).decode().startswith("slots")
