"""Write tests/golden/c1_trace.json: the CPU oracle's trace of the tiny decode
workload (1 request, 8/2 heads, 4096 tokens, top-k 8, 16 steps, seed 0), with
a tight budget (mandatory + 4 pages) and fast-changing queries so the bucketed
LRU fires.  Only the oracle and the seeded input generator run here.

    python tests/golden/make_c1_trace.py

The stored values are the oracle's own: they pin it against unintended
changes.  A change to the oracle's arithmetic that alters them must name, in
its commit message, the passage (or reading) of the pages that justifies it.
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from oracle.spin_oracle import SpinOracle  # noqa: E402
from sparse_attention_tiered_amd import workload as W  # noqa: E402

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_trace.json")


def trace():
    w = W.variant(W.C1, ar_coef=0.5, slots_per_request=2 * 8 + 4)
    geo = W.geometry(w)
    draws = W.draw_queries(w, geo)
    kv = W.host_kv_numpy(w, geo, draws, threads=1)
    o = SpinOracle(w.B, w.Hq, w.Hkv, w.k, w.slots_per_request, geo.max_pages, 2)
    o.index(0, kv[0], geo.lens[0])
    steps = []
    for t in range(w.steps):
        sel, blocks, out = o.step(draws.q_bits[t], t)
        st = o.stats[0]
        steps.append({
            "t": t,
            "sel": sel[0].tolist(),
            "hits": st["hits"], "misses": st["misses"], "evictions": st["evictions"],
            "cutoff": st["cutoff"],
            "owner": o.owner[0].tolist(),
            "out_sha256": hashlib.sha256(np.ascontiguousarray(out).tobytes()).hexdigest(),
            "out_sum": float(np.float64(out).sum()),
        })
    return {"workload": "c1_tiny, ar_coef 0.5, 20 slots, seed 0",
            "citation": "oracle trace; rules: Select per-head top-k, bucketed LRU with 64 buckets, "
                        "two-level page table (m.x-techcon article on SPIN, design parts 1-3)",
            "steps": steps}


if __name__ == "__main__":
    with open(PATH, "w") as f:
        json.dump(trace(), f, indent=1)
    print(f"wrote {PATH}")
