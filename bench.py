"""Sparse-decode benchmark on one MI355X.

A step is one pass of the whole decode path for a batch: select (score +
top-k), two-level resolve with bucketed-LRU eviction, retrieve of missed pages
from pinned host memory, and paged sparse attention.  Inputs (host KV, queries
for every step) are resident before the timed region.

Steps are numbered from 0 (every mandatory page a miss).  The timed window is
K consecutive steps: by default every configured step of the workload after a
warm-up of min(8, steps/4) (the 128K pressure workload: steps 8-127); with
--steps K, the last K configured steps, never starting before step W (the
query stream continues past the configured steps when W + K exceeds them).
Three contexts are indexed from the same pinned host KV and driven through
the same steps; the path is deterministic, so all pass through the same
states (their counters over the window are compared):

  context A  the steps before the window as untimed warm-up, then the window
             as replays of one captured HIP graph of the device-indexed
             whole-step call, back to back, events only at the window's
             ends: `mean_ms_per_step`, the whole window's throughput
             (`value_at_mean`);
  context C  the same, with a timing event between replays:
             `ms_per_step` is the median step of the window and `value` =
             B * Hq / ms_per_step (each event adds a few microseconds of idle
             to the step it closes: `mean_ms_per_step_with_step_events`
             minus `mean_ms_per_step`);
  context B  the same warm-up, then the same window with an event between
             stages on the stream each stage runs on: stage times per step,
             the transfer launch's duration (the roofline of the dominant
             kernel) and the device counters after each step (its bytes);
             then isolated replays of select, attention and the transfer on
             the window's last step, warm and after a 512 MB read that evicts
             the memory-side cache (cold).

Warm-up steps run the serial form of the step (the transfer, then attention),
so the one-launch transfer kernel runs only inside the three windows and a
kernel trace of this command averages it over exactly those steps.  Prints
one JSON line.

    python bench.py [--steps K] [--warmup W] [--config c4] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
PCIE_GEN5_X16_GBS = 63.0       # 32 GT/s x 16 lanes, 128b/130b, one direction
PAGE_BYTES = 32768


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pcie_link():
    """Negotiated link of the GPU from sysfs (best effort)."""
    try:
        import torch
        p = torch.cuda.get_device_properties(0)
        bus = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
        base = f"/sys/bus/pci/devices/{bus}"
        speed = open(f"{base}/current_link_speed").read().strip()
        width = open(f"{base}/current_link_width").read().strip()
        return {"bus": bus, "speed": speed, "width": width}
    except Exception as e:  # noqa: BLE001
        return {"error": str(e)}


def memcpy_h2d_gbs(nbytes=1 << 30):
    """Practical H2D ceiling: one pinned -> device copy engine transfer."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    gbs = 3 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


def kernel_sources_sha():
    """sha256 (12 hex digits) over every kernel source and header of the
    library, in name order: what a committed counter summary was taken with."""
    import hashlib
    csrc = os.path.join(ROOT, "sparse_attention_tiered_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:12]


def counter_traffic(cfg_key, stage, bytes_per_launch):
    """HBM-side bytes per launch of a stage from the committed rocprofv3 counter
    summary (traffic per algorithmic byte over the steps it counts), or None
    when any kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{cfg_key}_hbm_counters.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    lines = [l for l in text.splitlines() if l.startswith("machine-readable: traffic_ratio")]
    if not lines:
        return None
    kv = dict(t.split("=", 1) for t in lines[-1].split()[1:])
    if kv.get("sha_kernels") != kernel_sources_sha():
        return None
    ratio = kv.get(f"traffic_ratio_{stage}")
    return None if ratio is None else float(ratio) * bytes_per_launch


def select_kernels(B, Hkv, max_parts):
    """The select kernels the library launches for this shape: one workgroup
    per list for 128 or more (request, KV head) lists, several workgroups per
    list for lists of up to 4096 partitions, otherwise scoring and top-k as
    two launches."""
    if B * Hkv >= 128:
        return ["k_select_fused"]
    if max_parts <= 4096:
        return ["k_select_split"]
    return ["k_score", "k_topk"]




def timed_window(configured_steps, warmup=None, steps=None):
    """(start, end, steps to draw): the timed steps are start .. end-1.  By
    default every configured step after a warm-up of min(8, steps / 4); with
    an explicit step count K, the last K configured steps, never starting
    before the warm-up (the query stream then runs past the configured
    steps)."""
    warm = warmup if warmup is not None else min(8, configured_steps // 4)
    K = steps if steps is not None else configured_steps - warm
    start = max(warm, configured_steps - K)
    return start, start + K, max(configured_steps, start + K)


def cpu_baseline(w, geo, draws, host_np, start, end, budget_s=20.0):
    """The CPU oracle as it stands, on the same workload and the same steps as
    the GPU's timed window: steps 0 .. start-1 bring its state there untimed
    (select, resolve/evict and retrieve only: attention changes no state),
    then whole decode steps from `start` are timed, as many as fit in about
    budget_s seconds (at least one, at most the window).  BLAS is held to one
    thread and the control flow is single-threaded Python, so the oracle uses
    exactly one core."""
    import contextlib

    from oracle.spin_oracle import SpinOracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas_default = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
        one_thread = threadpool_limits(limits=1)
    except Exception:  # noqa: BLE001
        blas_default, one_thread = None, None
    with one_thread if one_thread is not None else contextlib.nullcontext():
        n_seg = min(w.B * w.slots_per_request, w.B * w.Hkv * ((geo.max_pages + 63) // 64))
        o = SpinOracle(w.B, w.Hq, w.Hkv, w.k, w.slots_per_request, geo.max_pages, n_seg)
        t0 = time.perf_counter()
        for b in range(w.B):
            o.index(b, host_np[b], geo.lens[b])
        for t in range(start):
            sel, _ = o.select(draws.q_bits[t])
            o.resolve_evict(sel, t)
            o.retrieve()
        t_setup = time.perf_counter() - t0
        steps, t0 = 0, time.perf_counter()
        while True:
            o.step(draws.q_bits[start + steps], start + steps)
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or start + steps >= end:
                break
    limit = one_thread
    return {"value": w.B * w.Hq * steps / el, "unit": "head-tokens/s",
            "cores": 1 if limit is not None else blas_default, "kind": "oracle",
            "host_cores_available": len(os.sched_getaffinity(0)),
            "blas_threads_default": blas_default, "blas_threads_used": 1 if limit is not None else blas_default,
            "steps_timed": [start, start + steps - 1],
            "sample": f"decode steps {start}-{start + steps - 1} of {w.name} (full batch; the first "
                      f"{steps} steps of the GPU's timed window), float64 numpy oracle, one thread, "
                      f"{el:.1f} s; index and steps 0-{start - 1} (untimed, no attention) took "
                      f"{t_setup:.1f} s"}


def prefill(args):
    """The prefill-side operations, timed on their own (--prefill): Index over
    the link (summaries read zero-copy from the pinned host KV), Offload (the
    device KV copied to its reserved host runs, then Index from the device
    copy) and decode-time append of one token to every request.  The first
    min(B, --prefill-requests) requests of the workload; each call is timed
    on the host around the call (Index and Offload synchronise), the appends
    with events around a run of them back to back.  Prints one JSON line."""
    import torch

    from sparse_attention_tiered_amd import binding as bd
    from sparse_attention_tiered_amd import workload as W

    w0 = W.get(args.config)
    n_req = max(1, min(w0.B, args.prefill_requests))
    w = W.variant(w0, B=n_req)
    n_app = args.appends
    extra = -(-n_app // W.PAGE_TOKENS) + 1          # host pages reserved per head for the appends
    t0 = time.time()
    geo = W.geometry(w)
    draws = W.draw_queries(w, geo, 1)
    src = [bd.pinned_u16(w.Hkv * geo.pages[b] * W.PAGE_ELEMS) for b in range(w.B)]
    W.fill_all(w, geo, draws, [h[1] for h in src])
    d_kv = [s[0].to("cuda") for s in src]
    dst = [torch.zeros(w.Hkv * (geo.pages[b] + extra) * W.PAGE_ELEMS, dtype=torch.int16, pin_memory=True)
           for b in range(w.B)]
    torch.cuda.synchronize()
    log(f"[prefill] {w.name}: {n_req} requests, inputs in {time.time() - t0:.1f}s")
    cfg = bd.make_config(w.B, w.Hq, w.Hkv, geo.max_parts + extra, geo.max_pages + extra, w.k,
                         w.slots_per_request, max_pages_per_partition=geo.max_ppp)
    spin = bd.Spin(cfg)
    S = torch.cuda.Stream()
    lens = [geo.lens[b] if w.var_len is not None else None for b in range(w.B)]
    tokens = [int(sum(geo.lens[b])) for b in range(w.B)]
    kv_bytes = [w.Hkv * geo.pages[b] * PAGE_BYTES for b in range(w.B)]
    key_bytes = [w.Hkv * tokens[b] * W.HEAD_DIM * 2 for b in range(w.B)]   # the valid tokens' keys

    def timed(fn):
        torch.cuda.synchronize()
        t = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3

    # untimed first calls (a kernel's first launch in a process costs ~0.6 ms)
    spin.index(0, src[0][0], w.ctx[0], lens[0], stream=S)
    spin.offload(0, d_kv[0], dst[0], w.ctx[0], lens[0], stream=S)
    idx_ms = [timed(lambda b=b: spin.index(b, src[b][0], w.ctx[b], lens[b], stream=S)) for b in range(w.B)]
    off_ms = [timed(lambda b=b: spin.offload(b, d_kv[b], dst[b], w.ctx[b], lens[b], stream=S))
              for b in range(w.B)]
    # the host copy must be the device KV, head by head in its reserved run
    for b in range(w.B):
        cap = geo.pages[b] + extra
        got = dst[b].view(w.Hkv, cap * W.PAGE_ELEMS)[:, : geo.pages[b] * W.PAGE_ELEMS]
        if not torch.equal(got, src[b][0].view(w.Hkv, geo.pages[b] * W.PAGE_ELEMS)):
            raise RuntimeError(f"offloaded host copy of request {b} differs from the device KV")
    # a plain device -> pinned host copy of the same bytes (one DMA transfer)
    flat = [dst[b][: w.Hkv * geo.pages[b] * W.PAGE_ELEMS] for b in range(w.B)]
    flat[0].copy_(d_kv[0], non_blocking=True)
    d2h_ms = [timed(lambda b=b: flat[b].copy_(d_kv[b], non_blocking=True)) for b in range(w.B)]
    # the appends: one token per request per call, on top of the offloaded KV
    g = torch.Generator().manual_seed(w.seed)
    dk = torch.randint(-16000, 16000, (n_app + 1, w.B, w.Hkv, W.HEAD_DIM), dtype=torch.int16, generator=g)
    dv = torch.randint(-16000, 16000, (n_app + 1, w.B, w.Hkv, W.HEAD_DIM), dtype=torch.int16, generator=g)
    dk, dv = (dk & 0x3FFF).to("cuda"), (dv & 0x3FFF).to("cuda")   # finite bf16 bit patterns
    with torch.cuda.stream(S):
        spin.append(dk[0], dv[0], stream=S)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(S)
        for i in range(1, n_app + 1):
            spin.append(dk[i], dv[i], stream=S)
        e1.record(S)
    torch.cuda.synchronize()
    app_ms = e0.elapsed_time(e1) / n_app
    spin.close()
    link = pcie_link()
    off_gbs = sum(kv_bytes) / (sum(off_ms) * 1e-3) / 1e9
    line = {
        "metric": "prefill offload GB/s (device KV to its host runs + Index from HBM)",
        "value": off_gbs, "unit": "GB/s", "n_gpus": 1, "steps": w.B, "warmup": 1,
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "requests": w.B, "kv_heads": w.Hkv, "context": w.ctx[0],
                   "partitions": "variable 16-256" if w.var_len else "fixed 64",
                   "parallelism": "single-gpu"},
        "offload": {"ms_per_request": float(np.mean(off_ms)), "bytes_per_request": float(np.mean(kv_bytes)),
                    "GBps": off_gbs, "frac_of_link": off_gbs / PCIE_GEN5_X16_GBS,
                    "plain_d2h_copy_ms_per_request": float(np.mean(d2h_ms)),
                    "plain_d2h_copy_GBps": sum(kv_bytes) / (sum(d2h_ms) * 1e-3) / 1e9,
                    "host_copy_checked": True},
        "index_over_link": {"ms_per_request": float(np.mean(idx_ms)),
                            "key_bytes_per_request": float(np.mean(key_bytes)),
                            "GBps": sum(key_bytes) / (sum(idx_ms) * 1e-3) / 1e9,
                            "frac_of_link": sum(key_bytes) / (sum(idx_ms) * 1e-3) / 1e9 / PCIE_GEN5_X16_GBS},
        "append": {"us_per_call": app_ms * 1e3, "calls": n_app, "tokens_per_call": w.B,
                   "timed_as": "back-to-back calls on one stream, events at the ends"},
        "pcie": {"link": link, "peak_GBps": PCIE_GEN5_X16_GBS},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: every configured step after the warm-up)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the window, at least (default: min(8, steps / 4))")
    ap.add_argument("--config", default="c4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--pps", type=int, default=0, help="attention pages per split (0 = auto)")
    ap.add_argument("--single-stream", action="store_true", help="retrieve on the compute stream")
    ap.add_argument("--no-overlap", action="store_true",
                    help="attention waits for the whole retrieve (no resident-page pass)")
    ap.add_argument("--budget-ratio", type=float, default=None,
                    help="buffer elasticity ablation: each request's budget = mandatory pages "
                         "x (1 + ratio), capped by its slots (0 = no buffer pages)")
    ap.add_argument("--eager", action="store_true",
                    help="time the steps as eager whole-step calls (spin_step) instead of replays "
                         "of one captured HIP graph (spin_step_at)")
    ap.add_argument("--host-segments", action="store_true",
                    help="keep the second-level segment tables in pinned host memory")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a plain elementwise copy of 256 MiB three times "
                         "(reference kernel for the HBM byte counters)")
    ap.add_argument("--prefill", action="store_true",
                    help="time Index, Offload and append on their own instead of decode steps")
    ap.add_argument("--prefill-requests", type=int, default=4,
                    help="with --prefill: how many of the workload's requests")
    ap.add_argument("--appends", type=int, default=256, help="with --prefill: appends timed")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the decode path shards by "
              "request with no exchange, so N GPUs run N independent copies of this benchmark.",
              file=sys.stderr)
        sys.exit(2)

    if args.prefill:
        prefill(args)
        return

    import torch

    from sparse_attention_tiered_amd import binding as bd
    from sparse_attention_tiered_amd import workload as W

    w = W.get(args.config)
    T = w.steps
    warm = args.warmup if args.warmup is not None else min(8, T // 4)
    if warm < 1:
        ap.error("--warmup must be at least 1 (step 0 is timed on its own)")
    if args.steps is not None and args.steps < 1:
        ap.error("--steps must be at least 1")
    start, end, n_steps = timed_window(T, warm, args.steps)   # the window: steps start .. end-1
    K = end - start
    use_graph = not args.eager and not args.no_overlap
    overlap = not args.single_stream and not args.no_overlap

    t0 = time.time()
    geo = W.geometry(w)
    draws = W.draw_queries(w, geo, n_steps)
    host = [bd.pinned_u16(w.Hkv * max(geo.pages[b], 1) * W.PAGE_ELEMS) for b in range(w.B)]
    W.fill_all(w, geo, draws, [h[1] for h in host])
    log(f"[bench] {w.name}: inputs generated in {time.time() - t0:.1f}s "
        f"({sum(h[0].numel() * 2 for h in host) / 1e9:.2f} GB pinned host KV); "
        f"timed window: steps {start}-{end - 1}")
    cfg = bd.make_config(w.B, w.Hq, w.Hkv, geo.max_parts, geo.max_pages, w.k, w.slots_per_request,
                         max_pages_per_partition=geo.max_ppp, attend_pages_per_split=args.pps,
                         host_segments=args.host_segments)
    budget = w.slots_per_request
    if args.budget_ratio is not None:
        mand = w.Hkv * w.k * geo.max_ppp
        budget = min(w.slots_per_request, int(round(mand * (1 + args.budget_ratio))))
    ctx = []
    for name in ("A", "B", "C"):
        spin = bd.Spin(cfg)
        t0 = time.time()
        for b in range(w.B):
            spin.index(b, host[b][0], w.ctx[b], geo.lens[b] if w.var_len is not None else None)
            if budget != w.slots_per_request:
                spin.set_budget(b, budget)
        log(f"[bench] context {name}: index (summaries over PCIe) {time.time() - t0:.2f}s; "
            f"attend splits={spin.splits}")
        ctx.append(spin)
    A, Bx, Cx = ctx
    q = torch.from_numpy(draws.q_bits.view(np.int16)).to("cuda")
    S = torch.cuda.Stream()  # a created stream: HIP graphs cannot capture the null stream
    Cs = S if args.single_stream else torch.cuda.Stream()
    torch.cuda.synchronize()

    def staged(spin, t, ev=None, ovl=overlap):
        # the stages of spin_step, one call each
        # events: 0 start, 1 select done, 2 resolve done; 3 / 4 around the
        # transfer (with the resident-page attention in the same launch when
        # overlapped); 6 attention done
        if ev is not None:
            ev[0].record(S)
        spin.select(q[t], stream=S)
        if ev is not None:
            ev[1].record(S)
        spin.resolve_evict(t, stream=S)
        if ev is not None:
            ev[2].record(S)
        if ovl:
            # as the whole-step call: one launch pulls the missed pages
            # (attending each on arrival) while it attends the resident ones
            if ev is not None:
                ev[3].record(S)
            spin.transfer_attend(q[t], stream=S)
            if ev is not None:
                ev[4].record(S)
            spin.attend_finish(q[t], stream=S)
        else:
            if ev is not None:
                if Cs is not S:
                    Cs.wait_stream(S)
                ev[3].record(Cs)
            spin.retrieve(copy_stream=Cs)
            if ev is not None:
                ev[4].record(Cs)
            spin.attend(q[t], stream=S)
        if ev is not None:
            ev[6].record(S)

    def warm_up(spin, t_from):
        # untimed steps in the serial form (transfer, then attention)
        for t in range(t_from, start):
            spin.step(q[t], t, stream=S, copy_stream=S)

    # ---- context A: step 0 (every mandatory page a miss, serial form, stage
    # events), the rest of the warm-up, then the timed window
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
    staged(A, 0, ev0, ovl=False)
    torch.cuda.synchronize()
    st_s0, _ = A.stats()
    s0_ret_ms = ev0[3].elapsed_time(ev0[4])
    step0 = {"ms": ev0[0].elapsed_time(ev0[6]), "misses": st_s0.misses, "kernel": "k_retrieve",
             "retrieve_ms": s0_ret_ms, "bytes": st_s0.h2d_bytes,
             "retrieve_GBps": st_s0.h2d_bytes / (s0_ret_ms * 1e-3) / 1e9}
    warm_up(A, 1)
    torch.cuda.synchronize()
    stA0, _ = A.stats()

    def capture(spin):
        # one step captured with the device-side step index, replayed K times
        t_dev = torch.full((1,), start, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=S):
            spin.step_at(q, t_dev, stream=S, copy_stream=Cs)
        torch.cuda.synchronize()
        return g

    def window(spin, g, evt=None):
        # steps start .. end-1; an event after each step when evt is given.
        # The replays run inside one stream context, as a serving loop keeps
        # its stream: entering it per step cost the host a few microseconds
        # of Python a step, which the tiny workload's host-bound replay loop
        # felt.
        if g is not None:
            with torch.cuda.stream(S):
                for i in range(K):
                    g.replay()
                    if evt is not None:
                        evt[i + 1].record(S)
            return
        for i in range(K):
            t = start + i
            if overlap or args.single_stream:
                spin.step(q[t], t, stream=S, copy_stream=Cs)  # the library's whole-step call
            else:
                staged(spin, t)
            if evt is not None:
                evt[i + 1].record(S)

    graph = capture(A) if use_graph else None
    w0 = time.perf_counter()
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ends[0].record(S)
    window(A, graph)
    ends[1].record(S)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    stA1, _ = A.stats()
    mean_ms = ends[0].elapsed_time(ends[1]) / K

    # ---- context C: the same steps again, with a timing event between steps
    # (their median is the figure the measurement plan asks for; each event
    # adds a few microseconds of idle to the step it closes, which the
    # difference of the two means shows)
    staged(Cx, 0, None, ovl=False)
    warm_up(Cx, 1)
    torch.cuda.synchronize()
    stC0, _ = Cx.stats()
    graph_c = capture(Cx) if use_graph else None
    evt = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    evt[0].record(S)
    window(Cx, graph_c, evt)
    torch.cuda.synchronize()
    stC1, _ = Cx.stats()
    step_times = [evt[i].elapsed_time(evt[i + 1]) for i in range(K)]
    ms_per_step = float(np.median(step_times))
    mean_ms_evented = evt[0].elapsed_time(evt[K]) / K
    value = w.B * w.Hq / (ms_per_step * 1e-3)
    del graph, graph_c

    # ---- context B: the same warm-up, then the same window with stage events
    staged(Bx, 0, None, ovl=False)
    warm_up(Bx, 1)
    torch.cuda.synchronize()
    stB0, _ = Bx.stats()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(K)]
    step_miss, step_hit, step_bytes = [], [], []
    prev_m, prev_h, prev_b = stB0.misses, stB0.hits, stB0.h2d_bytes
    for i in range(K):
        staged(Bx, start + i, evs[i])
        st_i, _ = Bx.stats()
        step_miss.append(st_i.misses - prev_m)
        step_hit.append(st_i.hits - prev_h)
        step_bytes.append(st_i.h2d_bytes - prev_b)  # read over the link: valid chunks only
        prev_m, prev_h, prev_b = st_i.misses, st_i.hits, st_i.h2d_bytes
    stB1 = st_i

    def window_counts(s0, s1):
        return (s0.misses, s1.hits - s0.hits, s1.misses - s0.misses, s1.evictions - s0.evictions)

    same_steps = (window_counts(stA0, stA1) == window_counts(stB0, stB1) == window_counts(stC0, stC1))
    if not same_steps:
        log("[bench] WARNING: the contexts' counters differ over the window")
    stage = {"select": [], "resolve_evict": [], "retrieve": [], "attend": []}
    instr_step = []
    for e in evs:
        instr_step.append(e[0].elapsed_time(e[6]))
        stage["select"].append(e[0].elapsed_time(e[1]))
        stage["resolve_evict"].append(e[1].elapsed_time(e[2]))
        stage["retrieve"].append(e[3].elapsed_time(e[4]))
        # after the transfer: the merge (or the whole attention without overlap)
        stage["attend"].append(max(e[4].elapsed_time(e[6]), 0.0))
    stage_ms = {k: float(np.mean(v)) for k, v in stage.items()}
    ret_ms = stage["retrieve"]

    # ---- kernel-isolated replays on the window's last step (select and
    # attention only read the residency state), so the HBM rooflines are not
    # mixed with the transfer that overlaps them inside a step
    spin = Bx
    last = end - 1
    reps = 10
    iso = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    torch.cuda.synchronize()
    iso[0].record(S)
    for _ in range(reps):
        spin.select(q[last], stream=S)
    iso[1].record(S)
    iso[2].record(S)
    for _ in range(reps):
        spin.attend(q[last], stream=S)
    iso[3].record(S)
    torch.cuda.synchronize()
    iso_select_ms = iso[0].elapsed_time(iso[1]) / reps
    iso_attend_ms = iso[2].elapsed_time(iso[3]) / reps
    # the last step's transfer again, alone on the compute stream: the same
    # pages to the same slots (idempotent), no attention beside it, so the
    # rate is the transfer's own for this many pages
    iso_r = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    spin.retrieve(copy_stream=S)
    torch.cuda.synchronize()
    h2d0 = spin.stats()[0].h2d_bytes
    iso_r[0].record(S)
    for _ in range(reps):
        spin.retrieve(copy_stream=S)
    iso_r[1].record(S)
    torch.cuda.synchronize()
    iso_retrieve_ms = iso_r[0].elapsed_time(iso_r[1]) / reps
    iso_retrieve_bytes = (spin.stats()[0].h2d_bytes - h2d0) / reps
    # cold replays: a 512 MB read before each one fills the 256 MB memory-side
    # cache with clean lines of another buffer, so the kernel reads HBM (a write
    # would leave dirty lines whose write-back the kernel would pay for); an
    # event pair brackets the kernel alone (the pair's own cost, timed with
    # nothing between, is reported beside it)
    scratch = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()  # (filled on the default stream)
    bd.read_stream(scratch, sink, S)  # written back once; later reads leave it clean

    def cold(fn):
        # reps of (cache-filling read, fn) back to back, less reps of the read
        # alone, with events only at the ends of each run: an event pair
        # around the launch itself would add its own cost (about 5 us here,
        # timed with nothing between) to a launch of 10-30 us
        creps = 20
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(S)
        for _ in range(creps):
            bd.read_stream(scratch, sink, S)
            fn()
        ev[1].record(S)
        ev[2].record(S)
        for _ in range(creps):
            bd.read_stream(scratch, sink, S)
        ev[3].record(S)
        torch.cuda.synchronize()
        return (ev[0].elapsed_time(ev[1]) - ev[2].elapsed_time(ev[3])) / creps

    cold_select_ms = cold(lambda: spin.select(q[last], stream=S))
    cold_attend_ms = cold(lambda: spin.attend(q[last], stream=S))

    def stream_floor(nbytes):
        """A plain read of as many bytes as a kernel's launch, timed as that
        kernel is: back to back (warm) and after the cache-filling read
        (cold)."""
        buf = torch.ones((nbytes + 15) // 16 * 4, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        bd.read_stream(buf, sink, S)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(S)
        for _ in range(reps):
            bd.read_stream(buf, sink, S)
        ev[1].record(S)
        torch.cuda.synchronize()
        warm_ms = ev[0].elapsed_time(ev[1]) / reps
        cold_ms = cold(lambda: bd.read_stream(buf, sink, S))
        return {"bytes": buf.numel() * 4, "launch_ms": warm_ms, "cold_launch_ms": cold_ms,
                "kernel": "k_read_stream"}

    n_parts = sum(len(l) for l in geo.lens)
    score_bytes = w.Hkv * n_parts * 128 * 4 + w.B * w.Hq * 128 * 2 + w.Hkv * n_parts * 4
    last_pages = int(spin.block_count.sum().item())
    iso_attend_bytes = last_pages * PAGE_BYTES + w.B * w.Hq * 128 * (2 + 4)
    floor_select = stream_floor(score_bytes)
    floor_attend = stream_floor(iso_attend_bytes)
    del scratch, sink
    # valid tokens of every (request, KV head) block table of the last step
    attended_tokens = int(spin.block_ntok.sum().item())

    hits = stA1.hits - stA0.hits
    misses = stA1.misses - stA0.misses
    evictions = stA1.evictions - stA0.evictions
    # algorithmic bytes per launch (one step)
    attend_bytes = (hits + misses) * PAGE_BYTES / K + w.B * w.Hq * 128 * (2 + 4)
    # the transfer's bytes per launch over the window (the same steps in both
    # contexts): what it read over the link (each missed page's chunks that
    # hold valid tokens, 32 KiB for a full page), and its duration per launch
    # measured in context B
    retrieve_bytes = sum(step_bytes) / K
    last_step_bytes = iso_retrieve_bytes
    # everything the transfer launch itself reads and writes: each missed page
    # read over the link and written whole to its slot; with the overlap,
    # also the resident pages it attends (read once) and the queries
    launch_bytes = retrieve_bytes + sum(step_miss) * PAGE_BYTES / K
    if overlap:
        launch_bytes += sum(step_hit) / K * PAGE_BYTES + w.B * w.Hq * 128 * 2
    link = pcie_link()
    memcpy_gbs = memcpy_h2d_gbs()
    transfer_ms = float(np.mean(ret_ms))
    rl = {
        "attend": {"bound": "hbm",
                   "achieved": iso_attend_bytes / (iso_attend_ms * 1e-3) / 1e9,
                   "launch_ms": iso_attend_ms,
                   "peak": HBM_PEAK_GBS, "unit": "GB/s", "bytes_per_launch": iso_attend_bytes,
                   "in_step_bytes_per_step": attend_bytes,
                   "kernels": ["k_attend", "k_attend_merge"]},
        "select": {"bound": "hbm", "achieved": score_bytes / (iso_select_ms * 1e-3) / 1e9,
                   "launch_ms": iso_select_ms,
                   "peak": HBM_PEAK_GBS, "unit": "GB/s", "bytes_per_launch": score_bytes,
                   "kernels": select_kernels(w.B, w.Hkv, geo.max_parts)},
        "retrieve": {"bound": "pcie",
                     "achieved": retrieve_bytes / (transfer_ms * 1e-3) / 1e9 if retrieve_bytes else 0.0,
                     "launch_ms": transfer_ms,
                     "launch_ms_median": float(np.median(ret_ms)),
                     "steps": [start, end - 1],
                     "peak": PCIE_GEN5_X16_GBS, "unit": "GB/s", "bytes_per_launch": retrieve_bytes,
                     "launch_work_bytes": launch_bytes,
                     "kernels": ["k_transfer_attend" if overlap else "k_retrieve"]},
    }
    # the transfer over the steps that move at least 8 MB (small transfers are
    # dominated by a fixed latency), and step 0 on its own
    big = [i for i in range(K) if step_bytes[i] >= 8e6]
    rl["retrieve"]["steps_ge_8MB"] = len(big)
    rl["retrieve"]["achieved_ge_8MB"] = (
        sum(step_bytes[i] for i in big) / (sum(ret_ms[i] for i in big) * 1e-3) / 1e9
        if big else None)
    rl["retrieve"]["step0"] = step0
    rl["retrieve"]["isolated_last_step"] = {
        "kernel": "k_retrieve", "bytes": last_step_bytes, "launch_ms": iso_retrieve_ms,
        "achieved": last_step_bytes / (iso_retrieve_ms * 1e-3) / 1e9 if last_step_bytes else 0.0,
        "frac": last_step_bytes / (iso_retrieve_ms * 1e-3) / 1e9 / PCIE_GEN5_X16_GBS if last_step_bytes else 0.0}
    rl["attend"]["cold"] = {"launch_ms": cold_attend_ms,
                            "achieved": iso_attend_bytes / (cold_attend_ms * 1e-3) / 1e9}
    rl["select"]["cold"] = {"launch_ms": cold_select_ms,
                            "achieved": score_bytes / (cold_select_ms * 1e-3) / 1e9}
    for k, fl in (("attend", floor_attend), ("select", floor_select)):
        rl[k]["cold"]["frac"] = rl[k]["cold"]["achieved"] / HBM_PEAK_GBS
        rl[k]["cold"]["timed_as"] = ("reps of (512 MB read, launch) less reps of the read alone, "
                                     "events only at the ends")
        # the same bytes as a plain read: the most a kernel that must read
        # them could reach here, warm and cold, and the kernel's share of it
        fl["frac_of_peak"] = fl["bytes"] / (fl["launch_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS
        fl["cold_frac_of_peak"] = fl["bytes"] / (fl["cold_launch_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS
        fl["kernel_vs_read"] = fl["launch_ms"] / rl[k]["launch_ms"]
        fl["cold_kernel_vs_read"] = fl["cold_launch_ms"] / rl[k]["cold"]["launch_ms"]
        rl[k]["stream_floor"] = fl
    for v in rl.values():
        v["frac"] = v["achieved"] / v["peak"]
    # dominant stage of the step: the transfer, or the HBM kernels run alone
    dominant = max(("attend", "select", "retrieve"), key=lambda k: rl[k]["launch_ms"])
    roof = dict(rl[dominant])
    roof["stage"] = dominant
    # counter traffic per launch: the transfer's counters cover the whole
    # launch, so they scale with all of its work (launch_work_bytes)
    for k, v in rl.items():
        v["traffic"] = counter_traffic(args.config, k, v.get("launch_work_bytes", v["bytes_per_launch"]))
    roof["traffic"] = rl[dominant]["traffic"]
    line = {
        "metric": "sparse decode head-tokens/s + achieved HBM GB/s vs peak; H2D GB/s vs PCIe",
        "value": value, "unit": "head-tokens/s", "n_gpus": 1, "steps": K, "warmup": start,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "context": w.ctx[0], "topk": w.k, "slots_per_request": w.slots_per_request,
                   "budget_per_request": budget,
                   "partitions": "variable 16-256" if w.var_len else "fixed 64",
                   "segment_tables": "host" if args.host_segments else "gpu",
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "timed_steps": [start, end - 1],
        "configured_steps": T,
        "ms_per_step_is": "median of the window's steps (an event between steps)",
        "mean_ms_per_step": mean_ms,
        "mean_ms_per_step_is": "the window's steps back to back, events only at its ends",
        "mean_ms_per_step_with_step_events": mean_ms_evented,
        "step_ms_p10_p90": [float(np.percentile(step_times, 10)), float(np.percentile(step_times, 90))],
        "value_at_mean": w.B * w.Hq / (mean_ms * 1e-3),
        "stages_ms": stage_ms,
        "instrumented_steps": [start, end - 1],
        "median_step_ms_instrumented": float(np.median(instr_step)),
        "contexts_agree_over_window": bool(same_steps),
        "attended_head_tokens_per_s": attended_tokens / (iso_attend_ms * 1e-3),
        "overlap_retrieve_attend": overlap,
        "timed_as_graph_replays": use_graph,
        "rooflines": rl,
        "residency": {"hits_per_step": hits / K, "misses_per_step": misses / K,
                      "evictions_per_step": evictions / K},
        "pcie": {"link": link, "memcpy_h2d_GBps": memcpy_gbs},
        "hbm_practical_read_GBps": bd.read_stream_gbs(),
        "wall_s": wall,
    }
    # metadata footprint (two-level table vs a flat one), measured now and
    # projected to a server provisioned for the worst case: 256 requests of
    # 1M tokens on every layer of the model, with this run's live working set
    md = A.metadata()
    prov_batch, prov_ctx = 256, 1 << 20
    prov_pages = prov_ctx // 64
    seg_b = 64 * 4 + 8
    flat_prov = prov_batch * w.layers * w.Hkv * prov_pages * 4
    dir_prov = prov_batch * w.layers * w.Hkv * ((prov_pages + 63) // 64) * 4
    two_level_prov = dir_prov + md["live_segments"] * w.layers * seg_b + w.B * w.layers * w.slots_per_request * 8
    # with the segment tables in host memory the GPU keeps the directory, the
    # segments' live counts and stack, and the reverse maps
    two_level_gpu_hs = dir_prov + md["live_segments"] * w.layers * 8 + w.B * w.layers * w.slots_per_request * 8
    line["metadata"] = {
        "measured": md,
        "segments_in_host_memory": bool(args.host_segments),
        "projection": {"provisioned_batch": prov_batch, "provisioned_context": prov_ctx,
                       "layers": w.layers, "active_batch": w.B,
                       "flat_table_bytes": flat_prov, "two_level_bytes": two_level_prov,
                       "ratio": flat_prov / two_level_prov,
                       "two_level_gpu_bytes_segments_in_host": two_level_gpu_hs,
                       "ratio_segments_in_host": flat_prov / two_level_gpu_hs},
    }
    if args.copy_calibration:
        n = 64 << 20  # 64 Mi float32 = 256 MiB read + 256 MiB written per launch
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        line["copy_calibration"] = {"kernel": "elementwise neg (torch)", "bytes_read": 4 * n,
                                    "bytes_written": 4 * n, "launches": 3}
    A.close()
    Bx.close()
    Cx.close()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(w, geo, draws, [h[1] for h in host], start, end,
                                            args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
