"""ctypes binding of libspin.so (C ABI in include/spin.h).

Argument marshalling only: every step of the decode path runs in the HIP
library.  PyTorch provides device memory (workspace, page pool, inputs,
outputs), pinned host memory and streams.  Loading fails loudly when the
library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_int, c_int32, c_int64, c_size_t, c_void_p

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspin.so")

SPIN_OK, SPIN_EINVAL, SPIN_ECAPACITY, SPIN_ESEGPOOL, SPIN_EHIP, SPIN_EDEVICE, SPIN_ESTATE = \
    0, -1, -2, -3, -4, -5, -6
SPIN_ESCRATCH = -7
NOALLOC_SCRATCH_BYTES = 32 << 20
DEVERR_PARTITION, DEVERR_SEGPOOL, DEVERR_STATE, DEVERR_STEP = 1, 2, 4, 8
PAGE_BYTES = 32768


class SpinConfig(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in (
        "max_batch", "num_q_heads", "num_kv_heads", "head_dim", "page_tokens", "max_partitions",
        "max_pages", "max_pages_per_partition", "topk", "slots_per_request", "num_segments",
        "seg_entries", "num_buckets", "attend_pages_per_split", "segments_in_host_memory")]


class SpinStats(ctypes.Structure):
    _fields_ = [("hits", ctypes.c_uint64), ("misses", ctypes.c_uint64),
                ("evictions", ctypes.c_uint64), ("h2d_bytes", ctypes.c_uint64),
                ("live_segments", c_int32), ("error_word", c_int32)]


class SpinMetadata(ctypes.Structure):
    _fields_ = [("directory_bytes", ctypes.c_uint64), ("segment_pool_bytes", ctypes.c_uint64),
                ("live_segment_bytes", ctypes.c_uint64), ("reverse_map_bytes", ctypes.c_uint64),
                ("flat_table_bytes", ctypes.c_uint64), ("live_segments", c_int32),
                ("num_segments", c_int32), ("host_segment_bytes", ctypes.c_uint64)]


_P = c_void_p
_I32P = POINTER(c_int32)
# name -> (restype, argtypes)
SIGNATURES = {
    "spin_config_init": (c_int, [POINTER(SpinConfig)]),
    "spin_config_check": (c_int, [POINTER(SpinConfig)]),
    "spin_workspace_size": (c_int, [POINTER(SpinConfig), POINTER(c_size_t), POINTER(c_size_t)]),
    "spin_derived": (c_int, [POINTER(SpinConfig), _I32P, _I32P, _I32P]),
    "spin_host_segment_bytes": (c_int, [POINTER(SpinConfig), POINTER(c_size_t)]),
    "spin_create": (c_int, [POINTER(SpinConfig), _P, c_size_t, _P, c_size_t, _P, POINTER(_P)]),
    "spin_create_ex": (c_int, [POINTER(SpinConfig), _P, c_size_t, _P, c_size_t, _P, c_size_t, _P,
                               POINTER(_P)]),
    "spin_destroy": (c_int, [_P]),
    "spin_index": (c_int, [_P, c_int32, _P, c_int64, _I32P, c_int32, _P]),
    "spin_release": (c_int, [_P, c_int32, _P]),
    "spin_offload": (c_int, [_P, c_int32, _P, _P, c_size_t, c_int64, _I32P, c_int32, _P]),
    "spin_append": (c_int, [_P, _P, _P, _P]),
    "spin_set_budget": (c_int, [_P, c_int32, c_int32, _P]),
    "spin_select": (c_int, [_P, _P, _P, _P, _P]),
    "spin_resolve_evict": (c_int, [_P, _P, c_int32, _P, _P, _P, _P]),
    "spin_retrieve": (c_int, [_P, _P]),
    "spin_retrieve_attend": (c_int, [_P, _P, _P]),
    "spin_transfer_attend": (c_int, [_P, _P, _P, _P, _P, _P]),
    "spin_attend": (c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "spin_attend_noalloc": (c_int, [_P, _P, c_int64, _P, _P, _P, _P, c_int32, c_int32, c_int32,
                                    c_int32, c_int32, _P]),
    "spin_attend_begin": (c_int, [_P, _P, _P, _P, _P, _P]),
    "spin_attend_finish": (c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "spin_step": (c_int, [_P, _P, c_int32, _P, _P, _P, _P, _P, _P, _P]),
    "spin_step_at": (c_int, [_P, _P, c_int64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "spin_get_stats": (c_int, [_P, POINTER(SpinStats), POINTER(c_int64)]),
    "spin_snapshot": (c_int, [_P, _I32P, _I32P, _I32P, _I32P, _I32P, _I32P, _I32P, _I32P]),
    "spin_read_summaries": (c_int, [_P, c_int32, POINTER(ctypes.c_float)]),
    "spin_metadata_footprint": (c_int, [_P, POINTER(SpinMetadata)]),
    "spin_sync_status": (c_int, [_P]),
    "spin_read_stream": (c_int, [_P, c_size_t, _P, _P]),
    "spin_strerror": (c_char_p, [c_int]),
    "spin_last_hip_error": (c_int, [_P]),
}

_lib = None


def load():
    """Load libspin.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_attention_tiered_amd.build_lib`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class SpinError(RuntimeError):
    def __init__(self, fn, code, hip=0):
        msg = load().spin_strerror(code).decode()
        super().__init__(f"{fn} failed: {code} ({msg}){f', hip error {hip}' if hip else ''}")
        self.code = code


def make_config(B, Hq, Hkv, max_partitions, max_pages, topk, slots_per_request,
                num_segments=None, max_pages_per_partition=1, attend_pages_per_split=0,
                host_segments=False):
    lib = load()
    c = SpinConfig()
    lib.spin_config_init(ctypes.byref(c))
    c.max_batch, c.num_q_heads, c.num_kv_heads = B, Hq, Hkv
    c.max_partitions, c.max_pages, c.max_pages_per_partition = max_partitions, max_pages, max_pages_per_partition
    c.topk, c.slots_per_request = topk, slots_per_request
    ndir = (max_pages + 63) // 64
    c.num_segments = num_segments if num_segments is not None else min(B * slots_per_request, B * Hkv * ndir)
    c.attend_pages_per_split = attend_pages_per_split
    c.segments_in_host_memory = 1 if host_segments else 0
    return c


def _ptr(x):
    if x is None:
        return None
    return c_void_p(x.data_ptr())


def _stream(s):
    import torch
    if s is None:
        s = torch.cuda.current_stream()
    return c_void_p(s.cuda_stream)


class Spin:
    """One context: caller-side (torch) device memory plus the library handle."""

    def __init__(self, cfg: SpinConfig, device="cuda:0", stream=None):
        import torch
        self.lib = load()
        self.cfg = cfg
        self.device = torch.device(device)
        ws, pool = c_size_t(), c_size_t()
        self._chk("spin_workspace_size", self.lib.spin_workspace_size(ctypes.byref(cfg), ctypes.byref(ws), ctypes.byref(pool)))
        nd, mb, sp = c_int32(), c_int32(), c_int32()
        self._chk("spin_derived", self.lib.spin_derived(ctypes.byref(cfg), ctypes.byref(nd), ctypes.byref(mb), ctypes.byref(sp)))
        self.ndir, self.max_blocks, self.splits = nd.value, mb.value, sp.value
        self.ws_bytes, self.pool_bytes = ws.value, pool.value
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.pool = torch.empty(self.pool_bytes, dtype=torch.uint8, device=self.device)
        B, Hq, Hkv, k = cfg.max_batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.topk
        i32 = dict(dtype=torch.int32, device=self.device)
        self.sel = torch.full((B, Hkv, k), -1, **i32)
        self.block_table = torch.full((B, Hkv, self.max_blocks), -1, **i32)
        self.block_ntok = torch.zeros((B, Hkv, self.max_blocks), **i32)
        self.block_count = torch.zeros((B, Hkv), **i32)
        self.out = torch.zeros((B, Hq, 128), dtype=torch.float32, device=self.device)
        h = c_void_p()
        hs = c_size_t()
        self._chk("spin_host_segment_bytes",
                  self.lib.spin_host_segment_bytes(ctypes.byref(cfg), ctypes.byref(hs)))
        self.host_segments = None
        if hs.value:
            # second-level segment tables in pinned host memory
            self.host_segments = torch.empty(hs.value // 4, dtype=torch.int32, pin_memory=True)
            self._chk("spin_create_ex", self.lib.spin_create_ex(
                ctypes.byref(cfg), c_void_p(self.ws.data_ptr()), self.ws_bytes,
                c_void_p(self.pool.data_ptr()), self.pool_bytes,
                c_void_p(self.host_segments.data_ptr()), hs.value, _stream(stream), ctypes.byref(h)))
        else:
            self._chk("spin_create", self.lib.spin_create(
                ctypes.byref(cfg), c_void_p(self.ws.data_ptr()), self.ws_bytes,
                c_void_p(self.pool.data_ptr()), self.pool_bytes, _stream(stream), ctypes.byref(h)))
        self.ctx = h
        self._host = {}

    def _chk(self, fn, rc):
        if rc != SPIN_OK:
            hip = self.lib.spin_last_hip_error(self.ctx) if getattr(self, "ctx", None) else 0
            raise SpinError(fn, rc, hip)

    # ---------------------------------------------------------------- setup
    def index(self, req, host_kv, n_tokens, part_lens=None, stream=None):
        """host_kv: pinned CPU torch tensor holding the request's pages."""
        if host_kv is not None and not host_kv.is_pinned():
            raise ValueError("host_kv must be pinned host memory")
        lens_p, n_parts = None, 0
        if part_lens is not None:
            arr = np.ascontiguousarray(part_lens, dtype=np.int32)
            lens_p = arr.ctypes.data_as(_I32P)
            n_parts = len(arr)
        self._chk("spin_index", self.lib.spin_index(
            self.ctx, req, c_void_p(host_kv.data_ptr()) if host_kv is not None else None,
            int(n_tokens), lens_p, n_parts, _stream(stream)))
        self._host[req] = host_kv  # keep the pinned buffer alive

    def set_budget(self, req, slots, stream=None):
        self._chk("spin_set_budget", self.lib.spin_set_budget(self.ctx, req, int(slots), _stream(stream)))

    def offload(self, req, d_kv, host_kv, n_tokens, part_lens=None, stream=None):
        """d_kv: device tensor with the request's pages; host_kv: pinned CPU tensor
        (its size sets the pages reserved per KV head for appends)."""
        if not host_kv.is_pinned():
            raise ValueError("host_kv must be pinned host memory")
        lens_p, n_parts = None, 0
        if part_lens is not None:
            arr = np.ascontiguousarray(part_lens, dtype=np.int32)
            lens_p = arr.ctypes.data_as(_I32P)
            n_parts = len(arr)
        self._chk("spin_offload", self.lib.spin_offload(
            self.ctx, req, _ptr(d_kv), c_void_p(host_kv.data_ptr()),
            host_kv.numel() * host_kv.element_size(), int(n_tokens), lens_p, n_parts, _stream(stream)))
        self._host[req] = host_kv

    def append(self, d_k, d_v, stream=None):
        self._chk("spin_append", self.lib.spin_append(self.ctx, _ptr(d_k), _ptr(d_v), _stream(stream)))

    def release(self, req, stream=None):
        self._chk("spin_release", self.lib.spin_release(self.ctx, req, _stream(stream)))
        self._host.pop(req, None)

    # ---------------------------------------------------------------- the step
    def select(self, q, sel=None, scores=None, stream=None):
        sel = self.sel if sel is None else sel
        self._chk("spin_select", self.lib.spin_select(self.ctx, _ptr(q), _ptr(sel), _ptr(scores), _stream(stream)))
        return sel

    def resolve_evict(self, t, sel=None, stream=None):
        sel = self.sel if sel is None else sel
        self._chk("spin_resolve_evict", self.lib.spin_resolve_evict(
            self.ctx, _ptr(sel), int(t), _ptr(self.block_table), _ptr(self.block_ntok),
            _ptr(self.block_count), _stream(stream)))

    def retrieve(self, copy_stream=None):
        self._chk("spin_retrieve", self.lib.spin_retrieve(self.ctx, _stream(copy_stream)))

    def transfer_attend(self, q, stream=None):
        self._chk("spin_transfer_attend", self.lib.spin_transfer_attend(
            self.ctx, _ptr(q), _ptr(self.block_table), _ptr(self.block_ntok), _ptr(self.block_count),
            _stream(stream)))

    def retrieve_attend(self, q, copy_stream=None):
        self._chk("spin_retrieve_attend",
                  self.lib.spin_retrieve_attend(self.ctx, _ptr(q), _stream(copy_stream)))

    def attend(self, q, out=None, stream=None, block_table=None, block_ntok=None, block_count=None):
        out = self.out if out is None else out
        bt = self.block_table if block_table is None else block_table
        bn = self.block_ntok if block_ntok is None else block_ntok
        bc = self.block_count if block_count is None else block_count
        self._chk("spin_attend", self.lib.spin_attend(
            self.ctx, _ptr(q), _ptr(bt), _ptr(bn), _ptr(bc), _ptr(out), _stream(stream)))
        return out

    def attend_begin(self, q, stream=None):
        """Attention over the resident pages of the last resolve (overlaps retrieve)."""
        self._chk("spin_attend_begin", self.lib.spin_attend_begin(
            self.ctx, _ptr(q), _ptr(self.block_table), _ptr(self.block_ntok),
            _ptr(self.block_count), _stream(stream)))

    def attend_finish(self, q, out=None, stream=None):
        """Waits for retrieve, attends the fetched pages, merges into out."""
        out = self.out if out is None else out
        self._chk("spin_attend_finish", self.lib.spin_attend_finish(
            self.ctx, _ptr(q), _ptr(self.block_table), _ptr(self.block_ntok),
            _ptr(self.block_count), _ptr(out), _stream(stream)))
        return out

    def step(self, q, t, stream=None, copy_stream=None):
        s = _stream(stream)
        cs = _stream(copy_stream) if copy_stream is not None else s
        self._chk("spin_step", self.lib.spin_step(
            self.ctx, _ptr(q), int(t), _ptr(self.sel), _ptr(self.block_table), _ptr(self.block_ntok),
            _ptr(self.block_count), _ptr(self.out), s, cs))
        return self.out

    def step_at(self, q_steps, t_dev, stream=None, copy_stream=None):
        """One step at the device-side index t_dev (int32 device tensor of one
        element, incremented on the device): q_steps[t] are its queries."""
        s = _stream(stream)
        cs = _stream(copy_stream) if copy_stream is not None else s
        step_elems = q_steps[0].numel() if q_steps.dim() > 1 else 0
        self._chk("spin_step_at", self.lib.spin_step_at(
            self.ctx, _ptr(q_steps), step_elems, _ptr(t_dev), _ptr(self.sel), _ptr(self.block_table),
            _ptr(self.block_ntok), _ptr(self.block_count), _ptr(self.out), s, cs))
        return self.out

    # ---------------------------------------------------------------- inspection
    def stats(self):
        st = SpinStats()
        per = np.zeros((self.cfg.max_batch, 4), np.int64)
        self._chk("spin_get_stats", self.lib.spin_get_stats(
            self.ctx, ctypes.byref(st), per.ctypes.data_as(POINTER(c_int64))))
        return st, per

    def snapshot(self):
        c = self.cfg
        B, Hkv, C, S = c.max_batch, c.num_kv_heads, c.slots_per_request, c.num_segments
        out = dict(directory=np.zeros((B, Hkv, self.ndir), np.int32),
                   segments=np.zeros((S, 64), np.int32), seg_live=np.zeros(S, np.int32),
                   seg_stack=np.zeros(S, np.int32), seg_top=np.zeros(1, np.int32),
                   owner=np.zeros((B, C), np.int32), last_use=np.zeros((B, C), np.int32),
                   free_count=np.zeros(B, np.int32))
        p = {k: v.ctypes.data_as(_I32P) for k, v in out.items()}
        self._chk("spin_snapshot", self.lib.spin_snapshot(
            self.ctx, p["directory"], p["segments"], p["seg_live"], p["seg_stack"], p["seg_top"],
            p["owner"], p["last_use"], p["free_count"]))
        return out

    def metadata(self):
        m = SpinMetadata()
        self._chk("spin_metadata_footprint", self.lib.spin_metadata_footprint(self.ctx, ctypes.byref(m)))
        return {f: getattr(m, f) for f, _ in SpinMetadata._fields_}

    def summaries(self, req, n_parts):
        out = np.zeros((self.cfg.num_kv_heads, n_parts, 128), np.float32)
        self._chk("spin_read_summaries", self.lib.spin_read_summaries(
            self.ctx, req, out.ctypes.data_as(POINTER(ctypes.c_float))))
        return out

    def sync_status(self):
        return self.lib.spin_sync_status(self.ctx)

    def close(self):
        if getattr(self, "ctx", None):
            self.lib.spin_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def attend_noalloc(q, pool, block_table, block_ntok, block_count, out, batch=None, Hq=None,
                   Hkv=None, pages_per_split=0, stream=None):
    """spin_attend_noalloc over device tensors: q [B][Hq][128] bf16 bits
    (int16), pool (any dtype, whole 32 KiB pages), block tables
    [>=batch][Hkv][max_blocks] int32, block_count [>=batch][Hkv] int32, out
    [>=batch][Hq][128] float32.  batch defaults to the tables' first
    dimension."""
    lib = load()
    Hkv = block_table.shape[1] if Hkv is None else Hkv
    Hq = q.shape[1] if Hq is None else Hq
    batch = block_table.shape[0] if batch is None else batch
    pool_pages = pool.numel() * pool.element_size() // PAGE_BYTES
    rc = lib.spin_attend_noalloc(_ptr(q), _ptr(pool), pool_pages, _ptr(block_table), _ptr(block_ntok),
                                 _ptr(block_count), _ptr(out), int(batch), int(Hq), int(Hkv),
                                 int(block_table.shape[2]), int(pages_per_split), _stream(stream))
    if rc != SPIN_OK:
        raise SpinError("spin_attend_noalloc", rc)
    return out


def read_stream(buf, sink, stream=None):
    """Enqueue spin_read_stream over the bytes of device tensor `buf` (a
    multiple of 16 bytes); `sink` is a device int32 tensor of 4 elements."""
    lib = load()
    rc = lib.spin_read_stream(c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                              c_void_p(sink.data_ptr()), _stream(stream))
    if rc != SPIN_OK:
        raise SpinError("spin_read_stream", rc)


def read_stream_gbs(nbytes=4 << 30, reps=5):
    """Practical HBM read ceiling: GB/s of spin_read_stream over nbytes."""
    import torch
    lib = load()
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    s = _stream(None)
    rc = lib.spin_read_stream(c_void_p(buf.data_ptr()), nbytes, c_void_p(sink.data_ptr()), s)
    if rc != SPIN_OK:
        raise SpinError("spin_read_stream", rc)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        lib.spin_read_stream(c_void_p(buf.data_ptr()), nbytes, c_void_p(sink.data_ptr()), s)
    e1.record()
    torch.cuda.synchronize()
    return reps * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9


def pinned_u16(n_elems: int):
    """A pinned host tensor of n_elems bf16 slots (int16 storage) and its uint16 numpy view."""
    import torch
    t = torch.empty(max(int(n_elems), 1), dtype=torch.int16, pin_memory=True)
    return t, t.numpy().view(np.uint16)
