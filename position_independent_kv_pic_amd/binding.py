"""ctypes binding of libpic (argument marshalling only).

Buffers are passed as raw device addresses (ints) or as objects with a
`data_ptr()` method (torch tensors); streams as a raw hipStream_t value or an
object with a `cuda_stream` attribute.  Nothing here computes any part of the
method: a missing library raises, it never falls back.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))

PIC_F32 = 0
PIC_BF16 = 1
TARGET_AUTO = -1
TARGET_ORIGINAL = -2
KEYS_ROTATED = 0
KEYS_UNROTATED = 1
PLAN_ONLY = 1
DRY_RUN = 2
DEFER_GATHER = 4
QUERY_ROTATION = 8
VALUES_IN_POOL = 16
VARIANT_MATERIALIZED = 0
VARIANT_FUSED = 1

_STATUS = {0: "PIC_OK", -1: "PIC_EINVAL", -2: "PIC_ERANGE", -3: "PIC_ENOMEM", -4: "PIC_EDEVICE",
           -5: "PIC_ESTATE", -6: "PIC_EALIGN", -7: "PIC_EUNSUPPORTED"}

EXPORTED = (
    "pic_pool_register", "pic_pool_release", "pic_plan_create", "pic_plan_release",
    "pic_assemble", "pic_query_prefill", "pic_plan_get_summary", "pic_plan_get_requests",
    "pic_plan_get_spans", "pic_plan_get_new_tokens", "pic_timing_enable", "pic_timing_read",
    "pic_timing_reset", "pic_last_error", "pic_version", "pic_plan_set_decode_rows", "pic_decode_layer",
    "pic_pool_register_host", "pic_gather_layers", "pic_plan_get_attention_work",
    "pic_query_prefill_noalloc", "pic_cache_create", "pic_cache_get_stats", "pic_cache_release",
    "pic_chunk_file_write", "pic_store_open", "pic_store_request", "pic_store_wait", "pic_store_forget",
    "pic_store_get_stats", "pic_store_release",
)


class PicError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = _STATUS.get(status, str(status))


class PicModel(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("q_heads", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("dtype", ctypes.c_int32),
                ("key_storage", ctypes.c_int32)]


class PicSpan(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int32), ("s", ctypes.c_int32), ("e", ctypes.c_int32),
                ("target", ctypes.c_int32)]


class PicCacheStats(ctypes.Structure):
    _fields_ = [("capacity_pages", ctypes.c_int64), ("resident_pages", ctypes.c_int64),
                ("hits", ctypes.c_int64), ("misses", ctypes.c_int64), ("evictions", ctypes.c_int64),
                ("layer_copies", ctypes.c_int64), ("bytes_copied", ctypes.c_int64)]


class PicStoreStats(ctypes.Structure):
    _fields_ = [("resident_pages", ctypes.c_int64), ("requested", ctypes.c_int64), ("hits", ctypes.c_int64),
                ("pages_read", ctypes.c_int64), ("bytes_read", ctypes.c_int64), ("reads", ctypes.c_int64),
                ("wait_seconds", ctypes.c_double)]


class PicPlanSummary(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_spans", ctypes.c_int32),
                ("prefix_rows", ctypes.c_int64), ("new_rows", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("max_position", ctypes.c_int32),
                ("materialized", ctypes.c_int32), ("fused_query_rotation", ctypes.c_int32),
                ("values_in_pool", ctypes.c_int32), ("attention_items", ctypes.c_int32),
                ("attention_workgroups", ctypes.c_int32), ("attention_item_workgroups", ctypes.c_int32)]


def library_path() -> str:
    return os.path.join(HERE, "libpic.so")


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libpic.so (built in-tree by build.py); raise if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m position_independent_kv_pic_amd.build`")
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I32 = ctypes.c_int32
    I64 = ctypes.c_int64
    pi32 = ctypes.POINTER(ctypes.c_int32)
    pi64 = ctypes.POINTER(ctypes.c_int64)
    sig = {
        "pic_pool_register": [ctypes.POINTER(PicModel), P, I64, I32, I32, I32, pi32, pi32, pi32, pi32,
                              ctypes.POINTER(P)],
        "pic_pool_register_host": [ctypes.POINTER(PicModel), P, I64, I32, I32, I32, pi32, pi32, pi32, pi32,
                                   ctypes.POINTER(P)],
        "pic_gather_layers": [P, I32, I32, P],
        "pic_pool_release": [P],
        "pic_cache_create": [P, I32, ctypes.POINTER(P)],
        "pic_cache_get_stats": [P, ctypes.POINTER(PicCacheStats)],
        "pic_cache_release": [P],
        "pic_chunk_file_write": [ctypes.POINTER(PicModel), I32, I32, I32, P, pi32, ctypes.c_char_p],
        "pic_store_open": [P, P, I64, ctypes.POINTER(ctypes.c_char_p), I32, ctypes.POINTER(P)],
        "pic_store_request": [P, I32, pi32, ctypes.POINTER(PicSpan)],
        "pic_store_wait": [P],
        "pic_store_forget": [P, I32],
        "pic_store_get_stats": [P, ctypes.POINTER(PicStoreStats)],
        "pic_store_release": [P],
        "pic_plan_create": [P, ctypes.POINTER(P)],
        "pic_plan_release": [P],
        "pic_assemble": [P, I32, pi32, ctypes.POINTER(PicSpan), pi32, pi32, P, P, I64, I32, P],
        "pic_query_prefill": [P, I32, P, P, P, P, I32, P],
        "pic_query_prefill_noalloc": [P, I32, P, P, P, P, I32, P],
        "pic_plan_set_decode_rows": [P, I32],
        "pic_decode_layer": [P, I32, I32, P, P, P, P, I32, P],
        "pic_plan_get_summary": [P, ctypes.POINTER(PicPlanSummary)],
        "pic_plan_get_requests": [P, pi64, pi32, pi32],
        "pic_plan_get_spans": [P, pi32, pi32, pi64],
        "pic_plan_get_new_tokens": [P, pi32, pi64],
        "pic_plan_get_attention_work": [P, pi32, pi32, pi32],
        "pic_timing_enable": [P, I32],
        "pic_timing_read": [P, I32, pi64, ctypes.POINTER(ctypes.c_double)],
        "pic_timing_reset": [P],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.pic_last_error.argtypes = []
    L.pic_last_error.restype = ctypes.c_char_p
    L.pic_version.argtypes = []
    L.pic_version.restype = ctypes.c_char_p
    _LIB = L
    return L


def _check(status: int):
    if status != 0:
        raise PicError(status, lib().pic_last_error().decode())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s) -> Optional[int]:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p32(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def model_struct(layers, q_heads, kv_heads, head_dim, theta, dtype, keys="rotated") -> PicModel:
    dt = {"bf16": PIC_BF16, "f32": PIC_F32}.get(dtype, dtype)
    ks = {"rotated": KEYS_ROTATED, "unrotated": KEYS_UNROTATED}.get(keys, keys)
    return PicModel(int(layers), int(q_heads), int(kv_heads), int(head_dim), float(theta), int(dt), int(ks))


class Pool:
    """A registered paged chunk-KV pool (the memory stays the caller's)."""

    def __init__(self, model: PicModel, pool, pool_bytes: int, page_tokens: int, n_pages: int,
                 chunk_len, chunk_page_ptr, page_ids, chunk_orig=None, host: bool = False):
        self.model = model
        self._keep = (_i32(chunk_len), _i32(chunk_page_ptr), _i32(page_ids),
                      None if chunk_orig is None else _i32(chunk_orig))
        cl, cp, pg, co = self._keep
        # the library reads n_chunks (+ 1) entries of these tables
        if cp.shape[0] != cl.shape[0] + 1:
            raise ValueError("chunk_page_ptr needs len(chunk_len) + 1 entries")
        if co is not None and co.shape[0] != cl.shape[0]:
            raise ValueError("chunk_orig needs len(chunk_len) entries")
        if cp.shape[0] and pg.shape[0] < int(cp[-1]):
            raise ValueError("page_ids is shorter than chunk_page_ptr[-1]")
        h = ctypes.c_void_p()
        reg = lib().pic_pool_register_host if host else lib().pic_pool_register
        _check(reg(ctypes.byref(model), _ptr(pool), int(pool_bytes), int(page_tokens),
                   int(n_pages), int(cl.shape[0]), _p32(cl), _p32(co), _p32(cp), _p32(pg), ctypes.byref(h)))
        self.handle = h

    def release(self):
        if self.handle:
            _check(lib().pic_pool_release(self.handle))
            self.handle = None


class Cache:
    """HBM hot set of `capacity_pages` page slots in front of a host pool."""

    def __init__(self, pool: Pool, capacity_pages: int):
        h = ctypes.c_void_p()
        _check(lib().pic_cache_create(pool.handle, int(capacity_pages), ctypes.byref(h)))
        self.handle = h

    def stats(self) -> dict:
        s = PicCacheStats()
        _check(lib().pic_cache_get_stats(self.handle, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in PicCacheStats._fields_}

    def release(self):
        if self.handle:
            _check(lib().pic_cache_release(self.handle))
            self.handle = None


def _span_array(spans):
    tbl = _i32(spans).reshape(-1, 4)
    arr = (PicSpan * max(1, tbl.shape[0]))()
    if tbl.shape[0]:
        ctypes.memmove(arr, tbl.ctypes.data, tbl.nbytes)
    return tbl, arr


def write_chunk_file(model: PicModel, page_tokens: int, length: int, orig: int, pages, page_list, path: str):
    """Write one chunk file: the chunk's pages, page j taken from host memory
    at pages + page_list[j] * page_bytes (`pages`: an address or a numpy
    array)."""
    pl = _i32(page_list)
    need = (int(length) + int(page_tokens) - 1) // int(page_tokens)
    if pl.shape[0] < need:
        raise ValueError(f"page_list needs {need} entries, got {pl.shape[0]}")
    base = pages if isinstance(pages, int) else pages.ctypes.data
    _check(lib().pic_chunk_file_write(ctypes.byref(model), int(page_tokens), int(length), int(orig),
                                      base, _p32(pl), os.fsencode(path)))


class Store:
    """Chunk files loaded on demand into host memory laid out like the pool
    (attached to the pool when `dst` is the host pool's own memory)."""

    def __init__(self, pool: Pool, dst, dst_bytes: int, paths, threads: int = 8):
        n_chunks = pool._keep[0].shape[0]
        if len(paths) != n_chunks:
            raise ValueError(f"{n_chunks} chunk paths needed, got {len(paths)}")
        self._paths = (ctypes.c_char_p * max(1, len(paths)))(*[os.fsencode(p) for p in paths])
        base = dst if isinstance(dst, int) else (dst.ctypes.data if isinstance(dst, np.ndarray) else _ptr(dst))
        h = ctypes.c_void_p()
        _check(lib().pic_store_open(pool.handle, base, int(dst_bytes), self._paths, int(threads),
                                    ctypes.byref(h)))
        self.handle = h

    def request(self, span_ptr, spans):
        """Start loading the pages a batch's spans cover; returns at once."""
        sp = _i32(span_ptr)
        tbl, arr = _span_array(spans)
        if sp.shape[0] < 1 or int(sp[-1]) != tbl.shape[0]:
            raise ValueError("span_ptr must end at the number of spans")
        self._keep = (sp, tbl, arr)
        _check(lib().pic_store_request(self.handle, int(sp.shape[0]) - 1, _p32(sp), arr))

    def wait(self):
        _check(lib().pic_store_wait(self.handle))

    def forget(self, drop_os_cache: bool = False):
        _check(lib().pic_store_forget(self.handle, 1 if drop_os_cache else 0))

    def stats(self) -> dict:
        s = PicStoreStats()
        _check(lib().pic_store_get_stats(self.handle, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in PicStoreStats._fields_}

    def release(self):
        if self.handle:
            _check(lib().pic_store_release(self.handle))
            self.handle = None


class Plan:
    """Plan object: assemble batches, then run the per-layer query prefill."""

    def __init__(self, pool: Pool):
        self.pool = pool
        h = ctypes.c_void_p()
        _check(lib().pic_plan_create(pool.handle, ctypes.byref(h)))
        self.handle = h
        self.batch = 0
        self.n_spans = 0

    def release(self):
        if self.handle:
            _check(lib().pic_plan_release(self.handle))
            self.handle = None

    def assemble(self, span_ptr, spans, new_ptr, new_pos=None, asm_k=None, asm_v=None,
                 capacity: int = 0, flags: int = 0, stream=None):
        sp = _i32(span_ptr)
        npt = _i32(new_ptr)
        tbl = _i32(spans).reshape(-1, 4)
        arr = (PicSpan * max(1, tbl.shape[0]))()
        if tbl.shape[0]:
            ctypes.memmove(arr, tbl.ctypes.data, tbl.nbytes)
        npos = None if new_pos is None else _i32(new_pos)
        batch = int(sp.shape[0]) - 1
        # the C side trusts the CSR ends to match the array lengths
        if batch < 0 or npt.shape[0] != sp.shape[0]:
            raise ValueError("span_ptr and new_ptr need batch + 1 entries")
        if int(sp[-1]) != tbl.shape[0]:
            raise ValueError(f"span_ptr ends at {int(sp[-1])} but {tbl.shape[0]} spans were given")
        if npos is not None and int(npt[-1]) != npos.shape[0]:
            raise ValueError(f"new_ptr ends at {int(npt[-1])} but {npos.shape[0]} positions were given")
        self._keep = (sp, npt, tbl, arr, npos)
        _check(lib().pic_assemble(self.handle, batch, _p32(sp), arr, _p32(npt), _p32(npos),
                                  _ptr(asm_k), _ptr(asm_v),
                                  int(capacity), int(flags), _stream(stream)))
        self.batch = batch
        self.n_spans = int(tbl.shape[0])

    def query_prefill(self, layer: int, q, k_new, v_new, out, variant: int = VARIANT_MATERIALIZED,
                      stream=None):
        _check(lib().pic_query_prefill(self.handle, int(layer), _ptr(q),
                                       _ptr(k_new), _ptr(v_new),
                                       _ptr(out), int(variant),
                                       _stream(stream)))

    def query_prefill_noalloc(self, layer: int, q, k_new, v_new, out, variant: int = VARIANT_MATERIALIZED,
                              stream=None):
        """pic_query_prefill with its scratch in the library's fixed device array."""
        _check(lib().pic_query_prefill_noalloc(self.handle, int(layer), _ptr(q),
                                               _ptr(k_new), _ptr(v_new),
                                               _ptr(out), int(variant),
                                               _stream(stream)))

    def gather_layers(self, layer_begin: int, layer_end: int, stream=None):
        """Gather layers [layer_begin, layer_end) after a DEFER_GATHER assemble."""
        _check(lib().pic_gather_layers(self.handle, int(layer_begin), int(layer_end),
                                       _stream(stream)))

    def set_decode_rows(self, rows: int):
        """Rows reserved per request for decode tokens at the next assemble."""
        _check(lib().pic_plan_set_decode_rows(self.handle, int(rows)))

    def decode_layer(self, layer: int, step: int, q, k_new, v_new, out, variant: int = VARIANT_MATERIALIZED,
                     stream=None):
        _check(lib().pic_decode_layer(self.handle, int(layer), int(step), _ptr(q),
                                      _ptr(k_new), _ptr(v_new),
                                      _ptr(out), int(variant),
                                      _stream(stream)))

    def summary(self) -> dict:
        s = PicPlanSummary()
        _check(lib().pic_plan_get_summary(self.handle, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in PicPlanSummary._fields_}

    def requests(self):
        rb = np.zeros(self.batch, np.int64)
        pr = np.zeros(self.batch, np.int32)
        fp = np.zeros(self.batch, np.int32)
        _check(lib().pic_plan_get_requests(self.handle, rb.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                           _p32(pr), _p32(fp)))
        return rb, pr, fp

    def spans(self):
        t = np.zeros(self.n_spans, np.int32)
        d = np.zeros(self.n_spans, np.int32)
        r = np.zeros(self.n_spans, np.int64)
        _check(lib().pic_plan_get_spans(self.handle, _p32(t), _p32(d),
                                        r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
        return t, d, r

    def new_tokens(self):
        n = self.summary()["new_rows"]
        p = np.zeros(n, np.int32)
        r = np.zeros(n, np.int64)
        _check(lib().pic_plan_get_new_tokens(self.handle, _p32(p),
                                             r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
        return p, r

    def attention_work(self, single_items: bool = False):
        """(items int32[n][7], launch order): see pic_plan_get_attention_work.
        The order is over item pairs, or over single items if `single_items`."""
        s = self.summary()
        items = np.zeros((s["attention_items"], 7), np.int32)
        order = np.zeros(s["attention_workgroups"], np.int32)
        item_order = np.zeros(s["attention_item_workgroups"], np.int32)
        _check(lib().pic_plan_get_attention_work(self.handle, _p32(items), _p32(order), _p32(item_order)))
        return items, (item_order if single_items else order)

    def timing(self, enable: bool):
        _check(lib().pic_timing_enable(self.handle, 1 if enable else 0))

    def timing_read(self, kernel: int):
        n = ctypes.c_int64()
        ms = ctypes.c_double()
        _check(lib().pic_timing_read(self.handle, int(kernel), ctypes.byref(n), ctypes.byref(ms)))
        return int(n.value), float(ms.value)

    def timing_reset(self):
        _check(lib().pic_timing_reset(self.handle))
