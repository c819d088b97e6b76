"""ctypes binding of the host-side metadata producer (``include/pka_sched.h``).

Argument marshalling only: the page allocator, the prefix cache and the batch
builder run in ``libpka.so`` (``csrc/sched.cpp``). A batch comes back as host
numpy arrays in the layout the attention calls take (int32; page_table
[batch, table_width]).

    s = Scheduler(page_size=16, num_pages=4096, policy="radix", max_prefill_tokens=8192)
    s.add_request(7, tokens)          # prompt token ids
    b = s.prefill_batch()             # chunked prefill over cached prefixes
    s.push_token(7, next_token)       # once its prompt is complete
    b = s.decode_batch()
    s.finish(7)                       # its whole pages join the prefix cache

A batch counts its new tokens as stored when it is built: run its store before
finishing a request it extended.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from . import PkaError, lib

PKA_CACHE_NAIVE = 0
PKA_CACHE_RADIX = 1
PKA_E_STATE = -6
PKA_E_CAPACITY = -7
PKA_E_NOMEM = -8

SCHED_SYMBOLS = (
    "pka_sched_create",
    "pka_sched_destroy",
    "pka_sched_add_request",
    "pka_sched_prefill_batch",
    "pka_sched_push_token",
    "pka_sched_push_tokens",
    "pka_sched_decode_batch",
    "pka_sched_finish",
    "pka_sched_request_pages",
    "pka_sched_get_stats",
)


class _Batch(ctypes.Structure):
    _fields_ = [
        ("max_batch", ctypes.c_int32),
        ("table_width", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("req_ids", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("prefix_lens", ctypes.c_void_p),
        ("extend_lens", ctypes.c_void_p),
        ("cu_extend", ctypes.c_void_p),
        ("out_loc", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32),
        ("max_extend", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
    ]


class _Stats(ctypes.Structure):
    _fields_ = [
        ("free_pages", ctypes.c_int64),
        ("cached_pages", ctypes.c_int64),
        ("locked_pages", ctypes.c_int64),
        ("private_pages", ctypes.c_int64),
        ("evicted_pages", ctypes.c_int64),
        ("waiting", ctypes.c_int32),
        ("prefilling", ctypes.c_int32),
        ("running", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_bound = False


def _lib():
    global _bound
    L = lib()
    if not _bound:
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.pka_sched_create.restype = ctypes.c_int
        L.pka_sched_create.argtypes = [i32, i64, i32, i32, ctypes.POINTER(vp)]
        L.pka_sched_destroy.restype = None
        L.pka_sched_destroy.argtypes = [vp]
        L.pka_sched_add_request.restype = ctypes.c_int
        L.pka_sched_add_request.argtypes = [vp, i64, vp, i32]
        L.pka_sched_prefill_batch.restype = ctypes.c_int
        L.pka_sched_prefill_batch.argtypes = [vp, ctypes.POINTER(_Batch)]
        L.pka_sched_push_token.restype = ctypes.c_int
        L.pka_sched_push_token.argtypes = [vp, i64, i32]
        L.pka_sched_push_tokens.restype = ctypes.c_int
        L.pka_sched_push_tokens.argtypes = [vp, vp, vp, i32]
        L.pka_sched_decode_batch.restype = ctypes.c_int
        L.pka_sched_decode_batch.argtypes = [vp, ctypes.POINTER(_Batch)]
        L.pka_sched_finish.restype = ctypes.c_int
        L.pka_sched_finish.argtypes = [vp, i64]
        L.pka_sched_request_pages.restype = ctypes.c_int
        L.pka_sched_request_pages.argtypes = [vp, i64, vp, i32, ctypes.POINTER(i32),
                                              ctypes.POINTER(i32)]
        L.pka_sched_get_stats.restype = ctypes.c_int
        L.pka_sched_get_stats.argtypes = [vp, ctypes.POINTER(_Stats)]
        _bound = True
    return L


def _check(status: int, what: str):
    if status != 0:
        raise PkaError(status, what)


@dataclass
class Batch:
    """One prefill or decode call's metadata (host numpy, int32 unless noted)."""
    req_ids: np.ndarray      # [batch] int64
    page_table: np.ndarray   # [batch, table_width]
    seq_lens: np.ndarray     # [batch]
    prefix_lens: np.ndarray  # [batch]
    extend_lens: np.ndarray  # [batch]
    cu_extend: np.ndarray    # [batch + 1]
    out_loc: np.ndarray      # [num_tokens]
    num_tokens: int
    max_extend: int
    max_seq_len: int

    @property
    def batch(self) -> int:
        return int(self.req_ids.shape[0])


class Scheduler:
    """Page allocator + prefix cache + chunked-prefill / decode batch builder."""

    def __init__(self, page_size: int, num_pages: int, policy: str = "radix",
                 max_prefill_tokens: int = 8192, max_batch: int = 1024, table_width: int = 4096,
                 max_tokens: int | None = None):
        pol = {"naive": PKA_CACHE_NAIVE, "radix": PKA_CACHE_RADIX}[policy]
        self._L = _lib()
        self._h = ctypes.c_void_p()
        _check(self._L.pka_sched_create(int(page_size), int(num_pages), pol,
                                        int(max_prefill_tokens), ctypes.byref(self._h)),
               "pka_sched_create")
        self.page_size = int(page_size)
        self.max_batch = int(max_batch)
        self.table_width = int(table_width)
        self.max_tokens = int(max_prefill_tokens if max_tokens is None else max_tokens)
        self._bufs = dict(
            req_ids=np.zeros(self.max_batch, np.int64),
            page_table=np.zeros((self.max_batch, self.table_width), np.int32),
            seq_lens=np.zeros(self.max_batch, np.int32),
            prefix_lens=np.zeros(self.max_batch, np.int32),
            extend_lens=np.zeros(self.max_batch, np.int32),
            cu_extend=np.zeros(self.max_batch + 1, np.int32),
            out_loc=np.zeros(max(self.max_tokens, 1), np.int32),
        )
        self._pages = np.zeros(self.table_width, np.int32)

    def close(self):
        if self._h:
            self._L.pka_sched_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_request(self, req_id: int, tokens):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(self._L.pka_sched_add_request(self._h, int(req_id), t.ctypes.data, int(t.size)),
               "pka_sched_add_request")

    def _descriptor(self) -> _Batch:
        b = self._bufs
        return _Batch(self.max_batch, self.table_width, self.max_tokens, 0,
                      b["req_ids"].ctypes.data, b["page_table"].ctypes.data,
                      b["seq_lens"].ctypes.data, b["prefix_lens"].ctypes.data,
                      b["extend_lens"].ctypes.data, b["cu_extend"].ctypes.data,
                      b["out_loc"].ctypes.data, 0, 0, 0, 0)

    def raw(self):
        """(library, handle, batch descriptor, buffers) for calling the C entry points
        directly, e.g. to time them without the Python-side copies: the descriptor points
        at this object's preallocated host buffers (a dict of numpy arrays), which the
        batch calls fill in place."""
        return self._L, self._h, self._descriptor(), self._bufs

    def _batch(self, fn, what) -> Batch:
        b = self._bufs
        c = self._descriptor()
        _check(fn(self._h, ctypes.byref(c)), what)
        n, t = c.batch, c.num_tokens
        return Batch(b["req_ids"][:n].copy(), b["page_table"][:n].copy(), b["seq_lens"][:n].copy(),
                     b["prefix_lens"][:n].copy(), b["extend_lens"][:n].copy(),
                     b["cu_extend"][:n + 1].copy(), b["out_loc"][:t].copy(), t, c.max_extend,
                     c.max_seq_len)

    def prefill_batch(self) -> Batch:
        return self._batch(self._L.pka_sched_prefill_batch, "pka_sched_prefill_batch")

    def decode_batch(self) -> Batch:
        return self._batch(self._L.pka_sched_decode_batch, "pka_sched_decode_batch")

    def push_token(self, req_id: int, token: int):
        _check(self._L.pka_sched_push_token(self._h, int(req_id), int(token)),
               "pka_sched_push_token")

    def push_tokens(self, req_ids, tokens):
        ids = np.ascontiguousarray(req_ids, dtype=np.int64)
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        assert ids.shape == tok.shape and ids.ndim == 1
        _check(self._L.pka_sched_push_tokens(self._h, ids.ctypes.data, tok.ctypes.data,
                                             int(ids.size)), "pka_sched_push_tokens")

    def finish(self, req_id: int):
        _check(self._L.pka_sched_finish(self._h, int(req_id)), "pka_sched_finish")

    def request_pages(self, req_id: int):
        n, cached = ctypes.c_int32(), ctypes.c_int32()
        _check(self._L.pka_sched_request_pages(self._h, int(req_id), self._pages.ctypes.data,
                                               self.table_width, ctypes.byref(n),
                                               ctypes.byref(cached)),
               "pka_sched_request_pages")
        return self._pages[:n.value].copy(), int(cached.value)

    def stats(self) -> dict:
        st = _Stats()
        _check(self._L.pka_sched_get_stats(self._h, ctypes.byref(st)), "pka_sched_get_stats")
        return {k: int(getattr(st, k)) for k, _ in _Stats._fields_ if k != "reserved"}
