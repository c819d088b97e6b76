"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libpka.so`` (declared in ``include/pka.h``): it only
marshals arguments. Every step of the computation runs in the library's HIP
kernels; PyTorch supplies device memory and the current stream. There is no
fallback: if the library is missing, every call raises.

Functions (same names as the C entry points, without the ``pka_`` prefix):
  store_kv(k_new, v_new, out_loc, k_pool, v_pool, page_size)
  paged_attn_decode(q, k_pool, v_pool, page_table, seq_lens, max_seq_len, page_size,
                    scale, out=None, workspace=None)
  paged_attn_prefill(q, k_pool, v_pool, page_table, seq_lens, prefix_lens, extend_lens,
                     cu_extend, max_extend, max_seq_len, page_size, scale, out=None,
                     workspace=None)
  decode_workspace_bytes(...), prefill_workspace_bytes(...)
Tensor conventions: bf16 tensors may be torch.bfloat16 or int16/uint16 bit
patterns; index tensors are int32; all tensors contiguous on the same GPU.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libpka.so")

PKA_OK = 0
PKA_E_NULLPTR = -1
PKA_E_SHAPE = -2
PKA_E_UNSUPPORTED = -3
PKA_E_WORKSPACE = -4
PKA_E_HIP = -5

# Every symbol include/pka.h and include/pka_sched.h declare (the latter bound in
# the `sched` submodule).
EXPORTED_SYMBOLS = (
    "pka_version",
    "pka_status_string",
    "pka_store_kv",
    "pka_paged_attn_decode",
    "pka_paged_attn_decode_store",
    "pka_decode_workspace_bytes",
    "pka_paged_attn_prefill",
    "pka_prefill_workspace_bytes",
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


class PkaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class Geom(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libpka.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m paged_kv_attention_25_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    gp = ctypes.POINTER(Geom)
    L.pka_version.restype = ctypes.c_int
    L.pka_version.argtypes = []
    L.pka_status_string.restype = ctypes.c_char_p
    L.pka_status_string.argtypes = [ctypes.c_int]
    L.pka_store_kv.restype = ctypes.c_int
    L.pka_store_kv.argtypes = [gp, vp, vp, vp, i32, vp, vp, vp]
    L.pka_paged_attn_decode.restype = ctypes.c_int
    L.pka_paged_attn_decode.argtypes = [gp, vp, vp, vp, vp, i32, vp, i32, i32, f32, vp, vp, sz,
                                        vp]
    L.pka_paged_attn_decode_store.restype = ctypes.c_int
    L.pka_paged_attn_decode_store.argtypes = [gp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32,
                                              f32, vp, vp, sz, vp]
    L.pka_decode_workspace_bytes.restype = sz
    L.pka_decode_workspace_bytes.argtypes = [gp, i32, i32]
    L.pka_paged_attn_prefill.restype = ctypes.c_int
    L.pka_paged_attn_prefill.argtypes = [gp, vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32,
                                         i32, f32, vp, vp, sz, vp]
    L.pka_prefill_workspace_bytes.restype = sz
    L.pka_prefill_workspace_bytes.argtypes = [gp, i32, i32, i32]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().pka_status_string(int(status)).decode()


def version() -> int:
    return int(lib().pka_version())


def _check(status: int, what: str):
    if status != PKA_OK:
        raise PkaError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_geom(num_q_heads, num_kv_heads, head_dim, page_size, num_pages) -> Geom:
    return Geom(int(num_q_heads), int(num_kv_heads), int(head_dim), int(page_size),
                int(num_pages))


def _pool_geom(q_heads, k_pool, page_size) -> Geom:
    slots, hkv, d = k_pool.shape
    if slots % page_size:
        raise ValueError("pool slots must be a whole number of pages")
    return make_geom(q_heads, hkv, d, page_size, slots // page_size)


def store_kv(k_new, v_new, out_loc, k_pool, v_pool, page_size=1):
    """pka_store_kv: k_pool[out_loc[t]] = k_new[t], v_pool[out_loc[t]] = v_new[t]."""
    g = _pool_geom(k_pool.shape[1], k_pool, page_size)
    _check(lib().pka_store_kv(ctypes.byref(g), _ptr(k_new), _ptr(v_new), _ptr(out_loc),
                              int(out_loc.shape[0]), _ptr(k_pool), _ptr(v_pool),
                              _stream(k_pool.device)), "pka_store_kv")


def decode_workspace_bytes(num_q_heads, num_kv_heads, head_dim, page_size, num_pages, batch,
                           max_seq_len) -> int:
    g = make_geom(num_q_heads, num_kv_heads, head_dim, page_size, num_pages)
    return int(lib().pka_decode_workspace_bytes(ctypes.byref(g), int(batch), int(max_seq_len)))


def prefill_workspace_bytes(num_q_heads, num_kv_heads, head_dim, page_size, num_pages, batch,
                            num_tokens, max_extend) -> int:
    g = make_geom(num_q_heads, num_kv_heads, head_dim, page_size, num_pages)
    return int(lib().pka_prefill_workspace_bytes(ctypes.byref(g), int(batch), int(num_tokens),
                                                 int(max_extend)))


def _alloc_like(q, nbytes):
    import torch
    return torch.empty(max(1, int(nbytes)), dtype=torch.uint8, device=q.device)


def paged_attn_decode(q, k_pool, v_pool, page_table, seq_lens, max_seq_len, page_size, scale,
                      out=None, workspace=None):
    """pka_paged_attn_decode. q [B, Hq, D]; returns out [B, Hq, D] (same dtype as q).
    Without a workspace, one of pka_decode_workspace_bytes is allocated for the call."""
    import torch
    g = _pool_geom(q.shape[1], k_pool, page_size)
    batch = int(q.shape[0])
    if out is None:
        out = torch.empty_like(q)
    need = int(lib().pka_decode_workspace_bytes(ctypes.byref(g), batch, int(max_seq_len)))
    if workspace is None and need > 0:
        workspace = _alloc_like(q, need)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pka_paged_attn_decode(ctypes.byref(g), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                       _ptr(page_table), int(page_table.shape[1]),
                                       _ptr(seq_lens), batch, int(max_seq_len), float(scale),
                                       _ptr(out), _ptr(workspace), ws_bytes,
                                       _stream(q.device)), "pka_paged_attn_decode")
    return out


def paged_attn_decode_store(q, k_new, v_new, out_loc, k_pool, v_pool, page_table, seq_lens,
                            max_seq_len, page_size, scale, out=None, workspace=None):
    """pka_paged_attn_decode_store: stores k_new[b], v_new[b] [B, Hkv, D] into slot
    out_loc[b] of the pools and decodes, in one launch (the same result as store_kv then
    paged_attn_decode). Returns out [B, Hq, D]."""
    import torch
    g = _pool_geom(q.shape[1], k_pool, page_size)
    batch = int(q.shape[0])
    if out is None:
        out = torch.empty_like(q)
    need = int(lib().pka_decode_workspace_bytes(ctypes.byref(g), batch, int(max_seq_len)))
    if workspace is None and need > 0:
        workspace = _alloc_like(q, need)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pka_paged_attn_decode_store(ctypes.byref(g), _ptr(q), _ptr(k_new),
                                             _ptr(v_new), _ptr(out_loc), _ptr(k_pool),
                                             _ptr(v_pool), _ptr(page_table),
                                             int(page_table.shape[1]), _ptr(seq_lens), batch,
                                             int(max_seq_len), float(scale), _ptr(out),
                                             _ptr(workspace), ws_bytes, _stream(q.device)),
           "pka_paged_attn_decode_store")
    return out


def paged_attn_prefill(q, k_pool, v_pool, page_table, seq_lens, prefix_lens, extend_lens,
                       cu_extend, max_extend, max_seq_len, page_size, scale, out=None,
                       workspace=None):
    """pka_paged_attn_prefill. q [T, Hq, D]; returns out [T, Hq, D] (same dtype as q)."""
    import torch
    g = _pool_geom(q.shape[1], k_pool, page_size)
    batch = int(seq_lens.shape[0])
    tokens = int(q.shape[0])
    if out is None:
        out = torch.empty_like(q)
    need = int(lib().pka_prefill_workspace_bytes(ctypes.byref(g), batch, tokens,
                                                 int(max_extend)))
    if workspace is None and need > 0:
        workspace = _alloc_like(q, need)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pka_paged_attn_prefill(ctypes.byref(g), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                        _ptr(page_table), int(page_table.shape[1]),
                                        _ptr(seq_lens), _ptr(prefix_lens), _ptr(extend_lens),
                                        _ptr(cu_extend), batch, tokens, int(max_extend),
                                        int(max_seq_len), float(scale), _ptr(out),
                                        _ptr(workspace), ws_bytes, _stream(q.device)),
           "pka_paged_attn_prefill")
    return out
