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
  paged_attn_decode_store(q, k_new, v_new, out_loc, ...), and its variant
    paged_attn_decode_store_noalloc(...) that uses the library's static scratch
  decode_workspace_bytes(...), prefill_workspace_bytes(...)
Tensor conventions: bf16 tensors may be torch.bfloat16 or int16/uint16 bit
patterns; index tensors are int32; all tensors contiguous on the same GPU. Each call
checks these conventions and the shape relations between its tensors on the host
before anything reaches the library, and raises ValueError on a mismatch (a CPU
tensor or a short metadata array would otherwise become a bad device pointer).

Debug mode (``PKA_DEBUG=1`` in the environment or ``set_debug(True)``): each call
also copies its device metadata to the host and checks it (``checks.py``: page ids
inside the pool, lengths within the host-known bounds, distinct and private
new-token slots), raising ``checks.MetadataError`` before any launch. It
synchronises with the device; leave it off when timing.
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
PKA_E_SCRATCH = -9

# Every symbol include/pka.h and include/pka_sched.h declare (the latter bound in
# the `sched` submodule).
EXPORTED_SYMBOLS = (
    "pka_version",
    "pka_status_string",
    "pka_store_kv",
    "pka_paged_attn_decode",
    "pka_paged_attn_decode_store",
    "pka_paged_attn_decode_store_noalloc",
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
    L.pka_paged_attn_decode_store_noalloc.restype = ctypes.c_int
    L.pka_paged_attn_decode_store_noalloc.argtypes = [gp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                                      i32, i32, f32, vp, vp]
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


_debug = os.environ.get("PKA_DEBUG", "0") not in ("", "0")


def set_debug(on: bool) -> None:
    """Turn the host-side metadata checks of every call on or off."""
    global _debug
    _debug = bool(on)


def debug_enabled() -> bool:
    return _debug


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_geom(num_q_heads, num_kv_heads, head_dim, page_size, num_pages) -> Geom:
    return Geom(int(num_q_heads), int(num_kv_heads), int(head_dim), int(page_size),
                int(num_pages))


# --- host-side tensor checks ------------------------------------------------------------

_torch_types = None


def _types():
    """(torch.Tensor, the bf16-carrying dtypes, torch.int32), looked up once."""
    global _torch_types
    if _torch_types is None:
        import torch
        _torch_types = (torch.Tensor, (torch.bfloat16, torch.int16, torch.uint16), torch.int32)
    return _torch_types


def _tensor(t, name, kind, shape):
    """`t` must be a contiguous torch tensor of `kind` ("bf16": bfloat16 or 16-bit
    integer bit patterns; "i32"; "bytes": any dtype) whose shape matches `shape`
    (None entries match any size), starting on a 16-byte boundary (4 for "i32")."""
    tensor_t, bf16_dtypes, i32 = _types()
    if not isinstance(t, tensor_t):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if kind == "bf16":
        if t.dtype not in bf16_dtypes:
            raise ValueError(f"{name} must hold bf16 values (torch.bfloat16 or 16-bit bit "
                             f"patterns), got {t.dtype}")
    elif kind == "i32" and t.dtype != i32:
        raise ValueError(f"{name} must be int32, got {t.dtype}")
    if shape is not None:
        got = t.shape
        bad = len(got) != len(shape)
        if not bad:
            for have, want in zip(got, shape):
                if want is not None and have != want:
                    bad = True
                    break
        if bad:
            want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
            raise ValueError(f"{name} has shape {list(got)}, expected {want}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    # The kernels read index arrays as int32 and move bf16 rows and workspace entries in
    # 16-byte pieces; the library rejects other starts too, with a less specific status.
    align = 4 if kind == "i32" else 16
    if t.numel() > 0 and t.data_ptr() % align:
        raise ValueError(f"{name} must start on a {align}-byte boundary "
                         f"(a view into another tensor may not)")


def _same_gpu(named):
    """Every tensor in `named` ({name: tensor or None}) lives on one and the same GPU."""
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} is on {t.device}; every tensor must be on the GPU")
        d = t.get_device()
        if dev is None:
            dev = d
        elif d != dev:
            raise ValueError(f"{name} is on cuda:{d}, other tensors on cuda:{dev}")
    return dev


def _pools(k_pool, v_pool, page_size):
    """Checks the two pools ([slots, Hkv, D], equal shapes, whole pages); returns
    (Hkv, D, num_pages)."""
    _tensor(k_pool, "k_pool", "bf16", (None, None, None))
    _tensor(v_pool, "v_pool", "bf16", tuple(k_pool.shape))
    if int(page_size) < 1:
        raise ValueError(f"page_size must be >= 1, got {page_size}")
    slots, hkv, d = (int(s) for s in k_pool.shape)
    if slots % int(page_size):
        raise ValueError(f"pool of {slots} slots is not a whole number of {page_size}-slot "
                         "pages")
    return hkv, d, slots // int(page_size)


def _workspace(ws):
    if ws is not None:
        _tensor(ws, "workspace", "bytes", None)
    return 0 if ws is None else ws.numel() * ws.element_size()


def _out(out, like, name="out"):
    if out is not None:
        _tensor(out, name, "bf16", tuple(like.shape))
        if out.data_ptr() == like.data_ptr():
            raise ValueError(f"{name} must not alias q")


def store_kv(k_new, v_new, out_loc, k_pool, v_pool, page_size=1):
    """pka_store_kv: k_pool[out_loc[t]] = k_new[t], v_pool[out_loc[t]] = v_new[t]."""
    hkv, d, num_pages = _pools(k_pool, v_pool, page_size)
    _tensor(out_loc, "out_loc", "i32", (None,))
    rows = int(out_loc.shape[0])
    _tensor(k_new, "k_new", "bf16", (rows, hkv, d))
    _tensor(v_new, "v_new", "bf16", (rows, hkv, d))
    if _debug:
        from . import checks
        checks.check_out_loc(out_loc, num_pages * int(page_size))
    _same_gpu(dict(k_new=k_new, v_new=v_new, out_loc=out_loc, k_pool=k_pool, v_pool=v_pool))
    g = make_geom(hkv, hkv, d, page_size, num_pages)
    _check(lib().pka_store_kv(ctypes.byref(g), _ptr(k_new), _ptr(v_new), _ptr(out_loc), rows,
                              _ptr(k_pool), _ptr(v_pool), _stream(k_pool.device)),
           "pka_store_kv")


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
    """A workspace for one call, zeroed (the decode's work counters start at zero)."""
    import torch
    return torch.zeros(max(1, int(nbytes)), dtype=torch.uint8, device=q.device)


def _decode_inputs(q, k_pool, v_pool, page_table, seq_lens, page_size, out, workspace,
                   extra=None, pools=None):
    """Checks shared by the decode entry points (`pools`: _pools' result when the caller
    has checked the pools and q already); returns (geometry, batch, the tensors by name
    for the device check)."""
    if pools is None:
        hkv, d, num_pages = _pools(k_pool, v_pool, page_size)
        _tensor(q, "q", "bf16", (None, None, d))
    else:
        hkv, d, num_pages = pools
    batch, hq = int(q.shape[0]), int(q.shape[1])
    if hq % hkv:
        raise ValueError(f"q has {hq} heads, not a multiple of the pools' {hkv} kv heads")
    _tensor(page_table, "page_table", "i32", (batch, None))
    _tensor(seq_lens, "seq_lens", "i32", (batch,))
    _out(out, q)
    _workspace(workspace)
    named = dict(q=q, k_pool=k_pool, v_pool=v_pool, page_table=page_table, seq_lens=seq_lens,
                 out=out, workspace=workspace, **(extra or {}))
    return make_geom(hq, hkv, d, page_size, num_pages), batch, named


def paged_attn_decode(q, k_pool, v_pool, page_table, seq_lens, max_seq_len, page_size, scale,
                      out=None, workspace=None):
    """pka_paged_attn_decode. q [B, Hq, D]; returns out [B, Hq, D] (same dtype as q).
    Without a workspace, one of pka_decode_workspace_bytes is allocated for the call."""
    import torch
    g, batch, named = _decode_inputs(q, k_pool, v_pool, page_table, seq_lens, page_size, out,
                                     workspace)
    if _debug:
        from . import checks
        checks.check_decode(seq_lens, int(max_seq_len), page_table, int(page_size), g.num_pages)
    _same_gpu(named)
    if out is None:
        out = torch.empty_like(q)
    need = int(lib().pka_decode_workspace_bytes(ctypes.byref(g), batch, int(max_seq_len)))
    if workspace is None and need > 0:
        workspace = _alloc_like(q, need)
    ws_bytes = _workspace(workspace)
    _check(lib().pka_paged_attn_decode(ctypes.byref(g), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                       _ptr(page_table), int(page_table.shape[1]),
                                       _ptr(seq_lens), batch, int(max_seq_len), float(scale),
                                       _ptr(out), _ptr(workspace), ws_bytes,
                                       _stream(q.device)), "pka_paged_attn_decode")
    return out


def _new_rows(k_new, v_new, out_loc, batch, hkv, d):
    _tensor(k_new, "k_new", "bf16", (batch, hkv, d))
    _tensor(v_new, "v_new", "bf16", (batch, hkv, d))
    _tensor(out_loc, "out_loc", "i32", (batch,))
    return dict(k_new=k_new, v_new=v_new, out_loc=out_loc)


def paged_attn_decode_store(q, k_new, v_new, out_loc, k_pool, v_pool, page_table, seq_lens,
                            max_seq_len, page_size, scale, out=None, workspace=None):
    """pka_paged_attn_decode_store: stores k_new[b], v_new[b] [B, Hkv, D] into slot
    out_loc[b] of the pools and decodes, in one launch (the same result as store_kv then
    paged_attn_decode). Returns out [B, Hq, D]."""
    import torch
    pools = _pools(k_pool, v_pool, page_size)
    hkv, d, _ = pools
    _tensor(q, "q", "bf16", (None, None, d))
    extra = _new_rows(k_new, v_new, out_loc, int(q.shape[0]), hkv, d)
    g, batch, named = _decode_inputs(q, k_pool, v_pool, page_table, seq_lens, page_size, out,
                                     workspace, extra, pools)
    if _debug:
        from . import checks
        checks.check_decode_store(out_loc, seq_lens, int(max_seq_len), page_table,
                                  int(page_size), g.num_pages)
    _same_gpu(named)
    if out is None:
        out = torch.empty_like(q)
    need = int(lib().pka_decode_workspace_bytes(ctypes.byref(g), batch, int(max_seq_len)))
    if workspace is None and need > 0:
        workspace = _alloc_like(q, need)
    ws_bytes = _workspace(workspace)
    _check(lib().pka_paged_attn_decode_store(ctypes.byref(g), _ptr(q), _ptr(k_new),
                                             _ptr(v_new), _ptr(out_loc), _ptr(k_pool),
                                             _ptr(v_pool), _ptr(page_table),
                                             int(page_table.shape[1]), _ptr(seq_lens), batch,
                                             int(max_seq_len), float(scale), _ptr(out),
                                             _ptr(workspace), ws_bytes, _stream(q.device)),
           "pka_paged_attn_decode_store")
    return out


def paged_attn_decode_store_noalloc(q, k_new, v_new, out_loc, k_pool, v_pool, page_table,
                                    seq_lens, max_seq_len, page_size, scale, out):
    """pka_paged_attn_decode_store_noalloc: the same call as paged_attn_decode_store with
    the split partials in the library's static device scratch; `out` [B, Hq, D] must be
    given (nothing is allocated). Returns out."""
    if out is None:
        raise ValueError("out must be given: this call allocates nothing")
    pools = _pools(k_pool, v_pool, page_size)
    hkv, d, _ = pools
    _tensor(q, "q", "bf16", (None, None, d))
    extra = _new_rows(k_new, v_new, out_loc, int(q.shape[0]), hkv, d)
    g, batch, named = _decode_inputs(q, k_pool, v_pool, page_table, seq_lens, page_size, out,
                                     None, extra, pools)
    if _debug:
        from . import checks
        checks.check_decode_store(out_loc, seq_lens, int(max_seq_len), page_table,
                                  int(page_size), g.num_pages)
    _same_gpu(named)
    _check(lib().pka_paged_attn_decode_store_noalloc(
        ctypes.byref(g), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out_loc), _ptr(k_pool),
        _ptr(v_pool), _ptr(page_table), int(page_table.shape[1]), _ptr(seq_lens), batch,
        int(max_seq_len), float(scale), _ptr(out), _stream(q.device)),
        "pka_paged_attn_decode_store_noalloc")
    return out


def paged_attn_prefill(q, k_pool, v_pool, page_table, seq_lens, prefix_lens, extend_lens,
                       cu_extend, max_extend, max_seq_len, page_size, scale, out=None,
                       workspace=None):
    """pka_paged_attn_prefill. q [T, Hq, D]; returns out [T, Hq, D] (same dtype as q)."""
    import torch
    hkv, d, num_pages = _pools(k_pool, v_pool, page_size)
    _tensor(q, "q", "bf16", (None, None, d))
    tokens, hq = int(q.shape[0]), int(q.shape[1])
    if hq % hkv:
        raise ValueError(f"q has {hq} heads, not a multiple of the pools' {hkv} kv heads")
    _tensor(seq_lens, "seq_lens", "i32", (None,))
    batch = int(seq_lens.shape[0])
    _tensor(prefix_lens, "prefix_lens", "i32", (batch,))
    _tensor(extend_lens, "extend_lens", "i32", (batch,))
    _tensor(cu_extend, "cu_extend", "i32", (batch + 1,))
    _tensor(page_table, "page_table", "i32", (batch, None))
    _out(out, q)
    _workspace(workspace)
    if _debug:
        from . import checks
        checks.check_prefill(seq_lens, prefix_lens, extend_lens, cu_extend, tokens,
                             int(max_extend), int(max_seq_len), page_table, int(page_size),
                             num_pages)
    _same_gpu(dict(q=q, k_pool=k_pool, v_pool=v_pool, page_table=page_table, seq_lens=seq_lens,
                   prefix_lens=prefix_lens, extend_lens=extend_lens, cu_extend=cu_extend,
                   out=out, workspace=workspace))
    g = make_geom(hq, hkv, d, page_size, num_pages)
    if out is None:
        out = torch.empty_like(q)
    need = int(lib().pka_prefill_workspace_bytes(ctypes.byref(g), batch, tokens,
                                                 int(max_extend)))
    if workspace is None and need > 0:
        workspace = _alloc_like(q, need)
    ws_bytes = _workspace(workspace)
    _check(lib().pka_paged_attn_prefill(ctypes.byref(g), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                        _ptr(page_table), int(page_table.shape[1]),
                                        _ptr(seq_lens), _ptr(prefix_lens), _ptr(extend_lens),
                                        _ptr(cu_extend), batch, tokens, int(max_extend),
                                        int(max_seq_len), float(scale), _ptr(out),
                                        _ptr(workspace), ws_bytes, _stream(q.device)),
           "pka_paged_attn_prefill")
    return out
