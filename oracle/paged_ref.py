"""Paged KV-cache attention, written out as its plain definition, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Conventions (readings of what the pages leave open are marked READING):

* Pools. ``k_pool`` and ``v_pool`` are uint16 bf16 bit patterns of shape
  [num_slots, Hkv, D] with num_slots = num_pages * page_size; a page is
  page_size consecutive slots [deployment guide (dpshk.com), section 6.2
  "Page Size": the page is the pool's allocation unit; default size 1].
  READING: K and V are separate tensors, slot-major.
* Page table. ``page_table[b, n]`` is the physical page holding logical
  tokens n*P .. n*P+P-1 of request b [miniSGLang intro blog (0539edu.com),
  section 1.3: attention finds each request's data through a page table].
  READING: entries are page ids, so token j of request b lives in slot
  page_table[b, j // P] * P + j % P.
* Lengths. seq_lens[b] = prefix_lens[b] + extend_lens[b]. The prefix is
  already in the pool (radix reuse or an earlier chunk; deployment guide,
  sections 6.1 "Chunked Prefill" and 6.5 "Radix Cache"); the extend tokens are
  new. READING: the new tokens' K/V are stored into the pool first, then
  attention reads every key, old and new, from the pool (intro blog,
  section 1.3: the K/V seen by attention are pool history plus new K/V).
* Causality. READING (bottom-right alignment): new token i of request b sits
  at absolute position prefix_lens[b] + i and sees keys 0 .. prefix_lens[b]+i.
* GQA. READING: contiguous groups; q head h reads kv head h // (Hq / Hkv).
* Queries of all requests are packed in batch order, rows in position order:
  q[t] for t in [sum(extend_lens[:b]), sum(extend_lens[:b+1])).
* Decode is the case extend_lens = 1, prefix_lens = seq_lens - 1
  (READING: a decode seq_len counts the new token, whose K/V was stored first).
* Output: float64, unrounded, shape [T, Hq, D].
"""
from __future__ import annotations

import numpy as np

from .bf16 import bf16_bits_to_f64


class OracleInputError(ValueError):
    """Raised for any input that breaks the conventions above."""


# --- the three small definitions everything else is built from ---------------------


def slot_of(page_table_row, j: int, page_size: int) -> int:
    """Physical slot of logical token j of one request (page id * P + offset)."""
    return int(page_table_row[j // page_size]) * page_size + (j % page_size)


def kv_head_of(h: int, group: int) -> int:
    """KV head read by q head h when every `group` consecutive q heads share one."""
    return h // group


def last_visible_key(prefix_len: int, i: int) -> int:
    """Largest logical key index that new token i (0-based) of a request may see."""
    return prefix_len + i


def request_slots(page_table_row, seq_len: int, page_size: int) -> np.ndarray:
    """Slots of logical tokens 0 .. seq_len-1 of one request, in order."""
    return np.array([slot_of(page_table_row, j, page_size) for j in range(seq_len)],
                    dtype=np.int64)


# --- validation ---------------------------------------------------------------------


def _as_u16(name, a, ndim):
    a = np.asarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise OracleInputError(f"{name}: expected bf16 bits as uint16, got {a.dtype}")
    if a.ndim != ndim:
        raise OracleInputError(f"{name}: expected {ndim} dims, got shape {a.shape}")
    return a


def validate_paged_batch(q, k_pool, v_pool, page_table, seq_lens, prefix_lens,
                         extend_lens, page_size):
    """Check shapes and metadata; return (B, T, Hq, Hkv, D, G, num_pages) or raise."""
    q = _as_u16("q", q, 3)
    k_pool = _as_u16("k_pool", k_pool, 3)
    v_pool = _as_u16("v_pool", v_pool, 3)
    if k_pool.shape != v_pool.shape:
        raise OracleInputError("k_pool and v_pool shapes differ")
    num_slots, hkv, d = k_pool.shape
    t_rows, hq, dq = q.shape
    if dq != d:
        raise OracleInputError("q and pool head_dim differ")
    if hkv < 1 or hq % hkv != 0:
        raise OracleInputError("num_q_heads must be a positive multiple of num_kv_heads")
    if page_size < 1 or num_slots % page_size != 0:
        raise OracleInputError("pool slots must be a whole number of pages")
    num_pages = num_slots // page_size
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    extend_lens = np.asarray(extend_lens, dtype=np.int64)
    page_table = np.asarray(page_table)
    b = seq_lens.shape[0]
    if prefix_lens.shape != (b,) or extend_lens.shape != (b,):
        raise OracleInputError("seq/prefix/extend lens must all have shape [B]")
    if page_table.ndim != 2 or page_table.shape[0] != b:
        raise OracleInputError("page_table must be [B, W]")
    if np.any(prefix_lens < 0) or np.any(extend_lens < 0):
        raise OracleInputError("negative prefix or extend length")
    if np.any(seq_lens != prefix_lens + extend_lens):
        raise OracleInputError("seq_len must equal prefix_len + extend_len")
    if int(extend_lens.sum()) != t_rows:
        raise OracleInputError("q rows must equal the sum of extend lens")
    width = page_table.shape[1]
    for r in range(b):
        pages_needed = -(-int(seq_lens[r]) // page_size)
        if pages_needed > width:
            raise OracleInputError(f"request {r}: page table row too short")
        ids = page_table[r, :pages_needed]
        if np.any(ids < 0) or np.any(ids >= num_pages):
            raise OracleInputError(f"request {r}: page id out of range")
    return b, t_rows, hq, hkv, d, hq // hkv, num_pages


def validate_out_loc(out_loc, num_slots, page_table, seq_lens, prefix_lens, extend_lens,
                     page_size):
    """out_loc must name, in order, the slots of every new token, all distinct, and
    no new token's slot may be read by another request (new slots are private)."""
    out_loc = np.asarray(out_loc, dtype=np.int64)
    if out_loc.ndim != 1:
        raise OracleInputError("out_loc must be 1-D")
    if np.any(out_loc < 0) or np.any(out_loc >= num_slots):
        raise OracleInputError("out_loc slot out of range")
    if np.unique(out_loc).size != out_loc.size:
        raise OracleInputError("duplicate slot in out_loc")
    if page_table is None:
        return
    t = 0
    owner = {}
    for r in range(len(seq_lens)):
        p, e = int(prefix_lens[r]), int(extend_lens[r])
        for i in range(e):
            want = slot_of(page_table[r], p + i, page_size)
            if int(out_loc[t]) != want:
                raise OracleInputError(f"out_loc[{t}] does not match request {r} token {p+i}")
            owner[want] = r
            t += 1
    if t != out_loc.size:
        raise OracleInputError("out_loc length must equal the sum of extend lens")
    for r in range(len(seq_lens)):
        for s in request_slots(page_table[r], int(seq_lens[r]), page_size):
            if int(s) in owner and owner[int(s)] != r:
                raise OracleInputError(f"request {r} reads a slot written for request "
                                       f"{owner[int(s)]}")


# --- store --------------------------------------------------------------------------


def store_kv_ref(k_pool, v_pool, k_new, v_new, out_loc):
    """Write new K/V rows into the pools: pool[out_loc[t]] = new[t] (bit copies).

    Returns new (k_pool, v_pool) arrays; the inputs are not modified.
    """
    k_pool = _as_u16("k_pool", k_pool, 3)
    v_pool = _as_u16("v_pool", v_pool, 3)
    k_new = _as_u16("k_new", k_new, 3)
    v_new = _as_u16("v_new", v_new, 3)
    if k_new.shape != v_new.shape or k_new.shape[1:] != k_pool.shape[1:]:
        raise OracleInputError("new K/V rows must be [T, Hkv, D] matching the pool")
    validate_out_loc(out_loc, k_pool.shape[0], None, None, None, None, 1)
    out_loc = np.asarray(out_loc, dtype=np.int64)
    if out_loc.size != k_new.shape[0]:
        raise OracleInputError("out_loc length must equal the number of new rows")
    k2 = k_pool.copy()
    v2 = v_pool.copy()
    for t in range(out_loc.size):
        k2[out_loc[t]] = k_new[t]
        v2[out_loc[t]] = v_new[t]
    return k2, v2


# --- attention ----------------------------------------------------------------------


def paged_attention_ref(q, k_pool, v_pool, page_table, seq_lens, prefix_lens, extend_lens,
                        page_size, scale):
    """Causal extend attention of every new token over its request's pool keys.

    For new token i of request b (row t), q head h, kv head g = h // G:
        s_j  = scale * sum_d q[t,h,d] * K_b[j,g,d]      for j = 0 .. p_b + i
        out  = sum_j exp(s_j - max s) V_b[j,g,:] / sum_j exp(s_j - max s)
    where K_b[j] = k_pool[slot of token j of request b] (likewise V_b).
    Keys are gathered one request and one kv head at a time, so a pool is never
    upcast whole. Rows are independent; they are processed in blocks only to
    bound memory, which changes no arithmetic.
    """
    b_count, t_rows, hq, hkv, d, group, _ = validate_paged_batch(
        q, k_pool, v_pool, page_table, seq_lens, prefix_lens, extend_lens, page_size)
    q = _as_u16("q", q, 3)
    k_pool = _as_u16("k_pool", k_pool, 3)
    v_pool = _as_u16("v_pool", v_pool, 3)
    page_table = np.asarray(page_table)
    out = np.empty((t_rows, hq, d), dtype=np.float64)
    row0 = 0
    for b in range(b_count):
        L = int(seq_lens[b])
        p = int(prefix_lens[b])
        e = int(extend_lens[b])
        if e == 0:
            continue
        slots = request_slots(page_table[b], L, page_size)
        for g in range(hkv):
            k_b = bf16_bits_to_f64(k_pool[slots, g, :])          # [L, D]
            v_b = bf16_bits_to_f64(v_pool[slots, g, :])          # [L, D]
            heads = [h for h in range(hq) if kv_head_of(h, group) == g]
            for i0 in range(0, e, 1024):
                i1 = min(e, i0 + 1024)
                # key j is visible to new token i iff j <= last_visible_key(p, i)
                limit = np.array([last_visible_key(p, i) for i in range(i0, i1)])
                visible = np.arange(L)[None, :] <= limit[:, None]       # [rows, L]
                for h in heads:
                    q_rows = bf16_bits_to_f64(q[row0 + i0: row0 + i1, h, :])   # [rows, D]
                    s = scale * (q_rows @ k_b.T)                                 # [rows, L]
                    s = np.where(visible, s, -np.inf)
                    m = s.max(axis=1, keepdims=True)
                    w = np.exp(s - m)                                            # 0 where masked
                    out[row0 + i0: row0 + i1, h, :] = (w @ v_b) / w.sum(axis=1, keepdims=True)
        row0 += e
    return out


def decode_ref(q, k_pool, v_pool, page_table, seq_lens, page_size, scale):
    """Batched decode: one new token per request, already stored at position L_b - 1.

    q is [B, Hq, D]; seq_lens[b] >= 1 counts the new token. Returns [B, Hq, D] f64.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    if np.any(seq_lens < 1):
        raise OracleInputError("decode needs seq_len >= 1 (the new token is stored first)")
    ones = np.ones_like(seq_lens)
    return paged_attention_ref(q, k_pool, v_pool, page_table, seq_lens, seq_lens - 1, ones,
                               page_size, scale)
