"""Host-side checks of the device metadata, for the binding's debug mode.

The kernels never read device metadata on the host, so a mis-built page table, a
duplicated new-token slot or a length past a host-known bound gives wrong results
without an error (the kernels stay in bounds: a page id outside the pool reads slot 0,
keys past max_seq_len are not attended, rows of tokens past max_extend are not
written). With debug mode on (``PKA_DEBUG=1`` in the environment, or
``paged_kv_attention_25_amd.set_debug(True)``) every call first copies its metadata
to the host and checks it here; a violation raises ``MetadataError`` before anything
is launched. This synchronises with the device, so it is for tests and debugging, not
for timed runs.

What is checked follows the rules the path relies on: a pool shared by all requests
whose unit is a page, located through each request's page-table row ("Mini-SGLang
deployment guide", sections 6.2 and 6.5; "miniSGLang intro blog", section 1.3);
requests may share read-only prefix pages (radix reuse), but the slots a step writes
belong to one request and are pairwise distinct.
"""
from __future__ import annotations

import numpy as np


class MetadataError(ValueError):
    """Device metadata that breaks the rules the kernels assume."""


def _np(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.asarray(a)


def check_out_loc(out_loc, num_slots: int) -> np.ndarray:
    """New-token slots: inside the pool and pairwise distinct."""
    loc = _np(out_loc).astype(np.int64).reshape(-1)
    bad = np.flatnonzero((loc < 0) | (loc >= num_slots))
    if bad.size:
        raise MetadataError(f"out_loc[{bad[0]}] = {loc[bad[0]]} is outside the pool "
                            f"[0, {num_slots})")
    uniq, counts = np.unique(loc, return_counts=True)
    if np.any(counts > 1):
        s = int(uniq[np.argmax(counts > 1)])
        raise MetadataError(f"slot {s} appears {int(counts.max())} times in out_loc")
    return loc


def request_slots(page_table: np.ndarray, b: int, length: int, page_size: int) -> np.ndarray:
    """Slots of keys 0 .. length-1 of request b: page_table[b, j // P] * P + j % P."""
    j = np.arange(length, dtype=np.int64)
    return page_table[b, j // page_size].astype(np.int64) * page_size + j % page_size


def check_page_table(page_table, seq_lens, page_size: int, num_pages: int) -> None:
    """Every entry a request reads (the first ceil(L_b / P) of its row) is a page of
    the pool; the row is long enough."""
    pt = _np(page_table)
    seq = _np(seq_lens).astype(np.int64)
    if pt.ndim != 2 or pt.shape[0] != seq.shape[0]:
        raise MetadataError(f"page_table shape {pt.shape} does not match {seq.shape[0]} requests")
    need = -(-seq // page_size)
    if need.size and int(need.max()) > pt.shape[1]:
        b = int(np.argmax(need))
        raise MetadataError(f"request {b} needs {int(need[b])} page-table entries, rows hold "
                            f"{pt.shape[1]}")
    for b in range(seq.shape[0]):
        row = pt[b, : need[b]].astype(np.int64)
        bad = np.flatnonzero((row < 0) | (row >= num_pages))
        if bad.size:
            raise MetadataError(f"page_table[{b}, {bad[0]}] = {row[bad[0]]} is not a page of "
                                f"the pool [0, {num_pages})")


def check_private(out_loc, owners, page_table, seq_lens, page_size: int) -> None:
    """The slot of every new token belongs to its own request only: no other request
    reads it as one of its keys (shared prefix pages are read-only)."""
    loc = _np(out_loc).astype(np.int64).reshape(-1)
    own = np.asarray(owners, dtype=np.int64).reshape(-1)
    pt = _np(page_table)
    seq = _np(seq_lens).astype(np.int64)
    slots, who = [], []
    for b in range(seq.shape[0]):
        s = request_slots(pt, b, int(seq[b]), page_size)
        slots.append(s)
        who.append(np.full(s.shape, b, dtype=np.int64))
    if not slots:
        return
    slots = np.concatenate(slots)
    who = np.concatenate(who)
    order = np.argsort(slots, kind="stable")
    slots, who = slots[order], who[order]
    lo = np.searchsorted(slots, loc, side="left")
    hi = np.searchsorted(slots, loc, side="right")
    for t in range(loc.shape[0]):
        readers = who[lo[t]:hi[t]]
        other = readers[readers != own[t]]
        if other.size:
            raise MetadataError(f"new-token slot {loc[t]} (row {t}, request {own[t]}) is read as "
                                f"a key by request {int(other[0])}")


def check_decode(seq_lens, max_seq_len: int, page_table, page_size: int, num_pages: int) -> None:
    """Decode: 1 <= L_b <= max_seq_len, and the page-table entries read are pool pages."""
    seq = _np(seq_lens).astype(np.int64)
    bad = np.flatnonzero((seq < 1) | (seq > max_seq_len))
    if bad.size:
        raise MetadataError(f"seq_lens[{bad[0]}] = {seq[bad[0]]} is outside [1, max_seq_len = "
                            f"{max_seq_len}]")
    check_page_table(page_table, seq, page_size, num_pages)


def check_decode_store(out_loc, seq_lens, max_seq_len: int, page_table, page_size: int,
                       num_pages: int) -> None:
    """Decode with the store of the new rows: the decode rules, plus distinct in-pool
    new-token slots private to their requests."""
    check_decode(seq_lens, max_seq_len, page_table, page_size, num_pages)
    loc = check_out_loc(out_loc, num_pages * page_size)
    check_private(loc, np.arange(loc.shape[0]), page_table, seq_lens, page_size)


def check_prefill(seq_lens, prefix_lens, extend_lens, cu_extend, num_tokens: int,
                  max_extend: int, max_seq_len: int, page_table, page_size: int,
                  num_pages: int) -> None:
    """Prefill: L_b = p_b + e_b with p_b, e_b >= 0; e_b <= max_extend; L_b <=
    max_seq_len; cu_extend is the exclusive prefix sum of e ending at num_tokens; the
    page-table entries read are pool pages."""
    seq = _np(seq_lens).astype(np.int64)
    pre = _np(prefix_lens).astype(np.int64)
    ext = _np(extend_lens).astype(np.int64)
    cu = _np(cu_extend).astype(np.int64)
    if np.any(pre < 0) or np.any(ext < 0):
        raise MetadataError("prefix_lens and extend_lens must be >= 0")
    bad = np.flatnonzero(seq != pre + ext)
    if bad.size:
        b = bad[0]
        raise MetadataError(f"seq_lens[{b}] = {seq[b]} != prefix {pre[b]} + extend {ext[b]}")
    bad = np.flatnonzero(ext > max_extend)
    if bad.size:
        raise MetadataError(f"extend_lens[{bad[0]}] = {ext[bad[0]]} exceeds max_extend = "
                            f"{max_extend}")
    bad = np.flatnonzero(seq > max_seq_len)
    if bad.size:
        raise MetadataError(f"seq_lens[{bad[0]}] = {seq[bad[0]]} exceeds max_seq_len = "
                            f"{max_seq_len}")
    want = np.concatenate([[0], np.cumsum(ext)])
    if cu.shape != want.shape or np.any(cu != want):
        raise MetadataError("cu_extend is not the exclusive prefix sum of extend_lens")
    if int(want[-1]) != num_tokens:
        raise MetadataError(f"extend_lens sum to {int(want[-1])}, q has {num_tokens} rows")
    check_page_table(page_table, seq, page_size, num_pages)
