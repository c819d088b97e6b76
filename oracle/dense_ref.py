"""Brute-force dense masked softmax attention in pure Python (tiny inputs only).

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is the pin for ``paged_ref``: it never sees a pool, a page table or a
slot. It takes the logical (already ordered) keys and values of one sequence,
an explicit boolean mask matrix and an explicit q-head -> kv-head list, and
evaluates softmax(scale * q.k) . v with Python floats and loops, one score at a
time. It shares no arithmetic with ``paged_ref`` (no numpy matmul, no
vectorised masking), so a dropped term, a wrong index or a transposed operand in
either one shows up as a disagreement.
"""
from __future__ import annotations

import math


def causal_extend_mask(prefix_len: int, extend_len: int):
    """Explicit mask for extend rows over prefix+extend keys, written as a matrix.

    Row i is the i-th new token; it sits at absolute position prefix_len + i, so
    columns 0 .. prefix_len + i are True and the rest False (bottom-right causal
    alignment; see the reading in ``paged_ref``).
    """
    n_keys = prefix_len + extend_len
    mask = []
    for i in range(extend_len):
        row = [False] * n_keys
        for j in range(prefix_len + i + 1):
            row[j] = True
        mask.append(row)
    return mask


def dense_attention_bruteforce(q, k, v, mask, scale, kv_head_map):
    """out[r][h][:] = sum_j w_j v[j][g] / sum_j w_j over columns j with mask[r][j].

    q: [R][Hq][D] floats; k, v: [N][Hkv][D] floats; mask: [R][N] bools;
    kv_head_map: list, kv_head_map[h] = kv head read by q head h.
    Returns nested lists [R][Hq][D] of floats. Rows with no visible key raise.
    """
    rows = len(q)
    hq = len(q[0]) if rows else 0
    d = len(q[0][0]) if rows else 0
    out = []
    for r in range(rows):
        out_r = []
        for h in range(hq):
            g = kv_head_map[h]
            cols = [j for j in range(len(k)) if mask[r][j]]
            if not cols:
                raise ValueError(f"row {r} sees no key")
            scores = []
            for j in cols:
                acc = 0.0
                for x in range(d):
                    acc += float(q[r][h][x]) * float(k[j][g][x])
                scores.append(scale * acc)
            top = max(scores)
            weights = [math.exp(s - top) for s in scores]
            total = sum(weights)
            vec = []
            for x in range(d):
                acc = 0.0
                for w, j in zip(weights, cols):
                    acc += w * float(v[j][g][x])
                vec.append(acc / total)
            out_r.append(vec)
        out.append(out_r)
    return out
