"""Tiny seeded cases for the oracle's CPU pins (numpy only, no GPU, no torch)."""
import numpy as np


def rand_bf16(rng, shape, scale=1.0):
    """Random valid bf16 bit patterns (float32 N(0, scale^2) draws, low half dropped)."""
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def layout_case(rng, logical_k, logical_v, page_size, num_pages=None, permute=True,
                fill=0x7FC0):
    """Lay logical per-request K/V ([L_b, Hkv, D] uint16 each) out in a paged pool.

    Pages are assigned page by page from a (optionally permuted) list of page ids;
    slots of a page are enumerated in order. Unused slots hold `fill` (bf16 NaN).
    Returns (k_pool, v_pool, page_table).
    """
    hkv, d = logical_k[0].shape[1:]
    need = [-(-k.shape[0] // page_size) for k in logical_k]
    if num_pages is None:
        num_pages = sum(need) + 3
    order = rng.permutation(num_pages) if permute else np.arange(num_pages)
    width = max(max(need), 1)
    table = np.zeros((len(logical_k), width), dtype=np.int32)
    k_pool = np.full((num_pages * page_size, hkv, d), fill, dtype=np.uint16)
    v_pool = np.full_like(k_pool, fill)
    cursor = 0
    for b, (kb, vb) in enumerate(zip(logical_k, logical_v)):
        pages = order[cursor: cursor + need[b]]
        cursor += need[b]
        table[b, : len(pages)] = pages
        owned = [int(p) * page_size + o for p in pages for o in range(page_size)]
        for j in range(kb.shape[0]):
            k_pool[owned[j]] = kb[j]
            v_pool[owned[j]] = vb[j]
    return k_pool, v_pool, table


def random_case(rng, hq, hkv, d, prefix_lens, extend_lens, page_size, permute=True):
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    extend_lens = np.asarray(extend_lens, dtype=np.int64)
    seq = prefix_lens + extend_lens
    logical_k = [rand_bf16(rng, (int(L), hkv, d)) for L in seq]
    logical_v = [rand_bf16(rng, (int(L), hkv, d)) for L in seq]
    q = rand_bf16(rng, (int(extend_lens.sum()), hq, d))
    k_pool, v_pool, table = layout_case(rng, logical_k, logical_v, page_size, permute=permute)
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, page_table=table, seq_lens=seq,
                prefix_lens=prefix_lens, extend_lens=extend_lens, page_size=page_size,
                logical_k=logical_k, logical_v=logical_v, hq=hq, hkv=hkv, d=d)


def oracle_args(case, scale):
    return (case["q"], case["k_pool"], case["v_pool"], case["page_table"], case["seq_lens"],
            case["prefix_lens"], case["extend_lens"], case["page_size"], scale)
