"""Seeded synthetic inputs for paged KV-cache attention.

This module only *generates inputs*: lengths, page assignments, page tables,
the slots of new tokens, and bf16 values. It contains none of the attention
arithmetic and no slot-translation formula: the slots of a request are
enumerated page by page (page id p owns slots p*P .. p*P+P-1), and new tokens
take the slots that follow the request's prefix in that enumeration.

Randomness:
  * metadata (lengths, page permutation) comes from ``numpy.random.default_rng(seed)``
    in a fixed draw order: lengths, then pages;
  * bulk values (q, pool K, pool V, new K, new V, in that order) come from a
    ``torch.Generator`` on the target device seeded with ``seed``; float32 N(0,1)
    draws are rounded to bf16 (round-to-nearest-even) and carried as int16 bits.
Unreferenced pool slots, and the slots of new tokens before ``store_kv`` runs,
hold a fill pattern: bf16 NaN (0x7FC0) for correctness runs, zero for timing.

Workloads (head shapes are the Qwen3 models named by the pages' benchmarks:
0.6B and 14B offline on one GPU, 32B with 4-way tensor parallelism online; see
"Mini-SGLang deployment guide" section 9 and "Mini-SGLang: Efficient Inference
Engine in a Nutshell", experiment setup):
  tiny_decode        16q/8kv, B=4, L={17,64,100,250}, P=1, 1024-slot pool
  decode_b256        16q/8kv, B=256, L~U[200,2048], P=1, 2^20-slot pool
  chunked_prefill    40q/8kv, 32 requests, prefix~U[0,4096], extend lens a random
                     composition of 8192, P=16, pages permuted in a 2x pool
  tp4_mixed          16q/2kv, 128 decode seqs (L = clip(round(2048 e^Z),1,8192))
                     plus one 8192-token chunk on a 1024-token prefix, P=1, 2^20 slots
  long_decode        40q/8kv, B=32, L=32768, P=64, 16384 pages permuted
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

NAN_BF16 = 0x7FC0
HEAD_DIM = 128


@dataclass
class AttnPart:
    """Metadata and queries of one attention call (decode or prefill)."""
    kind: str                      # "decode" or "prefill"
    seq_lens: np.ndarray           # int32 [B]
    prefix_lens: np.ndarray        # int32 [B]
    extend_lens: np.ndarray        # int32 [B]
    cu_extend: np.ndarray          # int32 [B+1], exclusive prefix sums of extend_lens
    page_table: np.ndarray         # int32 [B, W]
    q: torch.Tensor                # int16 bf16 bits [T, Hq, D]
    row_offset: int                # first row of this part in the step's new-token arrays

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.extend_lens.sum())

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.batch else 0

    @property
    def max_extend(self) -> int:
        return int(self.extend_lens.max()) if self.batch else 0


@dataclass
class Step:
    """One step's worth of inputs: a pool, the new tokens to store, attention calls."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    k_pool: torch.Tensor           # int16 [num_pages*P, Hkv, D]
    v_pool: torch.Tensor
    k_new: torch.Tensor            # int16 [T_all, Hkv, D]
    v_new: torch.Tensor
    out_loc: np.ndarray            # int32 [T_all]
    parts: List[AttnPart] = field(default_factory=list)
    scale: float = HEAD_DIM ** -0.5

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.page_size


def _bf16_normal(gen: torch.Generator, shape, device) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16).view(torch.int16)


def _enumerate_slots(pages: np.ndarray, page_size: int, count: int) -> np.ndarray:
    """The first `count` slots owned by `pages`, page by page, offsets in order."""
    owned = (pages.astype(np.int64)[:, None] * page_size
             + np.arange(page_size, dtype=np.int64)[None, :]).reshape(-1)
    return owned[:count]


def build_step(name, num_q_heads, num_kv_heads, page_size, num_pages, parts_spec, seed,
               device="cpu", fill="nan", head_dim=HEAD_DIM, permute_pages=True,
               scale=None) -> Step:
    """Build a step from per-part lengths.

    parts_spec: list of (kind, prefix_lens, extend_lens) with integer sequences.
    Every request gets private pages drawn without replacement from the pool
    (a random permutation of all page ids if permute_pages, else ascending ids).
    """
    rng = np.random.default_rng(seed)
    per_part = []
    total_pages = 0
    for kind, prefix, extend in parts_spec:
        prefix = np.asarray(prefix, dtype=np.int64)
        extend = np.asarray(extend, dtype=np.int64)
        seq = prefix + extend
        need = -(-seq // page_size)
        per_part.append((kind, prefix, extend, seq, need))
        total_pages += int(need.sum())
    if total_pages > num_pages:
        raise ValueError(f"{name}: needs {total_pages} pages, pool has {num_pages}")
    order = rng.permutation(num_pages) if permute_pages else np.arange(num_pages)
    spare = order[total_pages:]
    pad_page = int(spare[0]) if spare.size else 0   # never referenced when spare exists

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    slots_total = num_pages * page_size
    fill_bits = NAN_BF16 if fill == "nan" else 0

    parts = []
    prefix_slots_all = []
    new_slots_all = []
    cursor = 0
    row = 0
    for kind, prefix, extend, seq, need in per_part:
        bsz = seq.shape[0]
        width = max(1, int(need.max()) if bsz else 1)
        table = np.full((bsz, width), pad_page, dtype=np.int32)
        for b in range(bsz):
            pages = order[cursor: cursor + int(need[b])]
            cursor += int(need[b])
            table[b, : pages.size] = pages
            slots = _enumerate_slots(pages, page_size, int(seq[b]))
            prefix_slots_all.append(slots[: int(prefix[b])])
            new_slots_all.append(slots[int(prefix[b]):])
        cu = np.zeros(bsz + 1, dtype=np.int32)
        cu[1:] = np.cumsum(extend)
        parts.append(AttnPart(kind=kind, seq_lens=seq.astype(np.int32),
                              prefix_lens=prefix.astype(np.int32),
                              extend_lens=extend.astype(np.int32), cu_extend=cu,
                              page_table=table, q=None, row_offset=row))
        row += int(extend.sum())

    prefix_slots = (np.concatenate(prefix_slots_all) if prefix_slots_all
                    else np.zeros(0, np.int64))
    out_loc = (np.concatenate(new_slots_all) if new_slots_all
               else np.zeros(0, np.int64)).astype(np.int32)

    # bulk values, fixed order: q (per part), pool K, pool V, new K, new V
    for part in parts:
        part.q = _bf16_normal(gen, (part.num_tokens, num_q_heads, head_dim), device)
    k_pool = torch.full((slots_total, num_kv_heads, head_dim), fill_bits, dtype=torch.int16,
                        device=device)
    v_pool = torch.full_like(k_pool, fill_bits)
    idx = torch.from_numpy(prefix_slots).to(device)
    n_pre = int(prefix_slots.size)
    k_pool.index_copy_(0, idx, _bf16_normal(gen, (n_pre, num_kv_heads, head_dim), device))
    v_pool.index_copy_(0, idx, _bf16_normal(gen, (n_pre, num_kv_heads, head_dim), device))
    k_new = _bf16_normal(gen, (out_loc.size, num_kv_heads, head_dim), device)
    v_new = _bf16_normal(gen, (out_loc.size, num_kv_heads, head_dim), device)
    return Step(name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                head_dim=head_dim, page_size=page_size, num_pages=num_pages,
                k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new, out_loc=out_loc,
                parts=parts, scale=head_dim ** -0.5 if scale is None else scale)


def decode_spec(seq_lens):
    seq = np.asarray(seq_lens, dtype=np.int64)
    return ("decode", seq - 1, np.ones_like(seq))


def random_composition(rng, total, parts):
    """`parts` positive integers summing to `total` (distinct random cut points)."""
    cuts = np.sort(rng.choice(np.arange(1, total), size=parts - 1, replace=False))
    edges = np.concatenate([[0], cuts, [total]])
    return np.diff(edges)


# --- the five workloads ---------------------------------------------------------------

def tiny_decode(seed=1, device="cpu", fill="nan"):
    return build_step("tiny_decode", 16, 8, 1, 1024, [decode_spec([17, 64, 100, 250])],
                      seed, device, fill)


def decode_b256(seed=2, device="cpu", fill="nan", batch=256, page_size=1):
    """page_size other than 1: the same requests in a pool of 2^20 slots cut into pages
    of that size, pages drawn at random."""
    rng = np.random.default_rng(seed + 1000)
    seq = rng.integers(200, 2048, size=batch, endpoint=True)
    return build_step("decode_b256", 16, 8, page_size, (1 << 20) // page_size,
                      [decode_spec(seq)], seed, device, fill)


def chunked_prefill(seed=3, device="cpu", fill="nan", requests=32, total_extend=8192,
                    max_prefix=4096, page_size=16):
    rng = np.random.default_rng(seed + 1000)
    prefix = rng.integers(0, max_prefix, size=requests, endpoint=True)
    extend = random_composition(rng, total_extend, requests)
    seq = prefix + extend
    pages_needed = int((-(-seq // page_size)).sum())
    return build_step("chunked_prefill", 40, 8, page_size, 2 * pages_needed,
                      [("prefill", prefix, extend)], seed, device, fill)


def lognormal_lens(rng, count, median=2048, sigma=1.0, cap=8192):
    z = rng.standard_normal(count)
    return np.clip(np.rint(median * np.exp(sigma * z)), 1, cap).astype(np.int64)


def tp4_mixed(seed=4, device="cpu", fill="nan", decode_batch=128, chunk=8192, prefix=1024):
    rng = np.random.default_rng(seed + 1000)
    seq = lognormal_lens(rng, decode_batch)
    return build_step("tp4_mixed", 16, 2, 1, 1 << 20,
                      [decode_spec(seq), ("prefill", [prefix], [chunk])], seed, device, fill)


def long_decode(seed=5, device="cpu", fill="nan", batch=32, ctx=32768):
    return build_step("long_decode", 40, 8, 64, 16384, [decode_spec([ctx] * batch)], seed,
                      device, fill)


WORKLOADS = {
    "tiny_decode": tiny_decode,
    "decode_b256": decode_b256,
    "chunked_prefill": chunked_prefill,
    "tp4_mixed": tp4_mixed,
    "long_decode": long_decode,
}


def gather_request_rows(pool: torch.Tensor, table_row: np.ndarray, page_size: int,
                        seq_len: int) -> torch.Tensor:
    """Copy one request's pool rows (slots enumerated page by page) - a convenience
    for handing a sample of a large on-device pool to a host-side checker."""
    pages = np.asarray(table_row[: -(-seq_len // page_size)], dtype=np.int64)
    slots = torch.from_numpy(_enumerate_slots(pages, page_size, seq_len)).to(pool.device)
    return pool.index_select(0, slots)
