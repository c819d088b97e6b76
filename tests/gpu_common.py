"""Helpers for the GPU parity tests: run the HIP path through the C ABI, run the
oracle on host copies of the *inputs* (never on anything the HIP path produced),
and compare.
"""
import numpy as np
import torch

import oracle
import paged_kv_attention_25_amd as pka

# Attention parity bar for bf16 inputs (f32 accumulation on the GPU vs f64 oracle).
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host_u16(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint16)


def gpu_store(step):
    pka.store_kv(step.k_new, step.v_new, dev_i32(step.out_loc), step.k_pool, step.v_pool,
                 step.page_size)


def gpu_part(step, part, max_seq_len=None):
    pt = dev_i32(part.page_table)
    seq = dev_i32(part.seq_lens)
    msl = part.max_seq_len if max_seq_len is None else max_seq_len
    if part.kind == "decode":
        return pka.paged_attn_decode(part.q, step.k_pool, step.v_pool, pt, seq, msl,
                                     step.page_size, step.scale)
    return pka.paged_attn_prefill(part.q, step.k_pool, step.v_pool, pt, seq,
                                  dev_i32(part.prefix_lens), dev_i32(part.extend_lens),
                                  dev_i32(part.cu_extend), part.max_extend, msl,
                                  step.page_size, step.scale)


def gpu_decode_store(step, part, max_seq_len=None, out_loc=None):
    """The fused entry: store the part's new rows and decode in one launch."""
    r0, r1 = part.row_offset, part.row_offset + part.batch
    loc = step.out_loc[r0:r1] if out_loc is None else out_loc
    msl = part.max_seq_len if max_seq_len is None else max_seq_len
    return pka.paged_attn_decode_store(part.q, step.k_new[r0:r1], step.v_new[r0:r1],
                                       dev_i32(loc), step.k_pool, step.v_pool,
                                       dev_i32(part.page_table), dev_i32(part.seq_lens), msl,
                                       step.page_size, step.scale)


class HostInputs:
    """Host copies of a step's inputs, taken before any kernel runs, and the oracle's
    own store of the new rows into its copy of the pools."""

    def __init__(self, step):
        self.k_pool0 = host_u16(step.k_pool)
        self.v_pool0 = host_u16(step.v_pool)
        self.k_new = host_u16(step.k_new)
        self.v_new = host_u16(step.v_new)
        self.out_loc = step.out_loc.copy()
        self.q = [host_u16(p.q) for p in step.parts]
        self.k_pool, self.v_pool = oracle.store_kv_ref(self.k_pool0, self.v_pool0, self.k_new,
                                                       self.v_new, self.out_loc)


def oracle_decode(step, host, part_idx, requests=None):
    part = step.parts[part_idx]
    idx = np.arange(part.batch) if requests is None else np.asarray(requests)
    return oracle.decode_ref(host.q[part_idx][idx], host.k_pool, host.v_pool,
                             part.page_table[idx], part.seq_lens[idx], step.page_size,
                             step.scale), idx


def prefill_windows(part, windows):
    """windows: list of (request, first_token, end_token). Each window is the exact
    sub-problem prefix' = p + first, extend' = end - first on the same page-table row
    (rows of a token depend only on keys up to its position)."""
    q_rows, pre, ext, rows = [], [], [], []
    for b, a, c in windows:
        base = int(part.cu_extend[b])
        rows.append(np.arange(base + a, base + c))
        pre.append(int(part.prefix_lens[b]) + a)
        ext.append(c - a)
    bidx = np.array([w[0] for w in windows])
    return np.concatenate(rows), bidx, np.array(pre), np.array(ext)


def oracle_prefill(step, host, part_idx, windows):
    part = step.parts[part_idx]
    rows, bidx, pre, ext = prefill_windows(part, windows)
    out = oracle.paged_attention_ref(host.q[part_idx][rows], host.k_pool, host.v_pool,
                                     part.page_table[bidx], pre + ext, pre, ext,
                                     step.page_size, step.scale)
    return out, rows


def assert_close(got_bits, ref, what, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    got = oracle.bf16_bits_to_f64(got_bits)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    print(f"[gpu-case] {what}: max abs {mx:.3e}, mean abs {mean:.3e}", flush=True)
    assert mx <= max_abs and mean <= mean_abs, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean
