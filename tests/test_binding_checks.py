"""CPU tests of the binding's host-side checks.

Every call checks dtypes, contiguity, the shape relations between its tensors and
that all of them sit on one GPU before anything reaches the library; a mismatch
raises ValueError. With debug mode on it also checks the device metadata on the host
(checks.py) and raises MetadataError. Nothing here reaches a kernel launch: the
tensors are CPU tensors, so a call that passes every shape check still stops at the
device check.
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_25_amd as pka
from paged_kv_attention_25_amd import checks

HQ, HKV, D, P = 16, 2, 128, 4


def bf16(*shape):
    return torch.zeros(*shape, dtype=torch.int16)


def i32(*shape):
    return torch.zeros(*shape, dtype=torch.int32)


def pools(slots=64):
    return bf16(slots, HKV, D), bf16(slots, HKV, D)


def decode_args(B=3, W=5):
    k, v = pools()
    return dict(q=bf16(B, HQ, D), k_pool=k, v_pool=v, page_table=i32(B, W), seq_lens=i32(B),
                max_seq_len=20, page_size=P, scale=0.1)


def prefill_args(B=2, T=7, W=5):
    k, v = pools()
    return dict(q=bf16(T, HQ, D), k_pool=k, v_pool=v, page_table=i32(B, W), seq_lens=i32(B),
                prefix_lens=i32(B), extend_lens=i32(B), cu_extend=i32(B + 1), max_extend=4,
                max_seq_len=20, page_size=P, scale=0.1)


def store_args(T=3):
    k, v = pools()
    return dict(k_new=bf16(T, HKV, D), v_new=bf16(T, HKV, D), out_loc=i32(T), k_pool=k,
                v_pool=v, page_size=P)


def decode_store_args(B=3):
    a = decode_args(B)
    a.update(k_new=bf16(B, HKV, D), v_new=bf16(B, HKV, D), out_loc=i32(B))
    return a


def expect(fn, args, match):
    with pytest.raises(ValueError, match=match):
        fn(**args)


# --- every well-formed call stops at the device check on the CPU ---------------------------

@pytest.mark.parametrize("fn,make", [
    (pka.store_kv, store_args), (pka.paged_attn_decode, decode_args),
    (pka.paged_attn_decode_store, decode_store_args), (pka.paged_attn_prefill, prefill_args)])
def test_cpu_tensors_are_rejected(fn, make):
    expect(fn, make(), "on the GPU")


# --- dtype, contiguity and shape relations -------------------------------------------------

def test_store_kv_rejections():
    a = store_args()
    expect(pka.store_kv, {**a, "out_loc": torch.zeros(3, dtype=torch.int64)}, "out_loc must be int32")
    expect(pka.store_kv, {**a, "k_new": torch.zeros(3, HKV, D)}, "k_new must hold bf16")
    expect(pka.store_kv, {**a, "v_new": bf16(2, HKV, D)}, r"v_new has shape \[2, 2, 128\]")
    expect(pka.store_kv, {**a, "k_new": bf16(3, HKV + 1, D)}, "k_new has shape")
    expect(pka.store_kv, {**a, "v_pool": bf16(32, HKV, D)}, "v_pool has shape")
    expect(pka.store_kv, {**a, "k_pool": bf16(62, HKV, D), "v_pool": bf16(62, HKV, D)},
           "whole number")
    expect(pka.store_kv, {**a, "page_size": 0}, "page_size must be >= 1")
    expect(pka.store_kv, {**a, "k_new": bf16(HKV, 3, D).transpose(0, 1)}, "contiguous")
    expect(pka.store_kv, {**a, "out_loc": [0, 1, 2]}, "torch.Tensor")


def test_decode_rejections():
    a = decode_args()
    expect(pka.paged_attn_decode, {**a, "q": bf16(3, 15, D)}, "not a multiple")
    expect(pka.paged_attn_decode, {**a, "q": bf16(3, HQ, 64)}, "q has shape")
    expect(pka.paged_attn_decode, {**a, "seq_lens": i32(4)}, r"seq_lens has shape \[4\]")
    expect(pka.paged_attn_decode, {**a, "page_table": i32(2, 5)}, "page_table has shape")
    expect(pka.paged_attn_decode, {**a, "page_table": i32(15)}, "page_table has shape")
    expect(pka.paged_attn_decode, {**a, "seq_lens": torch.zeros(3, dtype=torch.int64)},
           "seq_lens must be int32")
    expect(pka.paged_attn_decode, {**a, "out": bf16(3, HQ, D + 1)}, "out has shape")
    expect(pka.paged_attn_decode, {**a, "out": a["q"]}, "must not alias q")
    expect(pka.paged_attn_decode, {**a, "v_pool": bf16(64, HKV, 64)}, "v_pool has shape")


def test_decode_store_rejections():
    a = decode_store_args()
    expect(pka.paged_attn_decode_store, {**a, "out_loc": i32(2)}, "out_loc has shape")
    expect(pka.paged_attn_decode_store, {**a, "k_new": bf16(3, 1, D)}, "k_new has shape")
    expect(pka.paged_attn_decode_store, {**a, "v_new": torch.zeros(3, HKV, D)},
           "v_new must hold bf16")


def test_prefill_rejections():
    a = prefill_args()
    expect(pka.paged_attn_prefill, {**a, "cu_extend": i32(2)}, r"cu_extend has shape \[2\]")
    expect(pka.paged_attn_prefill, {**a, "prefix_lens": i32(3)}, "prefix_lens has shape")
    expect(pka.paged_attn_prefill, {**a, "extend_lens": i32(1)}, "extend_lens has shape")
    expect(pka.paged_attn_prefill, {**a, "page_table": i32(3, 5)}, "page_table has shape")
    expect(pka.paged_attn_prefill, {**a, "q": bf16(7, 15, D)}, "not a multiple")
    expect(pka.paged_attn_prefill, {**a, "out": bf16(6, HQ, D)}, "out has shape")
    expect(pka.paged_attn_prefill, {**a, "workspace": [0]}, "workspace must be a torch.Tensor")


def misaligned_bf16(*shape, shift=1):
    """A contiguous bf16 view starting `shift` elements (2*shift bytes) into its storage."""
    n = int(np.prod(shape))
    return bf16(n + 8)[shift:shift + n].view(*shape)


def test_misaligned_views_are_rejected():
    a = decode_args()
    expect(pka.paged_attn_decode, {**a, "q": misaligned_bf16(3, HQ, D)}, "16-byte boundary")
    expect(pka.paged_attn_decode, {**a, "q": misaligned_bf16(3, HQ, D, shift=4)},
           "16-byte boundary")
    # 8 elements = 16 bytes in: aligned, so the call goes on to the device check
    expect(pka.paged_attn_decode, {**a, "q": misaligned_bf16(3, HQ, D, shift=8)}, "on the GPU")
    s = store_args()
    expect(pka.store_kv, {**s, "k_new": misaligned_bf16(3, HKV, D)}, "k_new must start")
    p = prefill_args()
    ws = torch.zeros(1 << 12, dtype=torch.uint8)[3:]
    expect(pka.paged_attn_prefill, {**p, "workspace": ws}, "workspace must start")


# --- debug-mode metadata checks (checks.py) ------------------------------------------------

def test_out_loc_checks():
    checks.check_out_loc(np.array([3, 0, 7]), 8)
    with pytest.raises(checks.MetadataError, match="outside the pool"):
        checks.check_out_loc(np.array([3, 8]), 8)
    with pytest.raises(checks.MetadataError, match="outside the pool"):
        checks.check_out_loc(np.array([-1]), 8)
    with pytest.raises(checks.MetadataError, match="slot 5 appears 2 times"):
        checks.check_out_loc(np.array([5, 1, 5]), 8)


def test_page_table_checks():
    pt = np.array([[3, 1, 0], [2, 9, 9]], np.int32)   # request 1 reads one entry only
    checks.check_page_table(pt, np.array([9, 4]), 4, 4)
    with pytest.raises(checks.MetadataError, match=r"page_table\[1, 1\] = 9"):
        checks.check_page_table(pt, np.array([9, 5]), 4, 4)
    with pytest.raises(checks.MetadataError, match="needs 4 page-table entries"):
        checks.check_page_table(pt, np.array([13, 1]), 4, 4)
    with pytest.raises(checks.MetadataError, match="is not a page"):
        checks.check_page_table(np.array([[-1]], np.int32), np.array([1]), 4, 4)


def test_decode_checks():
    pt = np.array([[0, 1], [2, 3]], np.int32)
    checks.check_decode(np.array([5, 8]), 8, pt, 4, 4)
    with pytest.raises(checks.MetadataError, match="outside \\[1, max_seq_len"):
        checks.check_decode(np.array([5, 9]), 8, pt, 4, 4)
    with pytest.raises(checks.MetadataError, match="outside \\[1, max_seq_len"):
        checks.check_decode(np.array([0, 8]), 8, pt, 4, 4)


def test_decode_store_privacy():
    # requests 0 and 1 share page 0 (a read-only prefix); their new tokens sit in their
    # own pages
    pt = np.array([[0, 1], [0, 2]], np.int32)
    seq = np.array([6, 7])
    ok = np.array([1 * 4 + 1, 2 * 4 + 2])             # key L-1 of each request
    checks.check_decode_store(ok, seq, 8, pt, 4, 3)
    with pytest.raises(checks.MetadataError, match="read as a key by request 1"):
        checks.check_decode_store(np.array([2, 10]), seq, 8, pt, 4, 3)   # slot 2: shared page
    with pytest.raises(checks.MetadataError, match="appears 2 times"):
        checks.check_decode_store(np.array([5, 5]), seq, 8, pt, 4, 3)


def test_prefill_checks():
    pt = np.array([[0, 1], [2, 3]], np.int32)
    good = dict(seq_lens=np.array([6, 3]), prefix_lens=np.array([2, 0]),
                extend_lens=np.array([4, 3]), cu_extend=np.array([0, 4, 7]), num_tokens=7,
                max_extend=4, max_seq_len=8, page_table=pt, page_size=4, num_pages=4)
    checks.check_prefill(**good)
    cases = [
        (dict(seq_lens=np.array([7, 3])), "!= prefix 2 \\+ extend 4"),
        (dict(max_extend=3), "exceeds max_extend"),
        (dict(max_seq_len=5), "exceeds max_seq_len"),
        (dict(cu_extend=np.array([0, 4, 6])), "exclusive prefix sum"),
        (dict(num_tokens=8), "q has 8 rows"),
        (dict(prefix_lens=np.array([-1, 0]), seq_lens=np.array([3, 3])), ">= 0"),
        (dict(page_table=np.array([[0, 4], [2, 3]], np.int32)), "is not a page"),
    ]
    for change, match in cases:
        with pytest.raises(checks.MetadataError, match=match):
            checks.check_prefill(**{**good, **change})


def test_debug_mode_routes_calls_through_the_checks(monkeypatch):
    """With debug mode on, a call's metadata is checked on the host before the device
    check (the tensors here are on the CPU: without debug mode every call below stops at
    the device check instead)."""
    monkeypatch.setattr(pka, "_debug", True)
    a = decode_store_args(B=2)
    a["seq_lens"] = torch.tensor([3, 0], dtype=torch.int32)
    with pytest.raises(checks.MetadataError, match="outside \\[1, max_seq_len"):
        pka.paged_attn_decode_store(**a)
    a["seq_lens"] = torch.tensor([3, 2], dtype=torch.int32)
    a["out_loc"] = torch.tensor([4, 4], dtype=torch.int32)
    with pytest.raises(checks.MetadataError, match="appears 2 times"):
        pka.paged_attn_decode_store(**a)
    a = decode_args(B=2)
    a["seq_lens"] = torch.tensor([21, 1], dtype=torch.int32)
    with pytest.raises(checks.MetadataError, match="max_seq_len"):
        pka.paged_attn_decode(**a)
    a = prefill_args(B=2, T=7)
    a.update(seq_lens=torch.tensor([6, 3], dtype=torch.int32),
             prefix_lens=torch.tensor([2, 0], dtype=torch.int32),
             extend_lens=torch.tensor([4, 3], dtype=torch.int32),
             cu_extend=torch.tensor([0, 4, 7], dtype=torch.int32), max_extend=3)
    with pytest.raises(checks.MetadataError, match="exceeds max_extend"):
        pka.paged_attn_prefill(**a)
    a = store_args(T=2)
    a["out_loc"] = torch.tensor([1, 64], dtype=torch.int32)
    with pytest.raises(checks.MetadataError, match="outside the pool"):
        pka.store_kv(**a)
    # well-formed metadata passes the checks and stops at the device check
    a["out_loc"] = torch.tensor([1, 63], dtype=torch.int32)
    expect(pka.store_kv, a, "on the GPU")
    pka.set_debug(False)
    assert not pka.debug_enabled()
