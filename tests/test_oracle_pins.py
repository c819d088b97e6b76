"""Pins of the float64 oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a closed form, a textbook library
routine (torch's scaled_dot_product_attention in float64 on the CPU), the
independent pure-Python brute force, a hand-derived worked example under
tests/golden/, or an invariance the definition implies. The last test plants
plausible mistakes in the oracle and checks that these pins catch each one.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import paged_ref
from tests.oracle_cases import layout_case, oracle_args, rand_bf16, random_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f64(x):
    return oracle.bf16_bits_to_f64(x)


def bruteforce_case(case, scale):
    """Dense brute force over each request's logical K/V, rows stacked like q."""
    g = case["hq"] // case["hkv"]
    kv_map = [kv for kv in range(case["hkv"]) for _ in range(g)]   # repeat each kv head G times
    out = []
    row = 0
    for b in range(len(case["seq_lens"])):
        p, e = int(case["prefix_lens"][b]), int(case["extend_lens"][b])
        if e == 0:
            continue
        q_rows = f64(case["q"][row: row + e]).tolist()
        k = f64(case["logical_k"][b]).tolist()
        v = f64(case["logical_v"][b]).tolist()
        out += oracle.dense_attention_bruteforce(q_rows, k, v, oracle.causal_extend_mask(p, e),
                                                 scale, kv_map)
        row += e
    return np.array(out, dtype=np.float64)


# --- the brute force itself, pinned to closed forms and a library routine -----------------

def test_bruteforce_closed_forms():
    # one visible key: output is that key's value row exactly
    out = oracle.dense_attention_bruteforce([[[1.0, -2.0]]], [[[0.5, 3.0]]], [[[7.0, -1.5]]],
                                            [[True]], 0.3, [0])
    assert out == [[[7.0, -1.5]]]
    # two keys with scores 0 and ln 3: weights 1/4 and 3/4
    q = [[[1.0, 0.0]]]
    k = [[[0.0, 5.0]], [[math.log(3.0), 9.0]]]
    v = [[[4.0, 8.0]], [[0.0, -4.0]]]
    out = oracle.dense_attention_bruteforce(q, k, v, [[True, True]], 1.0, [0])
    assert np.allclose(out[0][0], [1.0, -1.0], rtol=0, atol=1e-15)
    # a masked key contributes nothing
    out = oracle.dense_attention_bruteforce(q, k, v, [[True, False]], 1.0, [0])
    assert out[0][0] == [4.0, 8.0]


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (6, 1)])
def test_bruteforce_matches_torch_sdpa_causal(hq, hkv):
    rng = np.random.default_rng(11 + hq)
    n, d = 7, 8
    q = f64(rand_bf16(rng, (n, hq, d)))
    k = f64(rand_bf16(rng, (n, hkv, d)))
    v = f64(rand_bf16(rng, (n, hkv, d)))
    scale = 0.37
    kv_map = [kv for kv in range(hkv) for _ in range(hq // hkv)]
    ours = np.array(oracle.dense_attention_bruteforce(q.tolist(), k.tolist(), v.tolist(),
                                                      oracle.causal_extend_mask(0, n), scale,
                                                      kv_map))
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=True, scale=scale, enable_gqa=(hq != hkv))
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(ours - ref)) < 1e-13


# --- the oracle against the brute force ---------------------------------------------------

CASES = [
    # hq, hkv, prefix_lens, extend_lens, page_size
    (2, 2, [0], [5], 1),
    (4, 2, [3, 0, 6], [2, 4, 1], 1),
    (4, 1, [5, 9], [3, 2], 2),
    (6, 3, [0, 4, 7], [3, 1, 5], 4),
    (8, 2, [13, 1], [1, 1], 3),
    (4, 4, [2, 0, 17, 5], [0, 6, 2, 3], 16),
]


@pytest.mark.parametrize("hq,hkv,prefix,extend,page_size", CASES)
@pytest.mark.parametrize("seed", [0, 1])
def test_oracle_matches_bruteforce(hq, hkv, prefix, extend, page_size, seed):
    rng = np.random.default_rng(100 * seed + hq + page_size)
    case = random_case(rng, hq, hkv, 8, prefix, extend, page_size)
    scale = 8 ** -0.5
    ours = paged_ref.paged_attention_ref(*oracle_args(case, scale))
    brute = bruteforce_case(case, scale).reshape(ours.shape)
    assert np.max(np.abs(ours - brute)) < 1e-12


# --- textbook reduction ---------------------------------------------------------------------

def test_textbook_reduction_matches_sdpa():
    """p=0, P=1, identity slots and Hq=Hkv is textbook causal attention."""
    rng = np.random.default_rng(5)
    n, h, d = 9, 3, 16
    q = rand_bf16(rng, (n, h, d))
    k = rand_bf16(rng, (n, h, d))
    v = rand_bf16(rng, (n, h, d))
    table = np.arange(n, dtype=np.int32)[None]
    scale = 0.25
    ours = paged_ref.paged_attention_ref(q, k, v, table, [n], [0], [n], 1, scale)
    t = lambda a: torch.from_numpy(f64(a)).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True,
                                                           scale=scale)
    assert np.max(np.abs(ours - ref[0].permute(1, 0, 2).numpy())) < 1e-13


# --- invariances ----------------------------------------------------------------------------

def test_page_size_invariance_bit_identical():
    rng = np.random.default_rng(7)
    prefix, extend = np.array([70, 3, 0]), np.array([2, 9, 5])
    seq = prefix + extend
    hq, hkv, d = 4, 2, 8
    lk = [rand_bf16(rng, (int(L), hkv, d)) for L in seq]
    lv = [rand_bf16(rng, (int(L), hkv, d)) for L in seq]
    q = rand_bf16(rng, (int(extend.sum()), hq, d))
    outs = []
    for page_size in (1, 2, 16, 64):
        kp, vp, table = layout_case(np.random.default_rng(page_size), lk, lv, page_size)
        outs.append(paged_ref.paged_attention_ref(q, kp, vp, table, seq, prefix, extend,
                                                  page_size, 0.3))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_page_permutation_invariance_bit_identical():
    rng = np.random.default_rng(8)
    prefix, extend = np.array([33, 12]), np.array([4, 1])
    seq = prefix + extend
    lk = [rand_bf16(rng, (int(L), 2, 8)) for L in seq]
    lv = [rand_bf16(rng, (int(L), 2, 8)) for L in seq]
    q = rand_bf16(rng, (int(extend.sum()), 6, 8))
    base = None
    for perm_seed, permute in [(0, False), (1, True), (2, True)]:
        kp, vp, table = layout_case(np.random.default_rng(perm_seed), lk, lv, 4,
                                    num_pages=40, permute=permute)
        out = paged_ref.paged_attention_ref(q, kp, vp, table, seq, prefix, extend, 4, 0.5)
        if base is None:
            base = out
        assert np.array_equal(out, base)


def test_prefix_cached_equals_from_scratch():
    """Rows p..L-1 of a from-scratch prefill (p=0) equal a prefill of e=L-p rows on a
    cached prefix of p tokens (bottom-right causal alignment)."""
    rng = np.random.default_rng(9)
    L, p, hq, hkv, d = 23, 15, 4, 2, 8
    lk = [rand_bf16(rng, (L, hkv, d))]
    lv = [rand_bf16(rng, (L, hkv, d))]
    q_full = rand_bf16(rng, (L, hq, d))
    kp, vp, table = layout_case(rng, lk, lv, 2)
    full = paged_ref.paged_attention_ref(q_full, kp, vp, table, [L], [0], [L], 2, 0.3)
    tail = paged_ref.paged_attention_ref(q_full[p:], kp, vp, table, [L], [p], [L - p], 2, 0.3)
    assert np.max(np.abs(full[p:] - tail)) < 1e-12


def test_decode_equals_prefill_with_one_new_token():
    rng = np.random.default_rng(10)
    case = random_case(rng, 4, 2, 8, [6, 0, 11], [1, 1, 1], 2)
    a = paged_ref.decode_ref(case["q"], case["k_pool"], case["v_pool"], case["page_table"],
                             case["seq_lens"], 2, 0.4)
    b = paged_ref.paged_attention_ref(*oracle_args(case, 0.4))
    assert np.array_equal(a, b)


# --- softmax special cases --------------------------------------------------------------------

def test_single_key_returns_v_exactly():
    rng = np.random.default_rng(12)
    case = random_case(rng, 4, 2, 8, [0, 0], [1, 1], 1)
    out = paged_ref.paged_attention_ref(*oracle_args(case, 0.1))
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, h], f64(case["logical_v"][b][0, h // 2]))


def test_identical_keys_return_mean_v():
    rng = np.random.default_rng(13)
    L, hkv, d = 12, 2, 8
    key = rand_bf16(rng, (1, hkv, d))
    lk = [np.repeat(key, L, axis=0)]
    lv = [rand_bf16(rng, (L, hkv, d))]
    kp, vp, table = layout_case(rng, lk, lv, 4)
    q = rand_bf16(rng, (1, 4, d))
    out = paged_ref.decode_ref(q, kp, vp, table, [L], 4, 0.5)
    mean = f64(lv[0]).mean(axis=0)          # [Hkv, D]
    for h in range(4):
        assert np.max(np.abs(out[0, h] - mean[h // 2])) < 1e-12


def test_two_keys_closed_form():
    rng = np.random.default_rng(14)
    d = 8
    lk = [rand_bf16(rng, (2, 1, d))]
    lv = [rand_bf16(rng, (2, 1, d))]
    kp, vp, table = layout_case(rng, lk, lv, 1)
    q = rand_bf16(rng, (1, 1, d))
    scale = 0.7
    out = paged_ref.decode_ref(q, kp, vp, table, [2], 1, scale)
    qf, kf, vf = f64(q)[0, 0], f64(lk[0])[:, 0], f64(lv[0])[:, 0]
    s1, s2 = scale * float(qf @ kf[0]), scale * float(qf @ kf[1])
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    want = sig(s1 - s2) * vf[0] + sig(s2 - s1) * vf[1]
    assert np.max(np.abs(out[0, 0] - want)) < 1e-14


def test_gqa_constant_v_per_kv_head():
    """V rows of kv head g all equal g+1, so q head h must output h//G + 1 (up to the
    rounding of a weighted mean of equal values)."""
    rng = np.random.default_rng(15)
    hq, hkv, d = 8, 2, 8
    prefix, extend = [5, 2], [3, 1]
    seq = np.add(prefix, extend)
    lk = [rand_bf16(rng, (int(L), hkv, d)) for L in seq]
    lv = []
    for L in seq:
        v = np.zeros((int(L), hkv, d), dtype=np.float32)
        for g in range(hkv):
            v[:, g, :] = g + 1
        lv.append((v.view(np.uint32) >> np.uint32(16)).astype(np.uint16))
    kp, vp, table = layout_case(rng, lk, lv, 2)
    q = rand_bf16(rng, (4, hq, d))
    out = paged_ref.paged_attention_ref(q, kp, vp, table, seq, prefix, extend, 2, 0.2)
    for h in range(hq):
        assert np.max(np.abs(out[:, h, :] - (h // (hq // hkv) + 1))) < 1e-14


def test_scale_doubling_identity():
    """(2q, scale/2) gives bit-identical output to (q, scale): both are exact rescalings."""
    rng = np.random.default_rng(16)
    case = random_case(rng, 4, 2, 8, [4, 0], [3, 2], 2)
    q = case["q"]
    exp_field = (q >> 7) & 0xFF
    assert np.all((exp_field > 0) & (exp_field < 0xFE))   # normal numbers: doubling is exact
    q2 = (q + np.uint16(1 << 7)).astype(np.uint16)        # exponent + 1
    assert np.array_equal(f64(q2), 2 * f64(q))
    a = paged_ref.paged_attention_ref(*oracle_args(case, 0.5))
    case2 = dict(case, q=q2)
    b = paged_ref.paged_attention_ref(*oracle_args(case2, 0.25))
    assert np.array_equal(a, b)


# --- store, slot translation golden, validation --------------------------------------------------

def test_store_kv_ref_closed_form_and_sentinels():
    rng = np.random.default_rng(17)
    slots, hkv, d = 32, 2, 8
    kp = np.full((slots, hkv, d), 0x7FC0, dtype=np.uint16)
    vp = np.full_like(kp, 0x7FC0)
    out_loc = np.array([5, 31, 0, 17], dtype=np.int32)
    kn = rand_bf16(rng, (4, hkv, d))
    vn = rand_bf16(rng, (4, hkv, d))
    k2, v2 = oracle.store_kv_ref(kp, vp, kn, vn, out_loc)
    for t, s in enumerate(out_loc):
        assert np.array_equal(k2[s], kn[t]) and np.array_equal(v2[s], vn[t])
    untouched = np.setdiff1d(np.arange(slots), out_loc)
    assert np.all(k2[untouched] == 0x7FC0) and np.all(v2[untouched] == 0x7FC0)
    assert np.all(kp == 0x7FC0)      # inputs not modified
    with pytest.raises(oracle.OracleInputError):
        oracle.store_kv_ref(kp, vp, kn, vn, np.array([5, 5, 0, 1]))
    with pytest.raises(oracle.OracleInputError):
        oracle.store_kv_ref(kp, vp, kn, vn, np.array([5, 32, 0, 1]))


def _golden_slot_rows():
    rows = []
    with open(os.path.join(GOLDEN, "slot_translation.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            p, table, L, slots = [s.strip() for s in line.split("|")]
            rows.append((int(p), [int(x) for x in table.split()], int(L),
                         [int(x) for x in slots.split()]))
    return rows


@pytest.mark.parametrize("page_size,table,L,want", _golden_slot_rows())
def test_golden_slot_translation(page_size, table, L, want):
    got = oracle.request_slots(np.array(table), L, page_size)
    assert got.tolist() == want


def test_validation_raises():
    rng = np.random.default_rng(18)
    case = random_case(rng, 4, 2, 8, [3, 2], [2, 1], 2)
    base = oracle_args(case, 0.5)
    bad = list(base)
    bad[4] = np.array(case["seq_lens"]) + 1                      # L != p + e
    with pytest.raises(oracle.OracleInputError):
        paged_ref.paged_attention_ref(*bad)
    bad = list(base)
    t = case["page_table"].copy()
    t[0, 0] = case["k_pool"].shape[0] // 2 + 5                    # page id out of range
    bad[3] = t
    with pytest.raises(oracle.OracleInputError):
        paged_ref.paged_attention_ref(*bad)
    bad = list(base)
    bad[3] = case["page_table"][:, :1]                            # table row too short
    with pytest.raises(oracle.OracleInputError):
        paged_ref.paged_attention_ref(*bad)
    bad = list(base)
    bad[0] = rand_bf16(rng, (3, 3, 8))                            # Hq not a multiple of Hkv
    with pytest.raises(oracle.OracleInputError):
        paged_ref.paged_attention_ref(*bad)
    with pytest.raises(oracle.OracleInputError):                  # decode needs L >= 1
        paged_ref.decode_ref(rand_bf16(rng, (1, 4, 8)), case["k_pool"], case["v_pool"],
                             case["page_table"][:1], [0], 2, 0.5)


def test_out_loc_must_match_table_and_be_private():
    rng = np.random.default_rng(19)
    case = random_case(rng, 4, 2, 8, [3, 2], [2, 1], 2)
    t = case["page_table"]
    slots = [oracle.request_slots(t[b], int(case["seq_lens"][b]), 2) for b in range(2)]
    good = np.array([slots[0][3], slots[0][4], slots[1][2]])
    nslots = case["k_pool"].shape[0]
    oracle.validate_out_loc(good, nslots, t, case["seq_lens"], case["prefix_lens"],
                            case["extend_lens"], 2)
    with pytest.raises(oracle.OracleInputError):
        oracle.validate_out_loc(good[[1, 0, 2]], nslots, t, case["seq_lens"],
                                case["prefix_lens"], case["extend_lens"], 2)
    shared = t.copy()
    shared[1, 0] = t[0, 2]          # request 1 would read the page request 0 writes into
    with pytest.raises(oracle.OracleInputError):
        oracle.validate_out_loc(np.array([slots[0][3], slots[0][4],
                                          oracle.slot_of(shared[1], 2, 2)]), nslots, shared,
                                case["seq_lens"], case["prefix_lens"], case["extend_lens"], 2)


# --- the pins catch planted mistakes --------------------------------------------------------------

PINS = [
    lambda: test_oracle_matches_bruteforce(4, 2, [3, 0, 6], [2, 4, 1], 1, 0),
    lambda: test_oracle_matches_bruteforce(6, 3, [0, 4, 7], [3, 1, 5], 4, 1),
    test_textbook_reduction_matches_sdpa,
    test_page_size_invariance_bit_identical,
    test_prefix_cached_equals_from_scratch,
    test_single_key_returns_v_exactly,
    test_gqa_constant_v_per_kv_head,
    lambda: [test_golden_slot_translation(*r) for r in _golden_slot_rows()],
]

MISTAKES = {
    "gqa mapping h % G": ("kv_head_of", lambda h, g: h % g),
    "causal top-left": ("last_visible_key", lambda p, i: i),
    "causal excludes diagonal": ("last_visible_key", lambda p, i: p + i - 1),
    "causal off by one past": ("last_visible_key", lambda p, i: p + i + 1),
    "slot: pages and offsets swapped":
        ("slot_of", lambda row, j, P: int(row[j % P]) * P + j // P if j % P < len(row)
         else 0),
    "slot: offset dropped": ("slot_of", lambda row, j, P: int(row[j // P]) * P),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, bad = MISTAKES[name]
    monkeypatch.setattr(paged_ref, attr, bad)
    caught = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, oracle.OracleInputError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake: {name}"
