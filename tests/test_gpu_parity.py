"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

store_kv is compared bit for bit over the whole pools (untouched slots keep their
NaN sentinel). Attention outputs are compared element by element within max abs
2e-2 and mean abs 2e-3, on every row for small cases and on sampled requests or
exact token windows for the full-size workloads (a window [a, c) of request b is the
sub-problem with prefix p_b + a and extend c - a, which the oracle computes alone).
Unreferenced slots hold NaN, so any read outside a request's keys shows up.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_attention_25_amd import workloads as W
from tests.gpu_common import (HostInputs, announce, assert_close, dev_i32, gpu_decode_store,
                              gpu_part, gpu_store, host_u16, oracle_decode, oracle_prefill)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_25_amd as pka
    pka.lib()          # fail loudly if the library is missing


def check_store(step, host, what):
    gpu_store(step)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(step.k_pool), host.k_pool), f"{what}: k_pool differs"
    assert np.array_equal(host_u16(step.v_pool), host.v_pool), f"{what}: v_pool differs"


# --- store_kv -------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_decode", "chunked_prefill", "tp4_mixed"])
def test_store_kv_bit_exact(name):
    announce(f"store_kv {name}")
    step = W.WORKLOADS[name](device="cuda")
    host = HostInputs(step)
    check_store(step, host, name)


def test_store_kv_skips_out_of_pool_slots():
    announce("store_kv slot outside the pool is skipped")
    step = W.tiny_decode(device="cuda")
    host = HostInputs(step)
    import paged_kv_attention_25_amd as pka
    from tests.gpu_common import dev_i32
    bad = step.out_loc.copy()
    bad[1] = step.num_slots + 7
    bad[2] = -3
    pka.store_kv(step.k_new, step.v_new, dev_i32(bad), step.k_pool, step.v_pool, 1)
    torch.cuda.synchronize()
    kp, vp = host_u16(step.k_pool), host_u16(step.v_pool)
    for t in (0, 3):
        assert np.array_equal(kp[bad[t]], host.k_new[t])
        assert np.array_equal(vp[bad[t]], host.v_new[t])
    keep = np.setdiff1d(np.arange(step.num_slots), bad[[0, 3]])
    assert np.array_equal(kp[keep], host.k_pool0[keep])
    assert np.array_equal(vp[keep], host.v_pool0[keep])


# --- decode ---------------------------------------------------------------------------

def run_decode_case(step, what, requests=None):
    host = HostInputs(step)
    check_store(step, host, what)
    announce(f"decode {what}")
    out = gpu_part(step, step.parts[0])
    torch.cuda.synchronize()
    ref, idx = oracle_decode(step, host, 0, requests)
    assert_close(host_u16(out)[idx], ref, f"decode {what}")
    return step, host, out


def test_decode_tiny():
    run_decode_case(W.tiny_decode(device="cuda"), "tiny_decode (B=4, 16q/8kv)")


def test_decode_b256_full():
    run_decode_case(W.decode_b256(device="cuda"), "decode_b256 all requests")


@pytest.mark.parametrize("P", [16, 32, 64])
def test_decode_b256_page_sizes_sampled(P):
    # the decode_b256 requests in a 2^20-slot pool cut into pages of P slots
    step = W.decode_b256(device="cuda", page_size=P)
    run_decode_case(step, f"decode_b256 P={P} (16 requests)", requests=list(range(3, 256, 16)))


def test_decode_long_full():
    step = W.long_decode(device="cuda")
    run_decode_case(step, "long_decode 32x32768 P=64 (all 32 requests)")


def test_decode_tp4_part():
    step = W.tp4_mixed(device="cuda")
    host = HostInputs(step)
    check_store(step, host, "tp4_mixed")
    announce("decode tp4_mixed 128 seqs, 16q/2kv")
    out = gpu_part(step, step.parts[0])
    torch.cuda.synchronize()
    ref, idx = oracle_decode(step, host, 0)
    assert_close(host_u16(out)[idx], ref, "decode tp4_mixed")


@pytest.mark.parametrize("hq,hkv,page_size,lens", [
    (8, 8, 1, [1, 2, 63, 64, 65, 129]),      # G=1, split edges
    (16, 1, 3, [5, 100, 301]),               # G=16, non power-of-two page size
    (10, 2, 16, [16, 17, 1000, 4097]),       # G=5
    (16, 2, 64, [1, 64, 65, 9000]),          # G=8
    (16, 2, 96, [95, 96, 97, 3000]),         # G=8, pages of 96 slots (not a power of two)
    (12, 3, 1, [70, 2000, 4000, 129]),       # 3 kv heads: 682 groups of 3 wavefronts
    (16, 16, 16, [1, 300, 5000]),            # 16 kv heads, G=1: 128 groups of 16
])
def test_decode_edge_shapes(hq, hkv, page_size, lens):
    pages = sum(-(-L // page_size) for L in lens) + 8
    step = W.build_step("edge", hq, hkv, page_size, pages, [W.decode_spec(lens)], seed=21,
                        device="cuda")
    run_decode_case(step, f"edge hq={hq} hkv={hkv} P={page_size} L={lens}")


def test_decode_max_batch():
    """The largest supported batch (4096 requests, lengths 1..200): the per-request block
    prefix sums are built with 16 requests per thread, and most wavefront ranges hold
    several whole pairs (written directly) besides the split ones."""
    rng = np.random.default_rng(25)
    lens = rng.integers(1, 201, size=4096)
    step = W.build_step("max_batch", 16, 2, 1, int(lens.sum()) + 64, [W.decode_spec(lens)],
                        seed=25, device="cuda")
    run_decode_case(step, "max batch 4096, 16q/2kv, L in [1, 200]",
                    requests=list(range(0, 4096, 37)) + [4095])


def test_decode_keys_past_max_seq_len_are_not_attended():
    """A request longer than the max_seq_len hint attends only its first max_seq_len
    keys (the documented clamp): the same as the oracle on the truncated length."""
    step = W.build_step("clamp", 16, 2, 1, 2048, [W.decode_spec([100, 900, 700])], seed=27,
                        device="cuda")
    host = HostInputs(step)
    check_store(step, host, "clamp")
    announce("decode with seq_lens above the max_seq_len hint")
    out = host_u16(gpu_part(step, step.parts[0], max_seq_len=640))
    torch.cuda.synchronize()
    part = step.parts[0]
    clamped = np.minimum(part.seq_lens, 640).astype(np.int32)
    ref = oracle.decode_ref(host.q[0], host.k_pool, host.v_pool, part.page_table, clamped,
                            step.page_size, step.scale)
    assert_close(out, ref, "decode clamped to max_seq_len")


def test_decode_single_key_is_v_exactly():
    step = W.build_step("single", 16, 8, 1, 64, [W.decode_spec([1, 1, 1])], seed=22,
                        device="cuda")
    _, host, out = run_decode_case(step, "single key")
    got = host_u16(out)
    for b in range(3):
        for h in range(16):
            assert np.array_equal(got[b, h], host.v_new[b, h // 2])


def test_decode_split_count_invariance():
    """Requests split at different keys agree within tolerance: three requests decoded
    alone (992 blocks of 64 keys for 992 wavefronts, one block each, so every (request,
    kv head) pair is merged from many splits) and inside a batch of 23 (6112 blocks for
    2048 wavefronts, about three each, other split points), and with a max_seq_len hint
    far above the lengths (the plan's wavefront count is capped by the actual blocks)."""
    lens = [3000, 4096, 777] + [2000] * 20
    step = W.build_step("splits", 16, 8, 1, 1 << 16, [W.decode_spec(lens)], seed=23,
                        device="cuda")
    big = step.parts[0]
    hint = 200000
    small = W.AttnPart(kind="decode", seq_lens=big.seq_lens[:3], prefix_lens=big.prefix_lens[:3],
                       extend_lens=big.extend_lens[:3], cu_extend=big.cu_extend[:4],
                       page_table=np.pad(big.page_table[:3],
                                         ((0, 0), (0, hint - big.page_table.shape[1])),
                                         mode="edge"),
                       q=big.q[:3].contiguous(), row_offset=0)
    host = HostInputs(step)
    check_store(step, host, "splits")
    announce("decode split-count invariance")
    a = host_u16(gpu_part(step, small))
    b = host_u16(gpu_part(step, big))[:3]
    c = host_u16(gpu_part(step, small, max_seq_len=hint))
    torch.cuda.synchronize()
    ref, _ = oracle_decode(step, host, 0, requests=[0, 1, 2])
    assert_close(a, ref, "alone")
    assert_close(b, ref, "in a batch of 23")
    assert_close(c, ref, "alone, large max_seq_len hint")
    assert_close(a, oracle.bf16_bits_to_f64(b), "alone vs in the batch")


@pytest.mark.parametrize("hq,hkv", [(16, 1), (16, 8), (40, 8)])
def test_decode_one_launch_and_split_paths_agree(hq, hkv):
    # Lengths up to 512 keys. With a max_seq_len hint of 512 the call runs in one launch
    # (a workgroup per (request, kv head), one wavefront per 64-key block, merged in LDS;
    # 8 wavefronts at the limit); with a hint of 1024 it takes the split kernel and its
    # merge launch. Both must match the oracle.
    lens = [1, 63, 64, 65, 200, 511, 512]
    pages = sum(-(-L // 16) for L in lens) + 8
    step = W.build_step("paths", hq, hkv, 16, pages, [W.decode_spec(lens)], seed=51,
                        device="cuda")
    part = step.parts[0]
    # room in the table for the 1024-key hint (columns past a request's pages are
    # never read)
    part.page_table = np.pad(part.page_table, ((0, 0), (0, 1024 // 16)))
    host = HostInputs(step)
    check_store(step, host, "paths")
    announce(f"decode one-launch vs split paths hq={hq} hkv={hkv}")
    one = host_u16(gpu_part(step, part, max_seq_len=512))
    split = host_u16(gpu_part(step, part, max_seq_len=1024))
    torch.cuda.synchronize()
    ref, _ = oracle_decode(step, host, 0)
    assert_close(one, ref, f"one launch hq={hq} hkv={hkv}")
    assert_close(split, ref, f"split hq={hq} hkv={hkv}")


# --- store and decode in one launch ------------------------------------------------------

def check_pools(step, host, what):
    assert np.array_equal(host_u16(step.k_pool), host.k_pool), f"{what}: k_pool differs"
    assert np.array_equal(host_u16(step.v_pool), host.v_pool), f"{what}: v_pool differs"


def run_decode_store_case(step, what, requests=None, max_seq_len=None):
    """pka_paged_attn_decode_store on a decode-only step whose pools do not yet hold the
    new rows (their slots are NaN): the pools must equal the oracle's store bit for bit
    and the outputs the oracle's decode over the stored pools."""
    host = HostInputs(step)
    announce(f"decode+store {what}")
    out = gpu_decode_store(step, step.parts[0], max_seq_len=max_seq_len)
    torch.cuda.synchronize()
    check_pools(step, host, what)
    part = step.parts[0]
    idx = np.arange(part.batch) if requests is None else np.asarray(requests)
    lens = part.seq_lens[idx] if max_seq_len is None else np.minimum(part.seq_lens[idx],
                                                                     max_seq_len)
    ref = oracle.decode_ref(host.q[0][idx], host.k_pool, host.v_pool, part.page_table[idx],
                            lens.astype(np.int32), step.page_size, step.scale)
    assert_close(host_u16(out)[idx], ref, f"decode+store {what}")
    return host, out


def test_decode_store_tiny():
    run_decode_store_case(W.tiny_decode(device="cuda"), "tiny_decode")


def test_decode_store_b256_full():
    run_decode_store_case(W.decode_b256(device="cuda"), "decode_b256 all requests")


@pytest.mark.parametrize("P", [16, 64])
def test_decode_store_b256_page_sizes_sampled(P):
    # the page-size sweep's launch: decode_b256 in pages of P slots, store inside
    run_decode_store_case(W.decode_b256(device="cuda", page_size=P), f"decode_b256 P={P}",
                          requests=list(range(5, 256, 16)))


@pytest.mark.parametrize("hq,hkv", [(16, 1), (40, 8)])
def test_decode_store_one_launch_path(hq, hkv):
    # the store inside the one-launch path, 8 wavefronts per pair at the limit
    lens = [1, 64, 65, 300, 512]
    pages = sum(-(-L // 16) for L in lens) + 8
    step = W.build_step("paths", hq, hkv, 16, pages, [W.decode_spec(lens)], seed=53,
                        device="cuda")
    run_decode_store_case(step, f"one launch hq={hq} hkv={hkv}", max_seq_len=512)


def test_decode_store_long_full():
    run_decode_store_case(W.long_decode(device="cuda"), "long_decode (all 32 requests)")


@pytest.mark.parametrize("hq,hkv,page_size,lens", [
    (8, 8, 1, [1, 2, 63, 64, 65, 129]),
    (16, 1, 3, [5, 100, 301]),
    (16, 2, 64, [1, 64, 65, 9000]),
    (12, 3, 1, [70, 2000, 4000, 129]),
])
def test_decode_store_edge_shapes(hq, hkv, page_size, lens):
    pages = sum(-(-L // page_size) for L in lens) + 8
    step = W.build_step("edge", hq, hkv, page_size, pages, [W.decode_spec(lens)], seed=31,
                        device="cuda")
    run_decode_store_case(step, f"edge hq={hq} hkv={hkv} P={page_size} L={lens}")


def test_decode_store_max_batch():
    """4096 short requests: most wavefronts meet several pairs' last blocks (each a
    store) in one stream."""
    rng = np.random.default_rng(33)
    lens = rng.integers(1, 201, size=4096)
    step = W.build_step("max_batch", 16, 2, 1, int(lens.sum()) + 64, [W.decode_spec(lens)],
                        seed=33, device="cuda")
    run_decode_store_case(step, "max batch 4096", requests=list(range(0, 4096, 41)) + [4095])


def test_decode_store_single_key_is_v_new_exactly():
    step = W.build_step("single", 16, 8, 1, 64, [W.decode_spec([1, 1, 1])], seed=32,
                        device="cuda")
    host, out = run_decode_store_case(step, "single key")
    got = host_u16(out)
    for b in range(3):
        for h in range(16):
            assert np.array_equal(got[b, h], host.v_new[b, h // 2])


def test_decode_store_past_max_seq_len():
    """Requests longer than the max_seq_len hint still store their new rows; their
    attention covers only the first max_seq_len keys."""
    step = W.build_step("clamp", 16, 2, 1, 2048, [W.decode_spec([100, 900, 700])], seed=34,
                        device="cuda")
    run_decode_store_case(step, "seq_lens above the hint", max_seq_len=640)


def test_decode_store_skips_out_of_pool_slots():
    """A slot outside the pool is not written (as in store_kv); the other requests are
    stored and decoded as usual."""
    step = W.build_step("skip", 16, 8, 1, 1024, [W.decode_spec([50, 300, 129, 7])], seed=35,
                        device="cuda")
    host = HostInputs(step)
    part = step.parts[0]
    bad = step.out_loc.copy()
    bad[1] = step.num_slots + 5
    announce("decode+store with one out-of-pool slot")
    out = host_u16(gpu_decode_store(step, part, out_loc=bad))
    torch.cuda.synchronize()
    kp, vp = host_u16(step.k_pool), host_u16(step.v_pool)
    keep = np.ones(step.num_slots, bool)
    keep[step.out_loc[1]] = False
    assert np.array_equal(kp[keep], host.k_pool[keep])
    assert np.array_equal(vp[keep], host.v_pool[keep])
    assert np.array_equal(kp[step.out_loc[1]], host.k_pool0[step.out_loc[1]])  # untouched
    ok = [0, 2, 3]
    ref = oracle.decode_ref(host.q[0][ok], host.k_pool, host.v_pool, part.page_table[ok],
                            part.seq_lens[ok], step.page_size, step.scale)
    assert_close(out[ok], ref, "decode+store, the requests with valid slots")


def test_decode_store_equals_store_then_decode():
    """The fused call and store_kv followed by decode give the same pools bit for bit
    and outputs within rounding order (the same kernels' arithmetic: identical here)."""
    a = W.decode_b256(device="cuda", batch=64)
    b = W.decode_b256(device="cuda", batch=64)
    announce("decode+store vs store then decode (64 requests)")
    out_a = host_u16(gpu_decode_store(a, a.parts[0]))
    gpu_store(b)
    out_b = host_u16(gpu_part(b, b.parts[0]))
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(a.k_pool), host_u16(b.k_pool))
    assert np.array_equal(host_u16(a.v_pool), host_u16(b.v_pool))
    assert np.array_equal(out_a, out_b)


def test_decode_gqa_constant_v():
    step = W.build_step("gqa", 16, 2, 16, 64, [W.decode_spec([37, 200])], seed=24, device="cuda")
    for g in range(2):
        step.v_pool[:, g, :] = torch.tensor(float(g + 1), dtype=torch.bfloat16).view(torch.int16)
        step.v_new[:, g, :] = torch.tensor(float(g + 1), dtype=torch.bfloat16).view(torch.int16)
    gpu_store(step)
    announce("decode gqa constant V")
    out = oracle.bf16_bits_to_f64(host_u16(gpu_part(step, step.parts[0])))
    for h in range(16):
        assert np.all(out[:, h, :] == h // 8 + 1)


# --- prefill --------------------------------------------------------------------------

def run_prefill_case(step, what, part_idx=0, windows=None):
    host = HostInputs(step)
    check_store(step, host, what)
    part = step.parts[part_idx]
    announce(f"prefill {what}")
    out = gpu_part(step, part)
    torch.cuda.synchronize()
    if windows is None:
        windows = [(b, 0, int(part.extend_lens[b])) for b in range(part.batch)
                   if part.extend_lens[b] > 0]
    ref, rows = oracle_prefill(step, host, part_idx, windows)
    assert_close(host_u16(out)[rows], ref, f"prefill {what}")
    return step, host, out


@pytest.mark.parametrize("hq,hkv,page_size,prefix,extend", [
    (8, 8, 1, [0], [1]),
    (8, 8, 1, [0], [200]),
    (10, 2, 16, [0, 37, 500, 3], [129, 0, 64, 1]),      # G=5, an empty request
    (16, 2, 1, [1024, 0], [300, 77]),                    # G=8
    (16, 1, 3, [7, 100], [45, 130]),                     # G=16, P=3
    (40, 8, 64, [4096, 0, 130], [33, 257, 64]),          # 14B heads, P=64
    (16, 2, 128, [200, 0], [100, 300]),                  # pages longer than a key tile
    (16, 2, 96, [500, 31], [70, 200]),                   # 96-slot pages
])
def test_prefill_edge_shapes(hq, hkv, page_size, prefix, extend):
    seq = np.add(prefix, extend)
    pages = int(sum(-(-int(L) // page_size) for L in seq)) + 8
    step = W.build_step("edge", hq, hkv, page_size, pages, [("prefill", prefix, extend)],
                        seed=31, device="cuda")
    run_prefill_case(step, f"edge hq={hq} hkv={hkv} P={page_size} p={prefix} e={extend}")


def test_prefill_many_small_requests():
    """600 requests of 0..12 new tokens on prefixes of 0..300: many one-block work items
    with mixed key counts through the dispatch-order plan (empty requests included)."""
    rng = np.random.default_rng(26)
    prefix = rng.integers(0, 301, size=600)
    extend = rng.integers(0, 13, size=600)
    pages = int(sum(-(-int(L) // 16) for L in prefix + extend)) + 8
    step = W.build_step("many_small", 16, 2, 16, pages, [("prefill", prefix, extend)], seed=26,
                        device="cuda")
    run_prefill_case(step, "600 small requests, P=16")


def test_prefill_chunked_sampled():
    step = W.chunked_prefill(device="cuda")
    part = step.parts[0]
    e, p = part.extend_lens, part.prefix_lens
    picks = sorted({int(np.argmax(e)), int(np.argmax(p)), int(np.argmin(e)), 0, 7, 19, 31})
    windows = []
    for b in picks:
        eb = int(e[b])
        windows.append((b, 0, min(eb, 40)))
        if eb > 40:
            windows.append((b, max(40, eb - 40), eb))
    run_prefill_case(step, "chunked_prefill 32 req, 8192 tokens, P=16 (windows)",
                     windows=windows)


def test_prefill_chunked_full():
    """Every output row of the chunked_prefill workload (32 requests, 8192 new tokens,
    40q/8kv, P=16) against the oracle."""
    run_prefill_case(W.chunked_prefill(device="cuda"),
                     "chunked_prefill 32 req, 8192 tokens, P=16 (every row)")


def test_prefill_tp4_chunk_full():
    """Every output row of the tensor-parallel step's 8192-token chunk on a 1024-token
    prefix (16q/2kv, P=1) against the oracle."""
    run_prefill_case(W.tp4_mixed(device="cuda"),
                     "tp4_mixed 8192-token chunk on 1024 prefix (every row)", part_idx=1)


@pytest.mark.parametrize("P", [1, 32, 64])
def test_prefill_chunked_page_sizes_sampled(P):
    # the chunked_prefill requests with the pool cut into other page sizes (the
    # page-size sweep of the benchmark)
    step = W.chunked_prefill(device="cuda", page_size=P)
    part = step.parts[0]
    e = part.extend_lens
    windows = []
    for b in sorted({int(np.argmax(e)), int(np.argmax(part.prefix_lens)), 0, 13, 31}):
        eb = int(e[b])
        windows.append((b, 0, min(eb, 32)))
        if eb > 32:
            windows.append((b, max(32, eb - 32), eb))
    run_prefill_case(step, f"chunked_prefill P={P} (windows)", windows=windows)


def test_prefill_tp4_chunk_sampled():
    step = W.tp4_mixed(device="cuda")
    run_prefill_case(step, "tp4_mixed 8192-token chunk on 1024 prefix (windows)", part_idx=1,
                     windows=[(0, 0, 64), (0, 3000, 3064), (0, 8128, 8192)])


def test_prefill_prefix_cached_equals_from_scratch():
    L, p = 700, 450
    full = W.build_step("full", 16, 2, 16, 64, [("prefill", [0], [L])], seed=41, device="cuda")
    gpu_store(full)
    announce("prefill from scratch vs prefix-cached")
    out_full = host_u16(gpu_part(full, full.parts[0]))
    part = full.parts[0]
    part_tail = W.AttnPart(kind="prefill", seq_lens=np.array([L], np.int32),
                           prefix_lens=np.array([p], np.int32),
                           extend_lens=np.array([L - p], np.int32),
                           cu_extend=np.array([0, L - p], np.int32), page_table=part.page_table,
                           q=part.q[p:].contiguous(), row_offset=0)
    out_tail = host_u16(gpu_part(full, part_tail))
    torch.cuda.synchronize()
    assert_close(out_tail, oracle.bf16_bits_to_f64(out_full[p:]), "tail vs full rows")


def test_decode_equals_prefill_extend_one():
    step = W.build_step("d_eq_p", 40, 8, 16, 1024, [W.decode_spec([900, 31, 2048])], seed=42,
                        device="cuda")
    gpu_store(step)
    announce("decode vs prefill with one new token")
    part = step.parts[0]
    d = host_u16(gpu_part(step, part))
    as_prefill = W.AttnPart(kind="prefill", seq_lens=part.seq_lens, prefix_lens=part.prefix_lens,
                            extend_lens=part.extend_lens, cu_extend=part.cu_extend,
                            page_table=part.page_table, q=part.q, row_offset=0)
    pf = host_u16(gpu_part(step, as_prefill))
    torch.cuda.synchronize()
    assert_close(d, oracle.bf16_bits_to_f64(pf), "decode vs prefill")


def scale_keys_by_position(step, part, every=64):
    """Multiply K of logical key j of every request of `part` by 2^(j // every) (exact in
    bf16 at these magnitudes), in the pool for prefix keys and in k_new for new ones."""
    P = step.page_size
    slots, slot_f, rows, row_f = [], [], [], []
    for b in range(part.batch):
        p, e = int(part.prefix_lens[b]), int(part.extend_lens[b])
        for j in range(p + e):
            f = float(2 ** (j // every))
            if j < p:
                slots.append(int(part.page_table[b, j // P]) * P + j % P)
                slot_f.append(f)
            else:
                rows.append(part.row_offset + int(part.cu_extend[b]) + j - p)
                row_f.append(f)
    for t, idx, f in ((step.k_pool, slots, slot_f), (step.k_new, rows, row_f)):
        if not idx:
            continue
        v = t.view(torch.bfloat16)
        i = torch.tensor(idx, device=v.device)
        v[i] = (v[i].float() * torch.tensor(f, device=v.device)[:, None, None]).to(torch.bfloat16)


def test_prefill_scores_growing_with_position():
    """Keys scaled by 2^(j // 64): from tile 3 on, row maxima exceed the running max by
    more than 27 in log2 units, so those tiles raise the max, rescale the output and
    redo their exponentials; the tiles before keep the max of the first tile."""
    step = W.build_step("growing", 16, 2, 1, 2048, [("prefill", [300, 0], [70, 360])],
                        seed=43, device="cuda")
    scale_keys_by_position(step, step.parts[0])
    run_prefill_case(step, "keys growing 2x per 64 positions")


@pytest.mark.parametrize("tiles", list(range(1, 10)))
@pytest.mark.parametrize("batch", [1, 2])
def test_prefill_block_tile_counts(tiles, batch):
    """Blocks with exactly 1..9 key tiles of 64: the load pipeline's prologue and the
    wait counts of its last iterations (tiles past the end are never loaded); batch 2
    also runs the dispatch-order plan."""
    # G = 8: 16 tokens are 128 rows, one block; keys 0 .. prefix + 15
    prefix = 64 * (tiles - 1) + 1
    pre, ext = [prefix] * batch, [16] * batch
    if batch == 2:
        pre[1], ext[1] = max(0, prefix - 40), 9   # a second, shorter request
    step = W.build_step("tiles", 16, 2, 1, 4 * (prefix + 64) * batch,
                        [("prefill", pre, ext)], seed=300 + tiles, device="cuda")
    run_prefill_case(step, f"tiles={tiles} batch={batch}")


def test_mixed_step_on_two_streams_matches_one_stream():
    """The mixed step with its decode on a second stream beside the prefill (the decode
    waits for the store through an event) gives outputs bit-identical to the one-stream
    order store, decode, prefill, and both match the oracle. The pools are put back to
    their state before the first store (new tokens' slots NaN) before the two-stream
    run, so a decode that ran before the store would read NaN."""
    step = W.build_step("mixed", 16, 2, 1, 1 << 17,
                        [W.decode_spec(list(range(300, 300 + 64 * 37, 37))),
                         ("prefill", [512], [2048])], seed=61, device="cuda")
    dec, pre = step.parts
    host = HostInputs(step)
    k0, v0 = step.k_pool.clone(), step.v_pool.clone()
    announce("mixed step: two streams vs one")
    gpu_store(step)
    d1 = gpu_part(step, dec)
    p1 = gpu_part(step, pre)
    torch.cuda.synchronize()
    step.k_pool.copy_(k0)
    step.v_pool.copy_(v0)
    torch.cuda.synchronize()
    s1 = torch.cuda.current_stream()
    s2 = torch.cuda.Stream()
    gpu_store(step)
    stored = torch.cuda.Event()
    stored.record(s1)
    with torch.cuda.stream(s2):
        s2.wait_event(stored)
        d2 = gpu_part(step, dec)
    p2 = gpu_part(step, pre)
    s1.wait_stream(s2)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(step.k_pool), host.k_pool)
    assert np.array_equal(host_u16(step.v_pool), host.v_pool)
    ref_d, idx = oracle_decode(step, host, 0)
    assert_close(host_u16(d2)[idx], ref_d, "two-stream decode")
    windows = [(0, 0, 2048)]
    ref_p, rows = oracle_prefill(step, host, 1, windows)
    assert_close(host_u16(p2)[rows], ref_p, "two-stream prefill")
    assert torch.equal(d1, d2) and torch.equal(p1, p2)


def test_step_graph_replay_matches_eager():
    """store + decode + prefill captured once in a HIP graph and replayed three times,
    with eager work and synchronisation between replays: every replay reproduces the
    eager outputs bit for bit (the calls allocate nothing and never synchronise)."""
    import paged_kv_attention_25_amd as pka
    step = W.build_step("graph", 16, 2, 16, 4096,
                        [W.decode_spec([300, 1500, 40, 2048]), ("prefill", [100, 0], [70, 33])],
                        seed=77, device="cuda", fill="zero")
    dec, pre = step.parts
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    out_loc = i32(step.out_loc)
    dpt, dseq = i32(dec.page_table), i32(dec.seq_lens)
    ppt, pseq = i32(pre.page_table), i32(pre.seq_lens)
    ppre, pext, pcu = i32(pre.prefix_lens), i32(pre.extend_lens), i32(pre.cu_extend)
    geom = (step.num_q_heads, step.num_kv_heads, 128, step.page_size, step.num_pages)
    dws = torch.zeros(max(1, pka.decode_workspace_bytes(*geom, dec.batch, dec.max_seq_len)),
                      dtype=torch.uint8, device="cuda")
    pws = torch.zeros(max(1, pka.prefill_workspace_bytes(*geom, pre.batch, pre.num_tokens,
                                                         pre.max_extend)),
                      dtype=torch.uint8, device="cuda")
    dout, pout = torch.empty_like(dec.q), torch.empty_like(pre.q)

    def run():
        pka.store_kv(step.k_new, step.v_new, out_loc, step.k_pool, step.v_pool, step.page_size)
        pka.paged_attn_decode(dec.q, step.k_pool, step.v_pool, dpt, dseq, dec.max_seq_len,
                              step.page_size, step.scale, out=dout, workspace=dws)
        pka.paged_attn_prefill(pre.q, step.k_pool, step.v_pool, ppt, pseq, ppre, pext, pcu,
                               pre.max_extend, pre.max_seq_len, step.page_size, step.scale,
                               out=pout, workspace=pws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                      # eager reference (also warms the library's caches)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref_d, ref_p = host_u16(dout).copy(), host_u16(pout).copy()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    announce("graph replay")
    for r in range(3):
        dout.fill_(0)
        pout.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(dout), ref_d), f"decode differs on replay {r}"
        assert np.array_equal(host_u16(pout), ref_p), f"prefill differs on replay {r}"
        run()                      # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("name,lens", [
    ("tiny_decode", None),                         # the one-launch path
    ("split", [300, 1500, 40, 2048, 700, 64, 129]),  # split kernel + merge in the graph
])
def test_decode_store_graph_replay_matches_oracle(name, lens):
    """The decode step as one pka_paged_attn_decode_store call captured in a HIP graph.
    Before every replay the pools are put back to their state before the store (the new
    tokens' slots NaN), so each replay must store the new rows itself; every replay's
    pools must equal the oracle's store bit for bit and its output must match the
    oracle. Eager work (the same call on other buffers) and synchronisation run between
    the replays."""
    import paged_kv_attention_25_amd as pka
    if lens is None:
        step = W.tiny_decode(device="cuda")
    else:
        step = W.build_step("graph_split", 16, 8, 16, 1024, [W.decode_spec(lens)], seed=78,
                            device="cuda")
    part = step.parts[0]
    host = HostInputs(step)
    k0, v0 = step.k_pool.clone(), step.v_pool.clone()
    pt, seq, loc = dev_i32(part.page_table), dev_i32(part.seq_lens), dev_i32(step.out_loc)
    ws = torch.zeros(max(1, pka.decode_workspace_bytes(step.num_q_heads, step.num_kv_heads,
                                                       128, step.page_size, step.num_pages,
                                                       part.batch, part.max_seq_len)),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(part.q)
    # eager work between replays: the same call on copies of the inputs
    ek, ev = k0.clone(), v0.clone()
    eout = torch.empty_like(part.q)
    ews = torch.zeros_like(ws)

    def run():
        pka.paged_attn_decode_store(part.q, step.k_new, step.v_new, loc, step.k_pool,
                                    step.v_pool, pt, seq, part.max_seq_len, step.page_size,
                                    step.scale, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                      # eager (loads the kernels before capture)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = host_u16(out).copy()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    ref, idx = oracle_decode(step, host, 0)
    announce(f"decode_store graph replay ({name})")
    for r in range(3):
        step.k_pool.copy_(k0)
        step.v_pool.copy_(v0)
        out.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(step.k_pool), host.k_pool), f"k_pool, replay {r}"
        assert np.array_equal(host_u16(step.v_pool), host.v_pool), f"v_pool, replay {r}"
        got = host_u16(out)
        assert np.array_equal(got, eager), f"replay {r} differs from the eager call"
        assert_close(got[idx], ref, f"graph replay {r} ({name})")
        ek.copy_(k0)
        ev.copy_(v0)
        pka.paged_attn_decode_store(part.q, step.k_new, step.v_new, loc, ek, ev, pt, seq,
                                    part.max_seq_len, step.page_size, step.scale, out=eout,
                                    workspace=ews)
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(eout), eager)
