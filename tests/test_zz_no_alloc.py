"""GPU: pka_paged_attn_decode_store_noalloc (static device scratch, no workspace
argument) against pka_paged_attn_decode_store (caller workspace) through the C ABI.

Two calls in a row share the library's static scratch, the second with a smaller batch
and another geometry, so the second reads a scratch that still holds the first call's
partials: each must give the same pools (bit for bit) and the same output as the
workspace entry point on the same inputs, and both must match the float64 oracle
within the attention bar (max abs 2e-2, mean abs 2e-3).
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_25_amd as pka
from paged_kv_attention_25_amd import workloads as W
from tests.gpu_common import HostInputs, announce, assert_close, dev_i32, host_u16, oracle_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pka.lib()


def decode_store_both(step, requests):
    """Run the step's decode part through both entry points on identical copies of the
    pools; compare them with each other and with the oracle."""
    part = step.parts[0]
    host = HostInputs(step)
    pt, seq, loc = dev_i32(part.page_table), dev_i32(part.seq_lens), dev_i32(step.out_loc)
    k2, v2 = step.k_pool.clone(), step.v_pool.clone()
    out_ws = pka.paged_attn_decode_store(part.q, step.k_new, step.v_new, loc, step.k_pool,
                                         step.v_pool, pt, seq, part.max_seq_len,
                                         step.page_size, step.scale)
    out_na = torch.full_like(part.q, -1)
    pka.paged_attn_decode_store_noalloc(part.q, step.k_new, step.v_new, loc, k2, v2, pt, seq,
                                        part.max_seq_len, step.page_size, step.scale,
                                        out=out_na)
    torch.cuda.synchronize()
    assert torch.equal(k2, step.k_pool) and torch.equal(v2, step.v_pool), "pools differ"
    assert np.array_equal(host_u16(k2), host.k_pool), "k_pool differs from the oracle's store"
    assert np.array_equal(host_u16(v2), host.v_pool), "v_pool differs from the oracle's store"
    assert torch.equal(out_na, out_ws), "outputs differ between the two entry points"
    ref, idx = oracle_decode(step, host, 0, requests)
    assert_close(host_u16(out_na)[idx], ref, f"noalloc {step.name}")


def test_noalloc_decode_store_two_calls_second_smaller():
    rng = np.random.default_rng(91)
    # first call: 16q/2kv (G=8), 160 requests, lengths up to 8192: the split plan uses
    # 8.4 MB of the scratch
    lens1 = np.clip(np.rint(2048 * np.exp(rng.standard_normal(160))), 1, 8192).astype(np.int64)
    step1 = W.build_step("noalloc_big", 16, 2, 1, int(lens1.sum()) + 4096,
                         [W.decode_spec(lens1)], seed=91, device="cuda")
    need1 = pka.decode_workspace_bytes(16, 2, 128, 1, step1.num_pages, 160, int(lens1.max()))
    announce(f"noalloc call 1: 160 requests, 16q/2kv, workspace need {need1} B")
    assert 4 << 20 < need1 <= 16 << 20
    decode_store_both(step1, list(range(0, 160, 9)) + [159])
    # second call: 16q/8kv (G=2), 12 requests, P=16: a smaller split plan over the
    # scratch the first call left behind
    lens2 = [700, 65, 1, 3000, 129, 64, 2047, 300, 901, 5, 1500, 4096]
    pages2 = sum(-(-L // 16) for L in lens2) + 16
    step2 = W.build_step("noalloc_small", 16, 8, 16, pages2, [W.decode_spec(lens2)], seed=92,
                         device="cuda")
    need2 = pka.decode_workspace_bytes(16, 8, 128, 16, pages2, 12, max(lens2))
    announce(f"noalloc call 2: 12 requests, 16q/8kv, P=16, workspace need {need2} B")
    assert 0 < need2 < need1
    decode_store_both(step2, None)
