"""GPU parity with pools past 4 GiB: the used rows sit above byte offset 2^32.

The kernels address a pool row as slot * (Hkv * D * 2) bytes in 64-bit arithmetic. Here
the pools hold 1.25 * 2^20 slots of 4 KB (16 kv heads), 5 GiB each, and every request's
pages are drawn from above slot 2^20 (byte 2^32), with a few just below it, so a row
offset that wrapped at 32 bits would read the wrong row (or an unused NaN slot). The
oracle does not see the big pools: its result depends on the logical order of a
request's keys only (a pinned property), so it runs on compact host copies holding just
the used pages, with the page ids renumbered. store_kv, decode_store, decode and prefill
are each compared with it; the stored rows bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_25_amd as pka
from tests.gpu_common import announce, assert_close, dev_i32, host_u16

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 16, 128
ROW = HKV * D                      # bf16 elements per slot (4 KB)
SLOTS = (1 << 20) + (1 << 18)      # 5 GiB per pool; slot 2^20 starts at byte 2^32
NAN = np.uint16(0x7FC0)
SCALE = D ** -0.5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pka.lib()


def _bf16_bits(rng, shape):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


class Pools:
    """Big device pools (NaN everywhere but the cached rows) and compact host copies."""

    def __init__(self, rng, lens, page_size, cached):
        P = page_size
        self.P = P
        npages = [-(-int(L) // P) for L in lens]
        line = (1 << 20) // P                      # first page at or above byte 2^32
        low = min(4, sum(npages) // 4)             # a few pages just under the line
        high = rng.choice(np.arange(line, SLOTS // P), size=sum(npages) - low, replace=False)
        ids = rng.permutation(np.concatenate([high, np.arange(line - low, line)]))
        assert (ids >= line).sum() >= sum(npages) - low
        width = max(npages)
        self.table = np.zeros((len(lens), width), np.int32)       # big-pool page ids
        self.ctable = np.zeros((len(lens), width), np.int32)      # compact page ids
        k = 0
        for b, n in enumerate(npages):
            self.table[b, :n] = ids[k:k + n]
            self.ctable[b, :n] = np.arange(k, k + n)
            self.table[b, n:] = self.table[b, n - 1]
            self.ctable[b, n:] = self.ctable[b, n - 1]
            k += n
        cslots = sum(npages) * P
        self.kc = np.full((cslots, HKV, D), NAN, np.uint16)
        self.vc = np.full((cslots, HKV, D), NAN, np.uint16)
        self.k_pool = torch.full((SLOTS, HKV, D), int(NAN.view(np.int16)), dtype=torch.int16,
                                 device="cuda")
        self.v_pool = torch.full_like(self.k_pool, int(NAN.view(np.int16)))
        big, small = [], []
        for b, L in enumerate(lens):
            for j in range(int(cached[b])):        # the cached positions of request b
                big.append(self.slot(self.table, b, j))
                small.append(self.slot(self.ctable, b, j))
        big, small = np.array(big, np.int64), np.array(small, np.int64)
        kd, vd = _bf16_bits(rng, (len(big), HKV, D)), _bf16_bits(rng, (len(big), HKV, D))
        self.kc[small], self.vc[small] = kd, vd
        idx = torch.from_numpy(big).cuda()
        self.k_pool.view(SLOTS, ROW)[idx] = torch.from_numpy(kd.view(np.int16)).cuda().view(-1, ROW)
        self.v_pool.view(SLOTS, ROW)[idx] = torch.from_numpy(vd.view(np.int16)).cuda().view(-1, ROW)

    def slot(self, table, b, j):
        return int(table[b, j // self.P]) * self.P + j % self.P

    def rows(self, pool, slots):
        return host_u16(pool.view(SLOTS, ROW)[torch.from_numpy(np.asarray(slots, np.int64)).cuda()])


@pytest.mark.parametrize("page_size", [1, 16])
def test_decode_store_and_decode_above_4GiB(page_size):
    rng = np.random.default_rng(7 + page_size)
    lens = np.array([1, 17, 64, 65, 700, 2049, 4100], np.int32)
    announce(f"large pool decode P={page_size} lens={lens.tolist()}")
    pools = Pools(rng, lens, page_size, cached=lens - 1)
    B = len(lens)
    out_loc = np.array([pools.slot(pools.table, b, int(lens[b]) - 1) for b in range(B)], np.int32)
    c_loc = np.array([pools.slot(pools.ctable, b, int(lens[b]) - 1) for b in range(B)], np.int32)
    assert (out_loc >= (1 << 20)).sum() >= B - 1
    q = _bf16_bits(rng, (B, HQ, D))
    k_new, v_new = _bf16_bits(rng, (B, HKV, D)), _bf16_bits(rng, (B, HKV, D))
    t = lambda a: torch.from_numpy(a.view(np.int16)).cuda()
    kc, vc = oracle.store_kv_ref(pools.kc, pools.vc, k_new, v_new, c_loc)
    ref = oracle.decode_ref(q, kc, vc, pools.ctable, lens, page_size, SCALE)

    out = pka.paged_attn_decode_store(t(q), t(k_new), t(v_new), dev_i32(out_loc), pools.k_pool,
                                      pools.v_pool, dev_i32(pools.table), dev_i32(lens),
                                      int(lens.max()), page_size, SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(pools.rows(pools.k_pool, out_loc), k_new.reshape(B, ROW))
    assert np.array_equal(pools.rows(pools.v_pool, out_loc), v_new.reshape(B, ROW))
    assert_close(host_u16(out), ref, f"decode_store above 4 GiB, P={page_size}")

    out = pka.paged_attn_decode(t(q), pools.k_pool, pools.v_pool, dev_i32(pools.table),
                                dev_i32(lens), int(lens.max()), page_size, SCALE)
    torch.cuda.synchronize()
    assert_close(host_u16(out), ref, f"decode above 4 GiB, P={page_size}")
    del pools
    torch.cuda.empty_cache()


def test_store_and_prefill_above_4GiB():
    page_size = 16
    rng = np.random.default_rng(11)
    prefix = np.array([0, 333, 1000], np.int32)
    extend = np.array([200, 64, 129], np.int32)
    lens = prefix + extend
    announce(f"large pool prefill P={page_size} prefix={prefix.tolist()} extend={extend.tolist()}")
    pools = Pools(rng, lens, page_size, cached=prefix)
    B, T = len(lens), int(extend.sum())
    cu = np.concatenate([[0], np.cumsum(extend)]).astype(np.int32)
    out_loc = np.array([pools.slot(pools.table, b, int(prefix[b]) + i)
                        for b in range(B) for i in range(int(extend[b]))], np.int32)
    c_loc = np.array([pools.slot(pools.ctable, b, int(prefix[b]) + i)
                      for b in range(B) for i in range(int(extend[b]))], np.int32)
    q = _bf16_bits(rng, (T, HQ, D))
    k_new, v_new = _bf16_bits(rng, (T, HKV, D)), _bf16_bits(rng, (T, HKV, D))
    t = lambda a: torch.from_numpy(a.view(np.int16)).cuda()
    kc, vc = oracle.store_kv_ref(pools.kc, pools.vc, k_new, v_new, c_loc)
    ref = oracle.paged_attention_ref(q, kc, vc, pools.ctable, lens, prefix, extend, page_size,
                                     SCALE)

    pka.store_kv(t(k_new), t(v_new), dev_i32(out_loc), pools.k_pool, pools.v_pool, page_size)
    torch.cuda.synchronize()
    assert np.array_equal(pools.rows(pools.k_pool, out_loc), k_new.reshape(T, ROW))
    assert np.array_equal(pools.rows(pools.v_pool, out_loc), v_new.reshape(T, ROW))
    out = pka.paged_attn_prefill(t(q), pools.k_pool, pools.v_pool, dev_i32(pools.table),
                                 dev_i32(lens), dev_i32(prefix), dev_i32(extend), dev_i32(cu),
                                 int(extend.max()), int(lens.max()), page_size, SCALE)
    torch.cuda.synchronize()
    assert_close(host_u16(out), ref, "prefill above 4 GiB, P=16")
    del pools
    torch.cuda.empty_cache()
