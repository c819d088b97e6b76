"""Benchmark of the paged KV-cache attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]
    python bench.py --part WORKLOAD [--steps K] [--warmup W]   (one workload, for profiling)

Prints ONE JSON line. The headline workload is the offline-style decode batch
(Qwen3-0.6B heads 16q/8kv, d=128, bf16, batch 256, context lengths uniform in
[200, 2048], page size 1, slots scattered over a 2^20-slot pool). One step is the
whole decode step of the path: the store of the 256 new tokens' K/V rows and the
decode over all keys, made by pka_paged_attn_decode_store (the split decode kernel
with the store inside, then its merge pass); the same step as store_kv followed by
the decode call is timed beside it. `value` is the decode's algorithmic HBM bytes
(K+V of every attended token, q, out, page-table entries and seq_lens; the store's
bytes are reported separately) divided by the step's time, with inputs resident in
HBM and the caches flushed (a 1 GiB read) before every timed step.

The other workloads (chunked prefill over cached prefixes, the tensor-parallel
mixed step, long-context decode, tiny decode) are timed the same way and reported
under "parts": decode in GB/s against the 8 TB/s HBM peak, prefill in TFLOP/s
(4*D flops per unmasked (query, key) pair per q head) against the 2.5 PFLOP/s
dense bf16 MFMA peak.

Times come from HIP events recorded on the stream the kernels run on (torch's
current stream, which the binding passes to every call): a step's time between one
event before it and one after it; the per-call breakdown (store, decode, prefill) in a
second pass with an event after every call. The oracle (float64,
numpy) is timed on the host over the full decode batch as "cpu_baseline" (one BLAS
thread, and all the cores the process may use), on the chunked prefill as
"prefill_cpu_baseline", and on every other workload (bounded samples) under each
part's "oracle" record.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6
METRIC = "decode attn HBM GB/s (% peak) + prefill attn TFLOP/s (% MFMA peak), 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_b256_traffic.json")
PREFILL_COUNTERS_FILE = os.path.join(ROOT, "profiles", "prefill_counters.json")


def decode_bytes(part, step):
    """Algorithmic bytes of one decode call: K+V rows of every attended token, q, out,
    page-table entries and seq_lens."""
    d, hkv, hq = step.head_dim, step.num_kv_heads, step.num_q_heads
    seq = part.seq_lens.astype(np.int64)
    kv = int(seq.sum()) * hkv * d * 2 * 2
    qo = 2 * part.batch * hq * d * 2
    pt = 4 * int((-(-seq // step.page_size)).sum()) + 4 * part.batch
    return kv + qo + pt


def prefill_flops(part, step):
    """4*D flops per unmasked (query, key) pair per q head."""
    p = part.prefix_lens.astype(np.int64)
    e = part.extend_lens.astype(np.int64)
    pairs = int((e * p + e * (e + 1) // 2).sum())
    return 4 * step.head_dim * step.num_q_heads * pairs


def decode_flops(part, step):
    """4*D flops per (query, key) pair per q head, for context (decode is HBM-bound)."""
    return 4 * step.head_dim * step.num_q_heads * int(part.seq_lens.astype(np.int64).sum())


def prefill_bytes(part, step):
    """K+V rows of every referenced key plus q and out, for context (prefill is
    MFMA-bound)."""
    d, hkv, hq = step.head_dim, step.num_kv_heads, step.num_q_heads
    seq = part.seq_lens.astype(np.int64)
    return int(seq.sum()) * hkv * d * 4 + 2 * part.num_tokens * hq * d * 2


def store_bytes(step):
    rows = step.out_loc.size
    return rows * step.num_kv_heads * step.head_dim * 2 * 2 * 2 + 4 * rows


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_attention_25_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Runner:
    """Device-resident metadata and closures for one workload step. With `fused`, a
    decode-only step stores its new rows inside the decode launch
    (pka_paged_attn_decode_store) instead of a store_kv call before it."""

    def __init__(self, step, fused=False):
        import torch
        import paged_kv_attention_25_amd as pka
        self.step = step
        self.pka = pka
        self.fused = (fused and len(step.parts) == 1 and step.parts[0].kind == "decode"
                      and step.parts[0].batch == step.out_loc.size)
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        self.out_loc = i32(step.out_loc)
        self.meta = []
        for part in step.parts:
            m = dict(pt=i32(part.page_table), seq=i32(part.seq_lens))
            if part.kind == "decode":
                need = pka.decode_workspace_bytes(step.num_q_heads, step.num_kv_heads,
                                                  step.head_dim, step.page_size, step.num_pages,
                                                  part.batch, part.max_seq_len)
                m["ws"] = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
            else:
                m.update(pre=i32(part.prefix_lens), ext=i32(part.extend_lens),
                         cu=i32(part.cu_extend))
                need = pka.prefill_workspace_bytes(step.num_q_heads, step.num_kv_heads,
                                                   step.head_dim, step.page_size,
                                                   step.num_pages, part.batch, part.num_tokens,
                                                   part.max_extend)
                m["ws"] = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
            m["out"] = torch.empty_like(part.q)
            self.meta.append(m)

    def store(self):
        if self.fused:
            return
        s = self.step
        self.pka.store_kv(s.k_new, s.v_new, self.out_loc, s.k_pool, s.v_pool, s.page_size)

    def attend(self, i):
        s, part, m = self.step, self.step.parts[i], self.meta[i]
        if part.kind == "decode" and self.fused:
            self.pka.paged_attn_decode_store(part.q, s.k_new, s.v_new, self.out_loc, s.k_pool,
                                             s.v_pool, m["pt"], m["seq"], part.max_seq_len,
                                             s.page_size, s.scale, out=m["out"],
                                             workspace=m["ws"])
        elif part.kind == "decode":
            self.pka.paged_attn_decode(part.q, s.k_pool, s.v_pool, m["pt"], m["seq"],
                                       part.max_seq_len, s.page_size, s.scale, out=m["out"],
                                       workspace=m["ws"])
        else:
            self.pka.paged_attn_prefill(part.q, s.k_pool, s.v_pool, m["pt"], m["seq"], m["pre"],
                                        m["ext"], m["cu"], part.max_extend, part.max_seq_len,
                                        s.page_size, s.scale, out=m["out"], workspace=m["ws"])


PART_WARMUP = 60  # warmup steps of the workloads reported under "parts"
# ... and at least this much continuous work before their timing: under sustained
# matrix-core load the shader clock settles only after a few hundred ms (the prefill
# ran 301 us on its first timed pass after 300 calls and 268-269 us from then on, on
# one box), and a serving step runs at that steady state.
PART_WARM_SECONDS = 0.5


def time_step(runner, steps, warmup, flush, cold=True, warm_seconds=0.0):
    """Run warmup steps, then time `steps` steps twice. Pass 1 records one HIP event
    before and one after each step (the step's time: an event marker between calls
    holds the stream for a few µs, so none is placed inside the step). Pass 2 records
    an event after every call (store, then each attention part) for the per-call
    breakdown. A cache flush runs before each timed step, outside the events. Returns
    the per-call medians (ms, pass 2), the median step time (ms, pass 1) and the wall
    time of pass 1."""
    import torch
    nparts = len(runner.step.parts)

    def calls():
        runner.store()
        for i in range(nparts):
            runner.attend(i)

    for _ in range(warmup):
        calls()
    torch.cuda.synchronize()
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < warm_seconds:
        for _ in range(20):
            calls()
        torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        if cold:
            flush()
        ev[k][0].record()
        calls()
        ev[k][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nparts + 2)] for _ in range(steps)]
    for k in range(steps):
        if cold:
            flush()
        e = evs[k]
        e[0].record()
        runner.store()
        e[1].record()
        for i in range(nparts):
            runner.attend(i)
            e[i + 2].record()
    torch.cuda.synchronize()
    per_step = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(nparts + 1)] for e in evs])
    seg = np.median(per_step, axis=0)
    return seg, total, wall


def two_stream_step_us(runner, steps, warmup, flush):
    """A mixed step (a decode part and a prefill part) with the decode on a second
    stream: store_kv on the launch stream, then the decode on the second stream (after
    the store) beside the prefill on the launch stream; the step ends when both have.
    Both streams run at the default priority. Median step time, µs, over `steps`
    cold-cache steps."""
    import torch
    s1 = torch.cuda.current_stream()
    s2 = torch.cuda.Stream()
    kinds = [p.kind for p in runner.step.parts]
    di, pi = kinds.index("decode"), kinds.index("prefill")

    def calls():
        runner.store()
        stored = torch.cuda.Event()
        stored.record(s1)
        with torch.cuda.stream(s2):
            s2.wait_event(stored)
            runner.attend(di)
        runner.attend(pi)
        s1.wait_stream(s2)

    for _ in range(warmup):
        calls()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for k in range(steps):
        flush()
        ev[k][0].record()
        calls()
        ev[k][1].record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3


def prefill_alone_us(runner, idx, calls, warm_seconds):
    """The prefill call of part `idx` alone at a settled shader clock: after
    `warm_seconds` of continuous prefill calls, `calls` back-to-back calls between one
    pair of events (no cache flush, no marker between calls); mean µs per call."""
    import torch
    for _ in range(5):
        runner.attend(idx)
    torch.cuda.synchronize()
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < warm_seconds:
        for _ in range(20):
            runner.attend(idx)
        torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(calls):
        runner.attend(idx)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / calls


def _host_u16(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint16)


def _oracle_loop(fn, min_seconds, threads):
    """Run fn() with `threads` BLAS threads until at least min_seconds have passed."""
    from threadpoolctl import threadpool_limits
    reps = 0
    with threadpool_limits(threads):
        t0 = time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_seconds:
                return reps, el


def step_part_view(part, idx):
    """The requests `idx` of a decode part, as a part of their own (metadata only)."""
    from paged_kv_attention_25_amd import workloads as W
    return W.AttnPart(kind="decode", seq_lens=part.seq_lens[idx],
                      prefix_lens=part.prefix_lens[idx], extend_lens=part.extend_lens[idx],
                      cu_extend=np.arange(len(idx) + 1, dtype=np.int32),
                      page_table=part.page_table[idx], q=None, row_offset=0)


def oracle_for_part(name, step, min_seconds=2.0):
    """The oracle timed on a bounded sample of one workload's attention calls, with as
    many BLAS threads as the process may use. Decode samples are whole requests and are
    charged the decode's algorithmic bytes; prefill samples are whole requests or a
    window of tokens (an exact sub-problem) and are charged their algorithmic flops."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    kp, vp = _host_u16(step.k_pool), _host_u16(step.v_pool)
    out = {}
    for part in step.parts:
        q = _host_u16(part.q)
        if part.kind == "decode":
            idx = np.arange(part.batch)
            if name == "long_decode":
                idx = idx[::8]                      # 4 of the 32 requests
            sub = step_part_view(part, idx)
            reps, el = _oracle_loop(
                lambda: oracle.decode_ref(q[idx], kp, vp, sub.page_table, sub.seq_lens,
                                          step.page_size, step.scale), min_seconds, cores)
            nbytes = decode_bytes(sub, step)
            out["decode"] = {"value": round(nbytes * reps / el / 1e9, 4), "unit": "GB/s",
                             "cores": cores, "kind": "oracle",
                             "us_per_call": round(el / reps * 1e6, 1),
                             "sample": f"{len(idx)} of {part.batch} requests, {reps} pass(es) "
                                       f"in {el:.1f} s, float64 numpy"}
        else:
            if name == "chunked_prefill":
                bsel = np.arange(0, part.batch, 4)  # 8 of the 32 requests
                wins = [(int(b), 0, int(part.extend_lens[b])) for b in bsel]
                what = f"{len(bsel)} of {part.batch} requests (every 4th), all their rows"
            else:
                e = int(part.extend_lens[0])
                wins = [(0, e - 1024, e)]           # the last 1024 tokens: the heaviest rows
                what = "the chunk's last 1024 tokens (an exact sub-problem)"
            rows = np.concatenate([np.arange(int(part.cu_extend[b]) + a,
                                             int(part.cu_extend[b]) + c) for b, a, c in wins])
            bidx = np.array([w[0] for w in wins])
            pre = np.array([int(part.prefix_lens[b]) + a for b, a, c in wins])
            ext = np.array([c - a for b, a, c in wins])
            reps, el = _oracle_loop(
                lambda: oracle.paged_attention_ref(q[rows], kp, vp, part.page_table[bidx],
                                                   pre + ext, pre, ext, step.page_size,
                                                   step.scale), min_seconds, cores)
            flops = 4 * step.head_dim * step.num_q_heads * int((ext * pre +
                                                                ext * (ext + 1) // 2).sum())
            out["prefill"] = {"value": round(flops * reps / el / 1e12, 6), "unit": "TFLOP/s",
                              "cores": cores, "kind": "oracle",
                              "sample": f"{what}, {reps} pass(es) in {el:.1f} s, float64 numpy, "
                                        "same flop accounting as the GPU figure"}
    return out


QWEN3_06B_LAYERS = 28   # decoder layers of Qwen3-0.6B, the model whose heads tiny_decode has


def graph_vs_eager(runner, steps, flush):
    """The pages capture the decode step in a graph to cut CPU launch overhead. Times
    the tiny decode step (one decode_store call) eagerly and as a replayed HIP graph:
    GPU time per step with the host far ahead (events around the step, caches flushed
    before it) and wall time per step back to back (the host issues step after step,
    as a serving loop does). The same for a step over all 28 layers of the model (28
    calls, each on its own layer's pools), eager against one graph of the 28 calls."""
    import torch
    s = runner.step
    part = s.parts[0]

    def capture(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        return g

    def gpu_us(fn):
        ts = []
        for _ in range(steps):
            flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    def wall_us(fn, n=200):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / n

    def one():
        runner.attend(0)

    g1 = capture(one)
    # 28 layers: each layer's decode_store writes its own pools
    pools = [(s.k_pool.clone(), s.v_pool.clone()) for _ in range(QWEN3_06B_LAYERS)]
    m = runner.meta[0]
    outs = [torch.empty_like(part.q) for _ in range(QWEN3_06B_LAYERS)]

    def layers():
        for (kp, vp), o in zip(pools, outs):
            runner.pka.paged_attn_decode_store(part.q, s.k_new, s.v_new, runner.out_loc, kp, vp,
                                               m["pt"], m["seq"], part.max_seq_len, s.page_size,
                                               s.scale, out=o, workspace=m["ws"])

    gl = capture(layers)
    rec = {"graph_step_us": round(gpu_us(g1.replay), 2),
           "back_to_back_wall_us_per_step": {"eager": round(wall_us(one), 2),
                                             "graph": round(wall_us(g1.replay), 2)},
           f"{QWEN3_06B_LAYERS}_layers": {
               "gpu_us_per_step": {"eager": round(gpu_us(layers), 2),
                                   "graph": round(gpu_us(gl.replay), 2)},
               "back_to_back_wall_us_per_step": {"eager": round(wall_us(layers, 50), 2),
                                                 "graph": round(wall_us(gl.replay, 50), 2)}},
           "note": "gpu_us: events around one step with the host far ahead (after a cache "
                   "flush); back_to_back_wall: host wall time per step over consecutive "
                   "steps (the launch-overhead regime the graph is for)"}
    del gl, g1, pools, outs
    return rec


def cpu_baseline(step, min_seconds=10.0):
    """The oracle timed on the host over the whole decode batch, repeated until at least
    `min_seconds` have passed: with one BLAS thread (the reported figure) and with as many
    BLAS threads as this process may use (`all_cores`)."""
    import oracle
    from threadpoolctl import threadpool_limits
    part = step.parts[0]
    kp = step.k_pool.cpu().numpy().view(np.uint16)
    vp = step.v_pool.cpu().numpy().view(np.uint16)
    q = part.q.cpu().numpy().view(np.uint16)

    def timed(threads, seconds=min_seconds):
        reps = 0
        with threadpool_limits(threads):
            t0 = time.perf_counter()
            while True:
                oracle.decode_ref(q, kp, vp, part.page_table, part.seq_lens, step.page_size,
                                  step.scale)
                reps += 1
                el = time.perf_counter() - t0
                if el >= seconds:
                    break
        return decode_bytes(part, step) * reps / el / 1e9, reps, el

    gbs, reps, el = timed(1)
    cores = len(os.sched_getaffinity(0))
    gbs_n, reps_n, el_n = timed(cores, min_seconds / 2)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"full decode_b256 batch (256 requests), {reps} pass(es) in {el:.1f} s, "
                      "float64 numpy, one BLAS thread, same byte accounting as value",
            "all_cores": {"value": round(gbs_n, 4), "unit": "GB/s", "cores": cores,
                          "sample": f"the same, {reps_n} pass(es) in {el_n:.1f} s, "
                                    f"{cores} BLAS threads (the oracle's per-request, "
                                    "per-head products are small, so threads add little)"}}


def prefill_counters_for(kernel_hash):
    if not os.path.exists(PREFILL_COUNTERS_FILE):
        return None
    with open(PREFILL_COUNTERS_FILE) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_hash:
        return None
    return rec.get("workloads")


def traffic_for(kernel_hash):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_hash:
        return None      # counters were taken on an older kernel
    return rec.get("bytes_per_launch")


COPY_BYTES = 512 << 20   # the calibration copy: 512 MiB read, 512 MiB written


def _dispatch_counters(csv_dir, counter):
    """Per-dispatch values of one counter from a rocprofv3 counter_collection.csv:
    {kernel name: [(value, grid size) per dispatch, ...]}."""
    import csv
    import glob
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {csv_dir}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], r["Dispatch_Id"], int(r["Grid_Size"]))
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _, grid), v in per.items():
        out.setdefault(name, []).append((v, grid))
    return out


def write_traffic(fetch_dir, write_dir):
    """HBM bytes per decode launch on decode_b256 from two counter runs of
    `bench.py --quick --calibration-copy` (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch). Each counter is scaled by what it reads for the 512 MiB copy."""
    fetch = _dispatch_counters(fetch_dir, "FETCH_SIZE")
    write = _dispatch_counters(write_dir, "WRITE_SIZE")

    def mean_of(d, tag, largest_grid=False):
        vals = [vg for name, vs in d.items() if tag in name for vg in vs]
        if largest_grid:   # the 512 MiB copies, not the small metadata uploads
            g = max(grid for _, grid in vals) if vals else 0
            vals = [(v, grid) for v, grid in vals if grid == g]
        if not vals:
            raise SystemExit(f"no dispatch of a kernel named *{tag}*")
        return sum(v for v, _ in vals) / len(vals)

    kib = 1024.0
    fetch_scale = COPY_BYTES / (mean_of(fetch, "copyBuffer", True) * kib)
    write_scale = COPY_BYTES / (mean_of(write, "copyBuffer", True) * kib)
    f_split, f_merge = mean_of(fetch, "decode_split_kernel"), mean_of(fetch, "decode_merge_kernel")
    w_split, w_merge = mean_of(write, "decode_split_kernel"), mean_of(write, "decode_merge_kernel")
    total = ((f_split + f_merge) * fetch_scale + (w_split + w_merge) * write_scale) * kib
    rec = {"source_hash": source_hash("decode.hip", "pka_device.h"), "workload": "decode_b256",
           "kernels": "decode_split_kernel<true> (decode with the store) + decode_merge_kernel",
           "bytes_per_launch": int(round(total)),
           "fetch_kib": {"split": round(f_split, 1), "merge": round(f_merge, 1)},
           "write_kib": {"split": round(w_split, 1), "merge": round(w_merge, 1)},
           "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
           "calibration": "rocclr copyBuffer of 512 MiB in the same process",
           "commands": ["rocprofv3 --pmc FETCH_SIZE -d <fetch_dir> --output-format csv -- "
                        "python3 bench.py --quick --steps 3 --warmup 1 --no-cpu-baseline "
                        "--calibration-copy",
                        "rocprofv3 --pmc WRITE_SIZE -d <write_dir> --output-format csv -- "
                        "python3 bench.py --quick --steps 3 --warmup 1 --no-cpu-baseline "
                        "--calibration-copy",
                        "python3 bench.py --traffic-from <fetch_dir> <write_dir>"]}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def _dispatch_rows(csv_dir, counters):
    """Per-dispatch counter values and durations from rocprofv3 counter CSVs:
    {kernel name: [{counter: value, ..., "ns": duration}, ...]}."""
    import csv
    import glob
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {csv_dir}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] not in counters:
                    continue
                key = (r["Kernel_Name"], fn, r["Dispatch_Id"])
                d = per.setdefault(key, {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                                         "grid": int(r["Grid_Size"])})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _, _), d in per.items():
        out.setdefault(name, []).append(d)
    return out


def write_prefill_counters(workload, busy_dir, fetch_dir, write_dir):
    """MFMA busy fraction, shader clock and HBM bytes per prefill launch of one workload
    from three rocprofv3 counter runs of `bench.py --part W --calibration-copy`
    (SQ_VALU_MFMA_BUSY_CYCLES + GRBM_GUI_ACTIVE, then FETCH_SIZE, then WRITE_SIZE); the
    byte counters are scaled by what they read for the 512 MiB copy in the same run."""
    busy = _dispatch_rows(busy_dir, ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"))
    fetch = _dispatch_rows(fetch_dir, ("FETCH_SIZE",))
    write = _dispatch_rows(write_dir, ("WRITE_SIZE",))

    def rows(d, tag, largest_grid=False):
        vals = [v for name, vs in d.items() if tag in name for v in vs]
        if largest_grid and vals:
            g = max(v["grid"] for v in vals)
            vals = [v for v in vals if v["grid"] == g]
        if not vals:
            raise SystemExit(f"no dispatch of a kernel named *{tag}*")
        return vals

    b = [r for r in rows(busy, "prefill_kernel")]
    xcds = 8       # GRBM_GUI_ACTIVE is summed over the XCDs
    simds = 1024   # 256 CUs x 4 SIMDs
    active = np.mean([r["GRBM_GUI_ACTIVE"] / xcds for r in b])
    mfma = np.mean([r["SQ_VALU_MFMA_BUSY_CYCLES"] for r in b])
    ns = np.mean([r["ns"] for r in b])
    kib = 1024.0
    fscale = COPY_BYTES / (np.mean([r["FETCH_SIZE"] for r in rows(fetch, "copyBuffer", True)]) * kib)
    wscale = COPY_BYTES / (np.mean([r["WRITE_SIZE"] for r in rows(write, "copyBuffer", True)]) * kib)
    rd = np.mean([r["FETCH_SIZE"] for r in rows(fetch, "prefill_kernel")]) * kib * fscale
    wr = np.mean([r["WRITE_SIZE"] for r in rows(write, "prefill_kernel")]) * kib * wscale
    h = source_hash("prefill.hip", "pka_device.h")
    rec = {"source_hash": h, "workloads": {}}
    if os.path.exists(PREFILL_COUNTERS_FILE):
        with open(PREFILL_COUNTERS_FILE) as f:
            old = json.load(f)
        if old.get("source_hash") == h:
            rec = old
    rec["workloads"][workload] = {
        "mfma_busy": round(float(mfma / (active * simds)), 4),
        "shader_clock_ghz": round(float(active / ns), 3),
        "duration_us_under_counters": round(float(ns / 1e3), 1),
        "hbm_bytes": int(round(rd + wr)), "hbm_read_bytes": int(round(rd)),
        "hbm_write_bytes": int(round(wr)),
        "fetch_scale": round(float(fscale), 4), "write_scale": round(float(wscale), 4),
        "dispatches": len(b)}
    rec["commands"] = [
        "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE -d <busy_dir> "
        "--output-format csv -- python3 bench.py --part W --steps 3 --warmup 1 "
        "--no-cpu-baseline --calibration-copy",
        "rocprofv3 --pmc FETCH_SIZE -d <fetch_dir> --output-format csv -- (same command)",
        "rocprofv3 --pmc WRITE_SIZE -d <write_dir> --output-format csv -- (same command)",
        "python3 bench.py --prefill-counters-from W <busy_dir> <fetch_dir> <write_dir>"]
    with open(PREFILL_COUNTERS_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def calibration_copy(flush):
    """Two plain device copies of COPY_BYTES: the reference for the traffic counters."""
    import torch
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        flush()
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


# Decode-only workloads first: right after the prefill workloads' sustained MFMA load,
# a decode runs a few percent slow for longer than its warmup.
PART_NAMES = ("long_decode", "tiny_decode", "chunked_prefill", "tp4_mixed")


def time_part(name, steps, warmup, flush, log, cpu=True, warm_seconds=PART_WARM_SECONDS):
    """Time one of the non-headline workloads; per-segment medians in its record; with
    `cpu`, the oracle on a bounded sample of the same inputs under "oracle"."""
    import torch
    from paged_kv_attention_25_amd import workloads as W
    log(f"{name}: generating inputs")
    st = W.WORKLOADS[name](device="cuda", fill="zero")
    r = Runner(st, fused=True)
    torch.cuda.synchronize()
    seg, tot, _ = time_step(r, steps, warmup, flush, warm_seconds=warm_seconds)
    if r.fused:
        # The fused step and store_kv + decode, timed alternately (a second time each)
        # so that neither gains from the order; each reports the mean of its two medians.
        ru = Runner(st)
        _, tot_u1, _ = time_step(ru, steps, warmup, flush)
        _, tot_2, _ = time_step(r, steps, 5, flush)
        _, tot_u2, _ = time_step(ru, steps, 5, flush)
        tot, tot_u = (tot + tot_2) / 2, (tot_u1 + tot_u2) / 2
        del ru
    rec = {"step_us": round(tot * 1e3, 2)}
    if r.fused:
        rec["store"] = "inside the decode launch (pka_paged_attn_decode_store)"
    else:
        rec.update(store_us=round(seg[0] * 1e3, 2),
                   store_GBs=round(store_bytes(st) / (seg[0] * 1e-3) / 1e9, 1))
    for i, p in enumerate(st.parts):
        # a fused step is its one decode call: its time is the step's (no event inside)
        us = tot * 1e3 if r.fused else seg[i + 1] * 1e3
        if p.kind == "decode":
            # decode bytes only; a fused launch's store is reported beside them
            nbytes = decode_bytes(p, st)
            gbs = nbytes / (us * 1e-6) / 1e9
            rec["decode_us"] = round(us, 2)
            rec["decode_GBs"] = round(gbs, 1)
            rec["decode_frac_hbm"] = round(gbs / HBM_PEAK_GBS, 4)
            rec["decode_bytes"] = nbytes
            if r.fused:
                rec["store_bytes_in_call"] = store_bytes(st)
                rec["call_GBs_incl_store"] = round((nbytes + store_bytes(st)) /
                                                   (us * 1e-6) / 1e9, 1)
            rec["decode_TFLOPs_context"] = round(decode_flops(p, st) / (us * 1e-6) / 1e12, 2)
        else:
            tf = prefill_flops(p, st) / (us * 1e-6) / 1e12
            rec["prefill_us"] = round(us, 2)
            rec["prefill_TFLOPs"] = round(tf, 1)
            rec["prefill_frac_mfma"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
            rec["prefill_flops"] = prefill_flops(p, st)
            rec["prefill_GBs_context"] = round(prefill_bytes(p, st) / (us * 1e-6) / 1e9, 1)
            # context: the same call alone, back to back, once the clock has settled
            ua = prefill_alone_us(r, i, 50, max(warm_seconds, 0.5))
            ta = prefill_flops(p, st) / (ua * 1e-6) / 1e12
            rec["prefill_alone"] = {
                "us": round(ua, 2), "TFLOPs": round(ta, 1),
                "frac_mfma": round(ta / MFMA_BF16_PEAK_TFLOPS, 4),
                "how": "the prefill call alone: 50 back-to-back calls after half a second "
                       "of continuous prefill work, no cache flush, one event pair"}
    if r.fused:
        rec["unfused_step_us"] = round(tot_u * 1e3, 2)   # store_kv, then decode
    if name == "tiny_decode":
        rec.update(graph_vs_eager(r, steps, flush))
    kinds = {p.kind for p in st.parts}
    if kinds == {"decode", "prefill"}:
        # the same step with the decode beside the prefill on a second stream
        rec["two_stream_step_us"] = round(two_stream_step_us(r, steps, 10, flush), 2)
    if cpu:
        log(f"{name}: oracle on a sample")
        rec["oracle"] = oracle_for_part(name, st)
    log(f"{name}: {rec}")
    del r, st
    torch.cuda.empty_cache()
    return rec


PAGE_SIZES = (1, 16, 32, 64)


def page_size_sweep(steps, warmup, flush, log, warm_seconds=PART_WARM_SECONDS):
    """decode_b256 (the decode_store step) and chunked_prefill with the pool cut into
    pages of 1, 16, 32 and 64 slots: the same requests, pages drawn at random. The
    kernels take any page size at run time (powers of two by shift and mask)."""
    import torch
    from paged_kv_attention_25_amd import workloads as W
    out = {"decode_b256": {}, "chunked_prefill": {}}
    for P in PAGE_SIZES:
        st = W.decode_b256(device="cuda", fill="zero", page_size=P)
        r = Runner(st, fused=True)
        torch.cuda.synchronize()
        _, tot, _ = time_step(r, steps, warmup, flush, warm_seconds=warm_seconds)
        nbytes = decode_bytes(st.parts[0], st)   # decode bytes only, as the headline
        out["decode_b256"][f"P{P}"] = {"step_us": round(tot * 1e3, 2),
                                       "GBs": round(nbytes / (tot * 1e-3) / 1e9, 1)}
        del r, st
        torch.cuda.empty_cache()
    for P in PAGE_SIZES:
        st = W.chunked_prefill(device="cuda", fill="zero", page_size=P)
        r = Runner(st)
        torch.cuda.synchronize()
        seg, _, _ = time_step(r, steps, max(warmup, PART_WARMUP), flush,
                              warm_seconds=warm_seconds)
        us = seg[1] * 1e3
        tf = prefill_flops(st.parts[0], st) / (us * 1e-6) / 1e12
        out["chunked_prefill"][f"P{P}"] = {"prefill_us": round(us, 2),
                                           "TFLOPs": round(tf, 1)}
        del r, st
        torch.cuda.empty_cache()
    log(f"page sizes: {out}")
    return out


def host_sched_bench(log, decode_steps=20):
    """Host-side metadata producer (csrc/sched.cpp) on the decode_b256 request mix: 256
    prompts, lengths U[200, 2048], all starting with one 128-token system prompt, page
    size 1, a 2^20-page pool, radix cache, 8192-token prefill batches. Times (host
    µs, C calls made directly on preallocated buffers): the prefill batches that take
    every prompt in, a decode step (256 pushed tokens + the decode batch), finishing
    every request (its pages join the cache), and admitting 256 new requests of the same
    mix against that cache (prefix matches). The oracle (oracle/prefix_cache_ref.py)
    runs the prefill and decode part of the same stream beside it."""
    import ctypes
    from paged_kv_attention_25_amd import sched as S
    from oracle.prefix_cache_ref import PrefixCacheRef
    rng = np.random.default_rng(2)
    B, W = 256, 2048 + decode_steps + 1
    system = rng.integers(0, 32000, 128)

    def prompts():
        return [np.concatenate([system, rng.integers(0, 32000, int(n) - 128)]).astype(np.int32)
                for n in rng.integers(200, 2049, B)]

    first, second = prompts(), prompts()
    nxt = rng.integers(0, 32000, (decode_steps, B)).astype(np.int32)
    s = S.Scheduler(1, 1 << 20, "radix", 8192, max_batch=B, table_width=W, max_tokens=8192)
    L, h, c, bufs = s.raw()
    for a in bufs.values():   # fault the output buffers in before timing
        a.fill(1)
    ids = np.arange(B, dtype=np.int64)
    tc = time.perf_counter

    def prefill_all(offset, reqs):
        t0 = tc()
        for i, p in enumerate(reqs):
            L.pka_sched_add_request(h, offset + i, p.ctypes.data, int(p.size))
        t1 = tc()
        nb = 0
        while True:
            assert L.pka_sched_prefill_batch(h, ctypes.byref(c)) == 0
            if c.batch == 0:
                break
            nb += 1
        return (t1 - t0) * 1e6 / B, (tc() - t1) * 1e6, nb

    add_us, pre_us, n_pre = prefill_all(0, first)
    t0 = tc()
    entries = 0
    for k in range(decode_steps):
        assert L.pka_sched_push_tokens(h, ids.ctypes.data, nxt[k].ctypes.data, B) == 0
        assert L.pka_sched_decode_batch(h, ctypes.byref(c)) == 0 and c.batch == B
        entries += int(bufs["seq_lens"][:B].sum())
    dec_us = (tc() - t0) * 1e6 / decode_steps
    t0 = tc()
    for i in range(B):
        assert L.pka_sched_finish(h, i) == 0
    fin_us = (tc() - t0) * 1e6 / B
    add2_us, pre2_us, n_pre2 = prefill_all(B, second)
    st = s.stats()
    s.close()

    ref = PrefixCacheRef(1, 1 << 20, "radix", 8192)
    t0 = tc()
    for i, p in enumerate(first):
        ref.add_request(i, p.tolist())
    while ref.prefill_batch(B, 8192):
        pass
    t1 = tc()
    for k in range(decode_steps):
        for i in range(B):
            ref.push_token(i, int(nxt[k, i]))
        ref.decode_batch(B, 8192)
    t2 = tc()
    rec = {"workload": "decode_b256 request mix: 256 prompts U[200,2048] sharing a 128-token "
                       "system prompt, page_size 1, 2^20 pages, radix, 8192-token chunks",
           "prefill_batches": n_pre, "prefill_all_us": round(pre_us, 1),
           "prefill_us_per_batch": round(pre_us / n_pre, 1),
           "add_request_us": round(add_us, 2),
           "decode_step_us": round(dec_us, 1),
           "decode_step_page_table_entries": entries // decode_steps,
           "finish_us_per_request": round(fin_us, 2),
           "second_wave": {"prefill_all_us": round(pre2_us, 1), "prefill_batches": n_pre2,
                           "cached_pages": st["cached_pages"], "locked_pages": st["locked_pages"]},
           "oracle": {"prefill_all_us": round((t1 - t0) * 1e6, 1),
                      "decode_step_us": round((t2 - t1) * 1e6 / decode_steps, 1),
                      "note": "counts pages only: builds no page table"},
           "unit": "host us"}
    log(f"host_sched: {rec}")
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--hot", action="store_true", help="also report hot-cache times")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run two 512 MiB device copies (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the decode_b256 traffic record from two counter runs, then exit")
    ap.add_argument("--prefill-counters-from", nargs=4,
                    metavar=("WORKLOAD", "BUSY_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the prefill counter record of one workload from three counter "
                         "runs, then exit")
    ap.add_argument("--warm-seconds", type=float, default=PART_WARM_SECONDS,
                    help="continuous work before each timing (default %(default)s s; counter "
                         "runs that need no steady clock can pass 0)")
    ap.add_argument("--part", choices=PART_NAMES,
                    help="time only this workload (its warmup is --warmup), print its record, "
                         "exit (for profiling one workload)")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(*args.traffic_from)
        return
    if args.prefill_counters_from:
        write_prefill_counters(*args.prefill_counters_from)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the attention path here runs on one GPU only; --gpus must "
                          "be 1 (sharding across GPUs is a design note, not implemented)"}))
        sys.exit(2)

    import torch
    import paged_kv_attention_25_amd as pka
    from paged_kv_attention_25_amd import workloads as W
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    pka.lib()
    torch.cuda.set_device(0)
    # Cold caches without unrelated write-back: reading 1 GiB evicts the 4 MB L2s and
    # the 256 MB Infinity Cache with clean lines (a write-based flush would leave
    # dirty lines whose write-back would be charged to the timed kernels).
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush_sink = torch.empty((), dtype=torch.float32, device="cuda")
    flush = lambda: torch.sum(flush_buf, dim=0, out=flush_sink)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.part:
        if args.calibration_copy:
            calibration_copy(flush)
        print(json.dumps({"part": args.part,
                          **time_part(args.part, args.steps, args.warmup, flush, log,
                                      warm_seconds=args.warm_seconds,
                                      cpu=not args.no_cpu_baseline)}),
              flush=True)
        return

    # --- headline: decode_b256 ------------------------------------------------------
    log("decode_b256: generating inputs")
    step = W.decode_b256(device="cuda", fill="zero")
    run = Runner(step, fused=True)
    part = step.parts[0]
    torch.cuda.synchronize()
    seg, total_ms, wall = time_step(run, args.steps, args.warmup, flush,
                                    warm_seconds=args.warm_seconds)
    dec_bytes = decode_bytes(part, step)
    st_bytes = store_bytes(step)
    # decode bytes only (the store inside the same launch is reported beside them)
    value = dec_bytes / (total_ms * 1e-3) / 1e9
    launch_bytes = dec_bytes
    launch_ms = total_ms   # the step is the one decode_store call (split + merge)
    dec_gbs = launch_bytes / (launch_ms * 1e-3) / 1e9
    log(f"decode_b256: step {total_ms*1e3:.1f} us; {dec_gbs:.0f} GB/s")
    khash = source_hash("decode.hip", "pka_device.h")
    roofline = {"bound": "hbm",
                "kernel": "decode_split_kernel<store> + decode_merge_kernel",
                "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": traffic_for(khash),
                "algorithmic_bytes_per_launch": launch_bytes,
                "store_bytes_per_launch_not_counted": st_bytes,
                "avg_launch_us": round(launch_ms * 1e3, 2),
                "launch": "one pka_paged_attn_decode_store call (split kernel with the store "
                          "inside, then the merge kernel), timed with HIP events on its stream"}
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(total_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v; lengths and page permutations seeded)",
        "config": {"workload": "decode_b256: Qwen3-0.6B heads 16q/8kv, d=128, batch 256, "
                               "context U[200,2048], page_size 1, 2^20-slot pool; "
                               "step = decode_store (split decode with the store of the 256 "
                               "new rows inside) + merge",
                   "batch": part.batch, "sum_context": int(part.seq_lens.sum()),
                   "decode_bytes_per_step": dec_bytes, "store_bytes_per_step": st_bytes,
                   "step_GBs_incl_store": round((dec_bytes + st_bytes) / (total_ms * 1e-3) / 1e9,
                                                1),
                   "decode_TFLOPs_context": round(decode_flops(part, step) /
                                                  (total_ms * 1e-3) / 1e12, 2),
                   "timing": "HIP events on the launch stream, caches flushed before each step; "
                             "median over the timed steps, after half a second of continuous "
                             "steps",
                   "wall_s_timed_region_incl_flush": round(wall, 4)},
        "roofline": roofline,
    }
    if args.calibration_copy:
        calibration_copy(flush)
    if args.hot:
        _, tot_h, _ = time_step(run, args.steps, 0, flush, cold=False)
        result["config"]["hot_cache_decode_GBs"] = round(launch_bytes / (tot_h * 1e-3) / 1e9, 1)
    if not args.quick:
        # the same step as two calls: store_kv, then the decode
        run_u = Runner(step)
        seg_u, tot_u, _ = time_step(run_u, args.steps, args.warmup, flush)
        result["config"]["unfused_step"] = {
            "step_us": round(tot_u * 1e3, 2),
            "value_GBs": round(dec_bytes / (tot_u * 1e-3) / 1e9, 1),
            "with_an_event_after_each_call": {"store_us": round(seg_u[0] * 1e3, 2),
                                              "decode_us": round(seg_u[1] * 1e3, 2)}}
        del run_u

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on decode_b256")
        result["cpu_baseline"] = cpu_baseline(step)
    else:
        result["cpu_baseline"] = None
    del run, step
    torch.cuda.empty_cache()

    parts = {}
    if not args.quick:
        for name in PART_NAMES:
            parts[name] = time_part(name, args.steps, max(args.warmup, PART_WARMUP), flush, log,
                                    cpu=not args.no_cpu_baseline,
                                    warm_seconds=args.warm_seconds)
        parts["host_sched"] = host_sched_bench(log)
        parts["page_sizes"] = page_size_sweep(args.steps, args.warmup, flush, log,
                                              warm_seconds=args.warm_seconds)
        cp = parts["chunked_prefill"]
        result["prefill"] = {"workload": "chunked_prefill: Qwen3-14B heads 40q/8kv, 32 requests, "
                                         "prefixes U[0,4096], 8192 new tokens, page_size 16",
                             "value": cp["prefill_TFLOPs"], "unit": "TFLOP/s",
                             "peak": MFMA_BF16_PEAK_TFLOPS, "frac": cp["prefill_frac_mfma"]}
        counters = prefill_counters_for(source_hash("prefill.hip", "pka_device.h"))
        cw = (counters or {}).get("chunked_prefill", {})
        result["prefill_roofline"] = {
            "bound": "mfma", "kernel": "prefill_plan_kernel + prefill_kernel",
            "achieved": cp["prefill_TFLOPs"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": cp["prefill_frac_mfma"],
            "algorithmic_flops_per_launch": cp["prefill_flops"],
            "avg_launch_us": cp["prefill_us"],
            "launch": "one pka_paged_attn_prefill call, timed with HIP events on its stream",
            "mfma_busy": cw.get("mfma_busy"), "shader_clock_ghz": cw.get("shader_clock_ghz"),
            "traffic": cw.get("hbm_bytes"),
            "counters": "profiles/prefill_counters.json (rocprofv3 on the same source), or "
                        "null when the kernel changed since they were taken"}
        if "oracle" in cp:
            result["prefill_cpu_baseline"] = cp["oracle"]["prefill"]
    result["parts"] = parts
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
