#!/usr/bin/env python3
"""Benchmark of the quantized paged-KV decode step on one MI355X.

Default workload (the headline metric): INT4 split-KV decode at B=32,
Hq=32, Hk=8, D=128, block_size=16, seq_len ~ U[1024, 8192], 8 splits.
One step = write the step's new K/V token of every sequence into the paged
INT4 cache (tq_reshape_and_cache_int4, 32 tokens x 8 kv heads) + decode
attention over the whole cache (tq_decode_attention). Inputs are seeded
synthetic data already resident in HBM; the step rotates over enough cache
copies (> 512 MB in total) that the 256 MB Infinity Cache cannot serve
repeats.

Printed: one JSON line (rank 0). `value` is the step's algorithmic HBM
bytes / step time in TB/s. `roofline` covers the decode call (stage 1 +
stage 2 kernels), timed with HIP events on the stream it runs on.
`cpu_baseline` times the CPU oracle (tests' reference implementation) on a
bounded sample of the same step on the host cores, single-threaded and on
all the cores this process may use (at most 16), with the core count and
CPU model. `copy_calibration_TBps` is a 512 MiB device copy timed in the
same run. Every GPU time is the median of 5 event-timed runs.

Other workloads (--workload): llama8b_int4_8k, long_int4, tq_mixed_a,
tq_mixed_b, tq_fp8_values (the tq_mixed shape with FP8 keys and values),
tq_mixed_b_d256 (3-bit centroid keys and values at D=256), tq_mse4_u4 (the
tq_mixed shape with 4-bit centroid keys and 4-bit values), tq_mse3_fp8v (3-bit
centroid keys with FP8 values), tq_mixed_a_d256 (FP8 keys + 4-bit values at
D=256), write (65536
tokens x 8 heads x 128 bf16), tq_write_a / tq_write_b (the TurboQuant slot
writer on the same rows), fwht (1,048,576 rows), kpool (pooled-softmax key
compression: 262144 pools of 4 tokens), prefill_int4 (multi-query INT4
attention: 4 sequences of 1024 context + 1024 query tokens), tq_dequant
(bulk TurboQuant dequant of the tq_mixed cache to fp16), copy (device copy
used to calibrate the HBM byte counters).
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12  # bytes/s, MI355X HBM3E
HEADLINE = "INT4 split-KV decode attn: HBM TB/s (% of peak), µs/call at B=32, 8K ctx"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Events:
    """HIP events recorded on an explicit stream (torch.cuda.Event records on
    whichever stream it is given)."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def time(self, fn, n):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for i in range(n):
            fn(i)
        b.record(self.stream)
        b.synchronize()
        return a.elapsed_time(b) / n * 1e-3  # seconds per call

    def median(self, fn, n, reps=5):
        """Median over `reps` event-timed runs of n back-to-back calls (the
        call index keeps counting across runs, so cache copies keep
        rotating); returns (median, min, max) seconds per call."""
        ts = []
        for r in range(reps):
            ts.append(self.time(lambda i: fn(r * n + i), n))
        ts.sort()
        return ts[len(ts) // 2], ts[0], ts[-1]


def copy_calibration(torch, stream, warmup=3, n=20):
    """Device-to-device copy of 512 MiB on the same stream: the streaming
    rate this machine's HBM reaches with a plain copy (read + write bytes)."""
    dev = torch.device("cuda:0")
    nbytes = 512 * 2 ** 20
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(warmup):
        b.copy_(a)
    t, _, _ = Events(torch, stream).median(lambda i: b.copy_(a), n)
    del a, b
    return 2 * nbytes / t


def host_cpu():
    """Host CPU facts for the CPU baseline: logical CPUs, the ones this
    process may run on, and the model name."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count() or 1
    return dict(nproc=os.cpu_count() or 1, allowed=allowed, model=model)


# Worker threads of the CPU baselines: the host cores this process may use,
# at most 16 (the CPU share of one GPU on the measurement boxes).
CPU_THREAD_CAP = 16


def decode_bytes(w, splits_nonempty):
    kv = int(w.seq_lens.astype(np.int64).sum()) * w.hk * (w.d + 8)
    pages = int(sum((int(s) + w.block_size - 1) // w.block_size for s in w.seq_lens))
    parts = int(splits_nonempty.sum()) * w.hq * (w.d + 1) * 4 * 2
    qo = w.B * w.hq * (4 * w.d * 2 + 4) + w.B * 4
    return dict(kv=kv, partials=parts, q_out=qo, block_table=pages * 4, total=kv + parts + qo + pages * 4)


def profiled_traffic(name):
    """HBM bytes per call from a committed rocprofv3 counter summary
    (profiles/<name>.txt: FETCH_SIZE and WRITE_SIZE passes, scaled by the
    copy calibration). None when the summary is missing or the kernel
    sources it names have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name + ".txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if "traffic_bytes" not in fields or "sources_sha256" not in fields:
        return None
    h = hashlib.sha256()
    for src in fields.get("sources", "").split():
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != fields["sources_sha256"]:
        return None
    return int(fields["traffic_bytes"])


def nonempty_splits(seq_lens, S):
    out = []
    for s in seq_lens:
        s = int(s)
        if s == 0:
            out.append(0)
            continue
        L = (s + S - 1) // S
        out.append(sum(1 for k in range(S) if k * L < s))
    return np.array(out)


def run_int4(args, torch, tq, W, name):
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    w = W.decode_workload(name)
    if args.splits:
        w.num_splits = args.splits
    log("[bench] workload", name, "tokens", w.total_tokens, "splits", w.num_splits)
    kb, vb = W.kv_source(w)
    signs = torch.from_numpy(W.rht_signs(w.d)).to(dev)
    shape = (w.num_blocks, w.block_size, w.hk, w.d // 2)
    cache_bytes = int(np.prod(shape)) * 2 + int(np.prod(shape[:3])) * 8
    ncopies = max(2, -(-512 * 2 ** 20 // cache_bytes) + 1)
    key = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(dev)
    val = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(dev)
    slots = torch.from_numpy(w.slot_mapping).to(dev)
    sets = []
    for c in range(ncopies):
        kc = torch.empty(shape, dtype=torch.uint8, device=dev)
        vc = torch.empty_like(kc)
        ks = torch.empty(shape[:3], dtype=torch.float32, device=dev)
        vs = torch.empty_like(ks)
        tq.tq_reshape_and_cache_int4(key, val, kc, vc, slots, k_scale_cache=ks, v_scale_cache=vs,
                                     rht_signs=signs)
        sets.append((kc, vc, ks, vs))
    torch.cuda.synchronize()
    log("[bench] %d cache copies of %.1f MB written" % (ncopies, cache_bytes / 1e6))
    # the step's new token per sequence: the last position of each sequence
    last = np.cumsum(w.seq_lens.astype(np.int64)) - 1
    new_k, new_v = key[last].contiguous(), val[last].contiguous()
    new_slots = slots[last].contiguous()
    q = torch.from_numpy(W.query(w)).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    S = w.num_splits
    ws = torch.empty(tq.tq_decode_workspace_bytes(w.B, w.hq, w.hk, w.d, S) // 4, dtype=torch.float32,
                     device=dev)
    out = torch.empty(w.B, w.hq, w.d, dtype=torch.float32, device=dev)
    lse = torch.empty(w.B, w.hq, dtype=torch.float32, device=dev)
    del key, val

    sp = C.c_void_p(stream.cuda_stream)
    writes, decodes = [], []
    for kc, vc, ks, vs in sets:
        writes.append(tq.prepare_reshape(new_k, new_v, kc, vc, new_slots, k_scale_cache=ks,
                                         v_scale_cache=vs, rht_signs=signs))
        decodes.append(tq.prepare_decode(q, bt, sl, num_kv_splits=S, key_cache=kc, value_cache=vc,
                                         k_scale_cache=ks, v_scale_cache=vs, rht_signs=signs,
                                         workspace=ws, out=out, lse=lse,
                                         flags=(tq.FLAG_WIDE if args.wide else 0) |
                                         (tq.FLAG_GENERIC if args.generic else 0))[0])

    def decode(i):
        decodes[i % ncopies].run(sp)

    def step(i):
        writes[i % ncopies].run(sp)
        decodes[i % ncopies].run(sp)

    ev = Events(torch, stream)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    # decode call alone, HIP events on its stream: median of 5 runs
    t_dec, t_min, t_max = ev.median(decode, max(args.steps, 20))
    b = decode_bytes(w, nonempty_splits(w.seq_lens, S))
    wb = w.B * w.hk * (2 * w.d * 2 + (w.d + 8)) + w.B * 8
    step_bytes = b["total"] + wb
    res = dict(w=w, wall=wall, t_dec=t_dec, t_dec_range=(t_min, t_max), bytes=b,
               step_bytes=step_bytes, sets=sets, q=q, signs=signs)
    return res


def _cpu_rate(work, units, budget_s, threads):
    """Run work(i) over units 0, 1, ... (cycling) on `threads` threads until
    about budget_s seconds have passed; work returns the algorithmic bytes
    of its item. Returns (items, bytes, seconds). Each work item is one
    oracle call (ctypes releases the GIL)."""
    import concurrent.futures as cf
    done, nbytes, t0 = 0, 0, time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as pool:
        while time.perf_counter() - t0 < budget_s:
            batch = [(done + k) % units for k in range(threads)]
            nbytes += sum(pool.map(work, batch))
            done += len(batch)
    return done, nbytes, time.perf_counter() - t0


def cpu_baseline(work, units, budget_s, what):
    """The oracle on a bounded sample of the workload: single-thread, then
    on all the host cores this process may use (at most CPU_THREAD_CAP),
    each for about half of budget_s. Rates are algorithmic bytes per second
    (the same byte count as the GPU line), `value` the all-core one."""
    cpu = host_cpu()
    threads = max(1, min(CPU_THREAD_CAP, cpu["allowed"]))
    n1, b1, t1 = _cpu_rate(work, units, budget_s / 2, 1)
    nn, bn, tn = _cpu_rate(work, units, budget_s / 2, threads)
    r1 = b1 / t1
    rn = bn / tn
    return dict(value=rn / 1e12, unit="TB/s", cores=threads, kind="oracle",
                single_thread=r1 / 1e12, all_core=rn / 1e12, nproc=cpu["nproc"],
                cpus_allowed=cpu["allowed"], cpu_model=cpu["model"],
                sample="%s: %d items in %.1f s on 1 thread, %d items in %.1f s on %d threads "
                       "(the host's CPU share, at most %d)" % (
                           what, n1, t1, nn, tn, threads, CPU_THREAD_CAP))


def cpu_baseline_int4(res, W, budget_s):
    """The fp64 oracle decode of single (sequence, kv head) units -- all the
    query heads of one kv head of one sequence -- cycling over the batch,
    scaled to TB/s of the same KV bytes the GPU line counts."""
    import oracle
    w = res["w"]
    kc, vc, ks, vs = (t.cpu().numpy() for t in res["sets"][0])
    q = res["q"].cpu().numpy()
    signs = res["signs"].cpu().numpy()
    g = w.hq // w.hk
    units = [(b, h) for b in range(w.B) for h in range(w.hk)]
    kv_bytes = [int(w.seq_lens[b]) * (w.d + 8) for b, h in units]

    def work(i):
        b, h = units[i]
        rows = np.arange(b * w.hq + h * g, b * w.hq + (h + 1) * g, dtype=np.int32)
        oracle.int4_decode(q, kc, vc, ks, vs, w.block_table, w.seq_lens, signs, w.num_splits,
                           w.sm_scale, rows)
        return kv_bytes[i]

    return cpu_baseline(work, len(units), budget_s,
                        "fp64 oracle decode of (sequence, kv head) units of the %s batch "
                        "(%d query heads each), KV bytes" % (w.name, g))


def cpu_baseline_write(wl, W, budget_s):
    """The oracle INT4 cache writer on chunks of 512 tokens of the write
    workload (each into its own small cache), scaled to TB/s of the same
    algorithmic bytes as the GPU line (source rows read, codes and scale
    words written, slot indices read)."""
    import oracle
    T, hk, d = wl["key"].shape
    chunk = 512
    units = T // chunk
    signs = W.rht_signs(d)
    slots = wl["slot_mapping"]

    def work(i):
        sl = slots[i * chunk:(i + 1) * chunk]
        local = np.where(sl >= 0, np.arange(chunk, dtype=np.int64), -1)
        kc = np.zeros((chunk // 16, 16, hk, d // 2), np.uint8)
        vc = np.zeros_like(kc)
        ks = np.zeros((chunk // 16, 16, hk), np.float32)
        vs = np.zeros_like(ks)
        oracle.reshape_and_cache_int4(wl["key"][i * chunk:(i + 1) * chunk],
                                      wl["value"][i * chunk:(i + 1) * chunk], oracle.DT_BF16,
                                      local, signs, kc, vc, ks, vs)
        return int((sl >= 0).sum()) * hk * (2 * d * 2 + (d + 8)) + chunk * 8

    return cpu_baseline(work, units, budget_s,
                        "oracle reshape_and_cache_int4 of 512-token chunks of the 65536 x 8 x 128 "
                        "bf16 rows (5% skipped)")


def cpu_baseline_fwht(bits, budget_s):
    """The oracle fwht128_quant_fp8 on chunks of 4096 rows of the 1M-row
    input, scaled to TB/s of the same algorithmic bytes as the GPU line."""
    import oracle
    chunk = 4096
    units = bits.shape[0] // chunk

    def work(i):
        oracle.fwht128_quant_fp8(bits[i * chunk:(i + 1) * chunk])
        return chunk * (256 + 128 + 4)

    return cpu_baseline(work, units, budget_s,
                        "oracle fwht128_quant_fp8 of 4096-row chunks of the 1048576 x 128 bf16 rows")


# Secondary workloads time at least this many back-to-back calls per run: a
# run of a few milliseconds still sees the GPU's clocks ramping up after an
# idle spell (tens of milliseconds of load), which inflates per-call times
# by several percent.
MIN_TIMED_CALLS = 400


def _timed_calls(steps):
    return max(steps, MIN_TIMED_CALLS)


def set_min_timed_calls(n):
    """Counter-collection runs (one record per dispatch) time fewer calls."""
    global MIN_TIMED_CALLS
    MIN_TIMED_CALLS = max(1, int(n))


def _time_loop(torch, stream, fn, warmup, steps):
    """Median of 5 event-timed runs of max(steps, MIN_TIMED_CALLS) calls,
    after warmup."""
    for i in range(warmup):
        fn(i)
    return Events(torch, stream).median(fn, _timed_calls(steps))[0]


def run_other(args, torch, tq, W):
    """Secondary workloads: one JSON line each (not the headline metric)."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = C.c_void_p(stream.cuda_stream)
    name = args.workload
    if name == "write":
        wl = W.write_workload()
        T, hk, d = wl["key"].shape
        # enough source/cache copies to exceed the Infinity Cache
        per = T * hk * d * 2 * 2 + wl["num_blocks"] * 16 * hk * (d // 2 + 4) * 2
        ncopies = max(2, -(-1024 * 2 ** 20 // per))
        key = torch.from_numpy(wl["key"].view(np.int16)).view(torch.bfloat16).to(dev)
        val = torch.from_numpy(wl["value"].view(np.int16)).view(torch.bfloat16).to(dev)
        slots = torch.from_numpy(wl["slot_mapping"]).to(dev)
        signs = torch.from_numpy(W.rht_signs(d)).to(dev)
        calls = []
        for c in range(ncopies):
            k2, v2 = key.clone(), val.clone()
            kc = torch.zeros(wl["num_blocks"], 16, hk, d // 2, dtype=torch.uint8, device=dev)
            vc = torch.zeros_like(kc)
            ks = torch.zeros(wl["num_blocks"], 16, hk, dtype=torch.float32, device=dev)
            vs = torch.zeros_like(ks)
            calls.append(tq.prepare_reshape(k2, v2, kc, vc, slots, k_scale_cache=ks,
                                            v_scale_cache=vs, rht_signs=signs))
        t = _time_loop(torch, stream, lambda i: calls[i % ncopies].run(sp), args.warmup, args.steps)
        valid = int((wl["slot_mapping"] >= 0).sum())
        nbytes = valid * hk * (2 * d * 2 + (d + 8)) + T * 8
        line = dict(workload="write: tq_reshape_and_cache_int4 65536 tokens x 8 heads x 128 bf16, "
                             "5% slots skipped", us=t * 1e6, algorithmic_bytes=nbytes,
                    TBps=nbytes / t / 1e12, pct_peak=100 * nbytes / t / PEAK_HBM)
        if not args.no_cpu:
            line["cpu_baseline"] = cpu_baseline_write(wl, W, args.cpu_budget)
    elif name in ("tq_write_a", "tq_write_b"):
        wl = W.write_workload()
        T, hk, d = wl["key"].shape
        fmt = (tq.KEY_FP8, tq.VAL_U4) if name.endswith("a") else (tq.KEY_MSE3, tq.VAL_U3)
        sb = tq.tq_slot_bytes(d, *fmt)
        per = T * hk * d * 2 * 2 + wl["num_blocks"] * 16 * hk * sb
        ncopies = max(2, -(-1024 * 2 ** 20 // per))
        key = torch.from_numpy(wl["key"].view(np.int16)).view(torch.bfloat16).to(dev)
        val = torch.from_numpy(wl["value"].view(np.int16)).view(torch.bfloat16).to(dev)
        slots = torch.from_numpy(wl["slot_mapping"]).to(dev)
        cen = None
        if fmt[0] != tq.KEY_FP8:
            cen = torch.linspace(-0.2, 0.2, 8, device=dev)
        calls = []
        for c in range(ncopies):
            cache = torch.zeros(wl["num_blocks"], 16, hk, sb, dtype=torch.uint8, device=dev)
            calls.append(tq.prepare_encode(key.clone(), val.clone(), cache, slots, key_fmt=fmt[0],
                                           val_fmt=fmt[1], centroids=cen))
        t = _time_loop(torch, stream, lambda i: calls[i % ncopies].run(sp), args.warmup, args.steps)
        valid = int((wl["slot_mapping"] >= 0).sum())
        nbytes = valid * hk * (2 * d * 2 + sb) + T * 8
        line = dict(workload="%s: tq_encode_and_cache 65536 tokens x 8 heads x 128 bf16 -> %s "
                             "slots of %d B, 5%% slots skipped" % (
                                 name, "FP8 key / U4 value" if fmt[0] == tq.KEY_FP8
                                 else "3-bit centroid key / U3 value", sb),
                    us=t * 1e6, algorithmic_bytes=nbytes, TBps=nbytes / t / 1e12,
                    pct_peak=100 * nbytes / t / PEAK_HBM)
    elif name == "fwht":
        bits = W.fwht_rows()
        rows = bits.shape[0]
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        ncopies = 3
        xs = [x.clone() for _ in range(ncopies)]
        ys = [torch.empty(rows, 128, dtype=torch.uint8, device=dev) for _ in range(ncopies)]
        ss = [torch.empty(rows, dtype=torch.float32, device=dev) for _ in range(ncopies)]
        fn = tq.lib().fwht128_quant_fp8

        def call(i):
            j = i % ncopies
            tq._check(fn(xs[j].data_ptr(), rows, ys[j].data_ptr(), ss[j].data_ptr(), sp))
        t = _time_loop(torch, stream, call, args.warmup, args.steps)
        nbytes = rows * (256 + 128 + 4)
        line = dict(workload="fwht: fwht128_quant_fp8 1048576 rows x 128 bf16", us=t * 1e6,
                    algorithmic_bytes=nbytes, TBps=nbytes / t / 1e12,
                    pct_peak=100 * nbytes / t / PEAK_HBM)
        if not args.no_cpu:
            line["cpu_baseline"] = cpu_baseline_fwht(bits, args.cpu_budget)
    elif name == "kpool":
        wl = W.kpool_workload()
        n, P, hd = wl["slot_k"].shape
        bs = wl["block_size"]
        per = n * P * hd * 2 * 2 + wl["num_blocks"] * bs * (hd + 4)
        ncopies = max(2, -(-1024 * 2 ** 20 // per))
        sk = torch.from_numpy(wl["slot_k"].view(np.int16)).view(torch.bfloat16).to(dev)
        ss = torch.from_numpy(wl["slot_score"].view(np.int16)).view(torch.bfloat16).to(dev)
        ape = torch.from_numpy(wl["ape"]).to(dev)
        loc = torch.from_numpy(wl["loc"]).to(dev)
        calls = []
        for c in range(ncopies):
            cache = torch.zeros(wl["num_blocks"], bs, hd + 4, dtype=torch.uint8, device=dev)
            calls.append(tq.prepare_kpool(cache, sk.clone(), ss.clone(), ape, loc))
        t = _time_loop(torch, stream, lambda i: calls[i % ncopies].run(sp), args.warmup, args.steps)
        # per pool: P*128 bf16 keys and scores read, its location, one entry
        # (128 codes + 4-byte scale) written; the [P, 128] bias once
        nbytes = n * (P * hd * 2 * 2 + 8 + hd + 4) + P * hd * 4
        line = dict(workload="kpool: tq_kpool_compress_and_write_cache %d pools x %d tokens x %d, "
                             "bf16 keys and scores -> FP8 indexer entries (block %d)" % (n, P, hd, bs),
                    us=t * 1e6, algorithmic_bytes=nbytes, TBps=nbytes / t / 1e12,
                    pct_peak=100 * nbytes / t / PEAK_HBM)
    elif name == "prefill_int4":
        # chunked prefill at the Llama-3-8B head shape: 4 sequences, each with
        # 1024 cached context tokens and 1024 new query tokens
        ctx, ql = np.full(4, 1024), np.full(4, 1024)
        w = W.custom_decode_workload(12, 4, 32, 8, 128, 16, 1, ctx + ql)
        cu, q = W.prefill_queries(w, ql)
        g = torch.Generator(device=dev)
        g.manual_seed(5)
        shape = (w.num_blocks, w.block_size, w.hk, w.d // 2)
        kc = torch.randint(0, 256, shape, dtype=torch.uint8, device=dev, generator=g)
        vc = torch.randint(0, 256, shape, dtype=torch.uint8, device=dev, generator=g)
        # scale words: |scale| in [2^-6, 2^-2) with a zero point in the low nibble
        sc = torch.rand(shape[:3], device=dev, generator=g) * 0.24 + 0.016
        ks = (sc.view(torch.int32) & ~0xF | 7).view(torch.float32)
        vs = ks.clone()
        call, out = tq.prepare_prefill(
            torch.from_numpy(q).to(dev), kc, vc, torch.from_numpy(w.block_table).to(dev),
            torch.from_numpy(cu).to(dev), torch.from_numpy(w.seq_lens).to(dev),
            k_scale_cache=ks, v_scale_cache=vs,
            rht_signs=torch.from_numpy(W.rht_signs(w.d)).to(dev), sm_scale=w.sm_scale)
        t = _time_loop(torch, stream, lambda i: call.run(sp), args.warmup, args.steps)
        # the vector-ALU kernel (the path without a workspace), fewer calls
        vcall, _ = tq.prepare_prefill(
            torch.from_numpy(q).to(dev), kc, vc, torch.from_numpy(w.block_table).to(dev),
            torch.from_numpy(cu).to(dev), torch.from_numpy(w.seq_lens).to(dev),
            k_scale_cache=ks, v_scale_cache=vs,
            rht_signs=torch.from_numpy(W.rht_signs(w.d)).to(dev), sm_scale=w.sm_scale,
            workspace=None)
        for i in range(2):
            vcall.run(sp)
        tv = Events(torch, stream).median(lambda i: vcall.run(sp), 20)[0]
        pairs = int(sum(int(c) * int(n) + int(n) * (int(n) + 1) // 2 for c, n in zip(ctx, ql)))
        flops = 4 * pairs * w.hq * w.d
        line = dict(workload="prefill_int4: tq_prefill_attention_int4, 4 sequences x (1024 "
                             "context + 1024 query tokens), Hq=32 Hk=8 D=128 bs=16, INT4 K/V, "
                             "matrix-core path (query tokens as decode entries)",
                    us=t * 1e6, query_tokens_per_s=float(ql.sum()) / t,
                    visible_pairs=pairs, attention_TFLOPs=flops / t / 1e12,
                    vector_path_us=tv * 1e6, vector_path_TFLOPs=flops / tv / 1e12)
    elif name == "tq_dequant":
        # bulk dequant of the tq_mixed cache (B=16 Hk=4 D=128, 16384 tokens each,
        # FP8 keys + 4-bit values, 208-B slots) to fp16 K/V
        w = W.decode_workload("tq_mixed")
        sb = tq.tq_slot_bytes(w.d, tq.KEY_FP8, tq.VAL_U4)
        g = torch.Generator(device=dev)
        g.manual_seed(9)
        cache = torch.randint(0, 256, (w.num_blocks, w.block_size, w.hk, sb), dtype=torch.uint8,
                              device=dev, generator=g)
        cache[..., :w.d][(cache[..., :w.d] & 0x7F) == 0x7F] -= 1  # no E4M3 NaN codes
        # fp16 value scale 2^-4 and zero 0 (bits 0x2C00, 0x0000) after the indices
        cache[..., w.d + 64] = 0x00
        cache[..., w.d + 65] = 0x2C
        cache[..., w.d + 66:w.d + 68] = 0
        call, k, v = tq.prepare_full_dequant(cache, torch.from_numpy(w.block_table).to(dev),
                                             head_dim=w.d, key_fmt=tq.KEY_FP8, val_fmt=tq.VAL_U4,
                                             max_seq=int(w.seq_lens.max()))
        t = _time_loop(torch, stream, lambda i: call.run(sp), args.warmup, args.steps)
        rows = w.B * w.hk * int(w.seq_lens.max())
        nbytes = rows * (sb + 2 * w.d * 2) + w.block_table.size * 4
        line = dict(workload="tq_dequant: tq_full_dequant_kv B=16 Hk=4 D=128 16384 tokens, FP8 keys "
                             "+ U4 values (208-B slots) -> fp16 K/V", us=t * 1e6,
                    algorithmic_bytes=nbytes, TBps=nbytes / t / 1e12,
                    pct_peak=100 * nbytes / t / PEAK_HBM)
    elif name == "copy":
        n = 512 * 2 ** 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        t = _time_loop(torch, stream, lambda i: b.copy_(a), args.warmup, args.steps)
        line = dict(workload="copy: device-to-device copy of 512 MiB", us=t * 1e6,
                    read_bytes=n, write_bytes=n, TBps=2 * n / t / 1e12)
    elif name in TQ_DECODES:
        fmt, d = TQ_DECODES[name]
        fmt = tuple(getattr(tq, f) for f in fmt)
        w = W.decode_workload("tq_mixed", d=d)
        sb = tq.tq_slot_bytes(w.d, *fmt)
        shape = (w.num_blocks, w.block_size, w.hk, sb)
        nbytes_cache = int(np.prod(shape))
        ncopies = max(2, -(-512 * 2 ** 20 // nbytes_cache) + 1)
        g = torch.Generator(device=dev)
        g.manual_seed(3)
        kb = {tq.KEY_FP8: 8, tq.KEY_MSE3: 3, tq.KEY_MSE4: 4}[fmt[0]]
        vb = {tq.VAL_U3: 3, tq.VAL_U4: 4, tq.VAL_FP8: 8}[fmt[1]]
        kps = w.d if fmt[0] == tq.KEY_FP8 else (w.d * kb + 7) // 8 + 2
        vdb = (w.d * vb + 7) // 8
        caches = []
        for c in range(ncopies):
            cache = torch.randint(0, 256, shape, dtype=torch.uint8, device=dev, generator=g)
            if fmt[0] == tq.KEY_FP8:  # no NaN codes in the key bytes
                cache[..., :w.d] &= 0x77
            if fmt[1] == tq.VAL_FP8:  # nor in the value bytes
                cache[..., kps:kps + w.d] &= 0x77
            # fp16 scale / zero / norm fields: small positive values
            offs = ([kps + vdb, kps + vdb + 2] if fmt[1] != tq.VAL_FP8 else []) + \
                ([kps - 2] if fmt[0] != tq.KEY_FP8 else [])
            for off in offs:
                cache[..., off] = 0x00
                cache[..., off + 1] = 0x2C
            caches.append(cache)
        q = torch.from_numpy(W.query(w, bf16_valued=True)).to(dev)
        bt = torch.from_numpy(w.block_table).to(dev)
        sl = torch.from_numpy(w.seq_lens).to(dev)
        # an evenly spaced table, c[n - 1 - j] = -c[j] exactly (as in every
        # Lloyd-Max table), made on the host
        cen = torch.linspace(-0.2, 0.2, 1 << kb).to(dev) if fmt[0] != tq.KEY_FP8 else None
        ws = torch.empty(tq.tq_decode_workspace_bytes(w.B, w.hq, w.hk, w.d, w.num_splits) // 4,
                         dtype=torch.float32, device=dev)
        calls = [tq.prepare_decode(q, bt, sl, num_kv_splits=w.num_splits, kv_cache=c,
                                   key_fmt=fmt[0], val_fmt=fmt[1], centroids=cen,
                                   norm_correction=bool(args.norm_correction) and fmt[0] != tq.KEY_FP8,
                                   workspace=ws,
                                   flags=(tq.FLAG_WIDE if args.wide else 0) |
                                   (tq.FLAG_GENERIC if args.generic else 0))[0]
                 for c in caches]
        t = _time_loop(torch, stream, lambda i: calls[i % ncopies].run(sp), args.warmup, args.steps)
        slot_used = kps + vdb + (0 if fmt[1] == tq.VAL_FP8 else 4)  # padding not counted
        kv = int(w.seq_lens.sum()) * w.hk * slot_used
        parts = w.B * w.hq * w.num_splits * (w.d + 1) * 8
        nbytes = kv + parts + w.B * w.hq * (8 * w.d + 4)
        line = dict(workload="%s: B=16 Hq=32 Hk=4 D=%d seq 16384 S=32, %s keys + %s values%s" % (
                        name, w.d, TQ_KEY_NAMES[fmt[0]], TQ_VAL_NAMES[fmt[1]],
                        (", norm-corrected keys" if args.norm_correction and fmt[0] != tq.KEY_FP8 else "") +
                        (", generic kernel" if args.generic else "")), us=t * 1e6,
                    algorithmic_bytes=nbytes, TBps=nbytes / t / 1e12,
                    pct_peak=100 * nbytes / t / PEAK_HBM)
    else:
        raise SystemExit("unknown workload %s" % name)
    line.update(steps=args.steps, warmup=args.warmup,
                timing="us: median of 5 HIP-event runs of %d back-to-back calls" % _timed_calls(args.steps))
    print(json.dumps(line), flush=True)


# TurboQuant decode workloads: the tq_mixed shape (B=16 Hq=32 Hk=4, seq 16384) with the given slot format and D
TQ_DECODES = {
    "tq_mixed_a": (("KEY_FP8", "VAL_U4"), 128),
    "tq_mixed_b": (("KEY_MSE3", "VAL_U3"), 128),
    "tq_fp8_values": (("KEY_FP8", "VAL_FP8"), 128),
    "tq_mixed_b_d256": (("KEY_MSE3", "VAL_U3"), 256),
    "tq_mse4_u4": (("KEY_MSE4", "VAL_U4"), 128),
    "tq_mse3_fp8v": (("KEY_MSE3", "VAL_FP8"), 128),
    "tq_mixed_a_d256": (("KEY_FP8", "VAL_U4"), 256),
}
TQ_KEY_NAMES = {1: "FP8", 2: "3-bit centroid", 3: "4-bit centroid"}
TQ_VAL_NAMES = {1: "3-bit uniform", 2: "4-bit uniform", 3: "FP8"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_int4")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--min-calls", type=int, default=MIN_TIMED_CALLS,
                    help="secondary workloads: least calls per timed run (fewer for counter runs)")
    ap.add_argument("--splits", type=int, default=0, help="override num_kv_splits (sweeps)")
    ap.add_argument("--norm-correction", action="store_true",
                    help="TurboQuant decode workloads with centroid keys: the norm-corrected read")
    ap.add_argument("--generic", action="store_true",
                    help="decode workloads: force the generic (vector) kernel, for comparison")
    ap.add_argument("--wide", action="store_true",
                    help="decode through the 64-bit addressing variant (the one caches of "
                         "2 GiB and more take) whatever the cache size")
    args = ap.parse_args()
    set_min_timed_calls(args.min_calls)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path has no multi-GPU "
              "component in this build (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import quantized_paged_kv_tq_amd as tq
    from quantized_paged_kv_tq_amd import workloads as W
    tq.lib()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(2)

    if args.workload in ("llama8b_int4", "llama8b_int4_8k", "long_int4"):
        res = run_int4(args, torch, tq, W, args.workload)
        w, b = res["w"], res["bytes"]
        achieved = b["total"] / res["t_dec"]
        line = {
            "metric": HEADLINE,
            "value": round(res["step_bytes"] / res["wall"] / 1e12, 4),
            "unit": "TB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(res["wall"] * 1e3, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": "%s: B=%d Hq=%d Hk=%d D=%d block_size=%d seq_len %s "
                                   "(sum %d) num_kv_splits=%d, INT4 K/V" % (
                                       w.name, w.B, w.hq, w.hk, w.d, w.block_size,
                                       "U[1024,8192]" if w.name == "llama8b_int4" else str(int(w.seq_lens[0])),
                                       int(w.seq_lens.sum()), w.num_splits)
                                   + (", 64-bit addressing variant" if args.wide else "")
                                   + (", generic kernel" if args.generic else ""),
                       "global_batch": w.B, "seq_len": int(w.seq_lens.max()), "parallelism": "1 GPU"},
            "decode_us": round(res["t_dec"] * 1e6, 2),
            "decode_us_min_max": [round(res["t_dec_range"][0] * 1e6, 2),
                                  round(res["t_dec_range"][1] * 1e6, 2)],
            "timing": "decode_us: median of 5 HIP-event runs of %d back-to-back calls" % max(args.steps, 20),
            "decode_TBps": round(achieved / 1e12, 4),
            "decode_pct_peak": round(100 * achieved / PEAK_HBM, 2),
            "kv_only_TBps": round(b["kv"] / res["t_dec"] / 1e12, 4),
            "roofline": {"bound": "hbm", "kernel": "tq_decode_attention (stage 1 + stage 2)",
                         "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": round(achieved / PEAK_HBM, 4),
                         "traffic": profiled_traffic("decode_int4_" + w.name),
                         "algorithmic_bytes": b},
        }
        line["copy_calibration_TBps"] = round(copy_calibration(torch, torch.cuda.current_stream()) / 1e12, 4)
        if not args.no_cpu:
            log("[bench] cpu baseline")
            line["cpu_baseline"] = cpu_baseline_int4(res, W, args.cpu_budget)
        print(json.dumps(line), flush=True)
        return
    run_other(args, torch, tq, W)


if __name__ == "__main__":
    main()
