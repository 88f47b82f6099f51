"""Decode-step benchmark for paged decode attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step is one decode step of the whole path over the Llama-3-8B-shaped batch (64 sequences,
32 query heads, 8 KV heads, head_dim 128, page_size 16, bf16, contexts uniform in [512, 4096]),
made by one call of pkv_paged_decode_step (one kernel launch):
  1. paged KV append of each sequence's new token at position L - 1;
  2. attention of every sequence's query over its L tokens through the page table, the batch's
     tiles split evenly over the GPU's workgroups;
  3. log-sum-exp merge of the sequences that span several workgroups, into the bf16 output.
Inputs are seeded synthetic data, resident in HBM before timing starts.  The pools rotate over
several replicas so that no step finds the previous step's KV in the 256 MB Infinity Cache.

Timing: first a settle phase, untimed and reported on its own (`settle` in the line): real steps
until --settle-ms of host time (200 ms by default) have passed, because the device needs some tens
of milliseconds of continuous work to reach its steady clock and power state (after 10 steps the
timed steps read about 2 us longer than after 200, on the same device; a decode loop runs in the
steady state).  Then W untimed warmup steps (200 by default), then the timed region, K steps
launched back to back between two HIP
events on the launch stream (their average is the step kernel's average launch duration, and the
host clock around the same region gives the step rate), then K more steps each bracketed by its
own event pair for the median / p10 / p90 (an event pair per launch adds a few us to each).

Prints one JSON line: whole-step throughput in algorithmic GB/s (KV rows of every live token once,
q, out, page-table entries and the append rows), decode tokens/s (= sequences per step / step
time), the roofline of the dominant kernel (and the HBM traffic that rocprofv3 counters measured
for it, when those were taken on the current kernel source), a plain copy's and a plain read
stream's rate on the same device, every workload of the suite on its own paths (`configs`), and
the fp64 CPU oracle's rate on the host for reference.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention HBM GB/s (% of peak) + decode tokens/sec, 1 MI355X"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed steps before the warmup, for at least this much host time, so "
                         "that the device reaches its steady clock state (0 disables)")
    ap.add_argument("--config", type=int, default=2, help="workload index (default: 2)")
    ap.add_argument("--path", choices=["step", "split", "single", "cascade", "multiquery",
                                       "multiquery-step"],
                    default="step",
                    help="cascade: shared-prefix decode (prefix-shared workloads only); "
                         "multiquery: --q-tokens new tokens per sequence, causal, over fixed "
                         "partitions; multiquery-step: the same through the balanced step")
    ap.add_argument("--q-tokens", type=int, default=8,
                    help="multiquery paths: query tokens per sequence")
    ap.add_argument("--partition-tokens", type=int, default=None)
    ap.add_argument("--rope", action="store_true",
                    help="step path: rotate the new key and the query in the same launch "
                         "(rotary cache with base 500000)")
    ap.add_argument("--replicas", type=int, default=None,
                    help="pool replicas rotated per step (default: enough for >= 2 GB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum host time spent timing the CPU oracle (0 disables it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload sweep (every workload of the suite, its own paths)")
    ap.add_argument("--config-steps", type=int, default=50, help="timed calls per path in the sweep")
    ap.add_argument("--config-warmup", type=int, default=200)
    return ap.parse_args()


def step_bytes(w, partition_tokens, path):
    """Algorithmic bytes of one step and of its dominant kernel launch: every live token's K and
    V rows once, q, out, the live page-table entries and lengths, the append (new rows read and
    written) and, for the fixed-partition split, its partials (written and read back).  The fused
    step's piece partials are not counted: they are this implementation's, not the method's."""
    import numpy as np
    cfg = w.cfg
    e = cfg.elem_bytes
    B, Hq, D, Hkv, PS = cfg.batch, cfg.num_q_heads, cfg.head_dim, cfg.num_kv_heads, cfg.page_size
    L = np.maximum(w.context_lens.astype(np.int64), 0)
    kv = int(L.sum()) * 2 * Hkv * D * e
    q = out = B * Hq * D * e
    table = int((-(-L // PS)).sum()) * 4 + B * 4
    append = 2 * (2 * B * Hkv * D * e)
    if path == "split":
        nparts = -(-L // partition_tokens)
        partials = int(nparts.sum()) * Hq * (D + 1) * 4
        kernel = kv + q + table + partials            # partial-attention launch
        step = kv + q + out + table + append + 2 * partials + B * 4
    elif path == "step":
        kernel = step = kv + q + out + table + append   # one launch does all of it
    elif path == "multiquery":
        # K and V read once per sequence for all its query tokens; q and out per token; each
        # (sequence, token) row's partials written and read back.
        T = w.q_tokens
        Lj = np.maximum(L[:, None] - T + 1 + np.arange(T)[None, :], 0)
        partials = int((-(-Lj // partition_tokens)).sum()) * Hq * (D + 1) * 4
        qo = B * T * Hq * D * e
        kernel = kv + qo + table + partials             # partition launch
        step = kv + 2 * qo + table + 2 * partials + B * 4   # no append in this step
        return dict(kv=kv, step=step, kernel=kernel)
    elif path == "multiquery-step":
        # One launch: K and V once per sequence for all its query tokens, q and out per token.
        qo = B * w.q_tokens * Hq * D * e
        kernel = step = kv + 2 * qo + table
        return dict(kv=kv, step=step, kernel=kernel)
    elif path == "cascade":
        # The shared prefix pages are read once: unique KV bytes, plus every partition's partial
        # written and read back by the merge.
        P = w.shared_pages * PS
        uniq = (P + int(np.maximum(L - P, 0).sum())) * 2 * Hkv * D * e
        nparts = -(-L // partition_tokens)
        partials = int(nparts.sum()) * Hq * (D + 1) * 4
        kernel = uniq + q + out + table + 2 * partials + B * 4
        step = kernel + append
        return dict(kv=uniq, step=step, kernel=kernel)
    else:
        kernel = kv + q + out + table
        step = kernel + append
    return dict(kv=kv, step=step, kernel=kernel)


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "step_kernel_llama3-8b-bf16-b64_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_203_amd", "csrc", f)
                  for f in ("pkv_kernels.hip", "pkv_device.h", "pkv_launch.h", "pkv_arrival.h",
                            "pkv_prefix_body.h")] + \
                 [os.path.join(ROOT, "paged_kv_cache_203_amd", "build.py")]   # the compile flags


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the step kernel from the committed counter summary, or None when
    it is missing, covers another workload, or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            fields = dict(l.split(":", 1) for l in f.read().splitlines() if l.startswith("- ") and ":" in l)
    except OSError:
        return None
    get = lambda k: fields.get("- " + k, "").strip().strip("`")
    if get("workload") != workload or get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(get("hbm_bytes_per_launch"))
    except ValueError:
        return None


def copy_calibration(nbytes=2 << 30, reps=20):
    """A plain device copy of `nbytes` into another buffer (torch's copy kernel): the read + write
    rate, and the kernel the counter calibration reads."""
    import torch
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    log(f"plain copy: {nbytes / 2**30:.1f} GiB read + write, {ms:.3f} ms/launch, {gbs:.0f} GB/s")
    del a, b
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": round(ms, 5), "gbs": round(gbs, 1)}


def read_calibration(pkv, nbytes=4 << 30, reps=20):
    """The library's plain read stream over `nbytes` (each byte read once per launch): the read
    bandwidth this device reaches, the practical ceiling beside the 8 TB/s peak."""
    import torch
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").random_()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        pkv.read_stream(buf, sink)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        pkv.read_stream(buf, sink)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"plain read stream: {nbytes / 2**30:.1f} GiB, {ms:.3f} ms/launch, {gbs:.0f} GB/s")
    del buf
    return {"bytes_read": nbytes, "ms": round(ms, 5), "gbs": round(gbs, 1)}


def cpu_info():
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    return {"cpu": model, "affinity_cores": affinity, "os_cpu_count": os.cpu_count()}


def cpu_threads():
    """Host threads for the oracle: the affinity cores, capped at 16."""
    return max(1, min(16, cpu_info()["affinity_cores"]))


def run_oracle_rows(w, pools, threads):
    """The fp64 oracle over all rows of `w` against `pools`, rows spread over `threads` host
    threads (NumPy releases the interpreter lock inside its array operations); BLAS is limited to
    one thread per call, so `threads` is the core count the oracle uses."""
    import numpy as np
    import oracle as O
    import workloads as W
    from concurrent.futures import ThreadPoolExecutor
    B = w.cfg.batch
    chunks = [list(range(B))[i::threads] for i in range(min(threads, B))]

    def part(rows):
        sub = W.subset_rows(w, rows)
        O.paged_decode_attention(sub.q, pools[0], pools[1], sub.page_table, sub.context_lens,
                                 sub.scale, sub.dtype)

    with ThreadPoolExecutor(len(chunks)) as ex:
        list(ex.map(part, chunks))


def blas_limits():
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        import contextlib
        return contextlib.nullcontext()


def cpu_baseline(w, extra_new, seconds):
    """Time the fp64 oracle (append + attention) on the host over a bounded sample: whole steps
    of the workload, repeated until `seconds` have passed."""
    import numpy as np
    import oracle as O
    k_new, v_new, append_lens = extra_new
    threads = cpu_threads()
    with blas_limits():
        n = 0
        t0 = time.perf_counter()
        while True:
            kp, vp = O.paged_kv_append(w.k_pool, w.v_pool, k_new, v_new, w.page_table, append_lens)
            run_oracle_rows(w, (kp, vp), threads)
            n += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = (time.perf_counter() - t0) / n
    kv = int(np.maximum(w.context_lens.astype(np.int64), 0).sum()) * w.kv_bytes_per_token()
    info = cpu_info()
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "tokens_per_s": round(w.cfg.batch / dt, 3), "s_per_step": round(dt, 4),
            "sample": (f"{n} whole {w.cfg.name} step(s) (append + attention, all "
                       f"{w.cfg.batch} rows), float64 NumPy, rows over {threads} host threads, "
                       f"BLAS 1 thread per call"),
            "blas_threads_per_call": 1, **info}


def timed(fn, K, W, stream, settle_ms=0.0):
    """Run fn(i) untimed for at least `settle_ms` of host time (the device's steady state) and
    then W more times, then K times back to back between two events on `stream` (the timed
    region), then K more times with an event pair around each call (the spread).  Returns the
    per-call averages of the region (events and host wall clock) and the median, p10 and p90 of
    the individually bracketed calls."""
    import numpy as np
    import torch
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        for i in range(20):
            fn(i)
        torch.cuda.synchronize()
    for i in range(W):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        fn(W + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = e0.elapsed_time(e1) / K
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for i in range(K):
        evs[i][0].record(stream)
        fn(W + K + i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in evs])
    return {"wall_us": wall * 1e6 / K, "region_us": region_ms * 1e3,
            "median_us": float(np.median(per)) * 1e3, "p10_us": float(np.percentile(per, 10)) * 1e3,
            "p90_us": float(np.percentile(per, 90)) * 1e3, "mean_bracketed_us": float(per.mean()) * 1e3}


def to_device(arr, dtype, device):
    import numpy as np
    import torch
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


class Prepared:
    """One workload on the device: q, table, lengths, the new rows, and `R` replicas of the pools
    (rotated per call so that the 256 MB Infinity Cache never holds the next call's KV)."""

    def __init__(self, w, replicas, dev):
        import numpy as np
        import torch
        from workloads.generate import STREAM_KNEW, STREAM_VNEW, fill_normal
        cfg = w.cfg
        self.w, self.cfg = w, cfg
        B, Hkv, D = cfg.batch, cfg.num_kv_heads, cfg.head_dim
        if cfg.append:
            k_new, v_new, append_lens = w.k_new, w.v_new, w.append_lens
        else:
            # The step writes its own token: the new row lands at position L - 1, so that
            # attention covers exactly the workload's context lengths.
            k_new = fill_normal((B, Hkv, D), cfg.dtype, w.seed, STREAM_KNEW)
            v_new = fill_normal((B, Hkv, D), cfg.dtype, w.seed, STREAM_VNEW)
            append_lens = (w.context_lens - 1).astype(np.int32)
        self.new_rows = (k_new, v_new, append_lens)
        self.q = to_device(w.q, cfg.dtype, dev)
        self.table = torch.from_numpy(w.page_table).to(dev)
        self.lens = torch.from_numpy(w.context_lens).to(dev)
        self.alens = torch.from_numpy(append_lens).to(dev)
        self.kn = to_device(k_new, cfg.dtype, dev)
        self.vn = to_device(v_new, cfg.dtype, dev)
        k0 = to_device(w.k_pool, cfg.dtype, dev)
        v0 = to_device(w.v_pool, cfg.dtype, dev)
        self.pool_bytes = 2 * k0.numel() * k0.element_size()
        self.R = replicas or min(64, max(1, math.ceil((2 << 30) / self.pool_bytes)))
        self.pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(self.R - 1)]
        self.out = torch.empty_like(self.q)
        self.scale = float(w.scale)

    def release(self):
        self.pools = None


def config_sweep(pkv, dev, stream, read_gbs, K, W, cpu_seconds, settle_ms):
    """Every workload of the suite on its own paths: median / p10 / p90 per call, algorithmic
    GB/s, % of 8 TB/s and of this run's read-stream ceiling, decode tokens/s; pools rotated (and,
    where the KV fits in the Infinity Cache, also the same buffers every call); the fp64 oracle
    timed once per workload on the host.  Each path settles (--settle-ms) and warms up before its
    timed region, as the headline does."""
    import numpy as np
    import torch
    import oracle as O
    import workloads as W_
    res = {}
    for idx in (1, 2, 3, 4, 5):
        t_gen = time.perf_counter()
        cfg = W_.config(idx)
        w = W_.make_workload(cfg)
        log(f"[configs] {cfg.name}: generated in {time.perf_counter() - t_gen:.1f}s")
        pr = Prepared(w, None, dev)
        ws = torch.zeros(pkv.decode_step_workspace_bytes(pr.q, pr.pools[0][0], pr.table),
                         dtype=torch.uint8, device=dev)
        B = cfg.batch
        entry = {"description": cfg.description, "batch": B, "live_tokens": w.logical_tokens(),
                 "pool_replicas": pr.R, "paths": {}}
        PS = cfg.page_size
        P = cfg.partition_tokens or 512

        def rec(name, fn, nbytes, same_buffer=False, extra=None):
            r = timed(fn, K, W, stream, settle_ms)
            d = {"bytes": nbytes, "avg_us": round(r["region_us"], 3), "wall_us": round(r["wall_us"], 3),
                 "median_us": round(r["median_us"], 3), "p10_us": round(r["p10_us"], 3),
                 "p90_us": round(r["p90_us"], 3)}
            gbs = nbytes / (r["region_us"] * 1e-6) / 1e9
            d.update(gbs=round(gbs, 1), pct_of_hbm_peak=round(100 * gbs / HBM_PEAK_GBS, 2),
                     pct_of_read_stream=round(100 * gbs / read_gbs, 2) if read_gbs else None,
                     decode_tokens_per_s=round(B / (r["region_us"] * 1e-6), 1))
            if extra:
                d.update(extra)
            if same_buffer:
                r2 = timed(lambda i: fn(0), K, W, stream, settle_ms)
                d["same_buffer_avg_us"] = round(r2["region_us"], 3)
                d["same_buffer_gbs"] = round(nbytes / (r2["region_us"] * 1e-6) / 1e9, 1)
            entry["paths"][name] = d
            log(f"[configs] {cfg.name} {name}: {d['avg_us']:.1f} us/call, {d['gbs']:.0f} GB/s "
                f"({d['pct_of_hbm_peak']:.1f}% of 8 TB/s)"
                + (f", same buffers {d['same_buffer_avg_us']:.1f} us" if same_buffer else ""))

        kn, vn = pr.kn, pr.vn
        fits_cache = pr.pool_bytes < (1 << 30)

        def step(i):
            kp, vp = pr.pools[i % pr.R]
            pkv.paged_decode_step(pr.q, kp, vp, pr.table, pr.alens, pr.scale, k_new=kn, v_new=vn,
                                  out=pr.out, workspace=ws)

        nb = step_bytes(w, P, "step")
        extra = {}
        if cfg.lengths[0] == "prefix":
            uniq = w.unique_tokens() * w.kv_bytes_per_token()
            extra = {"effective_gbs_logical_bytes": None, "unique_kv_bytes": uniq}
        rec("step", step, nb["step"], same_buffer=fits_cache, extra=extra)
        if cfg.lengths[0] == "prefix":
            d = entry["paths"]["step"]
            d["effective_gbs_logical_bytes"] = d["gbs"]
            # headline for the shared-prefix batch: the unique physical bytes
            ub = nb["step"] - nb["kv"] + uniq
            d["unique_bytes"] = ub
            d["gbs"] = round(ub / (d["avg_us"] * 1e-6) / 1e9, 1)
            d["pct_of_hbm_peak"] = round(100 * d["gbs"] / HBM_PEAK_GBS, 2)
            # the shared-prefix (cascade) decode over the same batch
            Pc = 256
            maxp = pkv.partitions_needed(PS, w.page_table.shape[1], Pc)
            po = torch.empty((B, cfg.num_q_heads, maxp, cfg.head_dim), dtype=torch.float32, device=dev)
            pl = torch.empty((B, cfg.num_q_heads, maxp), dtype=torch.float32, device=dev)
            prefix_tokens = w.shared_pages * PS
            prefix_pages = torch.from_numpy(np.ascontiguousarray(w.page_table[0, :w.shared_pages])).to(dev)

            def cascade(i):
                kp, vp = pr.pools[i % pr.R]
                pkv.paged_decode_cascade(pr.q, kp, vp, prefix_pages, prefix_tokens, pr.table, pr.lens,
                                         Pc, pr.scale, out=pr.out, partial_out=po, partial_lse=pl)

            rec("cascade", cascade, step_bytes(w, Pc, "cascade")["kernel"], same_buffer=fits_cache,
                extra={"partition_tokens": Pc, "note": "without the append (attention only)"})
        if cfg.append:
            def separate(i):
                kp, vp = pr.pools[i % pr.R]
                pkv.paged_kv_append(kn, vn, kp, vp, pr.table, pr.alens)
                pkv.paged_decode_attention(pr.q, kp, vp, pr.table, pr.lens, pr.scale, pr.out)
            rec("append_then_single_pass", separate, nb["step"], same_buffer=fits_cache,
                extra={"note": "two launches: pkv_paged_kv_append, then pkv_paged_decode_attention"})
        if cfg.partition_tokens:
            maxp = pkv.partitions_needed(PS, w.page_table.shape[1], P)
            po = torch.empty((B, cfg.num_q_heads, maxp, cfg.head_dim), dtype=torch.float32, device=dev)
            pl = torch.empty((B, cfg.num_q_heads, maxp), dtype=torch.float32, device=dev)

            def split(i):
                kp, vp = pr.pools[i % pr.R]
                pkv.paged_decode_attention_partial(pr.q, kp, vp, pr.table, pr.lens, P, pr.scale, po, pl, maxp)
                pkv.lse_merge(po, pl, pr.lens, P, PS, w.page_table.shape[1], out=pr.out)

            append_bytes = 2 * (2 * B * cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes)
            rec("split_kv_and_merge", split, step_bytes(w, P, "split")["step"] - append_bytes,
                extra={"partition_tokens": P, "note": "attention only: partial launch + merge launch"})
        pr.release()
        del ws
        torch.cuda.empty_cache()
        # the oracle, once per workload (best of three for the tiny one)
        if cpu_seconds > 0:
            threads = cpu_threads()
            k_new, v_new, append_lens = pr.new_rows
            best = None
            with blas_limits():
                for _ in range(3 if idx == 1 else 1):
                    t0 = time.perf_counter()
                    kp, vp = O.paged_kv_append(w.k_pool, w.v_pool, k_new, v_new, w.page_table, append_lens)
                    run_oracle_rows(w, (kp, vp), threads)
                    dt = time.perf_counter() - t0
                    best = dt if best is None else min(best, dt)
            kvb = w.logical_tokens() * w.kv_bytes_per_token()
            entry["oracle"] = {"s_per_step": round(best, 4), "tokens_per_s": round(B / best, 2),
                               "logical_kv_gbs": round(kvb / best / 1e9, 4), "cores": threads,
                               "runs": 3 if idx == 1 else 1}
            log(f"[configs] {cfg.name} oracle: {best:.3f} s/step on {threads} threads")
        res[cfg.name] = entry
        del w, pr
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "this build has no multi-GPU path; run with --gpus 1.", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_203_amd as pkv
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        print(json.dumps({"copy_calibration": copy_calibration()}), flush=True)
        return

    cfg = W.config(args.config)
    t_gen = time.perf_counter()
    w = W.make_workload(cfg)
    B, Hq, Hkv, D, PS = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    mq = args.path in ("multiquery", "multiquery-step")
    one_launch = args.path in ("step", "multiquery-step")
    w.q_tokens = args.q_tokens if mq else 1
    if args.path == "cascade" and cfg.lengths[0] != "prefix":
        raise SystemExit("--path cascade needs a prefix-shared workload")
    P = args.partition_tokens or {"cascade": 256, "multiquery": 1024}.get(args.path) or \
        cfg.partition_tokens or 512
    log(f"workload {cfg.name}: generated in {time.perf_counter() - t_gen:.1f}s, "
        f"{w.logical_tokens()} live tokens, pool {w.k_pool.shape}")

    from workloads.generate import fill_normal
    dev = torch.device("cuda:0")
    pr = Prepared(w, args.replicas, dev)
    q, table, lens, alens, kn, vn, out = pr.q, pr.table, pr.lens, pr.alens, pr.kn, pr.vn, pr.out
    pools, R = pr.pools, pr.R
    maxp = pkv.partitions_needed(PS, w.page_table.shape[1], P)
    if mq:
        T = args.q_tokens
        qm = to_device(fill_normal((B, T, Hq, D), cfg.dtype, w.seed, 9), cfg.dtype, dev)
        outm = torch.empty_like(qm)
        pom = torch.empty((B, T, Hq, maxp, D), dtype=torch.float32, device=dev)
        plm = torch.empty((B, T, Hq, maxp), dtype=torch.float32, device=dev)
    po = torch.empty((B, Hq, maxp, D), dtype=torch.float32, device=dev)
    pl = torch.empty((B, Hq, maxp), dtype=torch.float32, device=dev)
    scale = pr.scale
    stream = torch.cuda.current_stream(dev)

    prefix_tokens = w.shared_pages * PS
    prefix_pages = torch.from_numpy(np.ascontiguousarray(
        w.page_table[int(np.argmax(w.context_lens > 0)), :w.shared_pages])).to(dev)
    rope = {}
    if args.rope:
        if args.path != "step":
            raise SystemExit("--rope applies to the step path")
        rc, rs = W.rope_tables(w.page_table.shape[1] * PS + 1, D, 500000.0)
        rope = dict(rope_cos=torch.from_numpy(rc).to(dev), rope_sin=torch.from_numpy(rs).to(dev))
    ws = None
    if args.path == "step":
        ws = torch.zeros(pkv.decode_step_workspace_bytes(q, pools[0][0], table), dtype=torch.uint8, device=dev)
    elif args.path == "multiquery-step":
        ws = torch.zeros(pkv.multi_query_step_workspace_bytes(qm, pools[0][0], table), dtype=torch.uint8,
                         device=dev)

    def step(i, ev=None):
        """One step; with `ev`, the event pair brackets the dominant kernel only."""
        kp, vp = pools[i % R]
        if args.path == "step":
            pkv.paged_decode_step(q, kp, vp, table, alens, scale, k_new=kn, v_new=vn, out=out,
                                  workspace=ws, **rope)
            return
        if args.path == "multiquery-step":
            pkv.paged_decode_multi_query_step(qm, kp, vp, table, lens, scale, out=outm, workspace=ws)
            return
        if args.path != "multiquery":   # the multi-query rows' K/V are already in the pages
            pkv.paged_kv_append(kn, vn, kp, vp, table, alens)
        if ev is not None:
            ev[0].record(stream)
        if args.path == "multiquery":
            pkv.paged_decode_multi_query(qm, kp, vp, table, lens, P, scale, out=outm,
                                         partial_out=pom, partial_lse=plm)
            if ev is not None:
                ev[1].record(stream)
        elif args.path == "cascade":
            pkv.paged_decode_cascade(q, kp, vp, prefix_pages, prefix_tokens, table, lens, P, scale,
                                     out=out, partial_out=po, partial_lse=pl)
            if ev is not None:
                ev[1].record(stream)
        elif args.path == "split":
            pkv.paged_decode_attention_partial(q, kp, vp, table, lens, P, scale, po, pl, maxp)
            if ev is not None:
                ev[1].record(stream)
            pkv.lse_merge(po, pl, lens, P, PS, w.page_table.shape[1], out=out)
        else:
            pkv.paged_decode_attention(q, kp, vp, table, lens, scale, out)
            if ev is not None:
                ev[1].record(stream)

    # ---- settle (reported apart from the warmup), then the W warmup steps ----
    settle_steps, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for i in range(20):
            step(settle_steps + i)
        settle_steps += 20
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    # ---- the timed region: K steps back to back between two events on the launch stream ----
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_us = e0.elapsed_time(e1) * 1e3 / K

    # ---- the spread: K more steps, each bracketed by its own event pair ----
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for i in range(K):
        if one_launch:
            evs[i][0].record(stream)
            step(args.warmup + K + i)
            evs[i][1].record(stream)
        else:
            step(args.warmup + K + i, evs[i])
    torch.cuda.synchronize()
    kernel_us = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3

    nb = step_bytes(w, P, args.path)
    ms_step = wall * 1e3 / K
    gbs = nb["step"] / (ms_step * 1e-3) / 1e9
    # One launch per step on the step paths: the region's average is the kernel's average launch
    # duration in a back-to-back stream.  Other paths time their dominant kernel alone.
    k_avg_us = region_us if one_launch else float(kernel_us.mean())
    k_gbs = nb["kernel"] / (k_avg_us * 1e-6) / 1e9
    log(f"{K} steps in {wall * 1e3:.2f} ms: {ms_step * 1e3:.1f} us/step, {gbs:.0f} GB/s step; "
        f"events over the region {region_us:.1f} us/step; dominant kernel {k_avg_us:.1f} us avg, "
        f"{k_gbs:.0f} GB/s; individually bracketed: median {np.median(kernel_us):.1f}, "
        f"p10 {np.percentile(kernel_us, 10):.1f}, p90 {np.percentile(kernel_us, 90):.1f} us")

    calib = {}
    configs = None
    if args.path == "step" and not args.rope and args.config == 2 and not args.no_configs:
        calib["copy"] = copy_calibration()
        calib["read_stream"] = read_calibration(pkv)
        pr.release()
        pools = None
        torch.cuda.empty_cache()
        configs = config_sweep(pkv, dev, stream, calib["read_stream"]["gbs"], args.config_steps,
                               args.config_warmup, args.cpu_seconds, args.settle_ms)

    cpu = None
    if args.cpu_seconds > 0:
        log(f"timing the CPU oracle for >= {args.cpu_seconds:.0f}s ...")
        cpu = cpu_baseline(w, pr.new_rows, args.cpu_seconds)
        log(f"CPU oracle: {cpu['s_per_step']:.3f} s/step, {cpu['value']} GB/s on {cpu['cores']} threads")

    kernel_name = {"split": "decode_kernel (split-KV partial attention)",
                   "cascade": "pkv_paged_decode_cascade (prefix on MFMA + suffix partitions + merge)",
                   "multiquery": "pkv_paged_decode_multi_query (partitions on MFMA + merge)",
                   "multiquery-step": "step_kernel (pkv_paged_decode_multi_query_step: balanced attention + merge)",
                   "single": "decode_kernel (single pass)",
                   "step": "step_kernel (pkv_paged_decode_step: append + balanced attention + merge)"}[args.path]
    traffic = measured_traffic(cfg.name) if args.path == "step" and not args.rope else None
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle": {"steps": settle_steps, "ms": round(settle_ms, 1),
                   "what": "untimed full steps run before the warmup steps, until the device reaches "
                           "its steady clock state (--settle-ms)"},
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": cfg.name,
            "description": {"split": "append + split-KV paged decode attention + LSE merge",
                            "cascade": "append + shared-prefix decode: prefix on the matrix cores, suffix partitions, LSE merge",
                            "multiquery": "causal decode of q_tokens new tokens per sequence (their K/V already paged) on the matrix cores + LSE merge",
                            "multiquery-step": "causal decode of q_tokens new tokens per sequence (their K/V already paged) in one launch: balanced split-KV attention, LSE merge",
                            "single": "append + single-pass paged decode attention",
                            "step": "one decode step in one launch: append, balanced split-KV attention, LSE merge"}[args.path],
            "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "page_size": PS,
            "context_lens": list(cfg.lengths), "seed": w.seed, "live_tokens": w.logical_tokens(),
            "partition_tokens": P if args.path in ("split", "cascade", "multiquery") else None,
            "path": args.path,
            "rope": bool(args.rope),
            "q_tokens": w.q_tokens,
            "pool_replicas": R,
            "step_bytes": nb["step"], "kv_bytes": nb["kv"],
        },
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(B * w.q_tokens / (ms_step * 1e-3), 1),
        "roofline": {
            "kernel": kernel_name,
            "bound": "hbm",
            "achieved": round(k_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(k_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_source": (f"profiles/{os.path.basename(TRAFFIC_SUMMARY)}: rocprofv3 FETCH_SIZE and "
                               "WRITE_SIZE per dispatch, scaled by a plain copy's, taken on kernel "
                               f"sources {kernel_source_hash()} (the current ones)") if traffic else None,
            "bytes_per_launch": nb["kernel"],
            "avg_launch_us": round(k_avg_us, 3),
            "timing": ("events on the launch stream around the K back-to-back steps of the timed "
                       "region, divided by K" if one_launch else
                       "an event pair around the dominant kernel of each step, averaged"),
            "median_bracketed_us": round(float(np.median(kernel_us)), 3),
            "p10_bracketed_us": round(float(np.percentile(kernel_us, 10)), 3),
            "p90_bracketed_us": round(float(np.percentile(kernel_us, 90)), 3),
            "pct_of_read_stream": round(100 * k_gbs / calib["read_stream"]["gbs"], 2) if calib else None,
            "kernel_source_sha256": kernel_source_hash(),
        },
        "cpu_baseline": cpu,
        "calibration": calib or None,
        "configs": configs,
        "device": torch.cuda.get_device_name(0),
        "gfx_arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None),
        "hip": getattr(torch.version, "hip", None),
        "torch": torch.__version__,
        "lib": pkv.version(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
