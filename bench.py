#!/usr/bin/env python3
"""Benchmark of the KV-cache write + chunk-attention hot path on one MI355X.

Headline workload (one "step" = one whole job): autoregressive decode with an active prefix,
B=1, 32 query heads on 8 KV heads, D=128, bf16, cache capacity 32768 rows: a 234-token causal
prefill (cursor advance, indexed write of 234 rows, flash attention) followed by 1024 decode
steps, each a cursor advance, a one-row indexed write and a split-K attention over the
active prefix kv_len = 235 ... 1258. The job is recorded once into a HIP graph and replayed;
all inputs are resident in HBM before the timed region starts.

Printed as one JSON line:
  value         decode KV-read throughput of the whole job: the K/V bytes the job's attention
                calls must read (active prefix only) / job time, in GB/s;
  roofline      the dominant kernel (split-K decode attention): algorithmic bytes per launch
                (K/V prefix + Q + O) / its mean duration, measured with HIP events around each
                launch on the launch stream, against 8 TB/s HBM;
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same job;
  rows          the other hot-path workloads measured in the same run (ring, multi-user slab,
                ragged cross-attention, decode kv_len sweep with cold caches, slab writes).

`python bench.py --gpus N` with N > 1 exits: the library runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2516.6    # MI355X dense bf16 matrix peak, published (256 CU x 2.4 GHz x 4096)
ELEM = 2                       # bytes per bf16/fp16 element


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true")
    ap.add_argument("--only", default="", help="profiling aid: run only this part "
                    "(decode | ring | multiuser | ragged | sweep | peaks)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="counter-profiling aid: finish with one plain device copy of 256 MiB "
                    "(fresh buffers), whose FETCH_SIZE / WRITE_SIZE readings scale the "
                    "counters of the other kernels in the same profile")
    return ap.parse_args()


def copy_calibration(torch, dev):
    """One torch device-to-device copy of exactly 256 MiB between fresh buffers: a kernel whose
    HBM traffic is known (256 MiB read + 256 MiB written)."""
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    return n


# ----------------------------------------------------------------------------------------
# timing helpers
# ----------------------------------------------------------------------------------------
def event_pair(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_gpu(torch, fn, reps=10, warm=2, flush=None):
    """Median GPU time (ms) of fn() measured with events on the current stream. If flush is
    given it runs (untimed) before every repetition to evict L2 and the Infinity Cache."""
    for _ in range(warm):
        fn()
    times = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b = event_pair(torch)
        a.record()
        fn()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    return statistics.median(times)


def make_flush(torch, dev):
    """Read a 1 GiB buffer: larger than 2 x (32 MB L2 + 256 MB Infinity Cache), and read, not
    written, so the timed kernel does not inherit dirty lines to write back."""
    buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    return lambda: buf.sum()


def graph_us_each(torch, fns, replays=4):
    """Mean GPU time (us) per call of the callables fns, run back to back once each inside one
    HIP graph (replayed `replays` times, the first untimed). Each call gets its own buffers, more
    bytes in all than L2 plus the Infinity Cache hold, so every call starts cold without a flush
    between calls (and without an event pair's dispatch latency around each call)."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for f in fns:
            f()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for f in fns:
                f()
        times = []
        for _ in range(replays):
            a, b = event_pair(torch)
            a.record(stream)
            g.replay()
            b.record(stream)
            b.synchronize()
            times.append(a.elapsed_time(b))
    torch.cuda.synchronize()
    return statistics.median(times[1:]) * 1e3 / len(fns)


# ----------------------------------------------------------------------------------------
# headline: decode job
# ----------------------------------------------------------------------------------------
class DecodeJob:
    """Prefill + 1024 decode steps through the device cursor; everything device-resident."""

    def __init__(self, torch, skv, SI, dev, dtype, fused=True):
        self.fused = fused
        W = SI.Decode()
        self.W, self.torch, self.skv = W, torch, skv
        n = W.prompt + W.steps
        td = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
        self.q = SI.per_batch_device_normal(1, (n, W.Hq, W.D), "decode", "q", dev, dtype, std=W.std)
        self.k = SI.per_batch_device_normal(1, (n, W.Hkv, W.D), "decode", "k", dev, dtype, std=W.std)
        self.v = SI.per_batch_device_normal(1, (n, W.Hkv, W.D), "decode", "v", dev, dtype, std=W.std)
        self.kc = torch.zeros(1, W.cap, W.Hkv, W.D, dtype=td, device=dev)
        self.vc = torch.zeros_like(self.kc)
        self.cursor = torch.zeros(1, dtype=torch.int32, device=dev)
        self.kv_len = torch.zeros(1, dtype=torch.int32, device=dev)
        self.idx_pre = torch.empty(W.prompt, dtype=torch.int64, device=dev)
        self.idx_one = torch.empty(1, dtype=torch.int64, device=dev)
        self.out_pre = torch.empty(1, W.prompt, W.Hq, W.D, dtype=td, device=dev)
        self.out = torch.empty(W.steps, 1, 1, W.Hq, W.D, dtype=td, device=dev)
        T = W.prompt
        # the job's longest prefix bounds the split-K grid (device kv_len, fixed launch shape)
        self.max_kv = T + W.steps
        self.ws = torch.zeros(skv.attn_workspace_bytes(self.q[:, T:T + 1], self.kc, kv_len=self.max_kv),
                              dtype=torch.uint8, device=dev)
        # prebuilt views so the replayed sequence does no tensor bookkeeping
        self.q_pre, self.k_pre, self.v_pre = self.q[:, :T], self.k[:, :T], self.v[:, :T]
        self.q_steps = [self.q[:, T + i:T + i + 1] for i in range(W.steps)]
        self.k_steps = [self.k[:, T + i:T + i + 1] for i in range(W.steps)]
        self.v_steps = [self.v[:, T + i:T + i + 1] for i in range(W.steps)]
        # algorithmic bytes: K/V of the active prefix (+ Q and O for the per-launch figure)
        self.kv_bytes_job = sum(2 * (T + i + 1) * W.Hkv * W.D * ELEM for i in range(W.steps)) \
            + 2 * T * W.Hkv * W.D * ELEM
        self.decode_launch_bytes = [2 * (T + i + 1) * W.Hkv * W.D * ELEM + 2 * W.Hq * W.D * ELEM
                                    for i in range(W.steps)]

    def run_steps(self):
        """The fused decode steps alone, from the cursor at the end of the prefill (the cache
        prefix is already in place; the steps rewrite their rows with the same values)."""
        skv, W = self.skv, self.W
        self.cursor.fill_(W.prompt)  # a fill kernel, safe to record in a graph
        for i in range(W.steps):
            skv.attn_decode_step(self.q_steps[i], self.k_steps[i], self.v_steps[i], self.kc, self.vc,
                                 self.cursor, self.out[i], kv_len_out=self.kv_len,
                                 max_seqlen_kv=self.max_kv, workspace=self.ws)

    def run(self, events=None):
        skv, W = self.skv, self.W
        self.cursor.zero_()  # a fill kernel, not a memset: safe to record in a graph
        skv.kv_cursor_advance(self.cursor, W.prompt, W.cap, self.idx_pre, self.kv_len)
        skv.kv_write_indexed(self.kc, self.vc, self.k_pre, self.v_pre, index=self.idx_pre)
        skv.attn_chunk_fwd(self.q_pre, self.kc, self.vc, self.out_pre, kv_len_dev=self.kv_len,
                           mask=skv.MASK_CAUSAL, max_seqlen_kv=W.cap)
        for i in range(W.steps):
            if self.fused:  # one launch: cursor read, row write, attention, cursor advance
                if events is not None:
                    events[i][0].record()
                skv.attn_decode_step(self.q_steps[i], self.k_steps[i], self.v_steps[i], self.kc, self.vc,
                                     self.cursor, self.out[i], kv_len_out=self.kv_len,
                                     max_seqlen_kv=self.max_kv, workspace=self.ws)
                if events is not None:
                    events[i][1].record()
                continue
            skv.kv_cursor_advance(self.cursor, 1, W.cap, self.idx_one, self.kv_len)
            skv.kv_write_indexed(self.kc, self.vc, self.k_steps[i], self.v_steps[i], index=self.idx_one)
            if events is not None:
                events[i][0].record()
            skv.attn_chunk_fwd(self.q_steps[i], self.kc, self.vc, self.out[i], kv_len_dev=self.kv_len,
                               max_seqlen_kv=self.max_kv, workspace=self.ws)
            if events is not None:
                events[i][1].record()


def bench_decode(torch, skv, SI, dev, args, fused=True):
    job = DecodeJob(torch, skv, SI, dev, args.dtype, fused)
    # eager warm-up (also builds every kernel), then record the job into a graph
    job.run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        job.run()  # one more eager run on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        job.run()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = event_pair(torch)
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    gpu_ms = e0.elapsed_time(e1) / args.steps

    # per-launch duration of the decode attention kernel. Fused job: a graph of the 1024 steps
    # alone, replayed and timed with one event pair -- back-to-back launches with nothing in
    # between, as a kernel-trace profile times them. Both jobs: events around each launch
    # (behind a GPU-side sleep, so host launch gaps do not enter) for the first / last step,
    # and for the unfused job's attention launch, which sits between two other kernels.
    steps_ms = None
    if fused:
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2):
            job.run_steps()
        for _ in range(2):
            g2.replay()
        torch.cuda.synchronize()
        reps = max(args.steps, 3)
        c0, c1 = event_pair(torch)
        c0.record()
        for _ in range(reps):
            g2.replay()
        c1.record()
        c1.synchronize()
        steps_ms = c0.elapsed_time(c1) / (reps * job.W.steps)
        del g2
    events = [event_pair(torch) for _ in range(job.W.steps)]
    t_host = time.perf_counter()
    job.run(events)  # host time to enqueue one job with its events
    t_host = time.perf_counter() - t_host
    torch.cuda.synchronize()
    a, b = event_pair(torch)
    a.record()
    torch.cuda._sleep(10_000_000)
    b.record()
    b.synchronize()
    sleep_cycles = int(10_000_000 * max(2.0 * t_host * 1e3, 20.0) / max(a.elapsed_time(b), 1e-3))
    durations = []
    for rep in range(3):
        torch.cuda._sleep(sleep_cycles)  # the GPU waits while the host enqueues the whole job
        job.run(events)
        torch.cuda.synchronize()
        durations.append([a.elapsed_time(b) for a, b in events])
    per_launch = [statistics.median(d[i] for d in durations) for i in range(job.W.steps)]
    mean_ms = steps_ms if steps_ms is not None else sum(per_launch) / len(per_launch)
    mean_bytes = sum(job.decode_launch_bytes) / len(job.decode_launch_bytes)
    achieved = mean_bytes / (mean_ms * 1e-3) / 1e9
    return {
        "job": job,
        "ms_per_step": wall * 1e3,
        "gpu_ms_per_step": gpu_ms,
        "value": job.kv_bytes_job / wall / 1e9,
        "decode_kernel": {"mean_us": mean_ms * 1e3, "mean_bytes": mean_bytes, "achieved_gbs": achieved,
                          "first_us": per_launch[0] * 1e3, "last_us": per_launch[-1] * 1e3},
        "decode_steps_per_s": job.W.steps / wall,
    }


# ----------------------------------------------------------------------------------------
# other hot-path workloads (reported under "rows")
# ----------------------------------------------------------------------------------------
def bench_ring(torch, skv, SI, dev):
    W = SI.Ring()
    rows = W.n_slots * W.C
    ks = torch.zeros(W.B, rows, W.H, W.D, dtype=torch.bfloat16, device=dev)
    vs = torch.zeros_like(ks)
    ring = skv.Ring(ks, vs, W.C, W.n_slots, W.sink)
    shape = (W.C, W.H, W.D)
    srcs = [(SI.per_batch_device_normal(W.B, shape, "ring", "q", dev, "bf16", chunk=c, rewrite=r),
             SI.per_batch_device_normal(W.B, shape, "ring", "k", dev, "bf16", chunk=c, rewrite=r),
             SI.per_batch_device_normal(W.B, shape, "ring", "v", dev, "bf16", chunk=c, rewrite=r))
            for c in range(2) for r in range(2)]
    out = torch.empty(W.B, W.C, W.H, W.D, dtype=torch.bfloat16, device=dev)
    # workspace for the tail split of the attention grid (37 query tiles x 24 heads leave the
    # second round of workgroups 73% full; its items run as key-range pieces)
    ws = torch.zeros(max(16, skv.attn_workspace_bytes(srcs[0][0], ks, kv_len_dev=ring.kv_len,
                                                      max_seqlen_kv=rows)), dtype=torch.uint8, device=dev)
    no_ws = torch.zeros(16, dtype=torch.uint8, device=dev)  # too small: every item runs whole

    def sequence(marks=None):
        ring.reset()
        for c in range(W.n_chunks):
            if marks is not None:
                marks[c].record()
            ring.reserve()
            for r in range(W.rewrites):
                q, k, v = srcs[(c % 2) * 2 + (r % 2)]
                ring.write(k, v)
                skv.attn_chunk_fwd(q, ks, vs, out, kv_len_dev=ring.kv_len, max_seqlen_kv=rows, workspace=ws)
        if marks is not None:
            marks[W.n_chunks].record()

    seq_ms = time_gpu(torch, sequence, reps=3, warm=1)
    # one more pass with an event at every chunk boundary: the step time of each chunk
    # (reserve + rewrites x (write + attention)); chunk n_slots is the first to evict
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(W.n_chunks + 1)]
    sequence(marks)
    marks[-1].synchronize()
    chunk_ms = [marks[c].elapsed_time(marks[c + 1]) for c in range(W.n_chunks)]

    def rolling_sequence():
        # the comparison arm: the same chunk lifecycle on a chronological buffer that moves its
        # retained non-sink rows left by one chunk whenever a new chunk does not fit
        filled = 0
        for c in range(W.n_chunks):
            if filled + W.C > rows:
                skv.kv_roll_left(ks, vs, W.sink * W.C, W.C)
            else:
                filled += W.C
            for r in range(W.rewrites):
                q, k, v = srcs[(c % 2) * 2 + (r % 2)]
                skv.kv_write_indexed(ks, vs, k, v, start=filled - W.C)
                skv.attn_chunk_fwd(q, ks, vs, out, kv_len=filled, workspace=ws)

    def clone_rolling_sequence():
        # the same arm with the page's roll as written there: clone the retained non-sink rows,
        # then copy them back one chunk to the left (torch copies; twice the bytes of the
        # in-place roll, and a temporary as large as the moved rows)
        filled = 0
        for c in range(W.n_chunks):
            if filled + W.C > rows:
                lo = W.sink * W.C
                for st in (ks, vs):
                    kept = st[:, lo + W.C:].clone()
                    st[:, lo:rows - W.C].copy_(kept)
                    del kept
            else:
                filled += W.C
            for r in range(W.rewrites):
                q, k, v = srcs[(c % 2) * 2 + (r % 2)]
                skv.kv_write_indexed(ks, vs, k, v, start=filled - W.C)
                skv.attn_chunk_fwd(q, ks, vs, out, kv_len=filled, workspace=ws)

    def peak_mb(fn):
        """Peak device memory allocated through torch while fn runs (storage included)."""
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        fn()
        torch.cuda.synchronize()
        return torch.cuda.max_memory_allocated() / 1e6

    roll_seq_ms = time_gpu(torch, rolling_sequence, reps=3, warm=1)
    clone_seq_ms = time_gpu(torch, clone_rolling_sequence, reps=3, warm=1)
    peak = {"ring_sequence_mb": peak_mb(sequence), "inplace_roll_sequence_mb": peak_mb(rolling_sequence),
            "clone_roll_sequence_mb": peak_mb(clone_rolling_sequence)}
    # saturated step: 7 valid slots
    ring.reset()
    for c in range(W.n_slots):
        ring.reserve()
        ring.write(srcs[0][1], srcs[0][2])
    q = srcs[1][0]
    attn_ms = time_gpu(torch, lambda: skv.attn_chunk_fwd(q, ks, vs, out, kv_len_dev=ring.kv_len,
                                                         max_seqlen_kv=rows, workspace=ws), reps=10)
    attn_whole_ms = time_gpu(torch, lambda: skv.attn_chunk_fwd(q, ks, vs, out, kv_len_dev=ring.kv_len,
                                                               max_seqlen_kv=rows, workspace=no_ws), reps=10)
    flush = make_flush(torch, dev)
    write_ms = time_gpu(torch, lambda: ring.write(srcs[0][1], srcs[0][2]), reps=10, flush=flush)
    roll_ms = time_gpu(torch, lambda: skv.kv_roll_left(ks, vs, W.sink * W.C, W.C), reps=10, flush=flush)

    def clone_roll():
        lo = W.sink * W.C
        for st in (ks, vs):
            kept = st[:, lo + W.C:].clone()
            st[:, lo:rows - W.C].copy_(kept)

    clone_roll_ms = time_gpu(torch, clone_roll, reps=10, flush=flush)
    # keys rotated at their absolute positions before storage: fused into the ring write, and
    # the unfused path (a separate rotation by torch in fp32, then the plain write) beside it
    half = W.D // 2
    inv = torch.pow(torch.tensor(10000.0, dtype=torch.float64, device=dev),
                    -torch.arange(half, dtype=torch.float64, device=dev) * 2.0 / W.D)
    rope_ms = time_gpu(torch, lambda: ring.write_rope(srcs[0][1], srcs[0][2], inv), reps=10, flush=flush)
    ang = ((int(ring.counter[0].item()) - 1) * W.C
           + torch.arange(W.C, dtype=torch.float64, device=dev))[:, None] * inv[None, :]
    cos, sin = ang.cos().float()[None, :, None, :], ang.sin().float()[None, :, None, :]

    def unfused_rope_write():
        x = srcs[0][1].float()
        a, b = x[..., :half], x[..., half:]
        ring.write(torch.cat([a * cos - b * sin, a * sin + b * cos], dim=-1).to(torch.bfloat16),
                   srcs[0][2])

    unfused_ms = time_gpu(torch, unfused_rope_write, reps=10, flush=flush)
    del flush
    # the same write back to back on 6 distinct rings and sources (6 x 115 MB, > L2 + MALL)
    extra = [skv.Ring(torch.empty_like(ks), torch.empty_like(vs), W.C, W.n_slots, W.sink) for _ in range(6)]
    esrc = [(SI.per_batch_device_normal(W.B, shape, "ring", "k", dev, "bf16", chunk=2 + i),
             SI.per_batch_device_normal(W.B, shape, "ring", "v", dev, "bf16", chunk=2 + i)) for i in range(6)]
    for r in extra:
        r.reserve()
    write_b2b_us = graph_us_each(torch, [lambda r=r, e=e: r.write(e[0], e[1]) for r, e in zip(extra, esrc)])
    rope_b2b_us = graph_us_each(torch, [lambda r=r, e=e: r.write_rope(e[0], e[1], inv)
                                        for r, e in zip(extra, esrc)])
    for r in extra:
        r.close()
    del extra, esrc
    reset_ms = time_gpu(torch, lambda: ring.reset(), reps=10)
    flop_sat = 4 * W.D * W.H * W.B * W.C * (W.n_slots * W.C)
    flop_seq = sum(4 * W.D * W.H * W.B * W.C * (min(c + 1, W.n_slots) * W.C) * W.rewrites
                   for c in range(W.n_chunks))
    wbytes = 2 * 2 * W.B * W.C * W.H * W.D * ELEM
    moved = rows - W.sink * W.C - W.C  # retained non-sink rows moved per roll
    rbytes = 2 * 2 * W.B * moved * W.H * W.D * ELEM
    n_rolls = max(0, W.n_chunks - W.n_slots)
    return {
        "workload": "ring: B=2, 12 heads, D=128, bf16, chunks of 4680, 7 slots (1 sink), 12 chunks x 4 rewrites",
        "sequence_ms": seq_ms, "sequence_tflops": flop_seq / seq_ms * 1e-9,
        "ms_per_rewrite_step": seq_ms / (W.n_chunks * W.rewrites),
        "chunk_step_ms": [round(x, 4) for x in chunk_ms],
        "first_eviction_chunk": W.n_slots,
        "saturated_attn_ms": attn_ms, "saturated_attn_tflops": flop_sat / attn_ms * 1e-9,
        "saturated_attn_frac_mfma": flop_sat / attn_ms * 1e-9 / MFMA_BF16_PEAK_TFS,
        "saturated_attn_tail_split_workspace_mb": ws.numel() / 1e6,
        "saturated_attn_whole_items_ms": attn_whole_ms,
        "saturated_attn_whole_items_tflops": flop_sat / attn_whole_ms * 1e-9,
        "ring_write_ms_cold": write_ms, "ring_write_gbs": wbytes / write_ms * 1e-6,
        "ring_write_frac_hbm": wbytes / write_ms * 1e-6 / HBM_PEAK_GBS,
        "ring_write_us_back_to_back": write_b2b_us,
        "ring_write_gbs_back_to_back": wbytes / write_b2b_us * 1e-3,
        "ring_write_frac_hbm_back_to_back": wbytes / write_b2b_us * 1e-3 / HBM_PEAK_GBS,
        "reset_us": reset_ms * 1e3,
        "rope_write": {
            "what": "kv_ring_write_rope: K rotated at chunk_id*C+t (fp64) as it is written, V copied; "
                    "unfused arm: torch fp32 rotation of K, then kv_ring_write",
            "fused_ms_cold": rope_ms, "fused_gbs": wbytes / rope_ms * 1e-6,
            "fused_frac_hbm": wbytes / rope_ms * 1e-6 / HBM_PEAK_GBS,
            "unfused_ms_cold": unfused_ms, "unfused_vs_fused": unfused_ms / rope_ms,
            "fused_us_back_to_back": rope_b2b_us, "fused_gbs_back_to_back": wbytes / rope_b2b_us * 1e-3,
            "vs_plain_write": rope_ms / write_ms},
        "rolling_arm": {
            "what": "chronological buffer with roll-left past the sink (the path the ring replaces): "
                    "same chunk lifecycle, host kv_len; in place (kv_roll_left, ordered chunk-sized "
                    "copies) and as the page writes it (clone the retained rows, copy them back)",
            "sequence_ms": roll_seq_ms, "vs_ring_sequence": roll_seq_ms / seq_ms,
            "roll_ms_cold": roll_ms, "roll_rows_moved": moved, "roll_bytes": rbytes,
            "roll_gbs": rbytes / roll_ms * 1e-6, "rolls_per_sequence": n_rolls,
            "clone_then_copy": {"sequence_ms": clone_seq_ms, "vs_ring_sequence": clone_seq_ms / seq_ms,
                                "roll_ms_cold": clone_roll_ms, "roll_bytes": 2 * rbytes,
                                "roll_gbs": 2 * rbytes / clone_roll_ms * 1e-6,
                                "temporary_mb": rbytes / 2 / 2 / 1e6},
            "ring_maintenance_bytes": 0,
            "peak_allocated_mb": peak},
    }


def bench_multiuser(torch, skv, SI, dev):
    W = SI.MultiUser()
    kc = torch.zeros(W.B, W.cap, W.H, W.D, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    shape = (W.chunk, W.H, W.D)
    q = SI.per_batch_device_normal(W.B, shape, "multiuser", "q", dev, "bf16")
    k = SI.per_batch_device_normal(W.B, shape, "multiuser", "k", dev, "bf16")
    v = SI.per_batch_device_normal(W.B, shape, "multiuser", "v", dev, "bf16")
    cursor = torch.zeros(1, dtype=torch.int32, device=dev)
    kv_len = torch.zeros(W.B, dtype=torch.int32, device=dev)
    idx = torch.empty(W.chunk, dtype=torch.int64, device=dev)
    out = torch.empty_like(q)

    def sequence():
        cursor.zero_()
        for c in range(W.n_chunks):
            skv.kv_cursor_advance(cursor, W.chunk, W.cap, idx, kv_len)
            skv.kv_write_indexed(kc, vc, k, v, index=idx)
            skv.attn_chunk_fwd(q, kc, vc, out, kv_len_dev=kv_len, mask=skv.MASK_BLOCK_CAUSAL,
                               mask_block=W.block, max_seqlen_kv=W.cap)

    seq_ms = time_gpu(torch, sequence, reps=3, warm=1)
    last = W.cap
    c15_ms = time_gpu(torch, lambda: skv.attn_chunk_fwd(q, kc, vc, out, kv_len=last, mask=skv.MASK_BLOCK_CAUSAL,
                                                        mask_block=W.block), reps=10)
    flush = make_flush(torch, dev)
    index = torch.arange(W.cap - W.chunk, W.cap, device=dev)
    write_ms = time_gpu(torch, lambda: skv.kv_write_indexed(kc, vc, k, v, index=index), reps=10, flush=flush)
    del flush
    pairs = lambda c: W.chunk * (W.chunk * c) + W.chunk * (W.chunk + 1) // 2  # noqa: E731 (block 1)
    flop_seq = sum(4 * W.D * W.H * W.B * pairs(c) for c in range(W.n_chunks))
    flop_c15 = 4 * W.D * W.H * W.B * pairs(W.n_chunks - 1)
    wbytes = 2 * 2 * W.B * W.chunk * W.H * W.D * ELEM
    return {
        "workload": "multi-user slab: B=8, 40 heads, D=128, bf16, cap 16384, 16 chunks of 1024, causal in chunk",
        "sequence_ms": seq_ms, "sequence_tflops": flop_seq / seq_ms * 1e-9,
        "ms_per_chunk_step": seq_ms / W.n_chunks,
        "chunk15_attn_ms": c15_ms, "chunk15_attn_tflops": flop_c15 / c15_ms * 1e-9,
        "chunk15_attn_frac_mfma": flop_c15 / c15_ms * 1e-9 / MFMA_BF16_PEAK_TFS,
        "slab_write_ms_cold": write_ms, "slab_write_gbs": wbytes / write_ms * 1e-6,
        "slab_write_frac_hbm": wbytes / write_ms * 1e-6 / HBM_PEAK_GBS,
    }


def bench_ragged(torch, skv, SI, dev):
    W = SI.Ragged()
    q = SI.per_batch_device_normal(W.B, (W.Tq, W.H, W.D), "ragged", "q", dev, "bf16")
    out = torch.empty_like(q)
    res = {"workload": "ragged cross-attention: 2 branches, 40 heads, D=128, bf16, Q 75600 per branch"}
    for lens in W.skews:
        total = sum(lens)
        kp = SI.device_normal((total, W.H, W.D), SI.seed_key("ragged", "k", 0, lens[1]), "bf16", dev)
        vp = SI.device_normal((total, W.H, W.D), SI.seed_key("ragged", "v", 0, lens[1]), "bf16", dev)
        cu = torch.tensor([0, lens[0], total], dtype=torch.int32, device=dev)
        kpad = torch.zeros(W.B, W.max_kv, W.H, W.D, dtype=torch.bfloat16, device=dev)
        vpad = torch.zeros_like(kpad)
        kpad[0, :lens[0]], kpad[1, :lens[1]] = kp[:lens[0]], kp[lens[0]:]
        vpad[0, :lens[0]], vpad[1, :lens[1]] = vp[:lens[0]], vp[lens[0]:]
        used = torch.tensor(list(lens), dtype=torch.int32, device=dev)
        cu_buf = torch.empty(W.B + 1, dtype=torch.int32, device=dev)
        kpk = torch.empty(total, W.H, W.D, dtype=torch.bfloat16, device=dev)
        vpk = torch.empty_like(kpk)

        def packed_total():  # metadata + gather + attention, what a caller pays per call
            skv.kv_ragged_metadata(used, W.max_kv, cu_buf)
            skv.kv_pack_ragged(kpad, vpad, cu_buf, kpk, vpk)
            skv.attn_chunk_fwd(q, kpk, vpk, out, cu_seqlens_kv=cu_buf, max_seqlen_kv=W.max_kv)
        arms = {
            "packed_total": packed_total,
            "packed": lambda: skv.attn_chunk_fwd(q, kp, vp, out, cu_seqlens_kv=cu, max_seqlen_kv=W.max_kv),
            "seqused": lambda: skv.attn_chunk_fwd(q, kpad, vpad, out, kv_len_dev=used, max_seqlen_kv=W.max_kv),
            "padded_masked": lambda: skv.attn_chunk_fwd(q, kpad, vpad, out, kv_len_dev=used, max_seqlen_kv=W.max_kv,
                                                        full_capacity_masked=True),
        }
        flop = 4 * W.D * W.H * W.Tq * total
        byts = 2 * W.B * W.Tq * W.H * W.D * ELEM + 2 * total * W.H * W.D * ELEM
        entry = {}
        for name, fn in arms.items():
            ms = time_gpu(torch, fn, reps=10)
            entry[name] = {"ms": ms, "tflops": flop / ms * 1e-9, "gbs": byts / ms * 1e-6,
                           "roofline_frac": max(flop / ms * 1e-9 / MFMA_BF16_PEAK_TFS,
                                                byts / ms * 1e-6 / HBM_PEAK_GBS)}
        res[f"{lens[0]},{lens[1]}"] = entry
    return res


def bench_sweep(torch, skv, SI, dev):
    W = SI.Decode()
    kc = SI.device_normal((1, W.cap, W.Hkv, W.D), SI.seed_key("decode", "k", 0, 7), "bf16", dev, std=W.std)
    vc = SI.device_normal((1, W.cap, W.Hkv, W.D), SI.seed_key("decode", "v", 0, 7), "bf16", dev, std=W.std)
    q = SI.device_normal((1, 1, W.Hq, W.D), SI.seed_key("decode", "q", 0, 7), "bf16", dev, std=W.std)
    out = torch.empty_like(q)
    ws = torch.zeros(skv.attn_workspace_bytes(q, kc, kv_len=W.cap, full_capacity_masked=True),
                     dtype=torch.uint8, device=dev)  # the largest split count of the sweep
    flush = make_flush(torch, dev)
    res = {"workload": "decode attention alone, B=1, 32/8 heads, D=128, bf16, cold L2 and Infinity Cache"}
    res["method"] = ("us: one launch between an event pair after a 1 GiB read (includes the event "
                     "pair's dispatch latency); us_back_to_back: launches on distinct caches of "
                     "capacity kv_len (together > 600 MB, so each starts cold) back to back in a HIP graph")
    for L in (1258, 4096, 8192, 16384, 32768):
        ms = time_gpu(torch, lambda: skv.attn_chunk_fwd(q, kc, vc, out, kv_len=L, workspace=ws), reps=10,
                      flush=flush)
        byts = 2 * L * W.Hkv * W.D * ELEM + 2 * W.Hq * W.D * ELEM
        n_sets = max(6, -(-600_000_000 // byts))
        caches = [(kc[:, :L].clone(), vc[:, :L].clone()) for _ in range(n_sets)]
        b2b = graph_us_each(torch, [lambda c=c: skv.attn_chunk_fwd(q, c[0], c[1], out, kv_len=L, workspace=ws)
                                    for c in caches])
        del caches
        res[str(L)] = {"us": ms * 1e3, "gbs": byts / ms * 1e-6, "frac_hbm": byts / ms * 1e-6 / HBM_PEAK_GBS,
                       "us_back_to_back": b2b, "gbs_back_to_back": byts / b2b * 1e-3,
                       "frac_hbm_back_to_back": byts / b2b * 1e-3 / HBM_PEAK_GBS}
    ms = time_gpu(torch, lambda: skv.attn_chunk_fwd(q, kc, vc, out, kv_len=1258, full_capacity_masked=True,
                                                    workspace=ws), reps=10, flush=flush)
    byts = 2 * W.cap * W.Hkv * W.D * ELEM
    res["full_capacity_arm_kv1258"] = {"us": ms * 1e3, "gbs_visited": byts / ms * 1e-6,
                                       "slowdown_vs_active": ms * 1e3 / res["1258"]["us"]}
    return res


# ----------------------------------------------------------------------------------------
# measured ceilings: the library's MFMA-loop and copy probes, and a library GEMM
# ----------------------------------------------------------------------------------------
def bench_peaks(torch, skv, SI, dev, rows):
    res = {"what": "ceilings measured on this chip: skv_probe_mfma_bf16 (back-to-back 32x32x16 bf16 "
                   "MFMAs from registers), skv_probe_copy (1 GiB copy, the cache writes' access pattern; "
                   "also, cold, at the ring and slab writes' own sizes, since a copy's rate depends on "
                   "its size), and a bf16 GEMM 8192 x 8192 x 16384 through torch (hipBLASLt) as a "
                   "library reference"}
    out = torch.empty(2048 * 256, dtype=torch.float32, device=dev)
    flops = skv.probe_mfma_bf16(out, 2048, 2000)
    ms = time_gpu(torch, lambda: skv.probe_mfma_bf16(out, 2048, 2000), reps=5)
    res["mfma_bf16_tflops"] = flops / ms * 1e-9
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    byts = skv.probe_copy(dst, src)
    ms = time_gpu(torch, lambda: skv.probe_copy(dst, src), reps=5)
    res["copy_gbs"] = byts / ms * 1e-6
    del src, dst
    # the same copy at the sizes of one ring rewrite and one slab chunk write (K and V together,
    # read + written), each after a cache flush like the writes' own cold timings
    flush = make_flush(torch, dev)
    R, M = SI.Ring(), SI.MultiUser()
    same = {"ring_write": 2 * R.B * R.C * R.H * R.D * ELEM, "slab_write": 2 * M.B * M.chunk * M.H * M.D * ELEM}
    res["copy_gbs_cold_same_size"] = {}
    for name, each_way in same.items():
        src = torch.empty(each_way, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        byts = skv.probe_copy(dst, src)
        ms = time_gpu(torch, lambda: skv.probe_copy(dst, src), reps=10, flush=flush)
        res["copy_gbs_cold_same_size"][name] = {"bytes": byts, "us": ms * 1e3, "gbs": byts / ms * 1e-6}
        del src, dst
    # x @ w^T with w [N, K] row-major (the fastest of the layouts and shapes tried here)
    a = torch.randn(8192, 16384, dtype=torch.bfloat16, device=dev)
    w = torch.randn(8192, 16384, dtype=torch.bfloat16, device=dev)
    ms = time_gpu(torch, lambda: torch.nn.functional.linear(a, w), reps=5)
    res["gemm_bf16_tflops_library"] = 2 * 8192 * 8192 * 16384 / ms * 1e-9
    del a, w
    mf, cp = res["mfma_bf16_tflops"], res["copy_gbs"]
    frac = {}
    ring, mu = rows.get("ring", {}), rows.get("multiuser", {})
    if "saturated_attn_tflops" in ring:
        frac["ring_saturated_attn_vs_mfma_probe"] = ring["saturated_attn_tflops"] / mf
    if "chunk15_attn_tflops" in mu:
        frac["chunk15_attn_vs_mfma_probe"] = mu["chunk15_attn_tflops"] / mf
    same = res["copy_gbs_cold_same_size"]
    if "slab_write_gbs" in mu:
        frac["slab_write_vs_copy_probe"] = mu["slab_write_gbs"] / cp
        frac["slab_write_vs_copy_same_size"] = mu["slab_write_gbs"] / same["slab_write"]["gbs"]
    if "ring_write_gbs" in ring:
        frac["ring_write_vs_copy_probe"] = ring["ring_write_gbs"] / cp
        frac["ring_write_vs_copy_same_size"] = ring["ring_write_gbs"] / same["ring_write"]["gbs"]
    sweep = rows.get("decode_sweep", {})
    if "32768" in sweep:
        frac["decode_32768_vs_copy_probe"] = sweep["32768"]["gbs_back_to_back"] / cp
    res["fractions_of_measured"] = frac
    return res


# ----------------------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host cores (a reported baseline, not a target)
# ----------------------------------------------------------------------------------------
def _host_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        import threadpoolctl
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    return model, threads


def _median_of(fn, runs=3):
    """Median wall time of `runs` timed calls after one untimed warm call."""
    fn()
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return statistics.median(times), times


def cpu_baseline(SI, dtype):
    """The fp64 oracle's attention over the whole decode job (234-token causal prefill and all
    1024 single-token steps, kv_len 235 .. 1258), median of 3 warm runs. The oracle's caches
    are built once beforehand, untimed: its slab write copies the capacity-sized cache on every
    call, which would time numpy copies rather than attention; attend_prefix reads only rows
    [0, kv_len) of them. Bytes are the job's K/V bytes at 2 B per element, as for the GPU."""
    import numpy as np
    from oracle import attention as A
    from oracle import cache as Cc
    W = SI.Decode()
    n = W.prompt + W.steps
    q = SI.as_f64(SI.per_batch_normal(1, (n, W.Hq, W.D), "decode", "q", std=W.std, dtype=dtype))[0]
    k = SI.as_f64(SI.per_batch_normal(1, (n, W.Hkv, W.D), "decode", "k", std=W.std, dtype=dtype))
    v = SI.as_f64(SI.per_batch_normal(1, (n, W.Hkv, W.D), "decode", "v", std=W.std, dtype=dtype))
    kc, _ = Cc.slab_write_indexed(np.zeros((1, W.cap, W.Hkv, W.D)), k, np.arange(n))
    vc, _ = Cc.slab_write_indexed(np.zeros((1, W.cap, W.Hkv, W.D)), v, np.arange(n))
    T = W.prompt

    def job():
        A.attend_prefix(q[:T], kc[0], vc[0], T, A.MASK_CAUSAL)
        for i in range(W.steps):
            A.attend_prefix(q[T + i:T + i + 1], kc[0], vc[0], T + i + 1)

    secs, runs = _median_of(job)
    kv_bytes = 2 * T * W.Hkv * W.D * ELEM + sum(2 * (T + i + 1) * W.Hkv * W.D * ELEM for i in range(W.steps))
    model, threads = _host_info()
    return {"value": kv_bytes / secs / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": secs, "runs": len(runs), "run_seconds": [round(x, 4) for x in runs],
            "statistic": "median of 3 warm runs", "cpu_model": model, "host_cpus": os.cpu_count(),
            "blas_threads": threads,
            "sample": "the whole decode job: fp64 numpy oracle attention for the 234-token causal "
                      "prefill and all 1024 decode steps (caches built beforehand, untimed)"}


def cpu_baseline_rows(SI):
    """The fp64 oracle on the other workloads (median of 3 warm runs each, ~10 s in all): the
    tiny fp32 workload whole; attention over a sample of query rows of one (b, h) at each
    workload's key count (rates per query row scale linearly to the whole workload, which is
    rows x heads x batch times larger); one cache write of each workload's size."""
    import numpy as np
    from oracle import attention as A
    from oracle import cache as Cc
    rng = np.random.default_rng(0)

    def attn_rate(n_q, L, D, mask=A.MASK_NONE, Tq=None):
        Tq = Tq or n_q
        q = rng.standard_normal((n_q, 1, D))
        k = rng.standard_normal((L, 1, D))
        v = rng.standard_normal((L, 1, D))
        allowed = np.stack([A.visible_keys(Tq - n_q + i, Tq, L, mask) for i in range(n_q)])
        secs, _ = _median_of(lambda: A.attend_keys(q, k, v, allowed))
        flop = 4 * D * int(allowed.sum())
        return {"tflops": flop / secs * 1e-12, "seconds": round(secs, 4),
                "sample": f"{n_q} query rows x {L} keys, one head"}

    def write_rate(rows, H, D, fn):
        src = rng.standard_normal((1, rows, H, D))
        secs, _ = _median_of(lambda: fn(src))
        return {"gbs": 2 * src.size * ELEM / secs * 1e-9, "seconds": round(secs, 4),
                "sample": f"{rows} rows x {H} heads x {D}, bytes counted at 2 B per element"}

    def tiny_whole():
        W = SI.Tiny()
        qs = SI.as_f64(SI.per_batch_normal(W.B, (W.chunk * W.n_chunks, W.H, W.D), "tiny", "q"))
        ks = SI.as_f64(SI.per_batch_normal(W.B, (W.chunk * W.n_chunks, W.H, W.D), "tiny", "k"))
        vs = SI.as_f64(SI.per_batch_normal(W.B, (W.chunk * W.n_chunks, W.H, W.D), "tiny", "v"))

        def run():
            kc = np.zeros((W.B, W.cap, W.H, W.D))
            vc = np.zeros_like(kc)
            for c in range(W.n_chunks):
                idx = np.arange(W.chunk * c, W.chunk * (c + 1))
                kc, _ = Cc.slab_write_indexed(kc, ks[:, idx], idx)
                vc, _ = Cc.slab_write_indexed(vc, vs[:, idx], idx)
                A.attend_batch_prefix(qs[:, idx], kc, vc, [W.chunk * (c + 1)] * W.B)

        secs, _ = _median_of(run)
        return {"seconds": round(secs, 5), "us_per_chunk_step": secs / W.n_chunks * 1e6,
                "sample": "the whole tiny workload: B=2, 7 chunks of 8 tokens (writes + attention)"}

    R, M, G = SI.Ring(), SI.MultiUser(), SI.Ragged()
    model, threads = _host_info()
    res = {"what": "fp64 numpy oracle, median of 3 warm runs each", "cpu_model": model,
           "blas_threads": threads}
    res["tiny_workload"] = tiny_whole()
    res["ring_saturated_attention"] = attn_rate(256, R.n_slots * R.C, R.D)
    res["multiuser_chunk15_attention"] = attn_rate(256, M.cap, M.D, A.MASK_BLOCK_CAUSAL, Tq=M.chunk)
    for L0, L1 in G.skews:
        res[f"ragged_{L0}_{L1}_attention"] = attn_rate(4096, L1, G.D)
    ring = Cc.RingPhysical(R.n_slots, R.sink, R.C, (R.H, R.D))
    ring.reserve()
    res["ring_write"] = write_rate(R.C, R.H, R.D, lambda s: ring.write(s[0]))
    slab = np.zeros((1, M.cap, M.H, M.D))
    res["slab_write"] = write_rate(M.chunk, M.H, M.D,
                                   lambda s: Cc.slab_write_indexed(slab, s, np.arange(M.chunk)))
    return res


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("attn_decode.hip", "common.h"):
        with open(os.path.join(ROOT, "streaming_kv_cache_write_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "decode_attention_counters.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        d = json.load(fh)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch

    import seeded_inputs as SI
    import streaming_kv_cache_write_amd as skv
    dev = "cuda:0"
    torch.cuda.set_device(0)

    if args.only and args.only != "decode":
        fn = {"ring": bench_ring, "multiuser": bench_multiuser, "ragged": bench_ragged,
              "sweep": bench_sweep, "peaks": lambda t, k, S, d: bench_peaks(t, k, S, d, {})}[args.only]
        res = {args.only: fn(torch, skv, SI, dev)}
        if args.copy_calibration:
            res["copy_calibration_bytes"] = copy_calibration(torch, dev)
        print(json.dumps(res))
        return

    d = bench_decode(torch, skv, SI, dev, args)
    dk = d["decode_kernel"]
    line = {
        "metric": "chunk-attn TFLOP/s + decode KV-read GB/s (% of MI355X peak); ms per chunk step",
        "value": round(d["value"], 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": "decode with active prefix: B=1, 32 q heads / 8 kv heads, D=128, "
                               "capacity 32768, 234-token causal prefill + 1024 single-token steps "
                               "(kv_len 235..1258); one step = the whole job, replayed as a HIP graph",
                   "decode_step": "fused attn_decode_step (cursor read + row write + split-K attention "
                                  "+ cursor advance in one launch)",
                   "decode_steps_per_s": round(d["decode_steps_per_s"], 1),
                   "gpu_ms_per_step": round(d["gpu_ms_per_step"], 4)},
        "roofline": {"bound": "hbm", "achieved": round(dk["achieved_gbs"], 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dk["achieved_gbs"] / HBM_PEAK_GBS, 5),
                     "traffic": traffic_from_profile(),
                     "kernel": "k_attn_decode, fused step (row write + split-K attention)",
                     "mean_launch_us": round(dk["mean_us"], 3),
                     "algorithmic_bytes_per_launch": round(dk["mean_bytes"])},
    }
    if not args.no_rows:
        rows = {}
        u = bench_decode(torch, skv, SI, dev, args, fused=False)
        rows["decode_three_calls"] = {
            "workload": "same decode job with kv_cursor_advance + kv_write_indexed + attn_chunk_fwd per step",
            "ms_per_job": u["ms_per_step"], "kv_read_gbs": u["value"],
            "attn_kernel_mean_us": u["decode_kernel"]["mean_us"]}
        del u
        torch.cuda.empty_cache()
        for name, fn in (("ring", bench_ring), ("multiuser", bench_multiuser), ("ragged", bench_ragged),
                         ("decode_sweep", bench_sweep)):
            try:
                rows[name] = fn(torch, skv, SI, dev)
            except Exception as e:  # report, never hide
                rows[name] = {"error": repr(e)}
            torch.cuda.empty_cache()
        try:
            line["measured_peaks"] = bench_peaks(torch, skv, SI, dev, rows)
        except Exception as e:  # report, never hide
            line["measured_peaks"] = {"error": repr(e)}
        torch.cuda.empty_cache()
        line["rows"] = rows
        ring, mu = rows.get("ring", {}), rows.get("multiuser", {})
        line["chunk_attention"] = {
            "what": "the metric's chunk-attention part: bf16 TFLOP/s of the saturated ring step (7 "
                    "valid slots, 4680 queries over 32760 keys, B=2, 12 heads) and of multi-user chunk 15 "
                    "(1024 queries over 16384 keys causal in chunk, B=8, 40 heads), fraction of the "
                    "2516.6 TFLOP/s peak; ms per chunk step of both sequences (write + attention)",
            "ring_saturated_tflops": ring.get("saturated_attn_tflops"),
            "ring_saturated_frac_mfma": ring.get("saturated_attn_frac_mfma"),
            "multiuser_chunk15_tflops": mu.get("chunk15_attn_tflops"),
            "multiuser_chunk15_frac_mfma": mu.get("chunk15_attn_frac_mfma"),
            "ring_ms_per_rewrite_step": ring.get("ms_per_rewrite_step"),
            "multiuser_ms_per_chunk_step": mu.get("ms_per_chunk_step")}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(SI, args.dtype)
        if not args.no_rows:
            line["cpu_baseline_rows"] = cpu_baseline_rows(SI)
    if args.copy_calibration:
        line["copy_calibration_bytes"] = copy_calibration(torch, dev)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
