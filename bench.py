"""Benchmark of the narrow-batch q8_0 decode matmul on one MI355X.

A step is one pass of the whole hot path over one decode batch of a
Qwen3-14B-shaped decode layer (hidden 5120): for each of its four weight
matrices (QKV 5120->7168, O 5120->5120, gate+up 5120->34816, down
17408->5120) the 16-slot activation buffer is pre-quantised and the narrow
matmul runs for the live batch, gathered through a seeded random
batch_index (workspace entry point: K splits of small-N matrices spread
over separate workgroups).  Weights are packed once, outside the timed region.
Each matrix rotates, step by step, through enough packed copies to exceed
1 GiB on its own (28 of QKV, 39 of O, 6 of gate+up, 12 of down), so neither
a step nor a single matrix's timing finds its weights in the 256 MB
last-level cache.

Reported (one JSON line): the whole step's achieved GB/s from algorithmic
bytes (packed weights 34 B per 32 weights, the live tokens' activation
blocks, batch_index, Y, and the quantiser's fp32 input and q8_0 output), the
step time, the same at every live batch 1..16 with t(16)/t(1) and the
speedup n*t(1)/t(n) over n single-token calls ("Batched decode: co-decode N
live sessions in one GPU pass", section "Measured", compares ms/step against
n x single-token time the same way), the roofline of the dominant kernel
(the gate+up matmul) from HIP events on its stream, each matrix's launch
time as mean, median and p90 over 11 graph replays, the step time's median
and p90 over 11 windows, a plain read-only streaming kernel's rate over 2
GiB (the measured read ceiling, beside the 8 TB/s vendor peak), and the CPU
oracle's rate on the host cores.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, vendor figure
COLD_BYTES = 1 << 30    # rotate each matrix's weight copies past 1 GiB
MAX_COPIES = 256        # ... but no more copies than this (tiny matrices)
SETTLE_S = 0.25         # untimed steps before the warmup, so clocks have settled
STEP_REPEATS = 11       # windows for the step time's median and p90
PROFILE_DIR = os.path.join(ROOT, "profiles")


def speedup_vs_single(t1: float, tn: float, n: int) -> float:
    """Throughput of one n-token step against n single-token steps."""
    return n * t1 / tn


# ------------------------------------------------------------ byte counts

def matmul_bytes(N: int, K: int, n_live: int) -> int:
    """Algorithmic bytes of one narrow matmul: each weight block once (32
    int8 + a binary16 scale), the live tokens' activation blocks,
    batch_index and the fp32 output."""
    blocks = K // 32
    return N * blocks * 34 + n_live * blocks * 34 + 4 * n_live + 4 * n_live * N


def quantize_bytes(K: int, rows: int = 16) -> int:
    """Algorithmic bytes of pre-quantising `rows` fp32 rows of K values."""
    return rows * K * 4 + rows * (K // 32) * 34


def step_bytes(matrices, n_live: int) -> int:
    return sum(matmul_bytes(m.N, m.K, n_live) + quantize_bytes(m.K) for m in matrices)


# ------------------------------------------------------------------- GPU

def copies_for(nbytes: int) -> int:
    """Packed copies of a matrix whose rotation covers COLD_BYTES (at least
    2, at most MAX_COPIES)."""
    return int(min(MAX_COPIES, max(2, -(-COLD_BYTES // nbytes))))


class Layer:
    """Packed copies of a workload's matrices (each matrix its own rotation
    of at least 1 GiB, or of MAX_COPIES copies for matrices under 4 MiB),
    plus the activation buffers."""

    def __init__(self, key: str, fused: bool = False):
        import torch
        import quantized_weight_streaming_q8_amd as q8
        self.q8 = q8
        self.w = wl.WORKLOADS[key]
        self.mats = list(self.w.matrices)
        sizes = [q8.q8_packed_weight_bytes(m.N, m.K) for m in self.mats]
        self.copies = [copies_for(b) for b in sizes]
        self.packed = []
        self.fused = fused
        self.X, self.Xq, self.Y, self.ws, self.fws = [], [], [], [], []
        for i, m in enumerate(self.mats):
            W = torch.from_numpy(wl.weights(self.w.config, i, m.N, m.K)).cuda()
            base = q8.empty_packed_weights(m.N, m.K)
            q8.q8_pack_weights(W, m.N, m.K, base)
            del W
            self.packed.append([base] + [base.clone() for _ in range(self.copies[i] - 1)])
            self.X.append(torch.from_numpy(
                wl.activations(self.w.config, m.K, outliers=self.w.outliers)).cuda())
            self.Xq.append(q8.empty_act_slots(m.K))
            self.Y.append(torch.empty((16, m.N), dtype=torch.float32, device="cuda"))
            self.ws.append(q8.zeroed_workspace(m.N, m.K))
            self.fws.append(q8.zeroed_fused_workspace(m.N, m.K))
        torch.cuda.synchronize()
        self.packed_bytes = sum(sizes)
        self.cold_bytes = sum(c * b for c, b in zip(self.copies, sizes))

    def weights(self, i: int, step: int):
        """Matrix i's packed copy for step `step` of the rotation."""
        return self.packed[i][step % self.copies[i]]

    def launches(self, i: int) -> int:
        """Back-to-back launches of matrix i in one timed graph: every copy
        of its rotation at least once."""
        return max(64, self.copies[i])

    def batch_index(self, n_live: int):
        import torch
        bi = wl.batch_index(self.w.config, n_live, random=self.w.random_batch_index)
        return torch.from_numpy(bi).cuda()

    def step(self, s: int, bi, n_live: int, events=None) -> None:
        """Enqueue step s: for every matrix, pre-quantise the 16 slots and
        run the narrow matmul on that step's weight copy, either in one fused
        launch or as the two separate calls; with `events`, bracket every
        matrix's launches with a pair of events recorded on the launch
        stream."""
        q8 = self.q8
        for i, m in enumerate(self.mats):
            if events is not None:
                events[i][0].record()
            if self.fused:
                q8.q8_matmul_narrow_fused(self.weights(i, s), self.X[i], 16, self.Xq[i], bi,
                                          n_live, m.N, m.K, self.Y[i], self.fws[i])
            else:
                q8.q8_quantize_acts(self.X[i], 16, m.K, self.Xq[i])
                q8.q8_matmul_narrow_ws(self.weights(i, s), self.Xq[i], bi, n_live, m.N, m.K,
                                       self.Y[i], self.ws[i])
            if events is not None:
                events[i][1].record()

    def settle(self, n_live: int, seconds: float = SETTLE_S) -> None:
        """Untimed steps for `seconds` of wall time (setup: lets the clocks
        and the page tables of every weight copy settle before the warmup)."""
        import torch
        bi = self.batch_index(n_live)
        t0 = time.perf_counter()
        s = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                self.step(s, bi, n_live)
                s += 1
            torch.cuda.synchronize()


def _event_pair():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_steps(layer: Layer, n_live: int, steps: int, warmup: int, with_events: bool):
    """Run `warmup` untimed steps, then time exactly `steps` steps between a
    pair of HIP events on the launch stream, with a device synchronisation
    on both sides.  Returns (ms per step, per-matrix kernel ms lists)."""
    import torch
    bi = layer.batch_index(n_live)
    for s in range(warmup):
        layer.step(s, bi, n_live)
    torch.cuda.synchronize()
    ev = []
    if with_events:
        ev = [[list(_event_pair()) for _ in layer.mats] for _ in range(steps)]
    e0, e1 = _event_pair()
    e0.record()
    for s in range(steps):
        layer.step(warmup + s, bi, n_live, ev[s] if with_events else None)
    e1.record()
    torch.cuda.synchronize()
    kern = [[] for _ in layer.mats]
    if with_events:
        for s in range(steps):
            for i in range(len(layer.mats)):
                kern[i].append(ev[s][i][0].elapsed_time(ev[s][i][1]))
    return e0.elapsed_time(e1) / steps, kern


def steps_per_graph(steps: int, most: int = 40) -> int:
    """Steps one captured graph holds: the largest divisor of `steps` that
    is at most `most` (so exactly `steps` steps are replayed)."""
    return max(n for n in range(1, min(most, steps) + 1) if steps % n == 0)


def capture_step_graph(layer: Layer, n_live: int, spg: int):
    """One HIP graph holding `spg` whole steps (each the four quantise +
    matmul pairs, each matrix's weight copies in rotation), captured through
    torch's graph API on the stream the library launches on.  With several
    steps per graph, the host's cost of launching a graph is spread over
    them."""
    import torch
    bi = layer.batch_index(n_live)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for k in range(spg):
            layer.step(k, bi, n_live)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(spg):
            layer.step(k, bi, n_live)
    torch.cuda.synchronize()
    return g, bi


def time_graph_steps(layer: Layer, n_live: int, steps: int, warmup: int):
    """Step time with the steps replayed from captured graphs of several
    steps each (exactly `steps` steps in all), between a pair of HIP events.
    Returns (ms per step, True if every output of the last replay is
    bit-identical to an eager step on the same inputs, steps per graph)."""
    import torch
    spg = steps_per_graph(steps)
    g, bi = capture_step_graph(layer, n_live, spg)
    for _ in range(max(1, warmup // spg)):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = _event_pair()
    e0.record()
    for _ in range(steps // spg):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    got = [y.clone() for y in layer.Y]
    layer.step(spg - 1, bi, n_live)
    torch.cuda.synchronize()
    same = all(torch.equal(a.view(torch.int32), b.view(torch.int32)) for a, b in zip(got, layer.Y))
    del g
    return e0.elapsed_time(e1) / steps, same, spg


def run_schedule(layer: Layer, steps: int, warmup: int) -> dict:
    """The workload's seeded decode schedule: `steps` steps whose live batch
    is uniform on 1..16, each step's batch_index a random prefix of a slot
    permutation, every step the whole hot path (each matrix: pre-quantise,
    then the narrow matmul at that step's live batch) with the weight copies
    rotated.  Reports the aggregate GB/s over the whole schedule (eager
    launches, and one HIP graph of the whole schedule, checked bit-identical
    to eager on its last step) and, per live batch, the number of steps and
    their mean time from a pair of HIP events around every step."""
    import torch
    sched = wl.schedule(layer.w.config, steps)
    bis = [torch.from_numpy(b).cuda() for b in sched]
    ns = [int(b.size) for b in sched]
    total = sum(step_bytes(layer.mats, n) for n in ns)

    def run_all(events=None):
        for s in range(steps):
            if events is not None:
                events[s][0].record()
            layer.step(s, bis[s], ns[s])
            if events is not None:
                events[s][1].record()

    for s in range(min(warmup, steps)):
        layer.step(s, bis[s], ns[s])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run_all()
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s in range(min(steps, 40)):
            layer.step(s, bis[s], ns[s])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_graph = e0.elapsed_time(e1)
    got = [y.clone() for y in layer.Y]
    layer.step(steps - 1, bis[-1], ns[-1])
    torch.cuda.synchronize()
    same = all(torch.equal(a.view(torch.int32), b.view(torch.int32)) for a, b in zip(got, layer.Y))
    del g

    ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
          for _ in range(steps)]
    run_all(ev)
    torch.cuda.synchronize()
    per = {}
    for n, (a, b) in zip(ns, ev):
        per.setdefault(n, []).append(a.elapsed_time(b))
    by_n = {}
    for n in sorted(per):
        t = float(np.mean(per[n]))
        by_n[n] = {"steps": len(per[n]), "mean_us": round(t * 1e3, 2),
                   "GBps": round(step_bytes(layer.mats, n) / (t * 1e-3) / 1e9, 1)}
    ms = ms_graph if same and ms_graph < ms_eager else ms_eager
    return {
        "workload": layer.w.key, "matrices": {m.name: [m.K, m.N] for m in layer.mats},
        "steps": steps, "schedule": "live batch uniform on 1..16, seeded random prefix of a slot "
                                    "permutation per step",
        "bytes": total, "value": round(total / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
        "frac_peak": round(total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "ms_total": round(ms, 4), "us_per_step": round(ms * 1e3 / steps, 2),
        "ms_total_eager": round(ms_eager, 4), "ms_total_graph": round(ms_graph, 4),
        "graph_bit_identical": same,
        "timing": "one hip graph of the whole schedule" if ms is ms_graph else "eager launches",
        "weight_copies_rotated": dict(zip((m.name for m in layer.mats), layer.copies)),
        "by_n_live": by_n,
    }


def graph_replay_us(launch, launches: int, replays: int) -> list:
    """Per-launch duration of each of `replays` replays of one HIP graph that
    holds `launches` back-to-back launches (launch(c) for c in
    range(launches)), each replay between its own pair of HIP events on the
    launch stream."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in range(4):
            launch(c)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in range(launches):
            launch(c)
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / launches)
    del g
    return out


def graph_avg_us(launch, launches: int, replays: int = 3) -> float:
    """Average duration of one launch: `launches` back-to-back launches
    (launch(c) for c in range(launches)) captured in one HIP graph, replayed
    `replays` times between one pair of HIP events on the launch stream, so
    that neither the host's launch rate nor the events' own cost shows."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in range(4):
            launch(c)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in range(launches):
            launch(c)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (launches * replays)


def kernel_stats_us(layer: Layer, i: int, n_live: int, launches: int, replays: int = 11) -> dict:
    """Matrix i's narrow matmul, as kernel_avg_us, over `replays` graph
    replays: the mean launch duration and the median and p90 of the
    per-replay means."""
    q8, m = layer.q8, layer.mats[i]
    bi = layer.batch_index(n_live)
    r = graph_replay_us(lambda c: q8.q8_matmul_narrow_ws(
        layer.weights(i, c), layer.Xq[i], bi, n_live, m.N, m.K,
        layer.Y[i], layer.ws[i]), launches, replays)
    return {"mean": float(np.mean(r)), "median": float(np.median(r)),
            "p90": float(np.percentile(r, 90)), "replays": replays, "launches_each": launches}


def kernel_avg_us(layer: Layer, i: int, n_live: int, launches: int) -> float:
    """Average duration of one launch of matrix i's narrow matmul (the
    workspace entry point the step uses), back to back over the rotated
    weight copies."""
    q8, m = layer.q8, layer.mats[i]
    bi = layer.batch_index(n_live)
    return graph_avg_us(lambda c: q8.q8_matmul_narrow_ws(
        layer.weights(i, c), layer.Xq[i], bi, n_live, m.N, m.K,
        layer.Y[i], layer.ws[i]), launches)


def fused_avg_us(layer: Layer, i: int, n_live: int, launches: int) -> float:
    """Average duration of one fused pre-quantise + matmul launch of matrix i."""
    q8, m = layer.q8, layer.mats[i]
    bi = layer.batch_index(n_live)
    return graph_avg_us(lambda c: q8.q8_matmul_narrow_fused(
        layer.weights(i, c), layer.X[i], 16, layer.Xq[i], bi, n_live, m.N, m.K,
        layer.Y[i], layer.fws[i]), launches)


def quantize_avg_us(layer: Layer, i: int, launches: int = 100) -> float:
    """Average duration of one pre-quantize launch (16 rows of matrix i's K)."""
    q8, m = layer.q8, layer.mats[i]
    return graph_avg_us(lambda c: q8.q8_quantize_acts(layer.X[i], 16, m.K, layer.Xq[i]), launches)


def read_ceiling_gbs(q8, nbytes: int = 2 << 30, reps: int = 10) -> float:
    """Rate of the library's plain read-only streaming kernel over a 2 GiB
    buffer (every byte read once per pass): the measured HBM read ceiling."""
    import torch
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    for _ in range(2):
        q8.q8_stream_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        q8.q8_stream_read(buf, nbytes, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9


def copy_ceiling_gbs(nbytes: int = 1 << 30, reps: int = 20) -> float:
    """Read+write rate of a plain device-to-device copy (torch's copy
    kernel), for context."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


# ------------------------------------------------------------ CPU oracle

def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or '' if unknown."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(key: str, n_live: int, seconds: float = 10.0):
    """The oracle as it stands, on the host cores: full passes over the
    workload's matrices at this live batch, repeated until `seconds` of
    wall time have passed.  Returns a dict for the JSON line."""
    import oracle
    orc = oracle.get()
    w = wl.WORKLOADS[key]
    bi = wl.batch_index(w.config, n_live, random=w.random_batch_index)
    data = []
    for i, m in enumerate(w.matrices):
        qw, dw = orc.quantize_rows(wl.weights(w.config, i, m.N, m.K))
        data.append((m, qw, dw, wl.activations(w.config, m.K, outliers=w.outliers)))
    nbytes = 0
    passes = 0
    t0 = time.perf_counter()
    while True:
        for m, qw, dw, X in data:
            qx, dx = orc.quantize_rows(X)
            orc.matmul(qw, dw, qx, dx, bi)
            nbytes += matmul_bytes(m.N, m.K, n_live) + quantize_bytes(m.K)
        passes += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(nbytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": orc.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{passes} full pass(es) of the {key} step (all {len(data)} matrices, "
                   f"quantise + matmul) at n_live={n_live}, {dt:.1f} s wall"),
        "ms_per_step": round(dt * 1e3 / passes, 3),
    }


def _median_wall(fn, runs: int, min_s: float = 0.2, most: int = 200) -> float:
    """Median wall time of fn() over at least `runs` timed calls (more, up to
    `most`, until min_s seconds have been timed), after one untimed call: on
    small matrices a single call is shorter than the host's thread wake-ups."""
    fn()
    ts = []
    while len(ts) < runs or (sum(ts) < min_s and len(ts) < most):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def cpu_detail(key: str, runs: int = 3) -> dict:
    """The oracle as it stands, per matrix of the workload: its matmul at
    n_live 1 and 16, on all the host threads OpenMP uses and on one, each the
    median wall time of at least `runs` runs after an untimed one; and its
    pre-quantisation of the 16 slots per K, timed the same way (all
    threads)."""
    import oracle
    orc = oracle.get()
    w = wl.WORKLOADS[key]
    all_threads = orc.num_threads()
    out = {"workload": key, "threads_all": all_threads, "cpu_model": cpu_model(), "runs": runs,
           "matrices": {}, "quantize": {}}
    for i, m in enumerate(w.matrices):
        qw, dw = orc.quantize_rows(wl.weights(w.config, i, m.N, m.K))
        X = wl.activations(w.config, m.K, outliers=w.outliers)
        qx, dx = orc.quantize_rows(X)
        rec = {}
        for threads in (all_threads, 1):
            orc.set_num_threads(threads)
            for n in (1, 16):
                bi = wl.batch_index(w.config, n, random=w.random_batch_index)
                t = _median_wall(lambda: orc.matmul(qw, dw, qx, dx, bi), runs)
                rec[f"threads={threads} n_live={n}"] = {
                    "ms": round(t * 1e3, 2), "GBps": round(matmul_bytes(m.N, m.K, n) / t / 1e9, 4)}
            print(f"# oracle {m.name} threads={threads}: "
                  + ", ".join(f"{k.split()[1]} {v['ms']} ms" for k, v in rec.items()
                              if k.startswith(f"threads={threads} ")), file=sys.stderr, flush=True)
        orc.set_num_threads(all_threads)
        out["matrices"][m.name] = {"K": m.K, "N": m.N, **rec}
        if m.K not in out["quantize"]:
            t = _median_wall(lambda: orc.quantize_rows(X), runs)
            out["quantize"][m.K] = {"ms": round(t * 1e3, 3),
                                    "GBps": round(quantize_bytes(m.K) / t / 1e9, 4)}
    return out


# ------------------------------------------------------------- profiles

def _code_only(text: str) -> str:
    """C++ source without its comments, blank lines and trailing blanks (the
    kernel sources hold no string literal with a comment marker in it)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line.strip())


def kernel_source_hash() -> str:
    """Hash of the matmul kernel's code (comments and blank lines left out,
    so that a comment edit does not void the counter summaries)."""
    h = hashlib.sha256()
    for name in ("q8_matmul.hip", "q8_internal.h"):
        with open(os.path.join(ROOT, "quantized_weight_streaming_q8_amd", "csrc", name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def output_digest(layer: Layer, i: int, n_live: int) -> str:
    """First 16 hex digits of the SHA-256 of matrix i's output bits: its
    seeded activations pre-quantised, then the workspace matmul on its first
    weight copy for the workload's seeded batch_index at n_live.  A
    measurement to compare runs and commits by (a changed summation tree or
    a regression changes it), not an expected value any test holds."""
    import torch
    q8 = layer.q8
    m = layer.mats[i]
    bi = layer.batch_index(n_live)
    Y = torch.empty((n_live, m.N), dtype=torch.float32, device="cuda")
    q8.q8_quantize_acts(layer.X[i], 16, m.K, layer.Xq[i])
    q8.q8_matmul_narrow_ws(layer.weights(i, 0), layer.Xq[i], bi, n_live, m.N, m.K, Y, layer.ws[i])
    torch.cuda.synchronize()
    return hashlib.sha256(Y.cpu().numpy().tobytes()).hexdigest()[:16]


def dominant_matrix(key: str) -> int:
    """Index of a workload's dominant matrix: the largest (gate+up on the
    Qwen3-14B layer)."""
    return int(np.argmax([m.N * m.K for m in wl.WORKLOADS[key].matrices]))


def pmc_summary_path(workload: str, matrix: str, fused: bool) -> str:
    name = f"{matrix}_{'fused' if fused else 'matmul'}_{workload}_pmc.json"
    return os.path.join(PROFILE_DIR, name)


def measured_traffic(workload: str, matrix: str, n_live: int, fused: bool):
    """HBM bytes per launch of this workload's matrix from the committed PMC
    counter summary, if the summary covers that matrix and was taken on the
    current kernel source."""
    path = pmc_summary_path(workload, matrix, fused)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    if rec.get("workload") != workload or rec.get("matrix") != matrix:
        return None
    per = rec.get("traffic_bytes_per_launch", {}).get(str(n_live))
    return None if per is None else int(per)


# ------------------------------------------------- multi-token columns

def multi_columns(layer: Layer, widths) -> dict:
    """The multi-column matmul (q8_matmul_multi) on every matrix of the
    workload with n columns (n slots, all live, seeded random batch_index),
    e.g. n_seq sequences x (k+1) speculative tokens: kernel time per launch,
    algorithmic GB/s, and columns per microsecond."""
    import torch
    q8 = layer.q8
    w = layer.w
    out = {}
    for n in widths:
        rec = {}
        bi = torch.from_numpy(wl.batch_index(w.config, n, random=True, n_slots=n)).cuda()
        for i, m in enumerate(layer.mats):
            X = torch.from_numpy(wl.activations(w.config, m.K, n_slots=n, outliers=w.outliers)).cuda()
            Xq = q8.empty_act_slots(m.K, n_slots=n)
            q8.q8_quantize_acts_n(X, n, m.K, Xq, n)
            Y = torch.empty((n, m.N), dtype=torch.float32, device="cuda")
            us = graph_avg_us(lambda c: q8.q8_matmul_multi(
                layer.weights(i, c), Xq, n, bi, n, m.N, m.K, Y), layer.launches(i))
            rec[m.name] = {"us": round(us, 2), "GBps": round(matmul_bytes(m.N, m.K, n) / us / 1e3, 1)}
            del X, Xq, Y
        tot = sum(r["us"] for r in rec.values())
        rec["all"] = {"us": round(tot, 2),
                      "GBps": round(sum(matmul_bytes(m.N, m.K, n) for m in layer.mats) / tot / 1e3, 1),
                      "columns_per_us": round(n / tot, 3)}
        out[str(n)] = rec
        print(f"# {n} columns: matmuls {tot:.1f} us, {rec['all']['GBps']} GB/s", file=sys.stderr,
              flush=True)
    return out


# ------------------------------------------------------ pos-vector RoPE



def rope_after_qkv(layer: Layer, n_live: int, launches: int = 100):
    """The pos-vector RoPE on the QKV matmul's output rows (the workload's
    query and key heads, e.g. 40 + 8 heads of 128 on the Qwen3-14B layer, one
    position per live token): average launch duration and algorithmic GB/s
    (each rotated value read and written once in fp32, plus the positions).
    None for a workload without a QKV matrix or a RoPE configuration."""
    import torch
    q8 = layer.q8
    i = [k for k, m in enumerate(layer.mats) if m.name == "qkv"]
    if not i or layer.w.rope is None:
        return None
    heads, head_dim, base = layer.w.rope
    m = layer.mats[i[0]]
    if heads * head_dim > m.N:
        return None
    pos = torch.arange(1000, 1000 + n_live, dtype=torch.int32, device="cuda") * 37
    us = graph_avg_us(lambda c: q8.q8_rope_multi(layer.Y[i[0]], n_live, m.N, pos, heads,
                                                 head_dim, base), launches)
    nbytes = 2 * 4 * n_live * heads * head_dim + 4 * n_live
    return {"us": round(us, 2), "GBps": round(nbytes / us / 1e3, 1), "rows": n_live,
            "heads": heads, "head_dim": head_dim, "base": base}


# ------------------------------------------------------- engine A/B

def engine_ab(layer: Layer, n_values) -> dict:
    """Both int8 dot engines (MFMA tiles against all 16 slots; v_dot4 with
    one row per lane and the live tokens' blocks through scalar loads) on
    every matrix of the workload, plain entry point, per live batch: the
    evidence for the default engine."""
    q8 = layer.q8
    out = {}
    for i, m in enumerate(layer.mats):
        for n in n_values:
            bi = layer.batch_index(n)
            rec = {}
            for name, path in (("mfma", q8.Q8_PATH_MFMA), ("dot4", q8.Q8_PATH_DOT4)):
                us = graph_avg_us(lambda c: q8.q8_matmul_narrow_path(
                    layer.weights(i, c), layer.Xq[i], bi, n, m.N, m.K,
                    layer.Y[i], path=path), layer.launches(i))
                rec[name] = {"us": round(us, 2),
                             "GBps": round(matmul_bytes(m.N, m.K, n) / us / 1e3, 1)}
            out[f"{m.name} n_live={n}"] = rec
            print(f"# {m.name} n_live={n}: mfma {rec['mfma']['us']} us, dot4 {rec['dot4']['us']} us",
                  file=sys.stderr, flush=True)
    return out


# --------------------------------------------------- HBM traffic counters
#
# Two rocprofv3 counter passes over `bench.py --pmc-probe` (FETCH_SIZE, then
# WRITE_SIZE) read the HBM traffic of the dominant matmul.  The same probe
# runs a plain device copy of CAL_BYTES, whose true traffic is known (read
# CAL_BYTES, write CAL_BYTES); each counter is scaled by known / counted on
# that copy.  `bench.py --pmc-summarize FETCH_CSV WRITE_CSV` turns the two
# counter_collection.csv files into the committed summary that the JSON
# line's roofline.traffic reads back.

CAL_BYTES = 256 << 20


def pmc_probe(key: str, launches: int, n_live: int, fused: bool, columns: int = 16) -> None:
    """Every matrix of the workload's step in turn (the fused pre-quantise +
    matmul, or the matmul alone; with `columns` > 16 the multi-column matmul
    over that many slot columns, all live), `launches` times each over two
    weight copies, then the calibration copy three times."""
    import torch
    import quantized_weight_streaming_q8_amd as q8
    w = wl.WORKLOADS[key]
    bi = torch.from_numpy(wl.batch_index(w.config, n_live, random=w.random_batch_index)).cuda()
    for i, m in enumerate(w.matrices):
        W = torch.from_numpy(wl.weights(w.config, i, m.N, m.K)).cuda()
        packed = [q8.empty_packed_weights(m.N, m.K) for _ in range(2)]
        for P in packed:
            q8.q8_pack_weights(W, m.N, m.K, P)
        del W
        X = torch.from_numpy(wl.activations(w.config, m.K, n_slots=columns,
                                            outliers=w.outliers)).cuda()
        Xq = q8.empty_act_slots(m.K, n_slots=columns)
        q8.q8_quantize_acts_n(X, columns, m.K, Xq, columns)
        Y = torch.empty((columns, m.N), dtype=torch.float32, device="cuda")
        ws = q8.zeroed_workspace(m.N, m.K)
        fws = q8.zeroed_fused_workspace(m.N, m.K)
        if columns > 16:
            bi = torch.from_numpy(wl.batch_index(w.config, columns, random=True,
                                                 n_slots=columns)).cuda()
        torch.cuda.synchronize()
        for c in range(launches):
            if columns > 16:
                q8.q8_matmul_multi(packed[c % 2], Xq, columns, bi, columns, m.N, m.K, Y)
            elif fused:
                q8.q8_matmul_narrow_fused(packed[c % 2], X, 16, Xq, bi, n_live, m.N, m.K, Y, fws)
            else:
                q8.q8_matmul_narrow_ws(packed[c % 2], Xq, bi, n_live, m.N, m.K, Y, ws)
        torch.cuda.synchronize()
        del packed, X, Xq, Y, ws, fws
        torch.cuda.empty_cache()
        print(f"pmc probe: {launches} {'fused' if fused else 'matmul'} launches of {m.name} "
              f"at n_live={columns if columns > 16 else n_live} ({columns} slot columns)",
              flush=True)
    a = torch.empty(CAL_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"pmc probe: 3 copies of {CAL_BYTES} B", flush=True)


TICK_US = 0.01            # s_memrealtime: 100 MHz
TIMELINE_MAX_WAVES = 1 << 20
PCTS = (0, 10, 50, 90, 100)


def _pct(a) -> list:
    a = np.asarray(a, dtype=np.float64)
    a = a[~np.isnan(a)]
    return [round(float(v), 3) for v in np.percentile(a, PCTS)] if a.size else []


def timeline_summary(recs: list, split: bool) -> dict:
    """Phase durations (us, percentiles over every wave of every recorded
    launch) from timeline-build records (include/q8timeline.h), each launch
    taken from its own earliest wave start, plus each launch's span, the
    waves per CU against when each CU's last wave ended, and whether the
    same CUs end last from launch to launch."""
    ph = {k: [] for k in ("start", "first_chunk", "stream", "reduce", "stream_end", "end")}
    ph.update({k: [] for k in (("publish", "arrive", "combine", "last_tail") if split
                               else ("y_issue", "y_done"))})
    spans, cu_rows, xcc_rows, cu_keys = [], [], [], []
    for t in recs:
        t = t[t[:, 0] > 0]
        t0 = t[:, 0].min()
        r = (t[:, :7] - t0).astype(np.float64) * TICK_US
        r[t[:, :7] == 0] = np.nan
        ph["start"].append(r[:, 0])
        ph["first_chunk"].append(r[:, 1] - r[:, 0])
        ph["stream"].append(r[:, 2] - r[:, 1])
        ph["reduce"].append(r[:, 3] - r[:, 2])
        ph["stream_end"].append(r[:, 2])
        if split:
            last = ~np.isnan(r[:, 6])
            ph["publish"].append(r[:, 4] - r[:, 3])
            ph["arrive"].append(r[:, 5] - r[:, 4])
            ph["combine"].append((r[:, 6] - r[:, 5])[last])
            ph["last_tail"].append((r[:, 6] - r[:, 2])[last])
            end = np.where(last, r[:, 6], r[:, 5])
        else:
            ph["y_issue"].append(r[:, 4] - r[:, 3])
            ph["y_done"].append(r[:, 5] - r[:, 4])
            end = r[:, 5]
        ph["end"].append(end)
        spans.append(float(np.nanmax(end)))
        hw = t[:, 7].astype(np.uint64)
        xcc_rows.append(((hw >> np.uint64(32)) & np.uint64(0xF)).astype(np.int64))
        cu = ((hw >> np.uint64(32)) & np.uint64(0xF)) * np.uint64(256) + ((hw >> np.uint64(8)) & np.uint64(0xFF))
        keys, inv, counts = np.unique(cu, return_inverse=True, return_counts=True)
        last_end = np.full(keys.size, -np.inf)
        np.maximum.at(last_end, inv, end)
        cu_rows.append((counts, last_end))
        cu_keys.append(keys)
    out = {"launches": len(recs), "waves": int((recs[0][:, 0] > 0).sum()),
           "span_us": [round(v, 3) for v in spans], "span_us_median": round(float(np.median(spans)), 3),
           "phases_us": {k: _pct(np.concatenate(v)) for k, v in ph.items()},
           "percentiles": list(PCTS)}
    counts = np.concatenate([c for c, _ in cu_rows])
    ends = np.concatenate([e for _, e in cu_rows])
    out["cus_used"] = int(np.median([c.size for c, _ in cu_rows]))
    # do the same CUs end last in every launch?  Spearman rank correlation of
    # the CUs' last-wave end times between every pair of recorded launches
    # (CUs present in both), median over the pairs: near 1 for CUs that are
    # slow every time, near 0 for a spread that is new in each launch
    corr = []
    for i in range(len(cu_keys)):
        for j in range(i + 1, len(cu_keys)):
            _, a, b = np.intersect1d(cu_keys[i], cu_keys[j], return_indices=True)
            if a.size > 2:
                ra = np.argsort(np.argsort(cu_rows[i][1][a])).astype(np.float64)
                rb = np.argsort(np.argsort(cu_rows[j][1][b])).astype(np.float64)
                corr.append(float(np.corrcoef(ra, rb)[0, 1]))
    out["cu_end_rank_corr_median"] = round(float(np.median(corr)), 3) if corr else None
    out["cu_last_end_us"] = _pct(ends)  # when each CU's last wave ended, over the CUs
    out["waves_per_cu"] = {int(n): {"cus": int((counts == n).sum() // len(recs)),
                                    "last_end_us_median": round(float(np.median(ends[counts == n])), 3)}
                           for n in np.unique(counts)}
    xcc = np.concatenate(xcc_rows)
    end_all = np.concatenate(ph["end"])
    se_all = np.concatenate(ph["stream_end"])
    out["per_xcc"] = {int(x): {"waves": int((xcc == x).sum() // len(recs)),
                               "stream_end_us_p50": round(float(np.nanmedian(se_all[xcc == x])), 3),
                               "end_us_p50": round(float(np.nanmedian(end_all[xcc == x])), 3),
                               "end_us_max": round(float(np.nanmax(end_all[xcc == x])), 3)}
                      for x in np.unique(xcc)}
    return out


def timeline_run(key: str, n_live: int, recorded: int = 5, fused: bool = False) -> dict:
    """Per-wave timelines of every matrix's narrow matmul (workspace entry
    point, or with `fused` the fused pre-quantise + matmul, whose records
    are its matmul workgroups' waves) from the timeline build: for each
    matrix, warm-up replays, then
    `recorded` times a series of 8 back-to-back launches over the weight
    rotation with recording on; each series leaves the records of its last
    launch."""
    import torch
    import quantized_weight_streaming_q8_amd as q8
    if not q8.TIMELINE:
        raise RuntimeError("the timeline needs Q8_LIBRARY=timeline before the package is imported")
    layer = Layer(key)
    bi = layer.batch_index(n_live)
    rec = torch.zeros(TIMELINE_MAX_WAVES * q8.Q8_STAMP_WORDS, dtype=torch.int64, device="cuda")
    res = {}
    for i, m in enumerate(layer.mats):
        q8.q8_quantize_acts(layer.X[i], 16, m.K, layer.Xq[i])

        def launch(c, i=i, m=m):
            if fused:
                q8.q8_matmul_narrow_fused(layer.weights(i, c), layer.X[i], 16, layer.Xq[i], bi,
                                          n_live, m.N, m.K, layer.Y[i], layer.fws[i])
            else:
                q8.q8_matmul_narrow_ws(layer.weights(i, c), layer.Xq[i], bi, n_live, m.N, m.K,
                                       layer.Y[i], layer.ws[i])
        n = layer.launches(i)
        us = float(np.mean(graph_replay_us(launch, n, 3)))
        recs = []
        for r in range(recorded):
            rec.zero_()
            q8.q8_timeline_set(rec, TIMELINE_MAX_WAVES)
            for c in range(8):
                launch(8 * r + c)
            q8.q8_timeline_set(None, 0)
            torch.cuda.synchronize()
            recs.append(rec.view(-1, q8.Q8_STAMP_WORDS).cpu().numpy().copy())
        split = q8.q8_matmul_workspace_bytes(m.N, m.K) > 0  # the same tiling fused
        res[m.name] = dict(timeline_summary(recs, split), K=m.K, N=m.N, n_live=n_live,
                           split=split, timeline_build_us_per_launch=round(us, 3))
        print(f"timeline: {m.name} {m.K}->{m.N}: span {res[m.name]['span_us_median']} us "
              f"(timeline build, graph replays: {us:.2f} us per launch)", flush=True)
    return {"workload": key, "fused": fused, "kernel_source_hash": kernel_source_hash(),
            "matrices": res}


def _counter_rows(path: str, counter: str):
    import csv
    with open(path) as f:
        return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]


def pmc_summarize(fetch_csv: str, write_csv: str, key: str, n_live: int, fused: bool,
                  launches: int) -> dict:
    """Per-launch HBM bytes of each matrix's kernel from the two counter
    passes over `bench.py --pmc-probe LAUNCHES` (the matmul dispatches in
    dispatch order are LAUNCHES per matrix, in the workload's order), each
    counter scaled by what it reads on the calibration copy.  Writes one
    summary per matrix under profiles/ and returns them."""
    mats = wl.WORKLOADS[key].matrices
    per_m = {m.name: {} for m in mats}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, name)
        mm = sorted(((int(r["Dispatch_Id"]), float(r["Counter_Value"])) for r in rows
                     if "mm_mfma_kernel" in r["Kernel_Name"]))
        if len(mm) != launches * len(mats):
            raise SystemExit(f"{path}: {len(mm)} matmul dispatches for {name}, expected "
                             f"{launches} x {len(mats)}")
        last_mm = mm[-1][0]
        cal = [float(r["Counter_Value"]) for r in rows
               if "copyBuffer" in r["Kernel_Name"] and int(r["Dispatch_Id"]) > last_mm]
        if not cal:
            raise SystemExit(f"{path}: no calibration dispatches for {name}")
        scale = (CAL_BYTES / 1024.0) / float(np.median(cal))  # counters are in KiB
        for j, m in enumerate(mats):
            vals = [v for _, v in mm[j * launches:(j + 1) * launches]]
            per_m[m.name][name] = {"matmul_KiB_per_dispatch_median": float(np.median(vals)),
                                   "calibration_KiB_median": float(np.median(cal)),
                                   "scale": scale,
                                   "bytes_per_launch": float(np.median(vals)) * 1024.0 * scale,
                                   "dispatches": len(vals)}
    out = {}
    for m in mats:
        per = per_m[m.name]
        traffic = int(per["FETCH_SIZE"]["bytes_per_launch"] + per["WRITE_SIZE"]["bytes_per_launch"])
        res = {"kernel_source_hash": kernel_source_hash(), "workload": key, "matrix": m.name,
               "K": m.K, "N": m.N, "n_live": n_live, "fused": fused,
               "calibration_copy_bytes": CAL_BYTES, "counters": per,
               "algorithmic_bytes_per_launch": matmul_bytes(m.N, m.K, n_live)
               + (quantize_bytes(m.K) if fused else 0),
               "traffic_bytes_per_launch": {str(n_live): traffic}}
        res["traffic_over_algorithmic"] = round(traffic / res["algorithmic_bytes_per_launch"], 4)
        with open(pmc_summary_path(key, m.name, fused), "w") as f:
            json.dump(res, f, indent=1)
        out[m.name] = res
    return out


def pmc_table(path: str, key: str, launches: int, columns: int) -> dict:
    """Per-dispatch medians of every counter in one counter_collection.csv of
    `bench.py --pmc-probe LAUNCHES [--columns C]` (LAUNCHES matmul dispatches
    per matrix, in the workload's order; a counter's rows of one dispatch
    summed), with the VALU and MFMA instruction counts set against the
    work: a term is one block's int32 dot of one row against one slot column,
    scaled into fp32 (the kernel computes every slot column of its tiles)."""
    import csv
    mats = wl.WORKLOADS[key].matrices
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if "mm_mfma_kernel" not in r["Kernel_Name"]:
                continue
            d = per.setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(per)
    if len(ids) != launches * len(mats):
        raise SystemExit(f"{path}: {len(ids)} matmul dispatches, expected {launches} x {len(mats)}")
    out = {"workload": key, "columns": columns, "kernel_source_hash": kernel_source_hash(),
           "matrices": {}}
    for j, m in enumerate(mats):
        rows = [per[i] for i in ids[j * launches:(j + 1) * launches]]
        med = {c: float(np.median([r[c] for r in rows])) for c in sorted(rows[0])}
        G, KB = (m.N + 15) // 16, m.K // 32
        terms = G * 16 * KB * columns
        res = {"K": m.K, "N": m.N, "dispatches": len(rows), "counters_median": med,
               "terms": terms, "mfma_expected": G * KB * (columns // 16)}
        if "SQ_INSTS_VALU" in med:
            res["valu_insts_per_term"] = round(med["SQ_INSTS_VALU"] * 64 / terms, 3)
        if "SQ_INSTS_MFMA" in med and "SQ_INSTS_VALU" in med:
            res["valu_minus_mfma_per_term"] = round(
                (med["SQ_INSTS_VALU"] - med["SQ_INSTS_MFMA"]) * 64 / terms, 3)
        for c in ("SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU_FMA_F32", "SQ_INSTS_VALU_MUL_F32",
                  "SQ_INSTS_VALU_ADD_F32", "SQ_INSTS_VALU_INT32", "SQ_INSTS_SALU"):
            if c in med:
                res[c.replace("SQ_INSTS_", "").lower() + "_per_term"] = round(med[c] * 64 / terms, 3)
        out["matrices"][m.name] = res
    return out


def trace_table(trace_dir: str, prefix: str = "kt") -> str:
    """Markdown table of a rocprofv3 --kernel-trace --output-format csv run
    (files PREFIX_kernel_trace.csv and PREFIX_kernel_stats.csv in trace_dir):
    the library's kernels grouped by name and launch shape, with launches
    and the mean, median, min and max duration in us, then the library's
    rows of the stats file as written."""
    import csv
    import re

    def short(n):
        n = re.sub(r"^void ", "", n).replace("q8::(anonymous namespace)::", "")
        return re.sub(r"\(.*$", "", n)

    ours = ("mm_", "quantize", "rope", "stream_read", "pack_", "unpack", "clear_scratch")
    rows = {}
    with open(os.path.join(trace_dir, f"{prefix}_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            n = short(r["Kernel_Name"])
            if not n.startswith(ours):
                continue
            key = (n, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]), r["VGPR_Count"],
                   r["LDS_Block_Size"])
            rows.setdefault(key, []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    lines = ["| kernel | grid (threads) | block | VGPR_Count (trace field) | LDS B | launches | mean | "
             "median | min | max |", "|---|---|---|---|---|---|---|---|---|---|"]
    for key, v in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        n, g, b, vg, lds = key
        lines.append(f"| `{n}` | {g} | {b} | {vg} | {lds} | {len(v)} | {np.mean(v):.2f} | "
                     f"{np.median(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    stats = ["Name,Calls,TotalDurationNs,AverageNs,Percentage"]
    with open(os.path.join(trace_dir, f"{prefix}_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            n = short(r["Name"])
            if n.startswith(ours):
                stats.append(f'{n},{r["Calls"]},{r["TotalDurationNs"]},{r["AverageNs"]},'
                             f'{r["Percentage"]}')
    return ("\n".join(lines) + "\n\n" + f"{prefix}_kernel_stats.csv (rocprofv3 --stats, grouped by "
            "kernel name only; the library's rows):\n\n```\n" + "\n".join(stats) + "\n```\n")


# ------------------------------------------------------------------ main

def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="qwen3_layer", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--n-live", type=int, default=16)
    ap.add_argument("--sweep-steps", type=int, default=100,
                    help="steps per live batch in the 1..16 sweep (0: no sweep)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time of the CPU oracle baseline (0: skip)")
    ap.add_argument("--out", default=None, help="also write the JSON line here")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="time eager launches only (no HIP graph replay)")
    ap.add_argument("--pmc-probe", type=int, default=0, metavar="LAUNCHES",
                    help="only launch each matrix's matmul this many times, then the "
                         "calibration copy (for rocprofv3 --pmc)")
    ap.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the per-matrix traffic summaries from two counter_collection.csv "
                         "files of --pmc-probe runs")
    ap.add_argument("--pmc-table", metavar="CSV",
                    help="print per-matrix medians of every counter in one counter_collection.csv "
                         "of a --pmc-probe run (with --columns as in that run), with VALU and MFMA "
                         "instructions per term")
    ap.add_argument("--trace-table", metavar="DIR",
                    help="print the markdown table of a rocprofv3 --kernel-trace --stats "
                         "--output-format csv -o kt run written to DIR")
    ap.add_argument("--pmc-launches", type=int, default=20,
                    help="the LAUNCHES of the --pmc-probe runs being summarised")
    ap.add_argument("--columns", type=int, default=16, choices=(16, 32, 48, 64),
                    help="--pmc-probe only: slot columns of the matmul (above 16: the multi-column "
                         "matmul with every column live)")
    ap.add_argument("--fused", action="store_true",
                    help="run the step through the fused pre-quantise + matmul entry point "
                         "(one launch per matrix; default: separate launches, faster here)")
    ap.add_argument("--no-multi", dest="multi", action="store_false",
                    help="skip the 16..64-column multi-token measurement")
    ap.add_argument("--engine-ab", action="store_true",
                    help="only time both dot engines on every matrix at n_live 1, 2, 4, 8, 16")
    ap.add_argument("--cpu-detail", action="store_true",
                    help="only time the CPU oracle per matrix at n_live 1 and 16, on all host "
                         "threads and on one (median of 3), and its pre-quantisation")
    ap.add_argument("--timeline", action="store_true",
                    help="only record per-wave timelines of each matrix's matmul with the timeline "
                         "build (libq8narrow_timeline.so) and print their summary")
    ap.add_argument("--schedule", type=int, default=0, metavar="STEPS",
                    help="only run the workload's seeded decode schedule of this many steps "
                         "(live batch uniform on 1..16): aggregate GB/s and per-live-batch times")
    args = ap.parse_args(argv)

    if args.trace_table:
        print(trace_table(args.trace_table))
        return 0
    if args.pmc_table:
        print(json.dumps(pmc_table(args.pmc_table, args.workload, args.pmc_launches, args.columns),
                         indent=1))
        return 0
    if args.pmc_summarize:
        print(json.dumps(pmc_summarize(*args.pmc_summarize, args.workload, args.n_live, args.fused,
                                       args.pmc_launches), indent=1))
        return 0

    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the narrow matmul is a single-GPU kernel here).", file=sys.stderr)
        return 2
    if not 1 <= args.n_live <= 16:
        print("--n-live must be in 1..16", file=sys.stderr)
        return 2

    if args.cpu_detail:
        res = cpu_detail(args.workload)
        text = json.dumps(res)
        print(text, flush=True)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text + "\n")
        return 0

    if args.timeline:
        os.environ["Q8_LIBRARY"] = "timeline"  # before the package's first import
    import torch
    torch.cuda.set_device(0)
    if args.timeline:
        res = timeline_run(args.workload, args.n_live, fused=args.fused)
        text = json.dumps(res, indent=1)
        print(text, flush=True)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text + "\n")
        return 0
    if args.pmc_probe:
        pmc_probe(args.workload, args.pmc_probe, args.n_live, args.fused, args.columns)
        return 0
    layer = Layer(args.workload, fused=args.fused)
    mats = layer.mats
    if args.engine_ab:
        res = engine_ab(layer, (1, 2, 4, 8, 16))
        text = json.dumps({"engine_ab": res, "workload": args.workload})
        print(text, flush=True)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text + "\n")
        return 0
    if args.schedule:
        res = run_schedule(layer, args.schedule, args.warmup)
        text = json.dumps(res)
        print(text, flush=True)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text + "\n")
        return 0
    print(f"# {args.workload}: {len(mats)} matrices, {layer.packed_bytes / 1e6:.1f} MB packed, "
          f"copies rotated {dict(zip((m.name for m in mats), layer.copies))} "
          f"({layer.cold_bytes / 1e9:.2f} GB)", file=sys.stderr, flush=True)

    def step_time(n_live, steps, warmup):
        """(ms per step, eager ms, graph ms or None): the faster of eager
        launches and graph replay (the replay checked against eager)."""
        ms_e, _ = time_steps(layer, n_live, steps, warmup, with_events=False)
        ms_g, spg = None, None
        if args.graph:
            ms_g, ok, spg = time_graph_steps(layer, n_live, steps, warmup)
            if not ok:
                ms_g = None
        best = ms_e if ms_g is None or ms_e <= ms_g else ms_g
        return best, ms_e, ms_g, spg

    # the step the library's fused entry point runs (one launch per matrix),
    # and the same step as separate pre-quantise and matmul launches; first
    # (setup, untimed) a quarter second of steps so that the clocks and the
    # weight copies' page tables have settled
    layer.fused = args.fused
    layer.settle(args.n_live)
    ms, ms_eager, ms_graph, graph_spg = step_time(args.n_live, args.steps, args.warmup)
    layer.fused = not args.fused
    ms_other = step_time(args.n_live, args.steps, args.warmup)[0]
    layer.fused = args.fused
    nbytes = step_bytes(mats, args.n_live)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(f"# n_live={args.n_live}: {ms * 1e3:.1f} us/step "
          f"({'fused' if args.fused else 'separate'} launches; eager {ms_eager * 1e3:.1f}"
          f"{'' if ms_graph is None else f', graph {ms_graph * 1e3:.1f}'}), {gbs:.0f} GB/s; "
          f"{'separate' if args.fused else 'fused'}: {ms_other * 1e3:.1f} us/step",
          file=sys.stderr, flush=True)

    # each kernel alone: back-to-back launches between one pair of events
    per_matrix = {}
    kern_us, fused_us = [], []
    for i, m in enumerate(mats):
        st = kernel_stats_us(layer, i, args.n_live, layer.launches(i))
        us = st["mean"]
        fu = fused_avg_us(layer, i, args.n_live, layer.launches(i))
        kern_us.append(us)
        fused_us.append(fu)
        b = matmul_bytes(m.N, m.K, args.n_live)
        fb = b + quantize_bytes(m.K)
        per_matrix[m.name] = {
            "K": m.K, "N": m.N, "us": round(us, 2), "GBps": round(b / us / 1e3, 1),
            "us_median": round(st["median"], 2), "us_p90": round(st["p90"], 2),
            "replays": st["replays"], "launches_per_replay": st["launches_each"],
            "frac_peak": round(b / us / 1e3 / PEAK_HBM_GBS, 4),
            "quantize_us": round(quantize_avg_us(layer, i), 2),
            "fused_us": round(fu, 2), "fused_GBps": round(fb / fu / 1e3, 1),
            "traffic": measured_traffic(args.workload, m.name, args.n_live, False),
            "weight_copies_rotated": layer.copies[i],
            "output_sha16": output_digest(layer, i, args.n_live),
        }
    mm_bytes = sum(matmul_bytes(m.N, m.K, args.n_live) for m in mats)
    print(f"# matmuls alone: {sum(kern_us):.1f} us, {mm_bytes / sum(kern_us) / 1e3:.0f} GB/s; "
          + ", ".join(f"{m.name} {u:.2f} us" for m, u in zip(mats, kern_us)), file=sys.stderr, flush=True)
    print("# fused pre-quantise + matmul: "
          + ", ".join(f"{m.name} {u:.2f} us" for m, u in zip(mats, fused_us)), file=sys.stderr, flush=True)

    # roofline of the dominant kernel of the step as run
    di = dominant_matrix(args.workload)
    dm = mats[di]
    dom_bytes = matmul_bytes(dm.N, dm.K, args.n_live) + (quantize_bytes(dm.K) if args.fused else 0)
    dom_us = fused_us[di] if args.fused else kern_us[di]
    achieved = dom_bytes / dom_us / 1e3
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": round(achieved / PEAK_HBM_GBS, 4),
        "traffic": measured_traffic(args.workload, dm.name, args.n_live, args.fused),
        "kernel": (f"fused pre-quantise + q8 narrow matmul" if args.fused else "q8 narrow matmul")
        + f", {dm.name} {dm.K}->{dm.N}, n_live={args.n_live}",
        "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 2),
        # the launch the workspace entry point makes (the fused one adds its
        # producer workgroups and 4 chunks in flight)
        "launch": layer.q8.q8_matmul_launch_info(dm.N, dm.K, 16, True),
    }

    sweep = {}
    if args.sweep_steps > 0:
        for n in range(1, 17):
            ms_n, ms_e, _, _ = step_time(n, args.sweep_steps, min(args.warmup, 20))
            kn = [kernel_avg_us(layer, i, n, layer.launches(i)) for i in range(len(mats))]
            sweep[n] = {"ms_per_step": round(ms_n, 4), "ms_per_step_eager": round(ms_e, 4),
                        "GBps": round(step_bytes(mats, n) / (ms_n * 1e-3) / 1e9, 1),
                        "kernel_us": round(sum(kn), 2),
                        "kernel_GBps": round(sum(matmul_bytes(m.N, m.K, n) for m in mats)
                                             / sum(kn) / 1e3, 1)}
            print(f"# sweep n_live={n}: {ms_n * 1e3:.1f} us/step, matmuls {sum(kn):.1f} us",
                  file=sys.stderr, flush=True)
    ratio = None
    if sweep:
        t1 = sweep[1]["ms_per_step"]
        for n, rec in sweep.items():
            rec["t_over_t1"] = round(rec["ms_per_step"] / t1, 4)
            rec["speedup_vs_n_single"] = round(speedup_vs_single(t1, rec["ms_per_step"], n), 3)
            rec["kernel_t_over_t1"] = round(rec["kernel_us"] / sweep[1]["kernel_us"], 4)
        ratio = sweep[16]["t_over_t1"]

    multi = multi_columns(layer, (16, 32, 48, 64)) \
        if args.multi else None
    rope = rope_after_qkv(layer, args.n_live)
    if rope:
        print(f"# pos-vector RoPE on the QKV rows: {rope['us']} us", file=sys.stderr, flush=True)
    copy_gbs = copy_ceiling_gbs()
    read_gbs = read_ceiling_gbs(layer.q8)
    print(f"# read ceiling (plain streaming read of 2 GiB): {read_gbs:.0f} GB/s; "
          f"{dm.name} at {roofline['achieved'] / read_gbs:.0%} of it", file=sys.stderr, flush=True)
    # the spread of the step time: STEP_REPEATS more windows of as many eager
    # steps as the timed run, each between two device synchronisations
    layer.fused = args.fused
    win = [time_steps(layer, args.n_live, args.steps, 2, False)[0] for _ in range(STEP_REPEATS)]
    repeats = {"windows": STEP_REPEATS, "steps_each": args.steps,
               "median_ms": round(float(np.median(win)), 5),
               "p90_ms": round(float(np.percentile(win, 90)), 5), "timing": "eager launches"}
    cpu = cpu_baseline(args.workload, args.n_live, args.cpu_seconds) if args.cpu_seconds > 0 else None

    line = {
        "metric": "achieved HBM GB/s (% of peak) & step-time ratio vs n_tok=1 for q8_0 narrow matmul",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_eager": round(ms_eager, 5),
        "timing": (f"hip graph replay, {graph_spg} steps per graph (checked bit-identical to eager)"
                   if ms is not ms_eager else "eager launches on one stream")
        + "; the faster of the two, each between a pair of hip events on the launch stream",
        "ms_per_step_graph": round(ms_graph, 5) if ms_graph is not None else None,
        "step_launches": "fused pre-quantise + matmul, one launch per matrix" if args.fused
        else "separate pre-quantise and matmul launches",
        "ms_per_step_other": round(ms_other, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "accumulate": "exact i32 per 32-value block, f32 across blocks",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations, 1% outlier channels x20)",
        "config": {
            "workload": f"{args.workload}: Qwen3-14B-shaped decode layer" if args.workload == "qwen3_layer"
            else args.workload,
            "matrices": {m.name: [m.K, m.N] for m in mats},
            "n_live": args.n_live, "slots": 16,
            "batch_index": "seeded random prefix of a slot permutation"
            if layer.w.random_batch_index else "identity",
            "weight_copies_rotated": dict(zip((m.name for m in layer.mats), layer.copies)),
            "cold_bytes": layer.cold_bytes,
        },
        "frac_peak": round(gbs / PEAK_HBM_GBS, 4),
        "step_bytes": nbytes,
        "matmul_us": round(sum(kern_us), 2),
        "matmul_GBps": round(mm_bytes / sum(kern_us) / 1e3, 1),
        "t16_over_t1": ratio,
        "per_matrix": per_matrix,
        "sweep": sweep,
        "roofline": roofline,
        "multi_columns": multi,
        "rope_after_qkv": rope,
        "copy_ceiling_GBps": round(copy_gbs, 1),
        "read_ceiling_GBps": round(read_gbs, 1),
        "step_repeats": repeats,
        "cpu_baseline": cpu,
    }
    text = json.dumps(line)
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
