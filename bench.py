"""Benchmark of the narrow-batch q8_0 decode matmul on one MI355X.

A step is one pass of the whole hot path over one decode batch of a
Qwen3-14B-shaped decode layer (hidden 5120): for each of its four weight
matrices (QKV 5120->7168, O 5120->5120, gate+up 5120->34816, down
17408->5120) the 16-slot activation buffer is pre-quantised and the narrow
matmul runs for the live batch, gathered through a seeded random
batch_index (workspace entry point: K splits of small-N matrices spread
over separate workgroups).  Weights are packed once, outside the timed region, in enough
copies (rotated step by step) to exceed 1 GiB, so no step finds its weights
in the 256 MB last-level cache.

Reported (one JSON line): the whole step's achieved GB/s from algorithmic
bytes (packed weights 34 B per 32 weights, the live tokens' activation
blocks, batch_index, Y, and the quantiser's fp32 input and q8_0 output), the
step time, the same at every live batch 1..16 with t(16)/t(1) and the
speedup n*t(1)/t(n) over n single-token calls ("Batched decode: co-decode N
live sessions in one GPU pass", section "Measured", compares ms/step against
n x single-token time the same way), the roofline of the dominant kernel
(the gate+up matmul) from HIP events on its stream, and the CPU oracle's
rate on the host cores.
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
COLD_BYTES = 1 << 30    # rotate weight copies past 1 GiB
DOMINANT = "gate_up"
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

class Layer:
    """R packed copies of a workload's matrices, plus the activation buffers."""

    def __init__(self, key: str):
        import torch
        import quantized_weight_streaming_q8_amd as q8
        self.q8 = q8
        self.w = wl.WORKLOADS[key]
        self.mats = list(self.w.matrices)
        one = sum(q8.q8_packed_weight_bytes(m.N, m.K) for m in self.mats)
        self.copies = max(1, -(-COLD_BYTES // one))
        self.packed = [[None] * len(self.mats) for _ in range(self.copies)]
        self.X, self.Xq, self.Y, self.ws = [], [], [], []
        for i, m in enumerate(self.mats):
            W = torch.from_numpy(wl.weights(self.w.config, i, m.N, m.K)).cuda()
            base = q8.empty_packed_weights(m.N, m.K)
            q8.q8_pack_weights(W, m.N, m.K, base)
            del W
            for c in range(self.copies):
                self.packed[c][i] = base if c == 0 else base.clone()
            self.X.append(torch.from_numpy(
                wl.activations(self.w.config, m.K, outliers=self.w.outliers)).cuda())
            self.Xq.append(q8.empty_act_slots(m.K))
            self.Y.append(torch.empty((16, m.N), dtype=torch.float32, device="cuda"))
            self.ws.append(q8.zeroed_workspace(m.N, m.K))
        torch.cuda.synchronize()
        self.packed_bytes = one

    def batch_index(self, n_live: int):
        import torch
        bi = wl.batch_index(self.w.config, n_live, random=self.w.random_batch_index)
        return torch.from_numpy(bi).cuda()

    def step(self, copy: int, bi, n_live: int, events=None) -> None:
        """Enqueue one step; with `events`, bracket every matmul launch with
        a pair of events recorded on the launch stream."""
        q8 = self.q8
        for i, m in enumerate(self.mats):
            q8.q8_quantize_acts(self.X[i], 16, m.K, self.Xq[i])
            if events is not None:
                events[i][0].record()
            q8.q8_matmul_narrow_ws(self.packed[copy][i], self.Xq[i], bi, n_live, m.N, m.K,
                                   self.Y[i], self.ws[i])
            if events is not None:
                events[i][1].record()


def time_steps(layer: Layer, n_live: int, steps: int, warmup: int, with_events: bool):
    """Run `warmup` untimed steps, then time exactly `steps` steps between two
    device synchronisations.  Returns (ms per step, per-matrix kernel ms
    lists)."""
    import torch
    bi = layer.batch_index(n_live)
    for s in range(warmup):
        layer.step(s % layer.copies, bi, n_live)
    torch.cuda.synchronize()
    ev = []
    if with_events:
        ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in layer.mats] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        layer.step(s % layer.copies, bi, n_live, ev[s] if with_events else None)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kern = [[] for _ in layer.mats]
    if with_events:
        for s in range(steps):
            for i in range(len(layer.mats)):
                kern[i].append(ev[s][i][0].elapsed_time(ev[s][i][1]))
    return dt * 1e3 / steps, kern


def capture_step_graphs(layer: Layer, n_live: int):
    """One HIP graph per weight copy, each holding one whole step (the four
    quantise + matmul pairs), captured through torch's graph API on the
    stream the library launches on."""
    import torch
    bi = layer.batch_index(n_live)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in range(layer.copies):
            layer.step(c, bi, n_live)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for c in range(layer.copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.step(c, bi, n_live)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs, bi


def time_graph_steps(layer: Layer, n_live: int, steps: int, warmup: int):
    """Step time with each step replayed from a captured graph.  Returns
    (ms per step, True if every output of the last replay is bit-identical
    to an eager step on the same inputs)."""
    import torch
    graphs, bi = capture_step_graphs(layer, n_live)
    for s in range(warmup):
        graphs[s % layer.copies].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        graphs[s % layer.copies].replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    last = (steps - 1) % layer.copies
    got = [y.clone() for y in layer.Y]
    layer.step(last, bi, n_live)
    torch.cuda.synchronize()
    same = all(torch.equal(a.view(torch.int32), b.view(torch.int32)) for a, b in zip(got, layer.Y))
    del graphs
    return dt * 1e3 / steps, same


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
        "kind": "oracle",
        "sample": (f"{passes} full pass(es) of the {key} step (all {len(data)} matrices, "
                   f"quantise + matmul) at n_live={n_live}, {dt:.1f} s wall"),
        "ms_per_step": round(dt * 1e3 / passes, 3),
    }


# ------------------------------------------------------------- profiles

def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("q8_matmul.hip", "q8_internal.h"):
        with open(os.path.join(ROOT, "quantized_weight_streaming_q8_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(n_live: int):
    """HBM bytes per launch of the dominant kernel from the committed PMC
    counter summary, if it was taken on the current kernel source."""
    path = os.path.join(PROFILE_DIR, "gate_up_matmul_qwen3_layer_pmc.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    per = rec.get("traffic_bytes_per_launch", {}).get(str(n_live))
    return None if per is None else int(per)


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
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the narrow matmul is a single-GPU kernel here).", file=sys.stderr)
        return 2
    if not 1 <= args.n_live <= 16:
        print("--n-live must be in 1..16", file=sys.stderr)
        return 2

    import torch
    torch.cuda.set_device(0)
    layer = Layer(args.workload)
    mats = layer.mats
    print(f"# {args.workload}: {len(mats)} matrices, {layer.packed_bytes / 1e6:.1f} MB packed, "
          f"{layer.copies} copies rotated", file=sys.stderr, flush=True)

    ms_eager, kern = time_steps(layer, args.n_live, args.steps, args.warmup, with_events=True)
    graph_ok = None
    ms = ms_eager
    if args.graph:
        ms_graph, graph_ok = time_graph_steps(layer, args.n_live, args.steps, args.warmup)
        if graph_ok:
            ms = ms_graph
    nbytes = step_bytes(mats, args.n_live)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(f"# n_live={args.n_live}: {ms * 1e3:.1f} us/step ({'graph' if ms is not ms_eager else 'eager'}), "
          f"eager {ms_eager * 1e3:.1f} us/step, {gbs:.0f} GB/s", file=sys.stderr, flush=True)

    per_matrix = {}
    for i, m in enumerate(mats):
        k = np.array(kern[i])
        b = matmul_bytes(m.N, m.K, args.n_live)
        per_matrix[m.name] = {
            "K": m.K, "N": m.N, "us": round(float(k.mean()) * 1e3, 2),
            "us_p90": round(float(np.percentile(k, 90)) * 1e3, 2),
            "GBps": round(b / (k.mean() * 1e-3) / 1e9, 1),
            "frac_peak": round(b / (k.mean() * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        }

    dom = [i for i, m in enumerate(mats) if m.name == DOMINANT]
    di = dom[0] if dom else int(np.argmax([m.N * m.K for m in mats]))
    dm = mats[di]
    dom_bytes = matmul_bytes(dm.N, dm.K, args.n_live)
    dom_ms = float(np.mean(kern[di]))
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(args.n_live),
        "kernel": f"q8 narrow matmul, {dm.name} {dm.K}->{dm.N}, n_live={args.n_live}",
        "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_ms * 1e3, 2),
    }

    sweep = {}
    if args.sweep_steps > 0:
        for n in range(1, 17):
            ms_e, kn = time_steps(layer, n, args.sweep_steps, min(args.warmup, 20), with_events=True)
            ms_n = ms_e
            if args.graph:
                ms_g, ok = time_graph_steps(layer, n, args.sweep_steps, min(args.warmup, 20))
                if ok:
                    ms_n = ms_g
            kmean = [float(np.mean(x)) for x in kn]
            sweep[n] = {"ms_per_step": round(ms_n, 4), "ms_per_step_eager": round(ms_e, 4),
                        "GBps": round(step_bytes(mats, n) / (ms_n * 1e-3) / 1e9, 1),
                        "kernel_us": round(sum(kmean) * 1e3, 2),
                        "kernel_GBps": round(sum(matmul_bytes(m.N, m.K, n) for m in mats)
                                             / (sum(kmean) * 1e-3) / 1e9, 1)}
            print(f"# sweep n_live={n}: {ms_n * 1e3:.1f} us/step, kernels {sum(kmean) * 1e3:.1f} us",
                  file=sys.stderr, flush=True)
    ratio = None
    if sweep:
        t1 = sweep[1]["ms_per_step"]
        for n, rec in sweep.items():
            rec["t_over_t1"] = round(rec["ms_per_step"] / t1, 4)
            rec["speedup_vs_n_single"] = round(speedup_vs_single(t1, rec["ms_per_step"], n), 3)
            rec["kernel_t_over_t1"] = round(rec["kernel_us"] / sweep[1]["kernel_us"], 4)
        ratio = sweep[16]["t_over_t1"]

    copy_gbs = copy_ceiling_gbs()
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
        "timing": "hip graph replay per step (checked bit-identical to eager)" if ms is not ms_eager
        else "eager launches",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 dot, fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations, 1% outlier channels x20)",
        "config": {
            "workload": f"{args.workload}: Qwen3-14B-shaped decode layer" if args.workload == "qwen3_layer"
            else args.workload,
            "matrices": {m.name: [m.K, m.N] for m in mats},
            "n_live": args.n_live, "slots": 16,
            "batch_index": "seeded random prefix of a slot permutation"
            if layer.w.random_batch_index else "identity",
            "weight_copies_rotated": layer.copies, "cold_bytes": layer.copies * layer.packed_bytes,
        },
        "frac_peak": round(gbs / PEAK_HBM_GBS, 4),
        "step_bytes": nbytes,
        "t16_over_t1": ratio,
        "per_matrix": per_matrix,
        "sweep": sweep,
        "roofline": roofline,
        "copy_ceiling_GBps": round(copy_gbs, 1),
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
