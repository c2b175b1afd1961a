#!/usr/bin/env python3
"""Benchmark of the Q4_0 weight-only linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one decode step of the 26-layer decoder's linears at M=1 (fused
QKV 3072->4096+1024+1024, O 4096->3072, fused gate/up 3072->2x9216,
down 9216->3072 per layer: 104 launches, 1.70 GB of distinct Q4_0 weights),
with every input already resident in HBM.  The step is captured once in a HIP
graph and replayed; K replays are timed with HIP events on the replay stream.

Printed (one JSON line):
  value       eff. HBM GB/s of the whole step: algorithmic bytes per step
              (packed weights + x + y) * K / elapsed
  decode_m2   the same step at M=2 (the batched CFG pair): us/step and GB/s
  roofline    the dominant kernel (the M=1 decode kernel) against 8 TB/s:
              algorithmic bytes of its launches / their summed kernel-own
              durations, taken with events armed on each launch of the timed
              steps (q4_0_time_next_launch; an eager pass over the same K steps)
  prefill     M=2048 through the four decoder shapes: TFLOP/s (2*M*N*K / time)
              and the GEMM kernel's roofline against 2.5 PFLOP/s bf16
  swiglu      the fused gate/up + SwiGLU launch (q4_0_linear_swiglu) next to
              the unfused gate/up launch it replaces, at M = 1, 2 and 2048
              (kernel-own times; each kind walks the 26 layers' gate/up
              weights in turn, so every launch streams its weights from HBM)
  embed       Q4 embedding lookups of 32, 2048 and 16384 random ids from the
              131072 x 3072 table, packed (q4_0_embed) and as GGUF blocks
              (q4_0_embed_gguf, under "gguf"): kernel-own time per launch,
              each after a 512 MiB read (rows from HBM), and GB/s moved
  lm_head     the same table as the LM head linear at M = 1 and 32 (kernel-own
              times, each launch after a 512 MiB read so the table comes from HBM)
  other_workloads  the lone GEMV 3072->4096 at M=1 and the audio linears
              (5120->3072 and 3072->3072 at M=1505, 1280->5120 and 5120->1280
              at M=6020), timed like the LM head: median, p10 and p90
  cpu_baseline  the CPU oracle (dequantize + fp64 matmul) on a bounded sample
              of the same step, on the host cores
"""

from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q4_0 linear eff. HBM GB/s (M=1 decode) + TFLOP/s (M=2048 prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_m1.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--prefill-steps", type=int, default=10)
    p.add_argument("--layers", type=int, default=26, help="decoder layers in a step (26 = the full workload)")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-swiglu", action="store_true", help="skip the fused gate/up + SwiGLU timings")
    p.add_argument("--no-embed", action="store_true", help="skip the Q4 embedding lookup timings")
    p.add_argument("--no-others", action="store_true",
                   help="skip the single GEMV and the audio linears (M = 1505, 6020)")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the CPU oracle sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a 256 MiB device copy (reference kernel for PMC byte counters)")
    return p.parse_args()


# ------------------------------------------------------------- workload
def build_device_specs(specs, m_values, dev, threads=16):
    """Generate seeded fp32 weights on the host (thread pool), quantize and
    pack them on the device; return [(spec, [PackedWeight], {m: x})]."""
    import numpy as np  # noqa: F401
    import torch

    import q4_weight_only_amd as q4

    jobs = [(spec, si) for spec in specs for si in range(len(spec.Ns))]
    built = {}
    with ThreadPoolExecutor(threads) as ex:
        pending = collections.deque()
        it = iter(jobs)

        def submit_next():
            nxt = next(it, None)
            if nxt is not None:
                spec, si = nxt
                pending.append((spec, si, ex.submit(spec.weight, si)))

        for _ in range(2 * threads):
            submit_next()
        while pending:
            spec, si, fut = pending.popleft()
            w = fut.result()
            del fut
            wt = torch.from_numpy(w).to(dev)
            del w
            blocks = q4.quantize(wt)
            del wt
            built[(id(spec), si)] = q4.pack(blocks, spec.Ns[si], spec.K)
            del blocks
            submit_next()
    out = []
    for spec in specs:
        pws = [built.pop((id(spec), si)) for si in range(len(spec.Ns))]
        xs = {}
        for m in m_values:
            xb = spec.activations(m)
            xs[m] = torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        out.append((spec, pws, xs))
    torch.cuda.synchronize(dev)
    return out


def algorithmic_bytes(spec, m):
    """Packed weights + x (bf16) + y (fp32) of one launch."""
    return spec.weight_bytes() + m * spec.K * 2 + sum(m * n * 4 for n in spec.Ns)


def flops(spec, m):
    return sum(2 * m * n * spec.K for n in spec.Ns)


class Runner:
    """Launch sequence over prepared specs at one M, with preallocated outputs."""

    def __init__(self, prepared, m, dev):
        import torch

        self.items = []
        for spec, pws, xs in prepared:
            ys = [torch.empty((m, n), dtype=torch.float32, device=dev) for n in spec.Ns]
            self.items.append((spec, pws, xs[m], ys))
        self.m = m

    def launch(self, i):
        import q4_weight_only_amd as q4

        spec, pws, x, ys = self.items[i]
        if len(pws) > 1:
            q4.linear_multi(x, pws, ys)
        else:
            q4.linear(x, pws[0], ys[0])

    def step(self):
        for i in range(len(self.items)):
            self.launch(i)

    def bytes_per_step(self):
        return sum(algorithmic_bytes(spec, self.m) for spec, *_ in self.items)

    def flops_per_step(self):
        return sum(flops(spec, self.m) for spec, *_ in self.items)


def time_graph(runner, steps, warmup, dev):
    """Capture one step in a HIP graph; time `steps` replays with events (one
    between every two replays, so each step's time is kept too)."""
    import torch

    stream = torch.cuda.Stream(dev)
    stream.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(stream):
        runner.step()                      # eager warm-up of every launch
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        runner.step()
    torch.cuda.synchronize(dev)
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            graph.replay()
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize(dev)
        marks[0].record(stream)
        for i in range(steps):
            graph.replay()
            marks[i + 1].record(stream)
    marks[-1].synchronize()
    runner.step_times = [marks[i].elapsed_time(marks[i + 1]) / 1e3 for i in range(steps)]
    return marks[0].elapsed_time(marks[-1]) / 1e3, graph


def pctl_us(times):
    import numpy as np

    return [round(float(np.percentile(times, q)) * 1e6, 2) for q in (10, 50, 90)]


def time_kernels(runner, steps, dev):
    """Kernel-own durations of every launch over `steps` eager steps: each
    launch is armed with an event pair that its kernel records at start/end."""
    import torch

    import q4_weight_only_amd as q4

    n = len(runner.items)
    pairs = []
    stream = torch.cuda.current_stream(dev)
    for _ in range(steps):
        for i in range(n):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)               # creates the events
            b.record(stream)
            q4.time_next_launch(a, b)
            runner.launch(i)
            pairs.append((i, a, b))
    torch.cuda.synchronize(dev)
    per_item = [[] for _ in range(n)]
    for i, a, b in pairs:
        per_item[i].append(a.elapsed_time(b) / 1e3)
    return per_item


def time_swiglu(prepared, ms, reps, dev):
    """Kernel-own times of the fused gate/up + SwiGLU launch next to the
    unfused gate/up launch it replaces, over the decode workload's gate/up
    weights.  Each kind of launch walks all layers' weight pairs in turn, so
    25 other pairs (800 MB) stream through between two uses of one pair and
    every launch reads its weights from HBM, not from the infinity cache."""
    import numpy as np
    import torch

    import q4_weight_only_amd as q4

    gate_up = [(s, pws) for s, pws, _ in prepared if s.name.endswith(".gate_up")]
    spec0 = gate_up[0][0]
    n, k = spec0.Ns[0], spec0.K
    stream = torch.cuda.current_stream(dev)
    out = {}
    for m in ms:
        xb = spec0.activations(m)
        x = torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        h = torch.empty((m, n), dtype=torch.float32, device=dev)
        h16 = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ys = [torch.empty((m, n), dtype=torch.float32, device=dev) for _ in range(2)]
        pairs = {"fused": [], "fused_bf16": [], "unfused": []}
        for r in range(reps + 1):
            for kind in ("fused", "fused_bf16", "unfused"):
                for _, pws in gate_up:
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    b.record(stream)
                    q4.time_next_launch(a, b)
                    if kind == "fused":
                        q4.linear_swiglu(x, pws[0], pws[1], h)
                    elif kind == "fused_bf16":
                        q4.linear_swiglu(x, pws[0], pws[1], h16, dtype=torch.bfloat16)
                    else:
                        q4.linear_multi(x, pws, ys)
                    if r > 0:              # the first pass warms up
                        pairs[kind].append((a, b))
        torch.cuda.synchronize(dev)
        t = {kind: float(np.mean([a.elapsed_time(b) / 1e3 for a, b in v])) for kind, v in pairs.items()}
        wbytes = spec0.weight_bytes()
        fused_bytes = wbytes + m * k * 2 + m * n * 4
        unfused_bytes = wbytes + m * k * 2 + 2 * m * n * 4
        fl = 2 * m * (2 * n) * k
        out[f"M={m}"] = {
            "kernel": q4.linear_swiglu_kernel(m, k),
            "fused_us": round(t["fused"] * 1e6, 2),
            "fused_bf16_out_us": round(t["fused_bf16"] * 1e6, 2),
            "unfused_us": round(t["unfused"] * 1e6, 2),
            "fused_GBs": round(fused_bytes / t["fused"] / 1e9, 1),
            "unfused_GBs": round(unfused_bytes / t["unfused"] / 1e9, 1),
            "fused_TFLOPs": round(fl / t["fused"] / 1e12, 2),
            "unfused_TFLOPs": round(fl / t["unfused"] / 1e12, 2),
            "launches": len(pairs["fused"]),
        }
    return out


def time_embed(pw, counts, reps, dev, blocks=None):
    """Kernel-own times (armed events) of Q4 embedding lookups, each launch
    with fresh random ids and after a read of a 512 MiB buffer, so the table
    rows come from HBM: the 226 MB table would otherwise sit in the 256 MB
    infinity cache after the first launches.  With `blocks` (the same table
    as GGUF bytes) the lookups run q4_0_embed_gguf instead."""
    import numpy as np
    import torch

    import q4_weight_only_amd as q4

    rng = np.random.default_rng(7)
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for count in counts:
        ids = [torch.from_numpy(rng.integers(0, pw.n, count).astype(np.int32)).to(dev) for _ in range(reps + 1)]
        res = torch.empty((count, pw.k), dtype=torch.float32, device=dev)
        pairs = []
        for r, batch in enumerate(ids):
            torch.sum(flush, dim=0, out=sink)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            b.record(stream)
            q4.time_next_launch(a, b)
            if blocks is None:
                q4.embed(pw, batch, res)
            else:
                q4.embed_gguf(blocks, pw.n, pw.k, batch, res)
            if r > 0:                      # the first launch warms up
                pairs.append((a, b))
        torch.cuda.synchronize(dev)
        t = float(np.median([a.elapsed_time(b) / 1e3 for a, b in pairs]))
        moved = count * (pw.k // 32 * 18 + pw.k * 4 + 4)     # table rows read + fp32 rows written + ids
        out[f"ids={count}"] = {"us": round(t * 1e6, 2), "GBs": round(moved / t / 1e9, 1), "bytes": moved}
    del flush, sink
    return out


def time_single(spec, pw, ms, reps, dev):
    """One single-segment linear at each M: kernel-own time (armed events) of
    launches that each follow a read of a 512 MiB buffer, so the weights
    stream from HBM rather than from the 256 MB infinity cache (a read, not
    a fill, so no write-back competes with the launch).  Median and
    p10 / p90 over `reps` launches after one warm-up launch."""
    import numpy as np
    import torch

    import q4_weight_only_amd as q4

    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for m in ms:
        xb = spec.activations(m)
        x = torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        y = torch.empty((m, pw.n), dtype=torch.float32, device=dev)
        q4.linear(x, pw, y)
        pairs = []
        for _ in range(reps):
            torch.sum(flush, dim=0, out=sink)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            b.record(stream)
            q4.time_next_launch(a, b)
            q4.linear(x, pw, y)
            pairs.append((a, b))
        torch.cuda.synchronize(dev)
        ts = np.array([a.elapsed_time(b) / 1e3 for a, b in pairs])
        t = float(np.median(ts))
        moved = algorithmic_bytes(spec, m)
        out[f"M={m}"] = {"kernel": q4.linear_kernel(m, spec.K, spec.Ns), "us": round(t * 1e6, 2),
                         "p10_us": round(float(np.percentile(ts, 10)) * 1e6, 2),
                         "p90_us": round(float(np.percentile(ts, 90)) * 1e6, 2),
                         "GBs": round(moved / t / 1e9, 1), "frac_of_8TBs": round(moved / t / 1e9 / HBM_PEAK_GBS, 4),
                         "TFLOPs": round(flops(spec, m) / t / 1e12, 2),
                         "frac_of_bf16_peak": round(flops(spec, m) / t / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "launches": reps}
        del x, y
    del flush, sink
    return out


def kernel_source_digest():
    """Hash of the linear kernels' source with comments and whitespace
    removed, so the stored counter record stays valid across comment edits
    and goes stale on any change to the code."""
    import re

    h = hashlib.sha256()
    for f in ("q4_0_linear.hip", "q4_0_internal.h"):
        with open(os.path.join(ROOT, "q4_weight_only_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from committed rocprofv3 PMC runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a reference copy), if they were taken
    on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_digest() or t.get("kernel") != kernel:
        return None
    return t.get("hbm_bytes_per_launch")


# --------------------------------------------------------- CPU baseline
def cpu_baseline(specs, budget_s):
    """The oracle on a bounded sample of the decode step (whole launches,
    in step order, until the budget is spent), reported as GB/s."""
    import numpy as np

    from oracle import q4_0_oracle as O

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    done_bytes, elapsed, launches = 0, 0.0, 0
    for spec in specs:
        if elapsed >= budget_s:
            break
        blocks = [O.quantize(spec.weight(si)) for si in range(len(spec.Ns))]   # untimed input prep
        xb = spec.activations(1)
        t0 = time.perf_counter()
        for si, n in enumerate(spec.Ns):
            O.linear(xb, blocks[si], n, spec.K)
        elapsed += time.perf_counter() - t0
        done_bytes += algorithmic_bytes(spec, 1)
        launches += 1
    return {
        "value": round(done_bytes / elapsed / 1e9, 3),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"first {launches} of the 104 decode-step launches (M=1), dequantize + fp64 matmul, "
                  f"{elapsed:.1f} s of CPU time",
    }


# ------------------------------------------------------------------ main
def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("bench.py runs on one GPU only: this build measures the single-GPU hot path "
               "(no collectives); run with --gpus 1")
        print(msg, file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    import q4_weight_only_amd as q4
    from q4_weight_only_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    q4.lib()          # fail loudly if the library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- decode step (the headline)
    _, decode = inputs.workload(2)
    specs = [s for s, _ in decode][: 4 * args.layers]
    t0 = time.time()
    prepared = build_device_specs(specs, (1, 2), dev)
    log(f"decode workload ready: {len(specs)} launches, {sum(s.weight_bytes() for s in specs) / 1e9:.3f} GB "
        f"of Q4_0 weights ({time.time() - t0:.1f} s)")
    runner = Runner(prepared, 1, dev)
    elapsed, graph = time_graph(runner, args.steps, args.warmup, dev)
    step_bytes = runner.bytes_per_step()
    value = step_bytes * args.steps / elapsed / 1e9
    log(f"decode: {elapsed / args.steps * 1e6:.1f} us/step, {value:.1f} GB/s")
    del graph

    durations = time_kernels(runner, args.steps, dev)
    # group launches by the kernel instantiation that ran them
    by_kernel = collections.OrderedDict()
    per_op = collections.OrderedDict()
    per_op_times = {}
    for (spec, *_), d in zip(runner.items, durations):
        kname = q4.linear_kernel(1, spec.K, spec.Ns)
        b, t, c = by_kernel.get(kname, (0, 0.0, 0))
        by_kernel[kname] = (b + algorithmic_bytes(spec, 1) * len(d), t + sum(d), c + len(d))
        op = spec.name.split(".", 1)[1]
        per_op_times.setdefault(op, []).extend(d)
        b, t, c = per_op.get(op, (0, 0.0, 0))
        per_op[op] = (b + algorithmic_bytes(spec, 1) * len(d), t + sum(d), c + len(d))
    dominant = max(by_kernel, key=lambda k: by_kernel[k][1])
    kern_bytes, kern_time, launches = by_kernel[dominant]
    achieved = kern_bytes / kern_time / 1e9
    traffic = measured_traffic(dominant)
    roofline = {
        "bound": "hbm",
        "kernel": dominant,
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "avg_launch_us": round(kern_time / launches * 1e6, 3),
        "bytes_per_launch": round(kern_bytes / launches),
        "launches_timed": launches,
        "kernels": {k: {"GBs": round(b / t / 1e9, 1), "avg_us": round(t / c * 1e6, 3), "launches": c}
                    for k, (b, t, c) in by_kernel.items()},
        "per_op_GBs": {op: round(b / t / 1e9, 1) for op, (b, t, c) in per_op.items()},
        "per_op_avg_us": {op: round(t / c * 1e6, 2) for op, (b, t, c) in per_op.items()},
        "per_op_p10_p50_p90_us": {op: pctl_us(v) for op, v in per_op_times.items()},
    }
    log(f"dominant decode kernel {dominant}: {achieved:.1f} GB/s over {launches} launches; per op {roofline['per_op_GBs']}")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "step_us_p10_p50_p90": pctl_us(runner.step_times),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.layers}-layer decoder decode step at M=1 (Q4_0 weights, bf16 x, fp32 y): "
                        "fused QKV 3072->6144, O 4096->3072, fused gate/up 3072->2x9216, down 9216->3072",
            "M": 1,
            "layers": args.layers,
            "launches_per_step": len(specs),
            "bytes_per_step": step_bytes,
            "graph": "one HIP graph per step",
        },
        "roofline": roofline,
    }

    # ---- the same step at M=2 (the batched CFG pair of the decode workload)
    runner2 = Runner(prepared, 2, dev)
    el2, graph2 = time_graph(runner2, args.steps, args.warmup, dev)
    del graph2
    gbs2 = runner2.bytes_per_step() * args.steps / el2 / 1e9
    out["decode_m2"] = {
        "workload": "the decode step at M=2 (batched CFG pair), same weights and launches",
        "us_per_step": round(el2 / args.steps * 1e6, 1),
        "step_us_p10_p50_p90": pctl_us(runner2.step_times),
        "value": round(gbs2, 1),
        "unit": "GB/s",
        "frac_of_8TBs": round(gbs2 / HBM_PEAK_GBS, 4),
        "kernels": sorted({q4.linear_kernel(2, spec.K, spec.Ns) for spec, *_ in runner2.items}),
    }
    log(f"decode M=2: {out['decode_m2']['us_per_step']} us/step, {gbs2:.1f} GB/s")
    del runner2

    # ---- prefill (M=2048 through the four decoder shapes, layer-0 weights)
    if not args.no_prefill:
        _, pre = inputs.workload(4)
        pspecs = [s for s, _ in pre]
        # the prefill weights are the decode step's layer-0 weights
        layer0 = {s.w_tags: pws for s, pws, _ in prepared}
        pprep = []
        for s in pspecs:
            xb = s.activations(2048)
            x = torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(torch.bfloat16)
            pprep.append((s, layer0[s.w_tags], {2048: x}))
        prunner = Runner(pprep, 2048, dev)
        pel, pgraph = time_graph(prunner, args.prefill_steps, 2, dev)
        del pgraph
        tflops = prunner.flops_per_step() * args.prefill_steps / pel / 1e12
        pdur = time_kernels(prunner, args.prefill_steps, dev)
        pk_time = sum(sum(d) for d in pdur)
        pk_flops = sum(flops(spec, 2048) * len(d) for (spec, *_), d in zip(prunner.items, pdur))
        pach = pk_flops / pk_time / 1e12
        # the GEMM tile shape depends on the shape's work tiles: name the one
        # holding the most kernel time, and every op's
        pk_names = [q4.linear_kernel(2048, spec.K, spec.Ns) for spec, *_ in prunner.items]
        pk_by = collections.Counter()
        for name, d in zip(pk_names, pdur):
            pk_by[name] += sum(d)
        out["prefill"] = {
            "value": round(tflops, 2),
            "unit": "TFLOP/s",
            "workload": "M=2048 through QKV 3072->6144, O 4096->3072, gate/up 3072->18432, down 9216->3072",
            "ms_per_step": round(pel / args.prefill_steps * 1e3, 4),
            "step_us_p10_p50_p90": pctl_us(prunner.step_times),
            "steps": args.prefill_steps,
            "roofline": {
                "bound": "mfma",
                "kernel": pk_by.most_common(1)[0][0],
                "kernels": {spec.name.split(".", 1)[1]: name for (spec, *_), name in zip(prunner.items, pk_names)},
                "achieved": round(pach, 2),
                "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(pach / BF16_PEAK_TFLOPS, 4),
                "per_op_TFLOPs": {spec.name.split(".", 1)[1]: round(flops(spec, 2048) * len(d) / sum(d) / 1e12, 2)
                                  for (spec, *_), d in zip(prunner.items, pdur)},
            },
        }
        log(f"prefill: {tflops:.1f} TFLOP/s (kernel {pach:.1f})")

    # ---- NEXT-2: fused gate/up + SwiGLU against the unfused gate/up launch
    if not args.no_swiglu:
        out["swiglu"] = {
            "workload": "decoder gate/up 3072->2x9216 (one weight pair per layer, rotated), "
                        "h = silu(x Wg^T) * (x Wu^T), fp32 out (fused_bf16_out_us: bf16 out)",
            **time_swiglu(prepared, (1, 2, 2048), 3 if args.layers >= 8 else 6, dev),
        }
        log(f"swiglu: {out['swiglu']}")

    # ---- NEXT-3: Q4 embedding lookup from the LM head's table
    if not args.no_embed:
        _, lm = inputs.workload(3)
        lm_spec = lm[0][0]
        wt = torch.from_numpy(lm_spec.weight(0)).to(dev)
        lm_blocks = q4.quantize(wt)
        del wt
        lm_pws = [q4.pack(lm_blocks, lm_spec.Ns[0], lm_spec.K)]
        out["embed"] = {
            "table": f"{lm_spec.Ns[0]}x{lm_spec.K} Q4_0 (the LM head weights), fp32 rows out, random ids; "
                     "packed table (q4_0_embed) and GGUF block order (q4_0_embed_gguf, key gguf)",
            **time_embed(lm_pws[0], (32, 2048, 16384), 50, dev),
            "gguf": time_embed(lm_pws[0], (32, 2048, 16384), 50, dev, blocks=lm_blocks),
        }
        del lm_blocks
        log(f"embed: {out['embed']}")
        # the same table as the LM head linear (workload 3: M = 1 and 32)
        out["lm_head"] = {
            "workload": f"LM head {lm_spec.K}->{lm_spec.Ns[0]} (226 MB of Q4_0), one launch, streamed from HBM",
            **time_single(lm_spec, lm_pws[0], (1, 32), 20, dev),
        }
        log(f"lm_head: {out['lm_head']}")
        del lm_pws

    # ---- the other workloads' single launches: the lone GEMV and the audio
    # linears (ragged M = 1505 and 6020), each from HBM
    if not args.no_others:
        _, g1 = inputs.workload(1)
        _, a5 = inputs.workload(5)
        others = {}
        for spec, ms in g1 + a5:
            (_, pws, _), = build_device_specs([spec], (), dev)
            res = time_single(spec, pws[0], ms, 20, dev)
            for key, r in res.items():
                others[f"{spec.name} {spec.K}->{spec.Ns[0]} {key}"] = r
            del pws
        out["other_workloads"] = others
        log(f"other workloads: {others}")

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        out["copy_calibration"] = {"bytes_read": 256 << 20, "bytes_written": 256 << 20, "calls": 3}

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(specs, args.cpu_seconds)
        log(f"cpu baseline: {out['cpu_baseline']}")

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
