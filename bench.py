#!/usr/bin/env python3
"""Benchmark of the Q4_0 weight-only linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one decode step of the 26-layer decoder's linears at M=1 (fused
QKV 3072->4096+1024+1024, O 4096->3072, fused gate/up 3072->2x9216,
down 9216->3072 per layer: 104 launches, 1.70 GB of distinct Q4_0 weights),
with every input already resident in HBM.  The step is captured once in a HIP
graph and replayed; K replays are timed between two HIP events on the replay
stream (K more, with an event after each, give the single-step spread).

Printed (one JSON line):
  value        eff. HBM GB/s of the whole step: algorithmic bytes per step
               (packed weights + x + y) * K / elapsed
  roofline     the dominant kernel (the M=1 decode kernel) against 8 TB/s:
               algorithmic bytes of its launches / their summed kernel-own
               durations, taken with events armed on each launch of the timed
               steps (q4_0_time_next_launch; an eager pass over the same K steps,
               the launches held back until a whole step is queued so that they
               run back to back as in the graph; with --isolated also the same
               launches one at a time on an idle GPU, per_op_isolated_p10_p50_p90_us)
  workloads    one record per workload (1 the lone GEMV, 2 the decode step at
               M=1 and 2, 3 the LM head at M=1 and 32, 4 the M=2048 prefill,
               5 the audio linears): algorithmic bytes and flops, kernel-time
               p10/p50/p90, GB/s or TFLOP/s against the roofline, the kernel
               names, parity of the timed outputs against the oracle on sampled
               weight rows (max |err|/bound, cosine) and the oracle's own rate on
               the host cores over a stated sample
  prefill.arithmetic_ceiling  the GEMM's inner-loop arithmetic alone (MFMAs;
               + the exact rescale; + the decode), the rate the exact method
               allows apart from memory
  decode_floor the same 104-launch step with a plain read of the same weight
               bytes in each launch, and with 104 empty launches: what a step
               of this launch structure costs without the layer's arithmetic
  swiglu       the fused gate/up + SwiGLU launch next to the unfused gate/up
               launch it replaces, at M = 1, 2 and 2048 (kernel-own times);
               and, timed by stream events around the calls, the fused launch
               next to the unfused launch followed by torch's silu(g) * u (the
               whole unfused step)
  embed        Q4 embedding lookups of 32, 2048 and 16384 random ids from the
               131072 x 3072 table, packed and as GGUF blocks (key gguf)
  cpu_baseline the oracle (dequantize + fp64 matmul) over the whole decode step
               at M=1 on the host cores (workload 2's CPU record)
  seed, git_rev, host_cores, blas   run metadata
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
    p.add_argument("--isolated", action="store_true",
                   help="also time the decode launches one at a time on an idle GPU")
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
    """Capture one step in a HIP graph; time `steps` replays between two
    events, then `steps` more with an event after each replay (each step's
    time, kept in runner.step_times)."""
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
        # the timed region: K replays between two events and nothing else
        # (an event between every two replays costs about 4 us per step here)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        start.record(stream)
        for _ in range(steps):
            graph.replay()
        stop.record(stream)
        torch.cuda.synchronize(dev)
        # then K more replays with an event after each, for the spread of single steps
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        marks[0].record(stream)
        for i in range(steps):
            graph.replay()
            marks[i + 1].record(stream)
    marks[-1].synchronize()
    runner.step_times = [marks[i].elapsed_time(marks[i + 1]) / 1e3 for i in range(steps)]
    return start.elapsed_time(stop) / 1e3, graph


def pctl_us(times):
    import numpy as np

    return [round(float(np.percentile(times, q)) * 1e6, 2) for q in (10, 50, 90)]


class Hold:
    """Runs host-enqueued launches back to back on a busy GPU: a spin kernel
    holds the stream while the host enqueues a batch of launches, so the
    launches run one after another as inside a graph instead of one at a
    time after the host's own launch overhead.  The spin's length (its rate
    follows the clock) is raised whenever a batch's enqueue time comes within
    half of it; `held` counts the counted batches that were queued in full
    before the hold ended."""

    def __init__(self, dev, enqueue, warm=2):
        import torch

        self.stream = torch.cuda.current_stream(dev)
        self.held = self.batches = 0
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        torch.cuda._sleep(2_000_000)
        b.record(self.stream)
        b.synchronize()
        t0 = time.perf_counter()
        enqueue()                          # untimed: the host's enqueue time of a batch
        self.cycles = int((2.0 * (time.perf_counter() - t0) * 1e3 + 2.0) / (a.elapsed_time(b) / 2_000_000))
        torch.cuda.synchronize(dev)
        for _ in range(warm):              # untimed held batches size the hold
            self.run(enqueue, count=False)

    def run(self, enqueue, count=True):
        import torch

        h0 = torch.cuda.Event(enable_timing=True)
        h1 = torch.cuda.Event(enable_timing=True)
        t_hold = time.perf_counter()
        h0.record(self.stream)
        torch.cuda._sleep(self.cycles)
        h1.record(self.stream)
        enqueue()
        enqueue_ms = (time.perf_counter() - t_hold) * 1e3
        h1.synchronize()
        hold = h0.elapsed_time(h1)
        if count:
            self.held += enqueue_ms < hold
            self.batches += 1
        need = 2.0 * enqueue_ms + 2.0
        if hold < need:
            self.cycles = int(self.cycles * need / hold)


def time_kernels(runner, steps, dev, back_to_back=True):
    """Kernel-own durations of every launch over `steps` eager steps: each
    launch is armed with an event pair that its kernel records at start/end.

    back_to_back (the default): each step's launches are enqueued under a
    Hold and run one after another on a busy GPU, as inside the timed graph
    (`runner.held`: timed steps queued in full before the hold ended).
    Otherwise each launch follows the host's own launch overhead on an idle
    GPU (isolated launches)."""
    import torch

    import q4_weight_only_amd as q4

    n = len(runner.items)
    stream = torch.cuda.current_stream(dev)

    def enqueue_step(pairs):
        for i in range(n):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)               # creates the events
            b.record(stream)
            q4.time_next_launch(a, b)
            runner.launch(i)
            pairs.append((i, a, b))

    pairs = []
    if back_to_back:
        hold = Hold(dev, lambda: enqueue_step([]))
        for _ in range(steps):
            hold.run(lambda: enqueue_step(pairs))
        runner.held = (hold.held, hold.batches)
    else:
        for _ in range(steps):
            enqueue_step(pairs)
        runner.held = None
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
    every launch reads its weights from HBM, not from the infinity cache.
    Two more kinds are timed by events recorded on the stream around the
    calls (launch gaps included): the fused launch, and the unfused launch
    followed by torch's silu(g) * u into h (the unfused step in full).
    Each kind's pass over the pairs runs back to back under a Hold, as the
    step's launches do.  Each kind's time is the median over its launches;
    two untimed passes over every kind come first (the GPU has been idle through the host-side
    oracle timing before this, and a single pass left the first kind's
    launches up to a third slower in some runs)."""
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
        kinds = ("fused", "fused_bf16", "unfused", "fused_stream", "unfused_silu_stream")
        pairs = {kind: [] for kind in kinds}

        def batch(kind, keep):
            for _, pws in gate_up:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                if kind.endswith("_stream"):
                    a.record(stream)
                    if kind == "fused_stream":
                        q4.linear_swiglu(x, pws[0], pws[1], h)
                    else:
                        q4.linear_multi(x, pws, ys)
                        torch.mul(torch.nn.functional.silu(ys[0]), ys[1], out=h)
                    b.record(stream)
                else:
                    a.record(stream)
                    b.record(stream)
                    q4.time_next_launch(a, b)
                    if kind == "fused":
                        q4.linear_swiglu(x, pws[0], pws[1], h)
                    elif kind == "fused_bf16":
                        q4.linear_swiglu(x, pws[0], pws[1], h16, dtype=torch.bfloat16)
                    else:
                        q4.linear_multi(x, pws, ys)
                if keep:
                    pairs[kind].append((a, b))

        # each kind's pass over the 26 pairs runs back to back under a hold
        hold = Hold(dev, lambda: batch("fused", False), warm=0)
        for r in range(reps + 2):
            for kind in kinds:
                hold.run(lambda: batch(kind, r > 1), count=r > 1)   # the first two passes warm up
        torch.cuda.synchronize(dev)
        t = {kind: float(np.median([a.elapsed_time(b) / 1e3 for a, b in v])) for kind, v in pairs.items()}
        wbytes = spec0.weight_bytes()
        fused_bytes = wbytes + m * k * 2 + m * n * 4
        unfused_bytes = wbytes + m * k * 2 + 2 * m * n * 4
        fl = 2 * m * (2 * n) * k
        out[f"M={m}"] = {
            "kernel": q4.linear_swiglu_kernel(m, k),
            "fused_us": round(t["fused"] * 1e6, 2),
            "fused_bf16_out_us": round(t["fused_bf16"] * 1e6, 2),
            "unfused_us": round(t["unfused"] * 1e6, 2),
            "fused_stream_us": round(t["fused_stream"] * 1e6, 2),
            "unfused_with_silu_mul_stream_us": round(t["unfused_silu_stream"] * 1e6, 2),
            "fused_GBs": round(fused_bytes / t["fused"] / 1e9, 1),
            "unfused_GBs": round(unfused_bytes / t["unfused"] / 1e9, 1),
            "fused_TFLOPs": round(fl / t["fused"] / 1e12, 2),
            "unfused_TFLOPs": round(fl / t["unfused"] / 1e12, 2),
            "launches": len(pairs["fused"]),
            "passes_held": [hold.held, hold.batches],
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


def time_single(spec, pw, ms, reps, dev, linear=None, moved_fn=None):
    """One single-segment linear at each M: kernel-own time (armed events) of
    launches that each follow a read of a 512 MiB buffer, so the weights
    stream from HBM rather than from the 256 MB infinity cache (a read, not
    a fill, so no write-back competes with the launch).  Median and
    p10 / p90 over `reps` launches after one warm-up launch."""
    import numpy as np
    import torch

    import q4_weight_only_amd as q4

    linear = linear or q4.linear
    moved_fn = moved_fn or algorithmic_bytes
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    out, ys = {}, {}
    for m in ms:
        xb = spec.activations(m)
        x = torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        y = torch.empty((m, pw.n), dtype=torch.float32, device=dev)
        ys[m] = y
        linear(x, pw, y)
        pairs = []
        for _ in range(reps):
            torch.sum(flush, dim=0, out=sink)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            b.record(stream)
            q4.time_next_launch(a, b)
            linear(x, pw, y)
            pairs.append((a, b))
        torch.cuda.synchronize(dev)
        ts = np.array([a.elapsed_time(b) / 1e3 for a, b in pairs])
        t = float(np.median(ts))
        moved = moved_fn(spec, m)
        kname = (q4.q41_linear_kernel(m, spec.K, spec.Ns[0]) if linear is q4.q41_linear
                 else q4.linear_kernel(m, spec.K, spec.Ns))
        out[f"M={m}"] = {"kernel": kname, "us": round(t * 1e6, 2),
                         "p10_us": round(float(np.percentile(ts, 10)) * 1e6, 2),
                         "p90_us": round(float(np.percentile(ts, 90)) * 1e6, 2),
                         "GBs": round(moved / t / 1e9, 1), "frac_of_8TBs": round(moved / t / 1e9 / HBM_PEAK_GBS, 4),
                         "TFLOPs": round(flops(spec, m) / t / 1e12, 2),
                         "frac_of_bf16_peak": round(flops(spec, m) / t / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "bytes_alg": moved, "flops": flops(spec, m), "launches": reps}
        del x
    del flush, sink
    return out, ys


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


# ------------------------------------------------------------- metadata
def run_meta():
    """Seed, source revision, host cores and the BLAS the oracle runs on."""
    info = {"seed": 0, "git_rev": None, "host_cores": len(os.sched_getaffinity(0)), "blas": None}
    try:
        with open(os.path.join(ROOT, "q4_weight_only_amd", "_build", "build_info.json")) as f:
            b = json.load(f)
        info["git_rev"] = b.get("git_rev")
        info["source_dirty_at_build"] = b.get("dirty")
    except (OSError, ValueError):
        pass
    try:
        from threadpoolctl import threadpool_info

        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = {"vendor": blas[0].get("internal_api"), "version": blas[0].get("version"),
                            "threads": blas[0].get("num_threads")}
    except Exception:
        pass
    return info


# --------------------------------------------------------------- parity
def parity_rows(spec, si, m, y_dev, w=None, count=48):
    """The timed output y_dev [m, N] of segment si against the oracle on
    `count` sampled weight rows (every m row): (max |err|/bound, cosine).  The
    oracle quantizes those rows itself from the seeded fp32 weights."""
    import numpy as np

    from oracle import q4_0_oracle as O

    if w is None:
        w = spec.weight(si)
    n = w.shape[0]
    rng = np.random.default_rng(1000 + si)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(count, n), replace=False)]))
    blocks = O.quantize(np.ascontiguousarray(w[rows]))
    ref, bound = O.linear_with_bound(spec.activations(m), blocks, len(rows), spec.K)
    y = y_dev[:, rows].cpu().numpy().astype(np.float64)
    ratio = float(np.max(np.abs(y - ref) / bound))
    cos = float(np.dot(y.ravel(), ref.ravel()) / (np.linalg.norm(y) * np.linalg.norm(ref)))
    return ratio, cos


def parity_record(checks):
    """Summary of a list of (ratio, cosine) checks."""
    return {"max_err_over_bound": round(max(r for r, _ in checks), 6),
            "cosine_min": min(c for _, c in checks), "checks": len(checks), "rows_per_check": 48,
            "within_bound": bool(all(r <= 1.0 for r, _ in checks))}


# ------------------------------------------------------- CPU oracle rate
def oracle_threads():
    try:
        from threadpoolctl import threadpool_info

        return max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_oracle_rate(jobs, runs, unit, sample):
    """Time the oracle (dequantize + fp64 matmul, input quantization outside
    the timer) over `jobs` = [(x_bits, blocks, n, k, amount)], `runs` times;
    the median rate in `unit` ("GB/s": amount = algorithmic bytes,
    "GFLOP/s": amount = 2 m n k)."""
    import numpy as np

    from oracle import q4_0_oracle as O

    rates = []
    for _ in range(runs):
        t0 = time.perf_counter()
        for xb, blocks, n, k, _amount in jobs:
            O.linear(xb, blocks, n, k)
        dt = time.perf_counter() - t0
        rates.append(sum(j[4] for j in jobs) / dt / 1e9)
    return {"value": round(float(np.median(rates)), 4), "unit": unit, "runs": runs, "cores": oracle_threads(),
            "kind": "oracle", "seconds_per_run": round(dt, 2), "sample": sample}


# ---------------------------------------------------------- decode floor
def time_ceiling(dev, iterations=2000, reps=5):
    """The prefill GEMM's arithmetic alone (q4_0_reference_mfma): kernel-own
    TFLOP/s of the MFMAs, of the MFMAs with the exact fp32 rescale, of both
    with the nibble decode, and of the MFMAs beside as many fp32 FMAs that do
    not depend on them (can the rescale's VALU work hide under the MFMAs?),
    median of `reps` launches each."""
    import numpy as np
    import torch

    import q4_weight_only_amd as q4

    stream = torch.cuda.current_stream(dev)
    out = {}
    for mode, key in ((0, "mfma_only"), (1, "mfma_rescale"), (2, "mfma_rescale_decode"),
                      (3, "mfma_independent_fma")):
        q4.reference_mfma(mode, 10, dev)
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            b.record(stream)
            q4.time_next_launch(a, b)
            mfmas = q4.reference_mfma(mode, iterations, dev)
            b.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        t = float(np.median(ts))
        tf = mfmas * 16384 / t / 1e12
        out[key] = {"TFLOPs": round(tf, 1), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                    "us": round(t * 1e6, 1)}
    return out


def time_floor(runner, steps, warmup, dev):
    """The decode step's launch structure without its arithmetic: a graph of
    one reference read per launch over that launch's weight bytes, and a graph
    of as many empty launches (reference reads of zero bytes)."""
    import torch

    import q4_weight_only_amd as q4

    sizes = [spec.weight_bytes() // 16 * 16 for spec, *_ in runner.items]
    buf = torch.zeros(sum(sizes), dtype=torch.uint8, device=dev)
    sink = torch.empty(int(q4.lib().q4_0_reference_read_words(max(sizes))), dtype=torch.int32, device=dev)
    offs = [sum(sizes[:i]) for i in range(len(sizes))]

    class Reads:
        items = runner.items

        def __init__(self, empty):
            self.empty = empty

        def launch(self, i):
            q4.reference_read(buf[offs[i]:offs[i] + sizes[i]], 0 if self.empty else sizes[i], sink)

        def step(self):
            for i in range(len(sizes)):
                self.launch(i)

    out = {}
    for key, empty in (("read_us_per_step", False), ("empty_us_per_step", True)):
        r = Reads(empty)
        el, g = time_graph(r, steps, warmup, dev)
        del g
        out[key] = round(el / steps * 1e6, 1)
        out[key.replace("_us_per_step", "_p10_p50_p90_us")] = pctl_us(r.step_times)
    # each op's plain read on its own: kernel-own p10 / p50 / p90 over the layers and steps
    per = time_kernels(Reads(False), steps, dev)
    by_op = collections.defaultdict(list)
    for (spec, *_), d in zip(runner.items, per):
        by_op[spec.name.split(".", 1)[1]].extend(d)
    out["per_op_read_us_p10_p50_p90"] = {op: pctl_us(d) for op, d in by_op.items()}
    out["launches"] = len(sizes)
    out["read_bytes_per_step"] = sum(sizes)
    out["read_GBs"] = round(sum(sizes) / (out["read_us_per_step"] * 1e-6) / 1e9, 1)
    del buf, sink
    return out


# ------------------------------------------------------------------ main
def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("bench.py runs on one GPU only: this build measures the single-GPU hot path "
               "(no collectives); run with --gpus 1")
        print(msg, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import q4_weight_only_amd as q4
    from oracle import q4_0_oracle as O
    from q4_weight_only_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    q4.lib()          # fail loudly if the library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    meta = run_meta()
    do_cpu = not args.no_cpu_baseline

    # ---- workload 2: the decode step (the headline)
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
        "timing": "kernel-own (events armed on each launch), launches back to back as in the graph",
        "steps_held": list(runner.held),
        "step_kernel_sum_us": round(sum(sum(d) for d in durations) / args.steps * 1e6, 1),
    }
    if args.isolated:
        # the same launches one at a time on an otherwise idle GPU (host overhead between them)
        iso = time_kernels(runner, args.steps, dev, back_to_back=False)
        iso_op = collections.OrderedDict()
        for (spec, *_), d in zip(runner.items, iso):
            iso_op.setdefault(spec.name.split(".", 1)[1], []).extend(d)
        roofline["per_op_isolated_p10_p50_p90_us"] = {op: pctl_us(v) for op, v in iso_op.items()}
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
        **meta,
    }

    # the same step at M=2 (the batched CFG pair)
    runner2 = Runner(prepared, 2, dev)
    el2, graph2 = time_graph(runner2, args.steps, args.warmup, dev)
    del graph2
    gbs2 = runner2.bytes_per_step() * args.steps / el2 / 1e9
    log(f"decode M=2: {el2 / args.steps * 1e6:.1f} us/step, {gbs2:.1f} GB/s")

    # parity of the timed outputs (the last replay's): first and last layer
    checks = []
    for li in sorted({0, args.layers - 1}):
        for (spec, pws, xs, ys), (_, _, _, ys2) in zip(runner.items[4 * li:4 * li + 4], runner2.items[4 * li:4 * li + 4]):
            for si in range(len(spec.Ns)):
                w = spec.weight(si)
                checks.append(parity_rows(spec, si, 1, ys[si], w))
                checks.append(parity_rows(spec, si, 2, ys2[si], w))
                del w
    parity2 = parity_record(checks)
    log(f"decode parity: {parity2}")

    out["decode_floor"] = {
        "workload": "the decode step's 104 launches, each a plain 16-byte nontemporal read of that launch's "
                    "weight bytes (q4_0_reference_read), and 104 empty launches; one HIP graph per step",
        **time_floor(runner, args.steps, args.warmup, dev),
    }
    log(f"decode floor: {out['decode_floor']}")

    wl = {}
    wl["2"] = {
        "workload": f"{args.layers}-layer decode step, M=1 and M=2 (batched CFG pair), distinct weights per layer",
        "M=1": {"us_per_step": round(elapsed / args.steps * 1e6, 1), "step_us_p10_p50_p90": pctl_us(runner.step_times),
                "GBs": round(value, 1), "frac_of_8TBs": round(value / HBM_PEAK_GBS, 4), "bytes_alg": step_bytes,
                "kernels": sorted({q4.linear_kernel(1, sp.K, sp.Ns) for sp, *_ in runner.items})},
        "M=2": {"us_per_step": round(el2 / args.steps * 1e6, 1), "step_us_p10_p50_p90": pctl_us(runner2.step_times),
                "GBs": round(gbs2, 1), "frac_of_8TBs": round(gbs2 / HBM_PEAK_GBS, 4),
                "bytes_alg": runner2.bytes_per_step(),
                "kernels": sorted({q4.linear_kernel(2, sp.K, sp.Ns) for sp, *_ in runner2.items})},
        "parity": parity2,
    }
    del runner2

    # ---- workload 4: prefill M=2048 through the four decoder shapes (layer-0 weights)
    if not args.no_prefill:
        _, pre = inputs.workload(4)
        pspecs = [s for s, _ in pre]
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
        pk_names = [q4.linear_kernel(2048, spec.K, spec.Ns) for spec, *_ in prunner.items]
        pk_by = collections.Counter()
        for name, d in zip(pk_names, pdur):
            pk_by[name] += sum(d)
        pchecks = []
        for spec, pws, xs, ys in prunner.items:
            for si in range(len(spec.Ns)):
                pchecks.append(parity_rows(spec, si, 2048, ys[si]))
        wl["4"] = {
            "workload": "prefill M=2048 through QKV 3072->6144, O 4096->3072, gate/up 3072->18432, down 9216->3072",
            "TFLOPs_per_step": round(tflops, 2),
            "us_per_step": round(pel / args.prefill_steps * 1e6, 1),
            "step_us_p10_p50_p90": pctl_us(prunner.step_times),
            "flops": prunner.flops_per_step(),
            "bytes_alg": prunner.bytes_per_step(),
            "steps": args.prefill_steps,
            "roofline": {
                "bound": "mfma",
                "kernel": pk_by.most_common(1)[0][0],
                "achieved": round(pach, 2),
                "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(pach / BF16_PEAK_TFLOPS, 4),
                "timing": "kernel-own (events armed on each launch), launches back to back as in the graph",
                "steps_held": list(prunner.held),
            },
            "per_op": {spec.name.split(".", 1)[1]: {
                "kernel": name, "TFLOPs": round(flops(spec, 2048) * len(d) / sum(d) / 1e12, 2),
                "kernel_us_p10_p50_p90": pctl_us(d), "flops": flops(spec, 2048),
                "bytes_alg": algorithmic_bytes(spec, 2048)}
                for (spec, *_), name, d in zip(prunner.items, pk_names, pdur)},
            "parity": parity_record(pchecks),
        }
        out["prefill"] = {"value": wl["4"]["TFLOPs_per_step"], "unit": "TFLOP/s", "roofline": wl["4"]["roofline"]}
        log(f"prefill: {tflops:.1f} TFLOP/s (kernel {pach:.1f})")
        ceil = time_ceiling(dev)
        out["prefill"]["arithmetic_ceiling"] = {
            "workload": "the 128-row GEMM tiles' inner loop on register operands (q4_0_reference_mfma): "
                        "8 MFMAs per B fragment, 4 waves per SIMD, no memory traffic",
            **ceil,
            "kernel_own_over_ceiling": round(pach / ceil["mfma_rescale_decode"]["TFLOPs"], 3),
        }
        log(f"arithmetic ceiling: {out['prefill']['arithmetic_ceiling']}")
        if do_cpu:
            spec = pspecs[0]
            rows = 1024
            blocks = O.quantize(spec.weight(0)[:rows])
            wl["4"]["cpu"] = cpu_oracle_rate(
                [(spec.activations(2048), blocks, rows, spec.K, 2 * 2048 * rows * spec.K)], 1, "GFLOP/s",
                f"M=2048 through the first {rows} rows of the QKV weights (K={spec.K})")
        del prunner, pprep

    # ---- fused gate/up + SwiGLU against the unfused gate/up launch
    if not args.no_swiglu:
        out["swiglu"] = {
            "workload": "decoder gate/up 3072->2x9216 (one weight pair per layer, rotated), "
                        "h = silu(x Wg^T) * (x Wu^T), fp32 out (fused_bf16_out_us: bf16 out)",
            **time_swiglu(prepared, (1, 2, 2048), 3 if args.layers >= 8 else 6, dev),
        }
        log(f"swiglu: {out['swiglu']}")

    # ---- workload 3: the LM head (M = 1 and 32); the same table feeds the embedding lookups
    if not args.no_embed:
        _, lm = inputs.workload(3)
        lm_spec = lm[0][0]
        lm_w = lm_spec.weight(0)
        wt = torch.from_numpy(lm_w).to(dev)
        lm_blocks = q4.quantize(wt)
        del wt
        lm_pw = q4.pack(lm_blocks, lm_spec.Ns[0], lm_spec.K)
        out["embed"] = {
            "table": f"{lm_spec.Ns[0]}x{lm_spec.K} Q4_0 (the LM head weights), fp32 rows out, random ids; "
                     "packed table (q4_0_embed) and GGUF block order (q4_0_embed_gguf, key gguf)",
            **time_embed(lm_pw, (32, 2048, 16384), 50, dev),
            "gguf": time_embed(lm_pw, (32, 2048, 16384), 50, dev, blocks=lm_blocks),
        }
        del lm_blocks
        log(f"embed: {out['embed']}")
        res, ys = time_single(lm_spec, lm_pw, (1, 32), 20, dev)
        wl["3"] = {"workload": f"LM head {lm_spec.K}->{lm_spec.Ns[0]} (226 MB of Q4_0), one launch, from HBM",
                   **res, "parity": parity_record([parity_rows(lm_spec, 0, m, ys[m], lm_w) for m in (1, 32)])}
        log(f"lm_head: {wl['3']}")
        if do_cpu:
            rows = 16384
            blocks = O.quantize(lm_w[:rows])
            wl["3"]["cpu"] = cpu_oracle_rate(
                [(lm_spec.activations(1), blocks, rows, lm_spec.K,
                  rows * lm_spec.K // 32 * 18 + lm_spec.K * 2 + rows * 4)], 3, "GB/s",
                f"M=1 through the first {rows} of the {lm_spec.Ns[0]} rows (1/8 of the table)")
        del lm_pw, lm_w, ys

    # ---- workloads 1 and 5: the lone GEMV and the audio linears, each from HBM
    if not args.no_others:
        _, g1 = inputs.workload(1)
        _, a5 = inputs.workload(5)
        for key, items in (("1", g1), ("5", a5)):
            rec, checks, jobs = {}, [], []
            for spec, ms in items:
                w = spec.weight(0)
                (_, pws, _), = build_device_specs([spec], (), dev)
                res, ys = time_single(spec, pws[0], ms, 20, dev)
                for mk, r in res.items():
                    rec[f"{spec.name} {spec.K}->{spec.Ns[0]} {mk}"] = r
                for m in ms:
                    checks.append(parity_rows(spec, 0, m, ys[m], w))
                if do_cpu and key == "1":
                    jobs.append((spec.activations(1), O.quantize(w), spec.Ns[0], spec.K, algorithmic_bytes(spec, 1)))
                if do_cpu and key == "5" and spec.name == "adapter":
                    rows = 512
                    jobs.append((spec.activations(ms[0]), O.quantize(w[:rows]), rows, spec.K,
                                 2 * ms[0] * rows * spec.K))
                del pws, ys, w
            wl[key] = {"workload": ("one GEMV 3072->4096 at M=1" if key == "1" else
                                    "audio linears: 5120->3072, 3072->3072 at M=1505; 1280->5120, 5120->1280 at M=6020"),
                       **rec, "parity": parity_record(checks)}
            if jobs:
                wl[key]["cpu"] = (cpu_oracle_rate(jobs, 3, "GB/s", "the whole GEMV") if key == "1" else
                                  cpu_oracle_rate(jobs, 1, "GFLOP/s", "M=1505 through the first 512 rows of the "
                                                                         "adapter 5120->3072"))
            log(f"workload {key}: {wl[key]}")

    # ---- the asymmetric variant (w = q d + m per block): the decoder shapes, each
    # matrix alone, at M = 1 and 2048 (layer-0 weights, quantized on the device)
    if not args.no_others:
        from q4_weight_only_amd.inputs import LinearSpec

        rec, checks = {}, []
        for spec in specs[:4]:
            for si, n in enumerate(spec.Ns):
                one = LinearSpec(f"{spec.name}.{si}", spec.K, (n,), [spec.w_tags[si]], spec.x_tags)
                w = one.weight(0)
                pw = q4.q41_pack(q4.q41_quantize(torch.from_numpy(w).to(dev)), n, spec.K)
                res, ys = time_single(one, pw, (1, 2048), 10, dev, linear=q4.q41_linear,
                                      moved_fn=lambda sp, m: sp.Ns[0] * sp.K // 32 * 20 + m * sp.K * 2 + m * sp.Ns[0] * 4)
                for mk, r in res.items():
                    rec[f"{spec.name.split('.', 1)[1]}[{si}] {spec.K}->{n} {mk}"] = r
                rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(si).choice(n, 46, replace=False)]))
                blocks = O.q41_quantize(np.ascontiguousarray(w[rows]))
                for m in (1, 2048):
                    ref, bound = O.q41_linear_with_bound(one.activations(m), blocks, len(rows), spec.K)
                    yv = ys[m][:, rows].cpu().numpy().astype(np.float64)
                    checks.append((float(np.max(np.abs(yv - ref) / bound)),
                                   float(np.dot(yv.ravel(), ref.ravel()) / (np.linalg.norm(yv) * np.linalg.norm(ref)))))
                del pw, ys, w
        out["variant_q41"] = {
            "workload": "asymmetric 4-bit blocks (w = q d + m, 20 bytes per 32 weights): the decoder's seven weight "
                        "matrices of layer 0, one launch each, from HBM, at M=1 (GB/s) and M=2048 (TFLOP/s)",
            **rec, "parity": parity_record(checks)}
        log(f"variant q41: {out['variant_q41']}")

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        out["copy_calibration"] = {"bytes_read": 256 << 20, "bytes_written": 256 << 20, "calls": 3}

    if do_cpu:
        # the whole decode step at M=1 (input quantization outside the timer)
        jobs = []
        for spec in specs:
            for si, n in enumerate(spec.Ns):
                jobs.append((spec.activations(1), O.quantize(spec.weight(si)), n, spec.K,
                             n * spec.K // 32 * 18 + spec.K * 2 // len(spec.Ns) + n * 4))
        rec = cpu_oracle_rate(jobs, 1, "GB/s", f"the whole {args.layers}-layer decode step at M=1 "
                                               f"({len(specs)} launches)")
        wl["2"]["cpu"] = rec
        out["cpu_baseline"] = rec
        log(f"cpu baseline: {rec}")

    out["workloads"] = {k: wl[k] for k in sorted(wl)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
