"""The five workloads at full size, run exactly as the benchmark runs them
(same entry points, same launch configuration), checked against the oracle on
sampled weight rows (every M row of those columns).  The weights' quantized
bytes are checked bit-exactly against the oracle quantizer on the same rows."""

import collections
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import q4_0_oracle as O
import q4_weight_only_amd as q4
from q4_weight_only_amd import inputs

from gpu_helpers import DEV, assert_within_bound, sample_rows, say, to_dev_x

pytestmark = pytest.mark.gpu

ROWS_PER_SEGMENT = 48


def _prepare(spec, si, seed):
    w = spec.weight(si)
    rows = sample_rows(w.shape[0], ROWS_PER_SEGMENT, seed)
    return w, rows, np.ascontiguousarray(w[rows])


def _run_workload(cfg):
    desc, specs = inputs.workload(cfg)
    say("workload", cfg, desc)
    jobs = [(j, spec, si) for j, (spec, si) in
            enumerate((spec, si) for spec, _ in specs for si in range(len(spec.Ns)))]
    built = {}
    with ThreadPoolExecutor(8) as ex:
        pending = collections.deque()
        it = iter(jobs)

        def submit_next():
            nxt = next(it, None)
            if nxt is not None:
                j, spec, si = nxt
                pending.append((spec, si, ex.submit(_prepare, spec, si, cfg * 1000 + j)))

        for _ in range(12):
            submit_next()
        while pending:
            spec, si, fut = pending.popleft()
            w, rows, wrows = fut.result()
            del fut
            blocks = q4.quantize(torch.from_numpy(w).to(DEV))
            del w
            got_rows = blocks[torch.from_numpy(rows).to(DEV)].cpu().numpy()
            ref_rows = O.quantize(wrows)
            assert np.array_equal(got_rows, ref_rows), f"{spec.name} seg {si}: quantized bytes differ"
            built[(id(spec), si)] = (q4.pack(blocks, spec.Ns[si], spec.K), (rows, ref_rows))
            del blocks
            submit_next()
    prepared = []
    for spec, ms in specs:
        segs = [built.pop((id(spec), si)) for si in range(len(spec.Ns))]
        prepared.append((spec, ms, [s[0] for s in segs], [s[1] for s in segs]))
    worst, cos_min = 0.0, 1.0
    for spec, ms, pws, samples in prepared:
        for m in ms:
            xb = spec.activations(m)
            x = to_dev_x(xb)
            say("run", spec.name, "M", m)
            ys = q4.linear_multi(x, pws) if len(pws) > 1 else [q4.linear(x, pws[0])]
            for si, (y, (rows, ref_blocks)) in enumerate(zip(ys, samples)):
                yr = y[:, torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
                n = len(rows)
                ref = O.linear(xb, ref_blocks, n, spec.K)
                ratio = assert_within_bound(yr, ref, O.error_bound(xb, ref_blocks, n, spec.K),
                                            f"cfg{cfg} {spec.name} seg{si} M={m}")
                worst = max(worst, ratio)
                cos = float(np.dot(yr.ravel(), ref.ravel()) / (np.linalg.norm(yr) * np.linalg.norm(ref)))
                cos_min = min(cos_min, cos)
    # the pages report parity as cosine similarity to a reference output; within
    # the elementwise bound it is 1 to many digits
    say(f"cfg{cfg}: max |err|/bound = {worst:.4f}, min cosine = {cos_min:.12f}")
    assert cos_min > 1 - 1e-9
    return worst


@pytest.mark.parametrize("cfg", [1, 3, 4, 5, 2])
def test_workload_parity_sampled(cfg):
    _run_workload(cfg)


def test_gemv_workload_full_output():
    """The single GEMV compared on every output element."""
    desc, [(spec, ms)] = inputs.workload(1)
    w = spec.weight(0)
    blocks = O.quantize(w)
    pw = q4.pack(q4.quantize(torch.from_numpy(w).to(DEV)), 4096, 3072)
    xb = spec.activations(1)
    say("gemv full")
    y = q4.linear(to_dev_x(xb), pw).cpu().numpy()
    assert_within_bound(y, O.linear(xb, blocks, 4096, 3072), O.error_bound(xb, blocks, 4096, 3072), "gemv")
