"""The five workloads at full size, run exactly as the benchmark runs them
(same entry points, same launch configuration), checked against the oracle on
every output element at every M.  The device quantizer's bytes are checked
against the oracle quantizer on every block of every weight matrix.

The oracle side runs on a thread pool: a matrix is drawn whole (its random
stream is per matrix), then quantized and multiplied in row chunks, which is
the same definition applied row by row."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import q4_0_oracle as O
import q4_weight_only_amd as q4
from q4_weight_only_amd import inputs

from gpu_helpers import DEV, assert_within_bound, say, to_dev_x

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
CHUNK_ROWS = 4096


def _oracle_chunk(w, xbs, k):
    """Oracle blocks and (y, bound) per activation matrix for one row chunk."""
    blocks = O.quantize(w)
    return blocks, [O.linear_with_bound(xb, blocks, w.shape[0], k) for xb in xbs]


def _oracle_segment(pool, w, spec, ms):
    """(oracle blocks, {m: (y, bound)}) for the fp32 weights w of one segment."""
    n, k = w.shape
    xbs = [spec.activations(m) for m in ms]
    futs = [pool.submit(_oracle_chunk, w[r0:r0 + CHUNK_ROWS], xbs, k) for r0 in range(0, n, CHUNK_ROWS)]
    parts = [f.result() for f in futs]
    blocks = np.concatenate([p[0] for p in parts], axis=0)
    refs = {m: (np.concatenate([p[1][i][0] for p in parts], axis=1),
                np.concatenate([p[1][i][1] for p in parts], axis=1)) for i, m in enumerate(ms)}
    return blocks, refs


LOOKAHEAD = 6   # weight matrices drawn ahead of the one being checked


def _run_workload(cfg):
    from threadpoolctl import threadpool_limits

    desc, specs = inputs.workload(cfg)
    say("workload", cfg, desc)
    worst, cos_min, outputs = 0.0, 1.0, 0
    segs = [(spec, si) for spec, _ in specs for si in range(len(spec.Ns))]
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(THREADS) as pool, \
            ThreadPoolExecutor(LOOKAHEAD) as gen:
        drawn = {i: gen.submit(spec.weight, si) for i, (spec, si) in enumerate(segs[:LOOKAHEAD])}
        j = 0
        for spec, ms in specs:
            pws, refs = [], []
            for si, n in enumerate(spec.Ns):
                w = drawn.pop(j).result()
                if j + LOOKAHEAD < len(segs):
                    nspec, nsi = segs[j + LOOKAHEAD]
                    drawn[j + LOOKAHEAD] = gen.submit(nspec.weight, nsi)
                j += 1
                ref_blocks, ref = _oracle_segment(pool, w, spec, ms)
                blocks = q4.quantize(torch.from_numpy(w).to(DEV))
                del w
                assert torch.equal(blocks.cpu(), torch.from_numpy(ref_blocks)), \
                    f"{spec.name} seg {si}: device quantizer bytes differ from the oracle"
                pws.append(q4.pack(blocks, n, spec.K))
                del blocks, ref_blocks
                refs.append(ref)
            for m in ms:
                x = to_dev_x(spec.activations(m))
                say("run", spec.name, "M", m, q4.linear_kernel(m, spec.K, spec.Ns))
                ys = q4.linear_multi(x, pws) if len(pws) > 1 else [q4.linear(x, pws[0])]
                for si, y in enumerate(ys):
                    yr = y.cpu().numpy().astype(np.float64)
                    ref, bound = refs[si][m]
                    ratio = assert_within_bound(yr, ref, bound, f"cfg{cfg} {spec.name} seg{si} M={m}")
                    worst = max(worst, ratio)
                    cos = float(np.dot(yr.ravel(), ref.ravel()) / (np.linalg.norm(yr) * np.linalg.norm(ref)))
                    cos_min = min(cos_min, cos)
                    outputs += yr.size
                del ys, x
            del pws, refs
    # the pages report parity as cosine similarity to a reference output; within
    # the elementwise bound it is 1 to many digits
    say(f"cfg{cfg}: {outputs} outputs, max |err|/bound = {worst:.4f}, min cosine = {cos_min:.12f}")
    assert cos_min > 1 - 1e-9
    return worst


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [1, 3, 4, 5, 2])
def test_workload_parity_every_output(cfg):
    _run_workload(cfg)
