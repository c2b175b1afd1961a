"""Seeded random launches across the dispatch table: M from 1 to 300 (and a
few tall one-row launches that take the stream kernel), 1-4 segments of
ragged N, K any multiple of 32 up to 5120.  Every output element against the oracle's
bound; each case prints its shape and kernel first."""

import numpy as np
import pytest
import torch

from oracle import q4_0_oracle as O
import q4_weight_only_amd as q4
from q4_weight_only_amd import inputs

from gpu_helpers import DEV, assert_within_bound, device_weight_from_f32, say, to_dev_x

pytestmark = pytest.mark.gpu

BUDGET = 4e7          # M * sum(N) * K per case, so the fp64 oracle stays fast


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    if seed % 10 == 9:                         # tall one-row launch
        m, k = 1, int(rng.choice([1024, 2048, 3072]))
        ns = [int(rng.integers(2048 * 16, 2400 * 16))]
        return m, k, ns
    m = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 17, 24, 32, 33, 48, 64, 65, 100, 129, 200, 300]))
    k = 32 * int(rng.integers(1, 161))
    nseg = int(rng.integers(1, 5))
    ns = [int(rng.integers(1, 1600)) for _ in range(nseg)]
    while m * sum(ns) * k > BUDGET:
        ns = [max(1, n // 2) for n in ns]
    return m, k, ns


@pytest.mark.parametrize("seed", range(30))
def test_random_launch_within_bound(seed):
    m, k, ns = _case(seed)
    ws = [inputs.weights_f32((n, k), seed=2000 + seed, tags=(i,)) for i, n in enumerate(ns)]
    dev = [device_weight_from_f32(w) for w in ws]
    xb = inputs.activations_bf16((m, k), seed=2000 + seed, tags=(m, k))
    say("random", seed, m, k, ns, q4.linear_kernel(m, k, ns))
    x = to_dev_x(xb)
    ys = q4.linear_multi(x, [p for p, _ in dev]) if len(ns) > 1 else [q4.linear(x, dev[0][0])]
    for i, (w, (pw, blocks), y) in enumerate(zip(ws, dev, ys)):
        b = blocks.cpu().numpy()
        assert np.array_equal(b, O.quantize(w)), f"case {seed} segment {i}: quantized bytes"
        n = w.shape[0]
        assert_within_bound(y.cpu().numpy(), O.linear(xb, b, n, k), O.error_bound(xb, b, n, k),
                            f"case {seed}: M={m} K={k} N={ns} segment {i}")
    torch.cuda.synchronize()
