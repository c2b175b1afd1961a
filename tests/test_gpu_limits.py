"""Sizes at and near the interface limits (include/q4_0.h): K up to 2^17, M up
to the 2^20 maximum, N up to 2^20 rows, each kernel family, checked against the
oracle (every output, or sampled weight rows where N is large)."""

import numpy as np
import pytest

from oracle import q4_0_oracle as O
import q4_weight_only_amd as q4
from q4_weight_only_amd import inputs

from gpu_helpers import assert_within_bound, device_weight_from_f32, sample_rows, say, to_dev_x

pytestmark = pytest.mark.gpu

CASES = [
    (1, 48, 131072),       # long K: x does not fit LDS, decode kernel reads it from L2
    (2, 48, 131072),
    (17, 40, 131072),      # 17-64 rows, long K
    (2100, 40, 65536),     # prefill tiles, long K
    (1 << 20, 16, 32),     # M at its maximum, one block of K
]


@pytest.mark.parametrize("m,n,k", CASES)
def test_limit_shapes_every_output(m, n, k):
    w = inputs.weights_f32((n, k), seed=61, tags=(n, k))
    x = inputs.activations_bf16((m, k), seed=61, tags=(m, k))
    pw, blocks = device_weight_from_f32(w)
    b = blocks.cpu().numpy()
    say("limits", m, n, k, q4.linear_kernel(m, k, n))
    y = q4.linear(to_dev_x(x), pw).cpu().numpy()
    assert_within_bound(y, O.linear(x, b, n, k), O.error_bound(x, b, n, k), f"M={m} N={n} K={k}")


@pytest.mark.parametrize("m,n,k", [(1, 1 << 20, 32), (100, 1 << 18, 64)])
def test_limit_rows_sampled(m, n, k):
    w = inputs.weights_f32((n, k), seed=62, tags=(n, k))
    x = inputs.activations_bf16((m, k), seed=62, tags=(m, k))
    pw, blocks = device_weight_from_f32(w)
    say("limits rows", m, n, k, q4.linear_kernel(m, k, n))
    y = q4.linear(to_dev_x(x), pw).cpu().numpy()
    rows = sample_rows(n, 256, 62)
    b = blocks.cpu().numpy().reshape(n, -1)[rows]
    assert np.array_equal(b.reshape(-1), O.quantize(w[rows]).reshape(-1))
    ref, bound = O.linear_rows(x, b, len(rows), k, np.arange(len(rows)))
    assert_within_bound(y[:, rows], ref, bound, f"M={m} N={n} K={k}")
