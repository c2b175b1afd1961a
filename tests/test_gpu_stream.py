"""The one-row stream kernel (tall weights such as the LM head: a fixed grid
walking the row tiles, x staged once per workgroup, the next tile's loads
issued across each tile boundary).  Its arithmetic is the decode kernel's, so
the rows of a tall launch must equal, bit for bit, a launch of just those rows
(which runs the ordinary decode kernel); the segment walk of a fused launch
must route every tile; and sampled rows must meet the oracle's bound."""

import numpy as np
import pytest
import torch

from oracle import q4_0_oracle as O
import q4_weight_only_amd as q4
from q4_weight_only_amd import inputs

from gpu_helpers import DEV, assert_within_bound, sample_rows, say, to_dev_x

pytestmark = pytest.mark.gpu

STREAM = "skinny_stream_kernel<1, 8, 3, 6>"


def _blocks(n, k, seed, tag):
    w = inputs.weights_f32((n, k), seed=seed, tags=(n, k, tag))
    return w, q4.quantize(torch.from_numpy(w).to(DEV))


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


def _cus():
    return torch.cuda.get_device_properties(DEV).multi_processor_count


@pytest.mark.parametrize("n,k", [(40008, 1024), (8 * 16 * 256 + 5, 3072)])
def test_stream_rows_equal_short_launches(n, k):
    if (n + 15) // 16 < 8 * _cus():
        pytest.skip("needs at least 8 row tiles per CU to take the stream kernel")
    w, blocks = _blocks(n, k, 91, 0)
    pw = q4.pack(blocks, n, k)
    xb = inputs.activations_bf16((1, k), seed=91, tags=(k,))
    x = to_dev_x(xb)
    assert q4.linear_kernel(1, k, n) == STREAM
    say("stream", n, k)
    y = q4.linear(x, pw)
    # the first 1000 rows and the last ~1000 (from a tile boundary, so each row
    # keeps its place in its 16-row tile; the last tile is ragged) as short launches
    gb = blocks.view(n, -1)
    for lo, hi in ((0, 1000), ((n - 1000) // 16 * 16, n)):
        sub = q4.pack(gb[lo:hi].contiguous().view(-1), hi - lo, k)
        assert q4.linear_kernel(1, k, hi - lo) != STREAM
        ys = q4.linear(x, sub)
        assert np.array_equal(_bits(y[:, lo:hi]), _bits(ys)), f"rows {lo}:{hi}"
    rows = sample_rows(n, 64, 91)
    rb = gb[torch.from_numpy(rows).to(DEV)].cpu().numpy().reshape(len(rows), k // 32, 18)
    assert np.array_equal(rb, O.quantize(w[rows]).reshape(rb.shape))
    assert_within_bound(y.cpu().numpy()[:, rows], O.linear(xb, rb, len(rows), k),
                        O.error_bound(xb, rb, len(rows), k), f"stream N={n} K={k}")


def test_stream_fused_segments():
    """Three segments whose tiles together take the stream kernel: every
    segment's output equals its own (short) launch bit for bit."""
    k = 1024
    ns = (12000, 13000, 8 * 16 * _cus() - 25000 + 40)
    parts = [_blocks(n, k, 92, i) for i, n in enumerate(ns)]
    pws = [q4.pack(b, n, k) for (_, b), n in zip(parts, ns)]
    x = to_dev_x(inputs.activations_bf16((1, k), seed=92, tags=(k,)))
    assert q4.linear_kernel(1, k, ns) == STREAM
    say("stream fused", ns)
    ys = q4.linear_multi(x, pws)
    for i, (n, pw) in enumerate(zip(ns, pws)):
        assert q4.linear_kernel(1, k, n) != STREAM
        assert np.array_equal(_bits(ys[i]), _bits(q4.linear(x, pw))), f"segment {i}"


def test_stream_deterministic():
    n, k = 40000, 1024
    _, blocks = _blocks(n, k, 93, 0)
    pw = q4.pack(blocks, n, k)
    x = to_dev_x(inputs.activations_bf16((1, k), seed=93, tags=(k,)))
    say("stream determinism")
    a = _bits(q4.linear(x, pw))
    b = _bits(q4.linear(x, pw))
    assert np.array_equal(a, b)
