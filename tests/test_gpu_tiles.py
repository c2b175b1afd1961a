"""The GEMM tile shape (64 x 128, 128 x 128 or 128 x 192) is picked from the
launch's tile count, so one output can be computed under different shapes:
a single launch, the same matrix inside a fused launch, and fewer rows of x.
The shapes add the block results of an output in the same order, so all of
them must agree bit for bit, and the 128 x 192 shape (with a ragged last
tile in N and a K that is not a multiple of 128) must meet the oracle's
bound."""

import numpy as np
import pytest

from oracle import q4_0_oracle as O
import q4_weight_only_amd as q4
from q4_weight_only_amd import inputs

from gpu_helpers import DEV, assert_within_bound, device_weight_from_f32, sample_rows, say, to_dev_x

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


def test_tile_shapes_agree_bitwise():
    m, k = 2048, 992
    ns = (3000, 3072, 3072)
    ws = [inputs.weights_f32((n, k), seed=81, tags=(n, i)) for i, n in enumerate(ns)]
    dev = [device_weight_from_f32(w) for w in ws]
    pws = [p for p, _ in dev]
    xb = inputs.activations_bf16((m, k), seed=81, tags=(m, k))
    x = to_dev_x(xb)

    single = q4.linear_kernel(m, k, ns[0])
    fused = q4.linear_kernel(m, k, ns)
    say("tiles single", single, "fused", fused)
    y_single = q4.linear(x, pws[0])
    y_fused = q4.linear_multi(x, pws)
    assert np.array_equal(_bits(y_single), _bits(y_fused[0])), f"{single} vs {fused}"
    for i in (1, 2):
        assert np.array_equal(_bits(q4.linear(x, pws[i])), _bits(y_fused[i]))

    # fewer rows of x: other tile shapes
    for rows in (1500, 300):
        say("tiles rows", rows, q4.linear_kernel(rows, k, ns[0]))
        y = q4.linear(x[:rows], pws[0])
        assert np.array_equal(_bits(y), _bits(y_single[:rows])), f"M={rows}"
    # and the 17-64-row GEMM, on weights tall enough to take it
    tall = 8 * 16 * 129
    wt = inputs.weights_f32((tall, k), seed=81, tags=(tall,))
    pt, _ = device_weight_from_f32(wt)
    yt = q4.linear(x, pt)
    for rows in (64, 40):
        assert q4.linear_kernel(rows, k, tall).startswith("gemm_kernel<")
        say("tiles rows", rows, q4.linear_kernel(rows, k, tall))
        assert np.array_equal(_bits(q4.linear(x[:rows], pt)), _bits(yt[:rows])), f"M={rows}"

    # the single launch against the oracle on sampled rows of W
    cols = sample_rows(ns[0], 48, 81)
    blocks = dev[0][1].cpu().numpy().reshape(ns[0], -1)[cols]
    assert np.array_equal(blocks.reshape(-1), O.quantize(ws[0][cols]).reshape(-1))
    xs = xb[np.r_[0:64, m - 64:m]]
    ref, bound = O.linear_rows(xs, blocks, len(cols), k, np.arange(len(cols)))
    got = y_single.cpu().numpy()[np.r_[0:64, m - 64:m]][:, cols]
    assert_within_bound(got, ref, bound, f"{single} M={m} N={ns[0]} K={k}")


def test_tile_shape_names():
    """At 2048 rows on 256 CUs: N = 3072 alone fills exactly 256 tiles of
    128 x 192; three of them fused make 1152 tiles of 128 x 128; at 1505 rows
    N = 3072 fills 256 tiles of 96 x 192; few rows take 64 x 128."""
    import torch
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    if cus != 256:
        pytest.skip(f"tile counts here assume 256 compute units, the device has {cus}")
    assert q4.linear_kernel(2048, 4096, 3072) == "gemm3_kernel<8, 1, 1, 12, 0, 4, false>"
    assert q4.linear_kernel(1505, 3072, 3072) == "gemm3_kernel<6, 1, 1, 12, 0, 4, false>"
    assert q4.linear_kernel(2048, 3072, (3072, 3072, 3072)) == "gemm3_kernel<8, 1, 1, 8, 4, 4, false>"
    assert q4.linear_kernel(2048, 3072, (9216, 9216)) == "gemm3_kernel<8, 1, 1, 8, 4, 4, false>"
    assert q4.linear_kernel(300, 3072, 3072) == "gemm3_kernel<4, 1, 1, 8, 4, 8, false>"
