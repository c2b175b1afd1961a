"""Parity of the device linear with the oracle on sizes the oracle finishes in
seconds: every output element within 1e-3 * sum|x w| + 1e-6, across the
kernel variants (M = 1, 2, 3-4, 5-16, 17-32, 33-64 on short and on tall
weights, 65-2047, >= 2048), several tiles in N and K, ragged edges,
structured weights, fused segments and determinism."""

import numpy as np
import pytest
import torch

from oracle import q4_0_oracle as O
import q4_weight_only_amd as q4
from q4_weight_only_amd import inputs

from gpu_helpers import DEV, assert_within_bound, device_weight_from_blocks, device_weight_from_f32, say, to_dev_x

pytestmark = pytest.mark.gpu


def _run_and_check(w32, x_bits, what):
    n, k = w32.shape
    blocks = O.quantize(w32)
    pw, _ = device_weight_from_f32(w32)
    say("linear", what)
    y = q4.linear(to_dev_x(x_bits), pw).cpu().numpy()
    return assert_within_bound(y, O.linear(x_bits, blocks, n, k), O.error_bound(x_bits, blocks, n, k), what)


MS = [1, 2, 3, 4, 5, 16, 17, 31, 32, 33, 64, 100, 129, 300, 2100]
NKS = [(16, 32), (48, 128), (40, 96), (200, 384), (1040, 1280), (96, 3072), (72, 3104)]


@pytest.mark.parametrize("m", MS)
@pytest.mark.parametrize("n,k", NKS)
def test_linear_parity_grid(m, n, k):
    w = inputs.weights_f32((n, k), seed=21, tags=(n, k))
    x = inputs.activations_bf16((m, k), seed=21, tags=(m, k))
    _run_and_check(w, x, f"M={m} N={n} K={k}")


# up to four rows on long rows: 12 K-slices of up to 6 stages (K 4097-9216;
# where 12 does not divide the super-tiles some stages lie past K, and a last
# super-tile may be partial), the K-split kernel beyond 9216
LONG_NKS = [(40, 4128), (48, 5152), (24, 9184), (72, 9216), (16, 9248)]


@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("n,k", LONG_NKS)
def test_linear_long_rows(m, n, k):
    w = inputs.weights_f32((n, k), seed=23, tags=(n, k))
    x = inputs.activations_bf16((m, k), seed=23, tags=(m, k))
    say("long rows", q4.linear_kernel(m, k, [n]))
    _run_and_check(w, x, f"M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [1, 2, 4, 16, 32, 64])
def test_all_codes_eight_give_zero(m):
    n, k = 64, 512
    rng = np.random.default_rng(m)
    d = (rng.standard_normal((n, k // 32)) * 10).astype(np.float16)
    blocks = O.gguf_encode(d, np.full((n, k), 8, dtype=np.uint8))
    x = inputs.activations_bf16((m, k), seed=m)
    pw = device_weight_from_blocks(blocks, n, k)
    say("all-q8", m)
    y = q4.linear(to_dev_x(x), pw).cpu().numpy()
    assert np.all(np.abs(y) <= 1e-6)


@pytest.mark.parametrize("m", [1, 2, 5, 32, 33])
def test_single_nonzero_nibble(m):
    n, k = 48, 384
    rng = np.random.default_rng(100 + m)
    x = inputs.activations_bf16((m, k), seed=100 + m)
    for trial in range(4):
        q = np.full((n, k), 8, dtype=np.uint8)
        rows = rng.integers(0, n, size=3)
        cols = rng.integers(0, k, size=3)
        q[rows, cols] = rng.integers(0, 16, size=3)
        d = (rng.standard_normal((n, k // 32)) * 0.05).astype(np.float16)
        blocks = O.gguf_encode(d, q)
        pw = device_weight_from_blocks(blocks, n, k)
        say("single nibble", m, trial)
        y = q4.linear(to_dev_x(x), pw).cpu().numpy()
        assert_within_bound(y, O.linear(x, blocks, n, k), O.error_bound(x, blocks, n, k), f"nibble m={m}")


@pytest.mark.parametrize("m", [3, 40, 300])
@pytest.mark.parametrize("e", [-24, -10, 0, 7, 15])
def test_power_of_two_scales_and_wide_activations(e, m):
    n, k = 32, 256
    rng = np.random.default_rng(e + 50)
    q = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    sign = np.where(rng.random((n, k // 32)) < 0.5, -1.0, 1.0)
    d = (sign * 2.0**e).astype(np.float16)
    blocks = O.gguf_encode(d, q)
    # activations over many binades (bf16 keeps fp32's exponent range)
    xf = (rng.standard_normal((m, k)) * np.exp2(rng.integers(-60, 60, size=(m, k)))).astype(np.float32)
    x = inputs.bf16_bits_from_f32(xf)
    pw = device_weight_from_blocks(blocks, n, k)
    say("pow2 scales", e, m)
    y = q4.linear(to_dev_x(x), pw).cpu().numpy()
    assert_within_bound(y, O.linear(x, blocks, n, k), O.error_bound(x, blocks, n, k), f"e={e}")


@pytest.mark.parametrize("m", [1, 2, 32, 70, 2100])
def test_reads_no_activation_beyond_k(m):
    """x sits in a larger buffer whose tail is NaN; padded K must not touch it."""
    n, k = 32, 96                                     # K pads to 128 inside the layout
    w = inputs.weights_f32((n, k), seed=5)
    x = inputs.activations_bf16((m, k), seed=5)
    blocks = O.quantize(w)
    pw = device_weight_from_blocks(blocks, n, k)
    big = torch.full((m * k + 4096,), float("nan"), dtype=torch.bfloat16, device=DEV)
    xv = big[: m * k].view(m, k)
    xv.copy_(to_dev_x(x))
    say("nan tail", m)
    y = q4.linear(xv, pw).cpu().numpy()
    assert_within_bound(y, O.linear(x, blocks, n, k), O.error_bound(x, blocks, n, k), "nan tail")


@pytest.mark.parametrize("m", [17, 32, 40, 64])
def test_17_to_64_rows_on_tall_weights(m):
    """17-64 rows take the GEMM only on weights of at least half a tile per CU
    (129 tiles of 128 rows here); short weights, as in the grid above, take
    the K-split decode kernel.  Every output element against the oracle."""
    n, k = 16400, 256
    w = inputs.weights_f32((n, k), seed=22, tags=(n, k))
    x = inputs.activations_bf16((m, k), seed=22, tags=(m, k))
    name = q4.linear_kernel(m, k, n)
    if torch.cuda.get_device_properties(DEV).multi_processor_count <= 256:
        assert name.startswith("gemm_kernel<"), name
    _run_and_check(w, x, f"M={m} N={n} K={k} {name}")


@pytest.mark.parametrize("m", [1, 2, 3, 17, 32, 40, 300])
def test_multi_equals_separate_calls_bitwise(m):
    k = 384
    ns = (64, 16, 40, 200)
    ws = [inputs.weights_f32((n, k), seed=9, tags=(i,)) for i, n in enumerate(ns)]
    pws = [device_weight_from_f32(w)[0] for w in ws]
    x = to_dev_x(inputs.activations_bf16((m, k), seed=9))
    say("multi", m)
    ys = q4.linear_multi(x, pws)
    for w, pw, y in zip(ws, pws, ys):
        single = q4.linear(x, pw)
        assert torch.equal(y, single)
    xb = inputs.activations_bf16((m, k), seed=9)
    for w, y in zip(ws, ys):
        b = O.quantize(w)
        assert_within_bound(y.cpu().numpy(), O.linear(xb, b, w.shape[0], k), O.error_bound(xb, b, w.shape[0], k))


@pytest.mark.parametrize("m,k", [(1, 3072), (2, 4096), (1, 5120), (3, 384), (2, 9216), (40, 384)])
def test_eight_segments(m, k):
    """The most segments a launch takes (8, ragged and of different lengths):
    every segment's work tiles are found from the start tiles of the others,
    which the decode kernel receives as separate scalar arguments.  Each output
    against the oracle, and bit for bit against a separate launch where the
    two pick the same kernel (the decode sizes: the choice follows M and K)."""
    ns = (16, 40, 8, 136, 24, 1, 72, 33)
    ws = [inputs.weights_f32((n, k), seed=10, tags=(i, k)) for i, n in enumerate(ns)]
    pws = [device_weight_from_f32(w)[0] for w in ws]
    xb = inputs.activations_bf16((m, k), seed=10, tags=(m, k))
    x = to_dev_x(xb)
    say("eight segments", m, k, q4.linear_kernel(m, k, list(ns)))
    ys = q4.linear_multi(x, pws)
    for si, (w, pw, y) in enumerate(zip(ws, pws, ys)):
        b = O.quantize(w)
        assert_within_bound(y.cpu().numpy(), O.linear(xb, b, w.shape[0], k), O.error_bound(xb, b, w.shape[0], k),
                            f"M={m} K={k} segment {si}")
        if m <= 4:
            assert torch.equal(y, q4.linear(x, pw)), f"M={m} K={k} segment {si}: fused and separate differ"


@pytest.mark.parametrize("m", [1, 2, 32, 129])
def test_bitwise_deterministic(m):
    n, k = 512, 1024
    pw, _ = device_weight_from_f32(inputs.weights_f32((n, k), seed=3))
    x = to_dev_x(inputs.activations_bf16((m, k), seed=3))
    say("determinism", m)
    y0 = q4.linear(x, pw)
    for _ in range(3):
        assert torch.equal(q4.linear(x, pw), y0)


def test_m_zero_is_a_no_op():
    n, k = 32, 64
    pw, _ = device_weight_from_f32(inputs.weights_f32((n, k), seed=1))
    y = torch.full((0, n), 7.0, device=DEV)
    x = torch.empty((0, k), dtype=torch.bfloat16, device=DEV)
    q4.linear(x, pw, out=y)
    sentinel = torch.full((4, n), 7.0, device=DEV)
    assert q4.lib().q4_0_linear(x.data_ptr(), 0, pw.data.data_ptr(), n, k, sentinel.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0)


def test_binding_rejects_mismatched_arguments():
    n, k, m = 32, 64, 2
    pw, _ = device_weight_from_f32(inputs.weights_f32((n, k), seed=5))
    x = to_dev_x(inputs.activations_bf16((m, k), seed=5))
    say("binding validation")
    with pytest.raises(ValueError, match="outputs"):
        q4.linear_multi(x, [pw, pw], [torch.empty((m, n), device=DEV)])
    with pytest.raises(ValueError, match=r"\[M, K\]"):
        q4.linear_multi(x.view(-1), [pw])
    with pytest.raises(ValueError, match="CUDA/HIP"):
        q4.linear(x, pw, out=torch.empty((m, n)))
    torch.cuda.synchronize()


@pytest.mark.parametrize("m", [1, 3, 40, 130])
def test_non_finite_inputs_stay_non_finite_where_the_definition_is(m):
    """NaN / inf in x or in a scale d: an output is non-finite exactly where
    the dequantize-then-matmul definition's is, and every finite output is
    within the bound.  (With d = +-inf the kinds can differ: the kernel scales
    the block sum sum_k x (q - 8), the definition each weight (q - 8) d, so
    a zero x next to a nonzero code gives NaN there and +-inf here.)"""
    n, k = 80, 320
    blocks = O.quantize(inputs.weights_f32((n, k), seed=21)).copy()
    d_bits = blocks[:, :, :2].view(np.uint16)
    d_bits[3, 2, 0] = 0x7C00            # +inf
    d_bits[7, 0, 0] = 0x7E00            # NaN
    d_bits[9, 5, 0] = 0xFC00            # -inf, on a block of all codes 8 (w = 0 * inf)
    blocks[9, 5, 2:] = 0x88
    d_bits[60, 9, 0] = 0x7BFF           # 65504, finite
    xb = inputs.activations_bf16((m, k), seed=21).copy()
    if m >= 2:
        xb[0, 10] = 0x7FC0              # NaN in the first row
    if m >= 3:
        xb[m - 1, 100] = 0x7F80         # +inf in the last row
    pw = device_weight_from_blocks(blocks, n, k)
    say("non-finite", m)
    y = q4.linear(to_dev_x(xb), pw).cpu().numpy().astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = O.linear(xb, blocks, n, k)
        bound = O.error_bound(xb, blocks, n, k)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(y), fin)
    if m >= 2:
        assert np.all(np.isnan(y[0])), "a NaN in x poisons its whole output row"
    assert not fin.all() and fin.any()
    err = np.abs(y[fin] - ref[fin])
    assert np.all(err <= bound[fin]), float((err / bound[fin]).max())
