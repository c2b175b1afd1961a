"""The asymmetric 4-bit variant on the GPU (w = q * d + m per 32-weight
block): the device quantizer, pack and dequantization bit for bit against
the oracle, and q4_1_linear on every output element against the oracle's
fp64 result within its bound, for every kernel family the dispatch picks."""

import numpy as np
import pytest
import torch

from oracle import q4_0_oracle as O
import q4_weight_only_amd as q4
from q4_weight_only_amd import inputs

from gpu_helpers import DEV, assert_within_bound, say, to_dev_x

pytestmark = pytest.mark.gpu


def _weights(n, k, seed, tag=0):
    w = inputs.weights_f32((n, k), seed=seed, tags=(41, n, k, tag))
    blocks = q4.q41_quantize(torch.from_numpy(w).to(DEV))
    ref = O.q41_quantize(w)
    assert np.array_equal(blocks.cpu().numpy(), ref), "device quantizer differs from the oracle"
    return q4.q41_pack(blocks, n, k), ref


def test_quantizer_structured_blocks():
    """Constant blocks (d = 0), exact-scale blocks, ties, negative offsets."""
    w = np.zeros((4, 128), dtype=np.float32)
    w[0] = 0.3                                              # constant
    w[1, :32] = [1.0 + (j % 16) for j in range(32)]         # d = 1, m = 1
    w[1, 32:64] = 15.0
    w[1, 32], w[1, 33], w[1, 34] = 0.0, 2.5, 3.5            # ties in a d = 1, m = 0 block
    w[2] = np.linspace(-3.0, 1.0, 128, dtype=np.float32)
    w[3] = -np.abs(inputs.weights_f32((1, 128), seed=3, tags=(41,)))[0]
    got = q4.q41_quantize(torch.from_numpy(w).to(DEV)).cpu().numpy()
    assert np.array_equal(got, O.q41_quantize(w))


@pytest.mark.parametrize("n,k", [(40, 384), (16, 32), (300, 1280)])
def test_pack_and_dequant_bit_exact(n, k):
    pw, ref = _weights(n, k, 1)
    assert np.array_equal(pw.data.cpu().numpy(), O.q41_pack(ref, n, k))
    w = q4.q41_dequant(pw).cpu().numpy()
    want = O.q41_dequantize(ref, n, k).astype(np.float32)
    w[w == 0], want[want == 0] = 0.0, 0.0                   # -0 and +0 compare as values
    assert np.array_equal(w.view(np.uint32), want.view(np.uint32))


GRID = [(m, n, k) for m in (1, 2, 3, 4, 5, 17, 33, 64, 65, 130, 300) for n, k in ((64, 128), (40, 384), (200, 1280))]
GRID += [(1, 48, 9216), (2, 48, 12288), (4, 24, 4096), (3, 32, 20480), (1, 17, 32), (1505, 72, 640)]
# one and two rows at K 4097-9216: 12 K-slices, with stages past K (5152) and a partial last super-tile (9184)
GRID += [(1, 40, 5152), (2, 40, 5152), (1, 24, 9184), (2, 24, 9184)]


@pytest.mark.parametrize("m,n,k", GRID)
def test_linear_every_output(m, n, k):
    pw, ref = _weights(n, k, 2)
    xb = inputs.activations_bf16((m, k), seed=2, tags=(41, m, k))
    say("q41", m, n, k, q4.q41_linear_kernel(m, k, n))
    y = q4.q41_linear(to_dev_x(xb), pw).cpu().numpy()
    yr, bound = O.q41_linear_with_bound(xb, ref, n, k)
    assert_within_bound(y, yr, bound, f"q41 M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [1, 2048])
def test_linear_full_size_decoder_shape(m):
    """QKV at full size (3072 -> 6144): the decode and the prefill kernel."""
    n, k = 6144, 3072
    pw, ref = _weights(n, k, 4)
    xb = inputs.activations_bf16((m, k), seed=4, tags=(41, m))
    say("q41 full", m, q4.q41_linear_kernel(m, k, n))
    y = q4.q41_linear(to_dev_x(xb), pw).cpu().numpy()
    yr, bound = O.q41_linear_with_bound(xb, ref, n, k)
    ratio = assert_within_bound(y, yr, bound, f"q41 full M={m}")
    say(f"q41 full M={m}: max |err|/bound = {ratio:.3g}")


@pytest.mark.parametrize("m", [1, 130])
def test_linear_where_offset_cancels_scale(m):
    """Blocks with w = q d + m near zero (m = -q d at q = 8): both terms are
    large, their sum small; the bound is on the terms' magnitudes."""
    n, k = 32, 256
    rng = np.random.default_rng(9)
    d = (rng.uniform(0.5, 2.0, (n, k // 32))).astype(np.float16)
    mm = (-8.0 * d.astype(np.float32)).astype(np.float16)
    q = rng.integers(7, 10, size=(n, k), dtype=np.uint8)
    blocks = O.q41_encode(d, mm, q)
    pw = q4.q41_pack(torch.from_numpy(blocks.reshape(-1).copy()).to(DEV), n, k)
    xb = inputs.activations_bf16((m, k), seed=9, tags=(m,))
    y = q4.q41_linear(to_dev_x(xb), pw).cpu().numpy()
    yr, bound = O.q41_linear_with_bound(xb, blocks, n, k)
    assert_within_bound(y, yr, bound, f"q41 cancel M={m}")


@pytest.mark.parametrize("m", [1, 2, 300])
def test_deterministic(m):
    pw, _ = _weights(256, 1024, 5)
    x = to_dev_x(inputs.activations_bf16((m, 1024), seed=5, tags=(m,)))
    a = q4.q41_linear(x, pw).cpu().numpy()
    b = q4.q41_linear(x, pw).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_gemm_tile_shapes_agree_bitwise():
    """Above 4 rows every tile shape of the GEMM adds an output's block
    results, and the offsets' share of each 8-block window, in the same
    order, so a row computed in a 32-, 64- or 128-row tile (128 or 192
    columns wide) has the same bits.  K = 1280 has five windows, K = 1152 an
    odd step count (its last window has one step)."""
    for k, n in ((1280, 3072), (1152, 4096)):
        pw, _ = _weights(n, k, 6)
        x = to_dev_x(inputs.activations_bf16((2048, k), seed=6, tags=(41, k)))
        full = q4.q41_linear(x, pw)
        names = {q4.q41_linear_kernel(2048, k, n)}
        for m in (32, 64, 300):
            say("q41 tiles", k, m, q4.q41_linear_kernel(m, k, n))
            names.add(q4.q41_linear_kernel(m, k, n))
            part = q4.q41_linear(x[:m], pw)
            assert torch.equal(part.view(torch.int32), full[:m].view(torch.int32)), f"K={k} M={m}"
        assert len(names) >= 3, names


def _random_case(seed):
    rng = np.random.default_rng(4100 + seed)
    m = int(rng.choice([1, 2, 3, 4, 5, 17, 33, 64, 65, 129, 300, 1500]))
    k = 32 * int(rng.integers(1, 161))
    n = int(rng.integers(1, 1600))
    while m * n * k > 4e7:
        n = max(1, n // 2)
    return m, k, n


@pytest.mark.parametrize("seed", range(16))
def test_random_launch_within_bound(seed):
    """Seeded random shapes across the asymmetric dispatch (every kernel
    family, ragged N, any K that is a multiple of 32 up to 5120): every
    output element against the oracle's bound."""
    m, k, n = _random_case(seed)
    pw, ref = _weights(n, k, 7, seed)
    xb = inputs.activations_bf16((m, k), seed=7, tags=(41, seed, m, k))
    say("q41 random", seed, m, k, n, q4.q41_linear_kernel(m, k, n))
    y = q4.q41_linear(to_dev_x(xb), pw).cpu().numpy()
    yr, bound = O.q41_linear_with_bound(xb, ref, n, k)
    assert_within_bound(y, yr, bound, f"q41 random {seed}: M={m} N={n} K={k}")
