"""Bit-exact checks of the device format kernels against the oracle:
quantize (fp32 or bf16 -> GGUF), pack (GGUF -> tiled), unpack (inverse), dequant."""

import numpy as np
import pytest
import torch

from oracle import q4_0_oracle as O
import q4_weight_only_amd as q4
from q4_weight_only_amd import inputs

from gpu_helpers import DEV, canon_zero, device_weight_from_blocks, say, to_dev_bytes

pytestmark = pytest.mark.gpu


def _random_blocks(rng, n, k):
    blocks = rng.integers(0, 256, size=(n, k // 32, 18), dtype=np.uint8)
    d = (rng.standard_normal((n, k // 32)) * 0.01).astype(np.float16)
    blocks[:, :, 0:2] = d.view(np.uint8).reshape(n, k // 32, 2)
    return blocks


SHAPES = [(1, 32), (17, 96), (40, 384), (64, 1024), (130, 1280), (33, 4096)]


@pytest.mark.parametrize("n,k", SHAPES)
def test_quantize_matches_oracle_bytes(n, k):
    w = inputs.weights_f32((n, k), seed=11, tags=(n, k))
    say("quantize", n, k)
    got = q4.quantize(torch.from_numpy(w).to(DEV)).cpu().numpy()
    assert np.array_equal(got, O.quantize(w))


def test_quantize_structured_blocks():
    rows = []
    rows.append([-1.0, 0.5, 0.25, -0.25, 0.125] + [0.0] * 27)             # d = 0.125
    rows.append([0.1, -0.3, 0.8] + [0.0] * 29)                              # positive extreme
    rows.append([-2.0, 0.625, 0.875, -0.375, 0.125] + [0.0] * 27)          # half-even ties
    rows.append([-1.0, 1.0] + [0.0] * 30)                                   # clamp to 15
    rows.append([1.0, -1.0] + [0.0] * 30)
    rows.append([0.0] * 32)                                                 # zero block
    rows.append([-0.0] * 32)
    rows.append([1e-9, -5e-10] + [0.0] * 30)                                # d underflows
    rows.append([65504.0 * 8, 1.0] + [0.0] * 30)                            # d at fp16 max
    rows.append([3e-5 * (j - 16) for j in range(32)])                       # subnormal-ish d
    w = np.array(rows, dtype=np.float32)
    w = np.concatenate([w, -w], axis=0)
    w = np.tile(w, (1, 2))                                                  # K = 64
    say("quantize structured", w.shape)
    got = q4.quantize(torch.from_numpy(np.ascontiguousarray(w)).to(DEV)).cpu().numpy()
    assert np.array_equal(got, O.quantize(w))


@pytest.mark.parametrize("n,k", SHAPES)
def test_quantize_bf16_matches_oracle_bytes(n, k):
    """bf16 weights: the oracle's rule on the exactly widened values, and the
    same bytes as the fp32 quantizer given those widened values."""
    w = inputs.bf16_bits_from_f32(inputs.weights_f32((n, k), seed=12, tags=(n, k)))
    wt = torch.from_numpy(w.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    say("quantize bf16", n, k)
    got = q4.quantize(wt).cpu().numpy()
    assert np.array_equal(got, O.quantize_bf16(w))
    assert np.array_equal(got, q4.quantize(wt.float()).cpu().numpy())


@pytest.mark.parametrize("n,k", SHAPES)
def test_pack_matches_oracle_layout(n, k):
    rng = np.random.default_rng(n * 7 + k)
    blocks = _random_blocks(rng, n, k)
    say("pack", n, k)
    pw = device_weight_from_blocks(blocks, n, k)
    assert pw.data.numel() == O.packed_bytes(n, k)
    assert np.array_equal(pw.data.cpu().numpy(), O.pack(blocks, n, k))


@pytest.mark.parametrize("n,k", SHAPES)
def test_unpack_inverts_pack(n, k):
    rng = np.random.default_rng(n * 13 + k)
    blocks = rng.integers(0, 256, size=(n, k // 32, 18), dtype=np.uint8)   # any bytes, NaN d too
    say("unpack", n, k)
    pw = device_weight_from_blocks(blocks, n, k)
    assert np.array_equal(q4.unpack(pw).cpu().numpy(), blocks)


@pytest.mark.parametrize("n,k", SHAPES)
def test_dequant_matches_oracle_values(n, k):
    rng = np.random.default_rng(n * 17 + k)
    blocks = _random_blocks(rng, n, k)
    say("dequant", n, k)
    pw = device_weight_from_blocks(blocks, n, k)
    got = q4.dequant(pw).cpu().numpy()
    ref = O.dequantize(blocks, n, k)
    assert np.array_equal(canon_zero(got).view(np.uint32), canon_zero(ref).view(np.uint32))


def test_full_size_decode_matrix_bit_exact():
    """The 4096 x 3072 GEMV matrix: quantize, pack, dequant all bit-exact."""
    n, k = 4096, 3072
    w = inputs.weights_f32((n, k), seed=0, tags=(1, 0, 0, 0))
    say("full-size format", n, k)
    blocks = q4.quantize(torch.from_numpy(w).to(DEV))
    ref_blocks = O.quantize(w)
    assert np.array_equal(blocks.cpu().numpy(), ref_blocks)
    pw = q4.pack(blocks, n, k)
    assert np.array_equal(pw.data.cpu().numpy(), O.pack(ref_blocks, n, k))
    got = q4.dequant(pw).cpu().numpy()
    assert np.array_equal(canon_zero(got).view(np.uint32), canon_zero(O.dequantize(ref_blocks, n, k)).view(np.uint32))
