"""Pins for the oracle's asymmetric 4-bit variant (w = q * d + m, 32-weight
blocks of an fp16 scale d and an fp16 offset m).

The TTS card names group-wise asymmetric int4 without its group size, zero
point or layout; the oracle takes the GGUF asymmetric block as the reading.
These tests tie the block layout, the quantizer and the product to values
worked out by hand, to exact rational brute force, and to the packed layout's
index rule; planted mistakes (a flipped offset sign, min and max swapped, a
bound on |w| instead of |q d| + |m|) are shown to fail them.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import q4_0_oracle as O
from q4_weight_only_amd import inputs


def _f16_bits(v):
    return int(np.array([v], dtype=np.float16).view(np.uint16)[0])


def _hand_block(d_bits, m_bits, q32):
    b = np.zeros(20, dtype=np.uint8)
    b[0], b[1] = d_bits & 0xFF, d_bits >> 8
    b[2], b[3] = m_bits & 0xFF, m_bits >> 8
    for j in range(16):
        b[4 + j] = q32[j] | (q32[j + 16] << 4)
    return b


def test_quantize_block_with_exact_scale_by_hand():
    # w = 1, 2, ..., 16 twice: min 1, max 16, (16 - 1) / 15 = 1 -> d = 1.0 (0x3C00),
    # m = 1.0 (0x3C00), q_j = w_j - 1 = j % 16 exactly
    w = np.array([[1.0 + (j % 16) for j in range(32)]], dtype=np.float32)
    got = O.q41_quantize(w).reshape(20)
    want = _hand_block(0x3C00, 0x3C00, [j % 16 for j in range(32)])
    assert got.tolist() == want.tolist()
    assert O.q41_dequantize(got.reshape(1, 1, 20), 1, 32)[0].tolist() == [1.0 + (j % 16) for j in range(32)]


def test_quantize_negative_offset_by_hand():
    # w = -2 + 0.5 (j % 16): min -2 (0xC000), max 5.5, 7.5 / 15 = 0.5 (0x3800)
    w = np.array([[-2.0 + 0.5 * (j % 16) for j in range(32)]], dtype=np.float32)
    got = O.q41_quantize(w).reshape(20)
    assert got.tolist() == _hand_block(0x3800, 0xC000, [j % 16 for j in range(32)]).tolist()


def test_quantize_ties_go_to_even_and_constant_blocks():
    # min 0, max 15 -> d = 1, m = 0; 2.5 -> 2 and 3.5 -> 4 (half to even), 14.5 -> 14
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0], w[0, 1], w[0, 2], w[0, 3] = 15.0, 2.5, 3.5, 14.5
    d, m, q = O.q41_decode(O.q41_quantize(w), 1, 32)
    assert d.view(np.uint16)[0, 0] == 0x3C00 and m.view(np.uint16)[0, 0] == 0
    assert q[0, :4].tolist() == [15, 2, 4, 14]
    # a constant block: d = 0, q = 0, m = fp16(0.3) = 0x34CD
    c = O.q41_quantize(np.full((1, 32), 0.3, dtype=np.float32)).reshape(20)
    assert c.tolist() == _hand_block(0x0000, 0x34CD, [0] * 32).tolist()


def test_quantize_error_bound_on_seeded_weights():
    w = inputs.weights_f32((64, 256), seed=17, tags=(41,))
    blocks = O.q41_quantize(w)
    d, m, _ = O.q41_decode(blocks, 64, 256)
    err = np.abs(O.q41_dequantize(blocks, 64, 256) - w.astype(np.float64))
    # within half a step, plus the fp16 rounding of m and of 15 d
    step = np.repeat(np.abs(d.astype(np.float64)), 32, axis=1)
    slack = np.repeat(np.abs(m.astype(np.float64)), 32, axis=1) * 2.0**-10 + 15 * step * 2.0**-10
    assert np.all(err <= step / 2 + slack + 1e-12)


def test_linear_and_bound_by_hand():
    """Block A: d = 1, m = 1, q_j = j % 16 (w_j = 1 + j % 16).  Block B:
    d = 1, m = -8 (w_j = j % 16 - 8).  x = all ones.
      y_A = 2 * sum_{i<16} (1 + i) = 2 * 136 = 272,
      bound_A = 1e-3 * 2 * sum (i + 1) + 1e-6 = 0.272001;
      y_B = 2 * sum (i - 8) = 2 * (120 - 128) = -16,
      bound_B = 1e-3 * 2 * sum (i + 8) + 1e-6 = 0.496001
    (the magnitudes of both terms; sum |w| would give 0.128001)."""
    qs = [j % 16 for j in range(32)]
    blocks = np.stack([_hand_block(0x3C00, 0x3C00, qs), _hand_block(0x3C00, _f16_bits(-8.0), qs)]).reshape(2, 1, 20)
    x = inputs.bf16_bits_from_f32(np.ones((1, 32), dtype=np.float32))
    y, bound = O.q41_linear_with_bound(x, blocks, 2, 32)
    assert y[0].tolist() == [272.0, -16.0]
    assert bound[0].tolist() == pytest.approx([0.272001, 0.496001], rel=1e-12)


@pytest.mark.parametrize("m,n,k", [(1, 2, 32), (2, 3, 64), (3, 2, 96)])
def test_linear_matches_exact_rational_triple_loop(m, n, k):
    rng = np.random.default_rng(m * 100 + n * 10 + k)
    d = (rng.standard_normal((n, k // 32)) * 0.01).astype(np.float16)
    mm = (rng.standard_normal((n, k // 32)) * 0.05).astype(np.float16)
    q = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    blocks = O.q41_encode(d, mm, q)
    xb = inputs.bf16_bits_from_f32(rng.standard_normal((m, k)).astype(np.float32))
    y, _ = O.q41_linear_with_bound(xb, blocks, n, k)
    xf = O.bf16_bits_to_f64(xb).reshape(m, k)
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(float(xf[i, t])) * (int(q[j, t]) * Fraction(float(d[j, t // 32]))
                                                      + Fraction(float(mm[j, t // 32]))) for t in range(k))
            scale = sum(abs(float(xf[i, t])) * (abs(int(q[j, t]) * float(d[j, t // 32])) + abs(float(mm[j, t // 32])))
                        for t in range(k))
            assert abs(Fraction(y[i, j]) - exact) <= Fraction(k) * Fraction(2) ** -52 * Fraction(scale)


def kt_n_of(k):
    return -(-k // 128)


def test_pack_places_offset_and_keeps_the_q4_0_planes():
    n, k = 20, 160                      # pads to 32 rows and 256 columns
    rng = np.random.default_rng(5)
    d = (rng.standard_normal((n, k // 32)) * 0.01).astype(np.float16)
    mm = np.zeros((n, k // 32), dtype=np.float16)
    mm[17, 4] = 3.0                     # row 17 = tile 1, r = 1; block 4 = kt 1, i = 0
    q = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    blocks = O.q41_encode(d, mm, q)
    packed = O.q41_pack(blocks, n, k)
    assert packed.size == O.q41_packed_bytes(n, k) == 32 * (256 // 32) * 20
    front = O.pack(O.gguf_encode(d, q ^ 8), n, k)          # codes q themselves in the nibble slots
    assert np.array_equal(packed[:front.size], front)
    # code q of row 5, element 37 (block 1 = kt 0, i = 1; g = 0, j = 5) by the layout rule
    byte = packed[(0 * kt_n_of(k) + 0) * 1024 + 0 * 256 + 5 * 16 + 1 * 4 + 5 // 2]
    assert (byte >> 4) == q[5, 37]
    off = packed[front.size:].view(np.float16)
    kt_n = 2
    idx = (1 * kt_n + 1) * 64 + 1 * 4 + 0
    assert off[idx] == 3.0 and np.count_nonzero(off) == 1


def test_planted_mistakes_are_caught(monkeypatch):
    orig_decode, orig_quant = O.q41_decode, O.q41_quantize

    def flipped(blocks, n, k):                  # m subtracted instead of added
        d, m, q = orig_decode(blocks, n, k)
        return d, -m, q
    monkeypatch.setattr(O, "q41_decode", flipped)
    with pytest.raises(AssertionError):
        test_quantize_block_with_exact_scale_by_hand()
    monkeypatch.setattr(O, "q41_decode", orig_decode)

    def swapped(w):                             # max taken as the offset
        w32 = np.ascontiguousarray(w, dtype=np.float32)
        n, k = w32.shape
        wb = w32.reshape(n, k // 32, 32)
        mn, mx = wb.min(axis=2), wb.max(axis=2)
        d16 = ((mx - mn) / np.float32(15)).astype(np.float16)
        m16 = mx.astype(np.float16)
        r = np.clip(np.rint((wb - m16.astype(np.float32)[:, :, None]) / d16.astype(np.float32)[:, :, None]), 0, 15)
        return O.q41_encode(d16, m16, r.astype(np.uint8).reshape(n, k))
    monkeypatch.setattr(O, "q41_quantize", swapped)
    with pytest.raises(AssertionError):
        test_quantize_block_with_exact_scale_by_hand()
    monkeypatch.setattr(O, "q41_quantize", orig_quant)

    orig_lb = O.q41_linear_with_bound

    def abs_w_bound(xb, blocks, n, k, chunk_rows=8192):   # sum |x w| instead of the two terms
        y, _ = orig_lb(xb, blocks, n, k, chunk_rows)
        w = O.q41_dequantize(blocks, n, k)
        return y, 1e-3 * (np.abs(O.bf16_bits_to_f64(xb).reshape(-1, k)) @ np.abs(w).T) + 1e-6
    monkeypatch.setattr(O, "q41_linear_with_bound", abs_w_bound)
    with pytest.raises(AssertionError):
        test_linear_and_bound_by_hand()
