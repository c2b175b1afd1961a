"""Pins for the CPU oracle: closed forms, brute force, invariants, page sizes.

Each test checks the oracle against something other than itself, chosen so a
plausible slip (a swapped nibble half, a dropped -8, a transposed operand, an
unsigned absmax, round-half-up instead of half-even) fails at least one of
them; the mutation tests at the bottom plant such slips in copies of the
oracle functions and confirm the pins catch them.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import q4_0_oracle as O
from q4_weight_only_amd import inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_sizes():
    out = {}
    with open(os.path.join(GOLDEN, "sizes.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, val = line.split()
                out[key] = float(val)
    return out


def _block(d, q32):
    """One GGUF block from a float d and 32 codes, via explicit byte writes."""
    b = np.zeros(18, dtype=np.uint8)
    b[0:2] = np.array([d], dtype="<f2").view(np.uint8)
    for j in range(16):
        b[2 + j] = (q32[j] & 0xF) | ((q32[j + 16] & 0xF) << 4)
    return b


def _random_blocks(rng, n, k):
    blocks = rng.integers(0, 256, size=(n, k // 32, 18), dtype=np.uint8)
    # keep d finite: draw a finite fp16 for every block
    d = (rng.standard_normal((n, k // 32)) * 0.01).astype(np.float16)
    blocks[:, :, 0:2] = d.view(np.uint8).reshape(n, k // 32, 2)
    return blocks


# ------------------------------------------------------------- bf16 widening
def test_bf16_widening_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_rounding_used_for_inputs_is_round_to_nearest_even():
    # 1 + 2^-8 lies exactly halfway between bf16 neighbours 1 and 1 + 2^-7:
    # ties go to the even significand (1.0); 1 + 3*2^-8 goes up to 1 + 2^-6.
    x = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8)], dtype=np.float32)
    got = O.bf16_bits_to_f64(inputs.bf16_bits_from_f32(x))
    assert list(got) == [1.0, 1 + 2**-6, -1.0]


# ------------------------------------------------------------ GGUF bytes
def test_gguf_block_nibble_order_by_hand():
    # d = 1.0 is 0x3C00 little-endian; byte j = low nibble j%16, high nibble 15-j
    b = np.zeros(18, dtype=np.uint8)
    b[0], b[1] = 0x00, 0x3C
    for j in range(16):
        b[2 + j] = (j & 0xF) | ((15 - j) << 4)
    d, q = O.gguf_decode(b.reshape(1, 1, 18), 1, 32)
    assert d.view(np.uint16)[0, 0] == 0x3C00
    assert list(q[0, :16]) == list(range(16))
    assert list(q[0, 16:]) == [15 - j for j in range(16)]
    w = O.dequantize(b.reshape(1, 1, 18), 1, 32)
    assert list(w[0, :16]) == [j - 8.0 for j in range(16)]
    assert list(w[0, 16:]) == [7.0 - j for j in range(16)]


def test_gguf_roundtrip_random_bytes():
    rng = np.random.default_rng(1)
    blocks = rng.integers(0, 256, size=(7, 5, 18), dtype=np.uint8)
    d, q = O.gguf_decode(blocks, 7, 160)
    again = O.gguf_encode(d, q)
    assert np.array_equal(again, blocks)


def test_sizes_printed_on_the_pages():
    g = _golden_sizes()
    n, k = int(g["embedding_rows"]), int(g["embedding_cols"])
    assert O.gguf_bytes(n, k) == g["embedding_q4_mib"] * 2**20
    assert n * k * 4 == g["embedding_f32_gib"] * 2**30
    dim = int(g["decoder_dim"])
    per_layer = sum(k_ * sum(ns) for _, k_, ns in inputs.decoder_layer_ops())
    assert inputs.decoder_layer_ops()[0][2] == (4096, 1024, 1024)
    total = per_layer * int(g["decoder_layers"]) + n * k
    assert round(total / 1e9, 1) == g["decoder_params_billion"]
    assert dim == inputs.DECODER_DIM
    assert inputs.QKV_SEGMENTS[0] // int(g["query_heads"]) == inputs.QKV_SEGMENTS[1] // int(g["kv_heads"])


# -------------------------------------------------------------- dequantize
def test_dequant_fp32_product_is_exact_for_every_fp16_scale():
    dbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    d = dbits.view(np.float16)
    d = d[np.isfinite(d)]
    q = np.arange(16, dtype=np.float32) - 8
    prod32 = (q[:, None] * d.astype(np.float32)[None, :]).astype(np.float64)
    prod64 = q.astype(np.float64)[:, None] * d.astype(np.float64)[None, :]
    assert np.array_equal(prod32, prod64)


@pytest.mark.parametrize("e", [-24, -14, -3, 0, 5, 15])
def test_dequant_power_of_two_scales(e):
    rng = np.random.default_rng(e + 100)
    q = rng.integers(0, 16, size=(3, 64), dtype=np.uint8)
    for sign in (1.0, -1.0):
        d = np.full((3, 2), sign * 2.0**e, dtype=np.float16)
        w = O.dequantize(O.gguf_encode(d, q), 3, 64)
        assert np.array_equal(w.astype(np.float64), (q.astype(np.float64) - 8) * sign * 2.0**e)


# ------------------------------------------------------------------ linear
def _fraction_linear(x_bits, blocks, n, k):
    """Exact rational triple loop, straight from the definition."""
    x = [[Fraction(float(v)) for v in row] for row in O.bf16_bits_to_f64(x_bits).reshape(-1, k)]
    out = []
    for xm in x:
        row = []
        for j in range(n):
            acc = Fraction(0)
            for b in range(k // 32):
                blk = blocks[j, b]
                d = Fraction(float(blk[0:2].view("<f2")[0]))
                for e in range(32):
                    byte = int(blk[2 + (e % 16)])
                    q = (byte & 0xF) if e < 16 else (byte >> 4)
                    acc += xm[32 * b + e] * (q - 8) * d
            row.append(acc)
        out.append(row)
    return out


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (2, 3, 64), (3, 5, 96), (1, 4, 128)])
def test_linear_matches_exact_rational_triple_loop(m, n, k):
    rng = np.random.default_rng(m * 100 + n * 10 + k)
    blocks = _random_blocks(rng, n, k)
    x_bits = inputs.bf16_bits_from_f32(rng.standard_normal((m, k)).astype(np.float32))
    y = O.linear(x_bits, blocks, n, k)
    exact = _fraction_linear(x_bits, blocks, n, k)
    absw = np.abs(O.dequantize(blocks, n, k).astype(np.float64))
    absx = np.abs(O.bf16_bits_to_f64(x_bits).reshape(m, k))
    scale = absx @ absw.T
    for i in range(m):
        for j in range(n):
            # fp64 summation of k exact products: |error| <= k * 2^-53 * sum|x w|
            assert abs(Fraction(y[i, j]) - exact[i][j]) <= Fraction(k) * Fraction(2) ** -53 * Fraction(scale[i, j])


def test_all_codes_eight_give_exact_zero():
    rng = np.random.default_rng(3)
    n, k = 6, 256
    d = (rng.standard_normal((n, k // 32)) * 10).astype(np.float16)
    blocks = O.gguf_encode(d, np.full((n, k), 8, dtype=np.uint8))
    x_bits = inputs.activations_bf16((3, k), seed=3)
    y = O.linear(x_bits, blocks, n, k)
    assert np.all(y == 0.0)
    assert np.all(O.error_bound(x_bits, blocks, n, k) == 1e-6)


def test_single_nonzero_nibble_reproduces_product_exactly():
    rng = np.random.default_rng(4)
    n, k = 4, 128
    x_bits = inputs.activations_bf16((2, k), seed=4)
    x = O.bf16_bits_to_f64(x_bits)
    for trial in range(20):
        q = np.full((n, k), 8, dtype=np.uint8)
        row, col = rng.integers(0, n), rng.integers(0, k)
        code = rng.integers(0, 16)
        q[row, col] = code
        d = (rng.standard_normal((n, k // 32)) * 0.05).astype(np.float16)
        y = O.linear(x_bits, O.gguf_encode(d, q), n, k)
        expect = np.zeros((2, n))
        expect[:, row] = (float(code) - 8.0) * float(d[row, col // 32]) * x[:, col]
        assert np.array_equal(y, expect), trial


def test_doubling_every_scale_doubles_the_output_exactly():
    rng = np.random.default_rng(5)
    n, k = 9, 192
    q = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    d = (rng.standard_normal((n, k // 32)) * 0.01).astype(np.float16)
    x_bits = inputs.activations_bf16((2, k), seed=5)
    y1 = O.linear(x_bits, O.gguf_encode(d, q), n, k)
    y2 = O.linear(x_bits, O.gguf_encode((d.astype(np.float32) * 2).astype(np.float16), q), n, k)
    assert np.array_equal(y2, 2 * y1)


def test_output_row_follows_weight_row_not_activation_row():
    # A transposed operand would mix these up: row j of W only feeds column j.
    n, k = 3, 32
    q = np.full((n, k), 8, dtype=np.uint8)
    q[1, :] = 9                       # only row 1 is nonzero, w = +1 * d
    d = np.ones((n, 1), dtype=np.float16)
    x_bits = inputs.bf16_bits_from_f32(np.stack([np.ones(k), 2 * np.ones(k)]).astype(np.float32))
    y = O.linear(x_bits, O.gguf_encode(d, q), n, k)
    assert np.array_equal(y, np.array([[0.0, 32.0, 0.0], [0.0, 64.0, 0.0]]))


def _bound_blocks():
    """Two one-block rows built by hand, and two rows of x.

    W row 0: d = 0.5,   q_j = j % 16      -> w_0j = (j % 16 - 8) / 2
    W row 1: d = -0.25, q_j = 15 - j % 16 -> w_1j = (7 - j % 16) * -1/4
    x row 0: x_0j = (-1)^j (j + 1) / 4   (0.25, -0.5, ..., -8: bf16-exact)
    x row 1: x_1j = 1 for j < 16, -2 for j >= 16
    """
    k = 32
    rows = [_block(0.5, [j % 16 for j in range(k)]), _block(-0.25, [15 - j % 16 for j in range(k)])]
    blocks = np.stack(rows).reshape(2, 1, 18)
    x = np.array([[(-1) ** j * (j + 1) / 4 for j in range(k)],
                  [1.0 if j < 16 else -2.0 for j in range(k)]], dtype=np.float32)
    return inputs.bf16_bits_from_f32(x), blocks


def test_error_bound_by_hand():
    """1e-3 * sum_k |x_k w_k| + 1e-6 on hand-built blocks, worked on paper.

    With a_i = |i - 8| = 8,7,...,1,0,1,...,7 and b_i = |7 - i| = 7,...,1,0,1,...,8
    (i = 0..15; sum a = sum b = 64, sum (i+1) a_i = 512, sum (i+1) b_i = 576):
      sum |x_0 w_0| = 1/8  * (512 + (16*64 + 512))   = 256
      sum |x_0 w_1| = 1/16 * (576 + (16*64 + 576))   = 136
      sum |x_1 w_0| = 1/2 * 64 + 2 * 1/2 * 64       = 96
      sum |x_1 w_1| = 1/4 * 64 + 2 * 1/4 * 64       = 48
    The signed sums are -32, -17, 4, -2, and |x| against the signed w gives
    52, 59, -12, 6, so a bound built on either is caught here.
    """
    x_bits, blocks = _bound_blocks()
    got = O.error_bound(x_bits, blocks, 2, 32)
    want = np.array([[0.256001, 0.136001], [0.096001, 0.048001]])
    assert got.shape == (2, 2)
    assert np.allclose(got, want, rtol=1e-12, atol=0)


def test_error_bound_uses_each_blocks_own_scale():
    """One row of two blocks: w = +1 (d = 1, q = 9) on block 0 and
    w = (6 - 8) * -3 = +6 on block 1; x = 1 on block 0, 0.5 on block 1:
    sum |x w| = 32 * 1 + 32 * 0.5 * 6 = 128."""
    blocks = np.concatenate([_block(1.0, [9] * 32), _block(-3.0, [6] * 32)]).reshape(1, 2, 18)
    x_bits = inputs.bf16_bits_from_f32(np.array([[1.0] * 32 + [0.5] * 32], dtype=np.float32))
    assert O.error_bound(x_bits, blocks, 1, 64)[0, 0] == pytest.approx(0.128001, rel=1e-12)
    assert O.linear(x_bits, blocks, 1, 64)[0, 0] == 128.0


@pytest.mark.parametrize("m,n,k,chunk", [(3, 40, 256, 16), (1, 7, 96, 8192), (5, 33, 128, 1)])
def test_linear_with_bound_is_linear_and_error_bound(m, n, k, chunk):
    """The one-pass helper is exactly the two pinned functions."""
    rng = np.random.default_rng(m * 1000 + n)
    blocks = _random_blocks(rng, n, k)
    x_bits = inputs.activations_bf16((m, k), seed=n, tags=(k,))
    y, bound = O.linear_with_bound(x_bits, blocks, n, k, chunk_rows=chunk)
    assert np.array_equal(y, O.linear(x_bits, blocks, n, k, chunk_rows=chunk))
    assert np.array_equal(bound, O.error_bound(x_bits, blocks, n, k, chunk_rows=chunk))


def test_linear_rows_matches_full_linear():
    rng = np.random.default_rng(6)
    n, k = 40, 256
    blocks = _random_blocks(rng, n, k)
    x_bits = inputs.activations_bf16((3, k), seed=6)
    rows = np.array([0, 7, 39, 12])
    y, bound = O.linear_rows(x_bits, blocks, n, k, rows)
    assert np.array_equal(y, O.linear(x_bits, blocks, n, k)[:, rows])
    assert np.array_equal(bound, O.error_bound(x_bits, blocks, n, k)[:, rows])


# --------------------------------------------------------------- quantizer
def _q1(w32):
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, : len(w32)] = w32
    b = O.quantize(w)
    d, q = O.gguf_decode(b, 1, 32)
    return d.view(np.uint16)[0, 0], list(q[0])


def test_quantizer_negative_extreme_by_hand():
    # amax = -1.0 -> d = -1/-8 = 0.125 (fp16 0x3000); q = w/0.125 + 8
    dbits, q = _q1([-1.0, 0.5, 0.25, -0.25, 0.125])
    assert dbits == 0x3000
    assert q[:5] == [0, 12, 10, 6, 9] and q[5:] == [8] * 27


def test_quantizer_positive_extreme_by_hand():
    # amax = +0.8 -> d = fp16(-0.1) = -0.0999755859375 (0xAE66);
    # 0.8 / d = -8.0019... -> -8 -> q 0; -0.3 / d = 3.0007... -> 3 -> q 11
    dbits, q = _q1([0.1, -0.3, 0.8])
    assert dbits == 0xAE66
    assert q[:3] == [7, 11, 0]


def test_bf16_quantizer_by_hand():
    # bf16 0xBF80 = -1.0, 0x3F00 = 0.5, 0x3E80 = 0.25, 0xBE80 = -0.25,
    # 0x3E00 = 0.125: the negative-extreme block above, entered as bf16 bits
    bits = np.zeros((1, 32), dtype=np.uint16)
    bits[0, :5] = [0xBF80, 0x3F00, 0x3E80, 0xBE80, 0x3E00]
    blk = O.quantize_bf16(bits)
    d, q = O.gguf_decode(blk, 1, 32)
    assert d.view(np.uint16)[0, 0] == 0x3000
    assert list(q[0, :5]) == [0, 12, 10, 6, 9] and list(q[0, 5:]) == [8] * 27
    # bf16 0x3DCD = 0.10009765625: with the other values, the widened block
    # quantizes as its fp32 twin does (a byte-swapped or shifted widening fails)
    bits[0, 5] = 0x3DCD
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, :6] = [-1.0, 0.5, 0.25, -0.25, 0.125, 0.10009765625]
    assert np.array_equal(O.quantize_bf16(bits), O.quantize(w))


def test_quantizer_ties_round_half_to_even():
    # amax = -2 -> d = 0.25; 0.625/0.25 = 2.5 -> 2; 0.875/0.25 = 3.5 -> 4;
    # -0.375/0.25 = -1.5 -> -2; 0.125/0.25 = 0.5 -> 0
    dbits, q = _q1([-2.0, 0.625, 0.875, -0.375, 0.125])
    assert dbits == 0x3400
    assert q[:5] == [0, 10, 12, 6, 8]


def test_quantizer_clamps_opposite_extreme_and_takes_first_maximum():
    # |-1| = |1|: the first one is amax -> d = 0.125; 1/0.125 = 8 -> 16 -> 15
    dbits, q = _q1([-1.0, 1.0])
    assert dbits == 0x3000 and q[:2] == [0, 15]
    dbits, q = _q1([1.0, -1.0])        # amax = +1 -> d = -0.125 (0xB000)
    assert dbits == 0xB000 and q[:2] == [0, 15]


def test_quantizer_zero_and_underflowing_blocks():
    assert _q1([]) == (0x0000, [8] * 32)
    # amax/-8 underflows fp16 (smallest subnormal is 2^-24): stored as +0, q = 8
    assert _q1([1e-9, -5e-10]) == (0x0000, [8] * 32)
    w = np.zeros((1, 32), dtype=np.float32)
    assert np.array_equal(O.quantize(w)[0, 0], np.array([0, 0] + [0x88] * 16, dtype=np.uint8))


def test_quantizer_error_bounds_and_idempotence_on_seeded_weights():
    n, k = 64, 1024
    w = inputs.weights_f32((n, k), seed=7)
    b = O.quantize(w)
    d, q = O.gguf_decode(b, n, k)
    wq = O.dequantize(b, n, k).astype(np.float64)
    dabs = np.repeat(np.abs(d.astype(np.float64)), 32, axis=1)
    err = np.abs(w.astype(np.float64) - wq)
    clamped = q == 15
    tol = dabs * (1 + 2.0**-10)
    assert np.all(err[~clamped] <= tol[~clamped] / 2)
    assert np.all(err[clamped] <= tol[clamped])
    # the extreme element of each block maps to code 0
    wb = w.reshape(n, k // 32, 32)
    idx = np.argmax(np.abs(wb), axis=2)
    qb = q.reshape(n, k // 32, 32)
    assert np.all(np.take_along_axis(qb, idx[:, :, None], axis=2) == 0)
    # quantizing the dequantized weights gives back the same bytes
    assert np.array_equal(O.quantize(wq.astype(np.float32)), b)
    # value structure of the seeded workload
    assert 0.08 < np.mean(q == 8) < 0.16


# ----------------------------------------------------------- packed layout
def test_pack_places_a_single_nibble_where_the_layout_says():
    n, k = 40, 384                        # pads to Np=48, Kp=384
    np_, kp = O.padded_dims(n, k)
    assert (np_, kp) == (48, 384)
    KT = kp // 128
    for (row, col, code) in [(17, 6 * 32 + 13, 3), (0, 0, 15), (39, 383, 0), (31, 200, 12)]:
        q = np.full((n, k), 8, dtype=np.uint8)
        q[row, col] = code
        blocks = O.gguf_encode(np.ones((n, k // 32), dtype=np.float16), q)
        p = O.pack(blocks, n, k)
        nib = p[: np_ * kp // 2]
        rt, r = divmod(row, 16)
        b, e = divmod(col, 32)
        kt, i = divmod(b, 4)
        g, j = divmod(e, 8)
        off = (rt * KT + kt) * 1024 + g * 256 + r * 16 + i * 4 + j // 2
        expect = np.zeros_like(nib)
        expect[off] = (code ^ 8) << (4 * (j % 2))
        assert np.array_equal(nib, expect), (row, col)
        sc = p[np_ * kp // 2:].view(np.float16)
        live = np.zeros(np_ * kp // 32, dtype=bool)
        for rr in range(n):
            for bb in range(k // 32):
                rt2, r2 = divmod(rr, 16)
                kt2, i2 = divmod(bb, 4)
                live[(rt2 * KT + kt2) * 64 + r2 * 4 + i2] = True
        assert np.all(sc[live] == 1.0) and np.all(sc[~live] == 0.0)


def test_pack_size_and_padding():
    assert O.packed_bytes(4096, 3072) == O.gguf_bytes(4096, 3072)
    assert O.packed_bytes(20, 96) == 32 * 4 * 18
    rng = np.random.default_rng(8)
    blocks = _random_blocks(rng, 20, 96)
    p = O.pack(blocks, 20, 96)
    assert p.size == O.packed_bytes(20, 96)
    # every input nibble lands in exactly one place: popcount is preserved
    d, q = O.gguf_decode(blocks, 20, 96)
    nib = p[: 32 * 128 // 2]
    codes = np.concatenate([nib & 0xF, nib >> 4])
    hist = np.bincount(codes, minlength=16)
    expect = np.bincount((q ^ 8).ravel(), minlength=16)
    expect[0] += codes.size - q.size      # padding stores code 8 ^ 8 = 0
    assert np.array_equal(hist, expect)


# ---------------------------------------------------- planted mistakes
_ORIG_DECODE = O.gguf_decode
_ORIG_DEQUANT = O.dequantize


def _mutant_decode_swapped_halves(blocks, n, k):
    d, q = _ORIG_DECODE(blocks, n, k)
    q = q.reshape(n, k // 32, 32)
    q = np.concatenate([q[:, :, 16:], q[:, :, :16]], axis=2)
    return d, q.reshape(n, k)


def test_planted_mistakes_are_caught(monkeypatch):
    """Each mutant oracle must fail at least one of the pins above."""
    mutants = {
        "swapped nibble halves": ("gguf_decode", _mutant_decode_swapped_halves),
        "dropped -8": ("dequantize", lambda b, n, k: _ORIG_DECODE(b, n, k)[1].astype(np.float32)
                       * np.repeat(_ORIG_DECODE(b, n, k)[0].astype(np.float32), 32, axis=1)),
        "reversed output columns": ("linear", lambda x, b, n, k, chunk_rows=8192:
                                    (O.bf16_bits_to_f64(x).reshape(-1, k)
                                     @ _ORIG_DEQUANT(b, n, k).astype(np.float64).T)[:, ::-1].copy()),
    }
    checks = [
        test_gguf_block_nibble_order_by_hand,
        test_single_nonzero_nibble_reproduces_product_exactly,
        test_output_row_follows_weight_row_not_activation_row,
    ]
    for name, (attr, fn) in mutants.items():
        with monkeypatch.context() as mp:
            mp.setattr(O, attr, fn)
            failed = 0
            for chk in checks:
                try:
                    chk()
                except AssertionError:
                    failed += 1
            assert failed > 0, name


_ORIG_BOUND = O.error_bound


def _bound_mutant(kind):
    def fn(x_bits, blocks, n, k, chunk_rows=8192):
        x = O.bf16_bits_to_f64(x_bits).reshape(-1, k)
        w = _ORIG_DEQUANT(blocks, n, k).astype(np.float64)
        if kind == "factor 1e-2":
            return 1e-2 * (np.abs(x) @ np.abs(w).T) + 1e-6
        if kind == "signed sum":
            return 1e-3 * (x @ w.T) + 1e-6
        return 1e-3 * (np.abs(x) @ w.T) + 1e-6          # |x| without |w|
    return fn


def test_planted_error_bound_mistakes_are_caught(monkeypatch):
    """A wrong factor, the signed sum x w^T, or |x| against the signed w must
    each fail the hand-worked bound pins."""
    for kind in ("factor 1e-2", "signed sum", "abs x only"):
        with monkeypatch.context() as mp:
            mp.setattr(O, "error_bound", _bound_mutant(kind))
            failed = 0
            for chk in (test_error_bound_by_hand, test_error_bound_uses_each_blocks_own_scale):
                try:
                    chk()
                except AssertionError:
                    failed += 1
            assert failed > 0, kind
    assert O.error_bound is _ORIG_BOUND


def test_planted_quantizer_mistakes_are_caught():
    w = inputs.weights_f32((8, 256), seed=9)
    good = O.quantize(w)

    def unsigned_absmax(wm):
        wb = wm.reshape(8, 8, 32)
        amax = np.max(np.abs(wb), axis=2)
        d16 = (amax / np.float32(-8)).astype(np.float16)
        r = np.clip(np.rint(wb / d16.astype(np.float32)[:, :, None]) + 8, 0, 15)
        return O.gguf_encode(d16, r.astype(np.uint8).reshape(8, 256))

    def half_up(wm):
        wb = wm.reshape(8, 8, 32)
        idx = np.argmax(np.abs(wb), axis=2)
        amax = np.take_along_axis(wb, idx[:, :, None], axis=2)[:, :, 0]
        d16 = (amax / np.float32(-8)).astype(np.float16)
        r = np.clip(np.floor(wb / d16.astype(np.float32)[:, :, None] + np.float32(0.5)) + 8, 0, 15)
        return O.gguf_encode(d16, r.astype(np.uint8).reshape(8, 256))

    assert not np.array_equal(unsigned_absmax(w), good)
    tie = np.zeros((8, 256), dtype=np.float32)
    tie[:, 0], tie[:, 1] = -2.0, 0.625
    assert not np.array_equal(half_up(tie), O.quantize(tie))


# ---------------------------------------------------------------- embedding
def test_embed_rows_by_hand():
    """Three-row table with hand-built blocks: each looked-up row is (q-8)*d of
    that row, in the requested order, duplicates repeated, bad ids NaN."""
    k = 64
    rows = []
    for r, d in enumerate((0.5, -2.0, 0.125)):
        q = [(r * 5 + e) % 16 for e in range(k)]
        rows.append(np.concatenate([_block(d, q[:32]), _block(d * 3, q[32:])]))
    table = np.stack(rows)
    got = O.embed(table, 3, k, [2, 0, 2, -1, 3, 1])
    assert got.shape == (6, k) and got.dtype == np.float32
    for t, r in enumerate([2, 0, 2, None, None, 1]):
        if r is None:
            assert np.all(np.isnan(got[t]))
            continue
        d = (0.5, -2.0, 0.125)[r]
        want = [((r * 5 + e) % 16 - 8) * (d if e < 32 else d * 3) for e in range(k)]
        assert got[t].tolist() == want


def test_embed_matches_full_dequant():
    w = inputs.weights_f32((40, 96), seed=9, tags=(9,))
    blocks = O.quantize(w)
    ids = np.array([39, 0, 17, 17, 5])
    full = O.dequantize(blocks, 40, 96)
    assert np.array_equal(O.embed(blocks, 40, 96, ids), full[ids])
    assert O.embed(blocks, 40, 96, []).shape == (0, 96)
