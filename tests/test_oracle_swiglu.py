"""Pins for the oracle's SwiGLU step (h = silu(x Wg^T) * (x Wu^T)).

The pages name SwiGLU right after the Q4 matmul (Rust fork, "Architecture
Summary") without defining it; the oracle takes the usual gated-MLP reading.
These tests tie its silu to values that follow from the definition by hand
(not by re-evaluating the same formula), to the odd-part identity
silu(t) - silu(-t) = t, to brute force with Python's math.exp on tiny shapes,
and check that the tolerance swiglu_bound really covers every h reachable from
g and u inside their own linear bounds.  A planted sign slip and a swapped
gate/up are shown to fail.
"""

import math

import numpy as np
import pytest

from oracle import q4_0_oracle as O
from q4_weight_only_amd import inputs


def _block(d, q32):
    b = np.zeros(18, dtype=np.uint8)
    b[0:2] = np.array([d], dtype="<f2").view(np.uint8)
    q = np.asarray(q32, dtype=np.uint8)
    for j in range(16):
        b[2 + j] = (q[j] & 0xF) | ((q[j + 16] & 0xF) << 4)
    return b


def _bf16_bits(vals):
    f = np.asarray(vals, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)   # exact for these values


def test_silu_closed_forms():
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4, so silu(+-ln 3) = +-ln3 * (3/4 | 1/4)
    l3 = math.log(3.0)
    got = O.silu([0.0, l3, -l3, math.log(2.0)])
    assert got[0] == 0.0
    assert got[1] == pytest.approx(0.75 * l3, rel=1e-15)
    assert got[2] == pytest.approx(-0.25 * l3, rel=1e-15)
    assert got[3] == pytest.approx(math.log(2.0) * 2.0 / 3.0, rel=1e-15)   # sigmoid(ln 2) = 2/3


def test_silu_odd_part_and_limits():
    t = np.linspace(-30.0, 30.0, 1201)
    # sigmoid(t) + sigmoid(-t) = 1  =>  silu(t) - silu(-t) = t
    assert np.allclose(O.silu(t) - O.silu(-t), t, rtol=0, atol=1e-13)
    big = np.array([50.0, 700.0, 1e300])
    assert np.array_equal(O.silu(big), big)                  # e^-t below half an ulp of 1
    neg = O.silu(np.array([-50.0, -700.0, -1e300]))
    assert np.all(neg <= 0) and np.all(np.abs(neg) < 1e-19)
    assert np.all(np.isfinite(O.silu(np.array([-1e308, 1e308]))))


def test_silu_slope_bound():
    t = np.linspace(-20, 20, 400001)
    s = O.silu(t)
    slope = np.abs(np.diff(s) / np.diff(t))
    assert slope.max() <= O.SILU_SLOPE_MAX
    assert slope.max() > 1.09          # the bound is tight, not loose


def test_swiglu_hand_values_and_asymmetry():
    # K = 32, N = 1: gate row has one code q=10 (w = 2 d), up row one code q=11 (w = 3 d)
    k, n = 32, 1
    qg = [8] * 32
    qg[5] = 10
    qu = [8] * 32
    qu[5] = 11
    gate = _block(1.0, qg)[None, None, :]
    up = _block(1.0, qu)[None, None, :]
    x = np.zeros(k, dtype=np.float32)
    x[5] = 1.0
    xb = _bf16_bits(x)[None, :]
    h = O.swiglu(xb, gate, up, n, k)
    assert h.shape == (1, 1)
    assert h[0, 0] == pytest.approx(3.0 * 2.0 / (1.0 + math.exp(-2.0)), rel=1e-15)
    swapped = O.swiglu(xb, up, gate, n, k)
    assert swapped[0, 0] == pytest.approx(2.0 * 3.0 / (1.0 + math.exp(-3.0)), rel=1e-15)
    assert abs(h[0, 0] - swapped[0, 0]) > 0.1


def test_swiglu_zero_gate_or_up():
    rng = np.random.default_rng(3)
    n, k = 5, 64
    w = rng.normal(0, 0.02, (n, k)).astype(np.float32)
    blocks = O.quantize(w)
    zero = O.gguf_encode(np.ones((n, k // 32), dtype=np.float16), np.full((n, k), 8, dtype=np.uint8))
    x = inputs.activations_bf16((3, k), seed=4, tags=(1,))
    assert np.all(O.swiglu(x, zero, blocks, n, k) == 0.0)      # silu(0) = 0
    assert np.all(O.swiglu(x, blocks, zero, n, k) == 0.0)


def test_swiglu_brute_force_tiny():
    rng = np.random.default_rng(11)
    m, n, k = 2, 3, 64
    gq = rng.integers(0, 16, (n, k))
    uq = rng.integers(0, 16, (n, k))
    gd = rng.uniform(0.01, 0.1, (n, k // 32)).astype(np.float16)
    ud = rng.uniform(0.01, 0.1, (n, k // 32)).astype(np.float16)
    gate = O.gguf_encode(gd, gq.astype(np.uint8))
    up = O.gguf_encode(ud, uq.astype(np.uint8))
    xv = rng.normal(0, 1, (m, k)).astype(np.float32)
    xb = (xv.view(np.uint32) >> 16).astype(np.uint16)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    h = O.swiglu(xb, gate, up, n, k)
    for i in range(m):
        for j in range(n):
            g = sum(xf[i, t] * (int(gq[j, t]) - 8) * float(gd[j, t // 32]) for t in range(k))
            u = sum(xf[i, t] * (int(uq[j, t]) - 8) * float(ud[j, t // 32]) for t in range(k))
            want = g / (1.0 + math.exp(-g)) * u
            assert h[i, j] == pytest.approx(want, rel=1e-12, abs=1e-15)


def test_swiglu_bound_covers_perturbations():
    m, n, k = 4, 24, 256
    gw = inputs.weights_f32((n, k), seed=5, tags=(1,))
    uw = inputs.weights_f32((n, k), seed=5, tags=(2,))
    gb, ub = O.quantize(gw), O.quantize(uw)
    x = inputs.activations_bf16((m, k), seed=5, tags=(3,))
    g, u = O.linear(x, gb, n, k), O.linear(x, ub, n, k)
    bg, bu = O.error_bound(x, gb, n, k), O.error_bound(x, ub, n, k)
    h = O.silu(g) * u
    tol = O.swiglu_bound(x, gb, ub, n, k)
    rng = np.random.default_rng(7)
    worst = 0.0
    for _ in range(200):
        sg = rng.choice([-1.0, 1.0], g.shape) * rng.uniform(0.0, 1.0, g.shape) ** 0.1
        su = rng.choice([-1.0, 1.0], u.shape) * rng.uniform(0.0, 1.0, u.shape) ** 0.1
        hp = O.silu(g + sg * bg) * (u + su * bu)
        worst = max(worst, float(np.max(np.abs(hp - h) / tol)))
    assert worst <= 1.0
    assert worst > 0.3          # not vacuous


def test_swiglu_bound_by_hand():
    """Two outputs, K = 32, d = 1, x = (2, 1, 0, ..., 0), worked on paper:

    column 0: gate w = (+1, -2) -> g = 0, sum|x w| = 4 -> bg = 0.004001;
              up w_0 = +3      -> u = 6, sum|x w| = 6 -> bu = 0.006001;
              silu(0) = 0, so the bound is 1.1 * bg * (|u| + bu).
    column 1: gate w_0 = +1 -> g = 2, bg = 0.002001;
              up w_1 = +2   -> u = 2, bu = 0.002001;
              bound 1.1 bg (|u| + bu) + silu(2) bu + 1e-5 |silu(2) u|.
    """
    k, n = 32, 2
    qg0, qu0, qg1, qu1 = [8] * 32, [8] * 32, [8] * 32, [8] * 32
    qg0[0], qg0[1], qu0[0] = 9, 6, 11
    qg1[0], qu1[1] = 9, 10
    gate = np.stack([_block(1.0, qg0), _block(1.0, qg1)]).reshape(n, 1, 18)
    up = np.stack([_block(1.0, qu0), _block(1.0, qu1)]).reshape(n, 1, 18)
    x = np.zeros(k, dtype=np.float32)
    x[0], x[1] = 2.0, 1.0
    xb = _bf16_bits(x)[None, :]
    s2 = 2.0 / (1.0 + math.exp(-2.0))
    want = [1.1 * 0.004001 * (6 + 0.006001),
            1.1 * 0.002001 * (2 + 0.002001) + s2 * 0.002001 + 1e-5 * s2 * 2]
    got = O.swiglu_bound(xb, gate, up, n, k)
    assert got.shape == (1, 2)
    assert got[0].tolist() == pytest.approx(want, rel=1e-12)
    assert want[0] == pytest.approx(0.0264330110011, rel=1e-12)


def test_planted_sign_slip_is_caught(monkeypatch):
    orig = O.silu

    def wrong(t):                       # t * sigmoid(-t): a plausible sign slip
        return -orig(-np.asarray(t, dtype=np.float64))

    monkeypatch.setattr(O, "silu", wrong)
    with pytest.raises(AssertionError):
        test_silu_closed_forms()
    with pytest.raises(AssertionError):
        test_swiglu_hand_values_and_asymmetry()


def test_swiglu_bound_catches_a_wrong_linear_bound(monkeypatch):
    """swiglu_bound is built on error_bound; a tenfold error_bound must fail
    the hand-worked SwiGLU bound as well."""
    orig = O.error_bound
    monkeypatch.setattr(O, "error_bound", lambda *a, **kw: 10.0 * orig(*a, **kw))
    with pytest.raises(AssertionError):
        test_swiglu_bound_by_hand()
