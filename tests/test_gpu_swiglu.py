"""Parity of the fused gate/up + SwiGLU launch (q4_0_linear_swiglu) with the
oracle's silu(x Wg^T) * (x Wu^T), within the stated bound, for every kernel
configuration (decode-sized M through prefill M, ragged N and K), at the
decoder's full gate/up shape (sampled rows), on saturating gate values, and
against silu of the library's own unfused gate and up outputs."""

import numpy as np
import pytest
import torch

from oracle import q4_0_oracle as O
import q4_weight_only_amd as q4
from q4_weight_only_amd import inputs

from gpu_helpers import DEV, assert_within_bound, device_weight_from_f32, sample_rows, say, to_dev_x

pytestmark = pytest.mark.gpu

MS = [1, 2, 3, 5, 16, 17, 32, 33, 64, 100, 300, 2100]
NKS = [(16, 32), (40, 96), (200, 384), (1040, 1280), (96, 3072)]


def _pair(n, k, seed):
    gw = inputs.weights_f32((n, k), seed=seed, tags=(n, k, 1))
    uw = inputs.weights_f32((n, k), seed=seed, tags=(n, k, 2))
    return gw, uw


@pytest.mark.parametrize("m", MS)
@pytest.mark.parametrize("n,k", NKS)
def test_swiglu_parity_grid(m, n, k):
    gw, uw = _pair(n, k, 31)
    x = inputs.activations_bf16((m, k), seed=31, tags=(m, k))
    gpw, gblk = device_weight_from_f32(gw)
    upw, ublk = device_weight_from_f32(uw)
    gb, ub = gblk.cpu().numpy(), ublk.cpu().numpy()
    assert np.array_equal(gb, O.quantize(gw)) and np.array_equal(ub, O.quantize(uw))
    say("swiglu", m, n, k, q4.linear_swiglu_kernel(m, k))
    h = q4.linear_swiglu(to_dev_x(x), gpw, upw).cpu().numpy()
    assert_within_bound(h, O.swiglu(x, gb, ub, n, k), O.swiglu_bound(x, gb, ub, n, k), f"swiglu M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [1, 2, 4])
@pytest.mark.parametrize("n,k", [(40, 5152), (24, 9184), (16, 9248)])
def test_swiglu_long_rows(m, n, k):
    """Up to four rows on long rows: the gated 12-K-slice launch at one and two
    rows (dead and partial stages), the gated K-split kernel at four rows and
    beyond K = 9216."""
    test_swiglu_parity_grid(m, n, k)


@pytest.mark.parametrize("m", [1, 2, 16, 32, 100, 2048])
def test_swiglu_equals_silu_of_unfused_outputs(m):
    """The fused launch forms g and u as q4_0_linear_multi does, except that at
    some M it splits K over a different number of waves, so the fp32 partial
    sums may be added in another order.  h must equal fp32 silu(g) * u of the
    unfused outputs up to that reordering: each of g, u is a sum of at most K
    rounded additions, so two orders differ by at most 2 K 2^-24 sum|x w|,
    carried through silu (slope <= 1.1) and the product; 4e-6 |h| covers the
    exponential and the division."""
    n, k = 520, 1024
    gw, uw = _pair(n, k, 32)
    xb = inputs.activations_bf16((m, k), seed=32, tags=(m,))
    x = to_dev_x(xb)
    gpw, gblk = device_weight_from_f32(gw)
    upw, ublk = device_weight_from_f32(uw)
    say("swiglu vs unfused", m)
    h = q4.linear_swiglu(x, gpw, upw).cpu().numpy().astype(np.float64)
    g, u = (t.cpu().numpy() for t in q4.linear_multi(x, [gpw, upw]))
    with np.errstate(over="ignore"):
        want = ((g / (np.float32(1) + np.exp(-g))) * u).astype(np.float64)
    ax = np.abs(O.bf16_bits_to_f64(xb))
    sg = ax @ np.abs(O.dequantize(gblk.cpu().numpy(), n, k)).T
    su = ax @ np.abs(O.dequantize(ublk.cpu().numpy(), n, k)).T
    dg, du = 2 * k * 2.0**-24 * sg, 2 * k * 2.0**-24 * su
    g64, u64 = g.astype(np.float64), u.astype(np.float64)
    tol = O.SILU_SLOPE_MAX * dg * (np.abs(u64) + du) + np.abs(O.silu(g64)) * du + 4e-6 * np.abs(want) + 1e-30
    err = np.abs(h - want)
    assert np.all(err <= tol), f"M={m}: worst err/tol {np.max(err / tol):.3g}"


@pytest.mark.parametrize("m", [1, 2, 40, 300])
def test_swiglu_saturating_gate(m):
    """Gate outputs far past the knee (g = 112 or -128): silu -> g, or -> -0
    once e^128 overflows fp32, never NaN."""
    n, k = 64, 256
    gq = np.full((n, k), 8, dtype=np.uint8)
    gq[: n // 2, :] = 15          # w = 7 d
    gq[n // 2:, :] = 0            # w = -8 d
    d = np.full((n, k // 32), 0.25, dtype=np.float16)   # g = 256 * 0.25 * (7 | -8) * 0.25 = 112 | -128
    gate = O.gguf_encode(d, gq)
    uw = inputs.weights_f32((n, k), seed=33, tags=(3,))
    ub = O.quantize(uw)
    xv = np.full((m, k), 0.25, dtype=np.float32)
    x = inputs.bf16_bits_from_f32(xv)
    gpw = q4.pack(torch.from_numpy(gate.reshape(-1).copy()).to(DEV), n, k)
    upw = q4.pack(torch.from_numpy(ub.reshape(-1).copy()).to(DEV), n, k)
    say("swiglu saturating", m)
    h = q4.linear_swiglu(to_dev_x(x), gpw, upw).cpu().numpy()
    assert np.all(np.isfinite(h))
    assert_within_bound(h, O.swiglu(x, gate, ub, n, k), O.swiglu_bound(x, gate, ub, n, k), "saturating")
    assert np.all(h[:, n // 2:] == 0)      # silu(-128) * u underflows to zero in fp32


@pytest.mark.parametrize("m", [1, 2, 2048])
def test_swiglu_decoder_gate_up_full_size(m):
    """The decoder's gate/up (3072 -> 2 x 9216, layer-0 weights of the decode
    workload) at full size, checked on sampled rows."""
    spec = [s for s, _ in inputs.workload(2)[1] if s.name == "L0.gate_up"][0]
    gw, uw = spec.weight(0), spec.weight(1)
    n, k = gw.shape
    x = spec.activations(m)
    gpw, gblk = device_weight_from_f32(gw)
    upw, ublk = device_weight_from_f32(uw)
    say("swiglu full", m, q4.linear_swiglu_kernel(m, k))
    h = q4.linear_swiglu(to_dev_x(x), gpw, upw).cpu().numpy()
    rows = sample_rows(n, 64, 34)
    gb = gblk.cpu().numpy().reshape(n, -1)[rows]
    ub = ublk.cpu().numpy().reshape(n, -1)[rows]
    assert np.array_equal(gb.reshape(-1), O.quantize(gw[rows]).reshape(-1))
    ref, bound = O.swiglu_rows(x, gb, ub, len(rows), k, np.arange(len(rows)))
    assert_within_bound(h[:, rows], ref, bound, f"gate/up full size M={m}")


def test_swiglu_deterministic_and_empty():
    n, k, m = 300, 640, 37
    gw, uw = _pair(n, k, 35)
    gpw, _ = device_weight_from_f32(gw)
    upw, _ = device_weight_from_f32(uw)
    x = to_dev_x(inputs.activations_bf16((m, k), seed=35, tags=(m,)))
    say("swiglu determinism")
    a = q4.linear_swiglu(x, gpw, upw).cpu().numpy()
    b = q4.linear_swiglu(x, gpw, upw).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    empty = q4.linear_swiglu(x[:0], gpw, upw)
    assert tuple(empty.shape) == (0, n)


@pytest.mark.parametrize("m", [1, 2, 16, 40, 2048])
def test_swiglu_bf16_output(m):
    """bf16 output is the fp32 output rounded to nearest even, bit for bit, and
    so within bound + 2^-9 (|h| + bound) of the exact value."""
    n, k = 264, 1024
    gw, uw = _pair(n, k, 36)
    xb = inputs.activations_bf16((m, k), seed=36, tags=(m,))
    x = to_dev_x(xb)
    gpw, gblk = device_weight_from_f32(gw)
    upw, ublk = device_weight_from_f32(uw)
    say("swiglu bf16", m)
    h32 = q4.linear_swiglu(x, gpw, upw)
    h16 = q4.linear_swiglu(x, gpw, upw, dtype=torch.bfloat16)
    assert h16.dtype == torch.bfloat16
    assert torch.equal(h16.view(torch.int16), h32.to(torch.bfloat16).view(torch.int16))
    gb, ub = gblk.cpu().numpy(), ublk.cpu().numpy()
    ref = O.swiglu(xb, gb, ub, n, k)
    bound = O.swiglu_bound(xb, gb, ub, n, k)
    assert_within_bound(h16.float().cpu().numpy(), ref, bound + 2.0**-9 * (np.abs(ref) + bound), f"bf16 M={m}")
