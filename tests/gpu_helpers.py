"""Shared plumbing for the GPU parity tests: move seeded inputs to the device,
run the library, and compare with the oracle within the stated bound."""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import q4_0_oracle as O
import q4_weight_only_amd as q4

DEV = "cuda:0"


def say(*a):
    """Name the case before each GPU step so a fault can be attributed."""
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_x(x_bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16).copy())
    return t.to(DEV).view(torch.bfloat16)


def to_dev_bytes(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8).reshape(-1).copy()).to(DEV)


def device_weight_from_f32(w32: np.ndarray):
    """(PackedWeight, device GGUF bytes): quantized and packed by the library."""
    n, k = w32.shape
    wt = torch.from_numpy(np.ascontiguousarray(w32, dtype=np.float32)).to(DEV)
    blocks = q4.quantize(wt)
    pw = q4.pack(blocks, n, k)
    del wt
    return pw, blocks


def device_weight_from_blocks(blocks: np.ndarray, n: int, k: int):
    return q4.pack(to_dev_bytes(blocks), n, k)


def assert_within_bound(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, what: str = "") -> float:
    """|y - y_ref| <= 1e-3 * sum|x w| + 1e-6 elementwise; returns max(err / bound)."""
    y = np.asarray(y_gpu, dtype=np.float64)
    assert y.shape == y_ref.shape, (what, y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - y_ref)
    ratio = err / bound
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{what}: |err|/bound = {worst:.3g} at {idx}: gpu {y[idx]!r} ref {y_ref[idx]!r} "
                             f"bound {bound[idx]!r}")
    return worst


def canon_zero(a: np.ndarray) -> np.ndarray:
    """Map -0.0 to +0.0 (values compare equal; bit patterns may not)."""
    a = np.array(a, dtype=np.float32, copy=True)
    a[a == 0] = 0.0
    return a


def sample_rows(n: int, count: int, seed: int) -> np.ndarray:
    """First, last and a seeded spread of rows in between (sorted, unique)."""
    if n <= count:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    inner = rng.choice(np.arange(1, n - 1), size=count - 2, replace=False)
    return np.unique(np.concatenate([[0, n - 1], inner, [15, 16, n - 16] if n > 32 else []]).astype(np.int64))
