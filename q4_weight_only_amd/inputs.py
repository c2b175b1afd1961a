"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers; it holds none of the Q4_0 arithmetic
(no quantizer, no decode, no matmul).  Both the oracle side and the device
side receive exactly the arrays produced here.

Recipe (stands in for the Voxtral workloads on the pages, shapes only):
  * weights: fp32 draws from N(0, 0.02): standard_normal(float32) * 0.02;
  * activations: N(0, 1) in fp32, rounded to bf16 (round to nearest even, by
    torch's CPU conversion) and returned as uint16 bit patterns;
  * every array has its own stream: NumPy PCG64 seeded with
    SeedSequence([seed, *tags]), so an array is reproducible on its own.
"""

from __future__ import annotations

import numpy as np

WEIGHT_STD = np.float32(0.02)


def _gen(seed: int, tags) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, tags)])))


def weights_f32(shape, seed: int = 0, tags=()) -> np.ndarray:
    """fp32 weights ~ N(0, 0.02) of the given [N, K] shape."""
    g = _gen(seed, tuple(tags) + (0,))
    w = g.standard_normal(size=tuple(shape), dtype=np.float32)
    w *= WEIGHT_STD
    return w


def activations_bf16(shape, seed: int = 0, tags=()) -> np.ndarray:
    """bf16 activations ~ N(0, 1) as uint16 bit patterns of the given [M, K] shape."""
    import torch

    g = _gen(seed, tuple(tags) + (1,))
    x = g.standard_normal(size=tuple(shape), dtype=np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    return xb.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (torch's CPU RNE) and return the uint16 bits."""
    import torch

    xb = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return xb.view(torch.int16).numpy().view(np.uint16).copy()


# Linear shapes of the workloads (rows N = outputs, columns K = inputs).
DECODER_DIM = 3072
FFN_DIM = 9216
QKV_SEGMENTS = (4096, 1024, 1024)       # 32 query heads and 8 KV heads of 128
GATE_UP_SEGMENTS = (FFN_DIM, FFN_DIM)
DECODER_LAYERS = 26
VOCAB = 131072


def decoder_layer_ops():
    """The four linear launches of one decoder layer: (name, K, segment Ns)."""
    return (
        ("qkv", DECODER_DIM, QKV_SEGMENTS),
        ("o", 4096, (DECODER_DIM,)),
        ("gate_up", DECODER_DIM, GATE_UP_SEGMENTS),
        ("down", FFN_DIM, (DECODER_DIM,)),
    )
