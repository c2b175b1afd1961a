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


# ------------------------------------------------------------ workloads
class LinearSpec:
    """One launch of a workload: segment row counts share K and x."""

    __slots__ = ("name", "K", "Ns", "w_tags", "x_tags")

    def __init__(self, name, K, Ns, w_tags, x_tags):
        self.name, self.K, self.Ns = name, int(K), tuple(int(n) for n in Ns)
        self.w_tags = tuple(tuple(t) for t in w_tags)   # one tag tuple per segment
        self.x_tags = tuple(x_tags)

    def weight(self, seg: int, seed: int = 0) -> np.ndarray:
        return weights_f32((self.Ns[seg], self.K), seed=seed, tags=self.w_tags[seg])

    def activations(self, m: int, seed: int = 0) -> np.ndarray:
        return activations_bf16((m, self.K), seed=seed, tags=self.x_tags + (m,))

    def weight_bytes(self) -> int:
        return sum(n * (self.K // 32) * 18 for n in self.Ns)


def _decoder_specs(cfg: int, layers):
    out = []
    for layer in layers:
        for op, (name, k, ns) in enumerate(decoder_layer_ops()):
            out.append(LinearSpec(f"L{layer}.{name}", k, ns,
                                  [(2, layer, op, s) for s in range(len(ns))], (cfg, layer, op)))
    return out


def workload(cfg: int):
    """(description, [(LinearSpec, (M, ...))]) for the five workloads.

    1  one GEMV: M=1, K=3072, N=4096
    2  a decoder layer's decode step, 26 layers of distinct weights, M in {1, 2}:
       fused QKV 3072->4096+1024+1024, O 4096->3072, fused gate/up
       3072->9216+9216, down 9216->3072
    3  LM head K=3072, N=131072, M in {1, 32}
    4  prefill M=2048 through the four decoder shapes (layer-0 weights of 2)
    5  audio side: adapter 5120->3072 and 3072->3072 at M=1505, encoder
       1280->5120 and 5120->1280 at M=6020
    """
    if cfg == 1:
        return ("single Q4_0 GEMV M=1 K=3072 N=4096",
                [(LinearSpec("gemv", 3072, (4096,), [(1, 0, 0, 0)], (1, 0, 0)), (1,))])
    if cfg == 2:
        return ("26-layer decoder decode step, M=1 and M=2",
                [(s, (1, 2)) for s in _decoder_specs(2, range(DECODER_LAYERS))])
    if cfg == 3:
        return ("LM head K=3072 N=131072, M=1 and M=32",
                [(LinearSpec("lm_head", DECODER_DIM, (VOCAB,), [(3, 0, 0, 0)], (3, 0, 0)), (1, 32))])
    if cfg == 4:
        return ("prefill M=2048 through the decoder shapes",
                [(s, (2048,)) for s in _decoder_specs(4, [0])])
    if cfg == 5:
        return ("audio linears: adapter at M=1505, encoder at M=6020", [
            (LinearSpec("adapter", 5120, (3072,), [(5, 0, 0, 0)], (5, 0, 0)), (1505,)),
            (LinearSpec("adapter_out", 3072, (3072,), [(5, 0, 1, 0)], (5, 0, 1)), (1505,)),
            (LinearSpec("enc_up", 1280, (5120,), [(5, 0, 2, 0)], (5, 0, 2)), (6020,)),
            (LinearSpec("enc_down", 5120, (1280,), [(5, 0, 3, 0)], (5, 0, 3)), (6020,)),
        ])
    raise ValueError(f"no workload {cfg}")
