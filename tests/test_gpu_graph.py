"""The entry points under HIP graph capture, as the benchmark uses them: a
graph holding a decode-sized fused linear, a prefill-sized GEMM, a SwiGLU
launch and an embedding lookup is replayed several times, with eager work and
synchronizations in between, and every replay must equal the eager results
bit for bit."""

import numpy as np
import pytest
import torch

import q4_weight_only_amd as q4
from q4_weight_only_amd import inputs

from gpu_helpers import DEV, device_weight_from_f32, say, to_dev_x

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    k = 768
    ns = (256, 64, 64)
    ws = [inputs.weights_f32((n, k), seed=71, tags=(i,)) for i, n in enumerate(ns)]
    pws = [device_weight_from_f32(w)[0] for w in ws]
    gate, _ = device_weight_from_f32(inputs.weights_f32((96, k), seed=71, tags=(7,)))
    up, _ = device_weight_from_f32(inputs.weights_f32((96, k), seed=71, tags=(8,)))
    x1 = to_dev_x(inputs.activations_bf16((1, k), seed=71, tags=(1,)))
    x2 = to_dev_x(inputs.activations_bf16((300, k), seed=71, tags=(300,)))
    ids = torch.tensor([5, 0, 255, 17, 17, -3], dtype=torch.int32, device=DEV)
    # a tall one-row launch: the stream kernel (fixed grid walking 2560 tiles)
    tall, kt = 40960, 1024
    ptall, _ = device_weight_from_f32(inputs.weights_f32((tall, kt), seed=71, tags=(9,)))
    xt = to_dev_x(inputs.activations_bf16((1, kt), seed=71, tags=(9,)))
    yt = torch.empty((1, tall), device=DEV)
    assert q4.linear_kernel(1, kt, tall).startswith("skinny_stream_kernel") or \
        torch.cuda.get_device_properties(DEV).multi_processor_count > 256

    ys1 = [torch.empty((1, n), device=DEV) for n in ns]
    y2 = torch.empty((300, ns[0]), device=DEV)
    h = torch.empty((300, 96), device=DEV)
    e = torch.empty((len(ids), k), device=DEV)

    def work():
        q4.linear_multi(x1, pws, ys1)
        q4.linear(x2, pws[0], y2)
        q4.linear_swiglu(x2, gate, up, h)
        q4.embed(pws[0], ids, e)
        q4.linear(xt, ptall, yt)

    say("graph eager")
    work()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (*ys1, y2, h, e, yt)]

    stream = torch.cuda.Stream(DEV)
    stream.wait_stream(torch.cuda.current_stream(DEV))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        work()
    torch.cuda.synchronize()
    outs = (*ys1, y2, h, e, yt)
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        say("graph replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, eager):
            a = got.cpu().numpy().view(np.uint32)
            b = want.cpu().numpy().view(np.uint32)
            assert np.array_equal(a, b), f"replay {rep} differs"
