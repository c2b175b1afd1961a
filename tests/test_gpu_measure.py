"""The measurement-support kernels on the GPU: the reference read touches
every byte it is given (sink word 256 b + t is the XOR of the 32-bit words
of the input's 16-byte chunks 4096 b + 256 p + t, p = 0 .. 15, zero past the
input), and the arithmetic-only GEMM loop runs in every mode,
deterministically, with finite results."""

import numpy as np
import pytest
import torch

import q4_weight_only_amd as q4

from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 16400, 65536, 65552, 3 * 65536 + 4096])
def test_reference_read_folds_every_word(nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32).copy()).to(DEV)
    say("reference read", nbytes)
    sink = q4.reference_read(src, nbytes).cpu().numpy().view(np.uint32)
    groups = -(-nbytes // 65536)
    assert sink.size == int(q4.lib().q4_0_reference_read_words(nbytes)) == 256 * groups
    chunks = np.zeros((groups * 4096, 4), dtype=np.uint32)      # 16-byte chunks, zero past the input
    chunks.reshape(-1)[:host.size] = host
    want = np.bitwise_xor.reduce(chunks.reshape(groups, 16, 256, 4), axis=(1, 3)).reshape(-1)
    assert np.array_equal(sink, want)


def test_reference_read_of_nothing_is_one_launch():
    src = torch.zeros(16, dtype=torch.uint8, device=DEV)
    sink = q4.reference_read(src, 0)
    torch.cuda.synchronize()
    assert sink.numel() == 256 and int(sink.abs().sum()) == 0


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_reference_mfma_runs_deterministically(mode):
    say("reference mfma", mode)
    a = torch.empty(int(q4.lib().q4_0_reference_mfma_threads()), dtype=torch.float32, device=DEV)
    b = torch.empty_like(a)
    n = q4.reference_mfma(mode, 3, DEV, a)
    q4.reference_mfma(mode, 3, DEV, b)
    torch.cuda.synchronize()
    assert n == a.numel() // 64 * 3 * 32
    assert torch.isfinite(a).all()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
