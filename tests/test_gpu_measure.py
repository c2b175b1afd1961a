"""The measurement-support kernels on the GPU: the reference read touches
every byte it is given (its sink words are the XOR of each 64 KiB piece's
32-bit words), and the arithmetic-only GEMM loop runs in every mode,
deterministically, with finite results."""

import numpy as np
import pytest
import torch

import q4_weight_only_amd as q4

from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 65536, 65552, 3 * 65536 + 4096])
def test_reference_read_folds_every_word(nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32).copy()).to(DEV)
    say("reference read", nbytes)
    sink = q4.reference_read(src, nbytes).cpu().numpy().view(np.uint32)
    words = 65536 // 4
    want = [np.bitwise_xor.reduce(host[i:i + words]) for i in range(0, host.size, words)]
    assert np.array_equal(sink, np.array(want, dtype=np.uint32))


def test_reference_read_of_nothing_is_one_launch():
    src = torch.zeros(16, dtype=torch.uint8, device=DEV)
    sink = q4.reference_read(src, 0)
    torch.cuda.synchronize()
    assert sink.numel() == 1 and int(sink[0]) == 0


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
