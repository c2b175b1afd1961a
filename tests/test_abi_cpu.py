"""C-ABI checks that need no GPU: the library loads, exports every function
include/q4_0.h declares, sizes its buffers as documented, and rejects bad
arguments before touching the HIP runtime.

Only argument combinations that fail validation (or M == 0) are passed, so no
kernel is ever launched here; fake device addresses are never dereferenced.
"""

import ctypes
import os
import re

import pytest

from oracle import q4_0_oracle as O
import q4_weight_only_amd as q4
from q4_weight_only_amd import _binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "q4_0.h")

FAKE = 0x10000          # 16-byte aligned, never dereferenced
MISALIGNED = 0x10004

OK, NULL, SHAPE, ALIGN, SEGS = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(q4.library_path()):
        import subprocess, sys
        subprocess.run([sys.executable, "-m", "q4_weight_only_amd.build"], check=True)
    return q4.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4_\w+)\s*\(", text)))


def test_every_declared_function_is_exported(L):
    names = _declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(L, name), name
    assert sorted(B.EXPORTS) == names


def test_status_strings(L):
    for s in range(6):
        assert q4.status_str(s) and q4.status_str(s) != "unknown status"
    assert q4.status_str(99) == "unknown status"


@pytest.mark.parametrize("n,k", [(4096, 3072), (131072, 3072), (40, 384), (1, 32), (17, 96), (6020, 1280)])
def test_packed_bytes_matches_layout_definition(L, n, k):
    assert q4.packed_bytes(n, k) == O.packed_bytes(n, k)


@pytest.mark.parametrize("n,k", [(0, 32), (-1, 64), (16, 0), (16, 31), (16, 48), (2**30 + 1, 32), (16, 2**20 + 32)])
def test_packed_bytes_invalid_is_zero(L, n, k):
    assert q4.packed_bytes(n, k) == 0


@pytest.mark.parametrize("fn", ["q4_0_quantize", "q4_0_quantize_bf16", "q4_0_pack", "q4_0_unpack", "q4_0_dequant"])
def test_format_entry_points_validate_first(L, fn):
    f = getattr(L, fn)
    assert f(FAKE, 16, 48, FAKE, None) == SHAPE
    assert f(FAKE, 0, 64, FAKE, None) == SHAPE
    assert f(None, 16, 64, FAKE, None) == NULL
    assert f(FAKE, 16, 64, None, None) == NULL
    assert f(MISALIGNED, 16, 64, FAKE, None) == ALIGN
    assert f(FAKE, 16, 64, MISALIGNED, None) == ALIGN


def test_linear_validates_first(L):
    lin = L.q4_0_linear
    assert lin(FAKE, 1, FAKE, 16, 48, FAKE, None) == SHAPE        # K % 32
    assert lin(FAKE, -1, FAKE, 16, 64, FAKE, None) == SHAPE       # M < 0
    assert lin(FAKE, 2**20 + 1, FAKE, 16, 64, FAKE, None) == SHAPE
    assert lin(FAKE, 1, FAKE, 0, 64, FAKE, None) == SHAPE
    assert lin(None, 1, FAKE, 16, 64, FAKE, None) == NULL
    assert lin(FAKE, 1, None, 16, 64, FAKE, None) == NULL
    assert lin(FAKE, 1, FAKE, 16, 64, None, None) == NULL
    assert lin(MISALIGNED, 1, FAKE, 16, 64, FAKE, None) == ALIGN
    assert lin(FAKE, 1, MISALIGNED, 16, 64, FAKE, None) == ALIGN
    assert lin(FAKE, 1, FAKE, 16, 64, MISALIGNED, None) == ALIGN
    # M == 0 is a successful no-op, even with NULL pointers
    assert lin(None, 0, None, 16, 64, None, None) == OK


def test_linear_multi_validates_first(L):
    segs = (B.Segment * 9)()
    for i in range(9):
        segs[i] = B.Segment(FAKE, 16, FAKE)
    multi = L.q4_0_linear_multi
    assert multi(FAKE, 1, 64, None, 1, None) == NULL
    assert multi(FAKE, 1, 64, segs, 0, None) == SEGS
    assert multi(FAKE, 1, 64, segs, 9, None) == SEGS
    bad = (B.Segment * 3)(B.Segment(FAKE, 16, FAKE), B.Segment(FAKE, 0, FAKE), B.Segment(FAKE, 16, FAKE))
    assert multi(FAKE, 1, 64, bad, 3, None) == SHAPE
    nul = (B.Segment * 2)(B.Segment(FAKE, 16, FAKE), B.Segment(None, 16, FAKE))
    assert multi(FAKE, 1, 64, nul, 2, None) == NULL
    mis = (B.Segment * 2)(B.Segment(FAKE, 16, FAKE), B.Segment(FAKE, 16, MISALIGNED))
    assert multi(FAKE, 1, 64, mis, 2, None) == ALIGN
    assert multi(FAKE, 1, 48, segs, 2, None) == SHAPE
    assert multi(None, 0, 64, segs, 8, None) == OK


def test_linear_swiglu_validates_first(L):
    sw = L.q4_0_linear_swiglu
    assert sw(FAKE, 1, 48, FAKE, FAKE, 16, FAKE, 0, None) == SHAPE       # K % 32
    assert sw(FAKE, -1, 64, FAKE, FAKE, 16, FAKE, 0, None) == SHAPE      # M < 0
    assert sw(FAKE, 1, 64, FAKE, FAKE, 0, FAKE, 0, None) == SHAPE        # N < 1
    assert sw(FAKE, 1, 64, FAKE, FAKE, 2**30 + 1, FAKE, 0, None) == SHAPE
    assert sw(FAKE, 1, 64, FAKE, FAKE, 16, FAKE, 2, None) == SHAPE       # output type flag
    assert sw(None, 1, 64, FAKE, FAKE, 16, FAKE, 1, None) == NULL
    assert sw(FAKE, 1, 64, None, FAKE, 16, FAKE, 0, None) == NULL
    assert sw(FAKE, 1, 64, FAKE, None, 16, FAKE, 0, None) == NULL
    assert sw(FAKE, 1, 64, FAKE, FAKE, 16, None, 0, None) == NULL
    assert sw(MISALIGNED, 1, 64, FAKE, FAKE, 16, FAKE, 0, None) == ALIGN
    assert sw(FAKE, 1, 64, FAKE, MISALIGNED, 16, FAKE, 0, None) == ALIGN
    assert sw(FAKE, 1, 64, FAKE, FAKE, 16, MISALIGNED, 1, None) == ALIGN
    assert sw(None, 0, 64, None, None, 16, None, 0, None) == OK
    assert L.q4_0_linear_swiglu_kernel(0, 64) == b""
    assert b"true" in L.q4_0_linear_swiglu_kernel(1, 3072)        # the gated instantiation


def test_linear_kernel_names(L):
    """The kernel-name query is host logic: invalid arguments give "", decode
    sizes name a decode kernel (its stage count follows from K), and above 64 rows the GEMM tile shape follows
    the launch's tile count (256 compute units are assumed without a device)."""
    import ctypes
    kn = L.q4_0_linear_kernel

    def arr(*ns):
        return (ctypes.c_int64 * len(ns))(*ns)
    assert kn(0, 64, arr(16), 1) == b""
    assert kn(1, 48, arr(16), 1) == b""                 # K % 32
    assert kn(1, 64, arr(0), 1) == b""                  # N < 1
    assert kn(1, 64, arr(16), 0) == b""                 # no segment
    assert kn(1, 64, arr(*([16] * 9)), 9) == b""        # too many segments
    assert kn(1, 64, None, 1) == b""
    assert kn(1, 3072, arr(4096, 1024, 1024), 3) == b"gemv_kernel<1, 8, 3, 6, false>"
    assert kn(1, 4096, arr(3072), 1) == b"gemv_kernel<1, 16, 2, 0, false>"
    assert kn(1, 9216, arr(3072), 1) == b"gemv_kernel<1, 12, 6, 0, false>"   # long K: 12 K-slices
    assert kn(2, 5120, arr(3072), 1) == b"gemv_kernel<2, 12, 4, 0, false>"
    assert kn(1, 9248, arr(3072), 1) == b"skinny_kernel<1, 1, 16, 2, true, 0, false>"   # past 12 x 6 stages
    assert kn(3, 9216, arr(3072), 1) == b"gemv_kernel<4, 12, 6, 0, false>"
    assert kn(4, 5120, arr(3072), 1) == b"gemv_kernel<4, 12, 4, 0, false>"
    assert kn(4, 9248, arr(3072), 1) == b"skinny_kernel<4, 1, 16, 2, true, 0, false>"
    assert L.q4_0_linear_swiglu_kernel(4, 9216) == b"skinny_kernel<4, 1, 8, 3, true, 0, true>"   # gated: K-split
    assert L.q4_0_linear_swiglu_kernel(3, 4096) == b"gemv_kernel<4, 16, 2, 0, true>"
    assert L.q4_0_linear_swiglu_kernel(1, 9216) == b"gemv_kernel<1, 12, 6, 0, true>"
    assert L.q4_0_linear_swiglu_kernel(2, 9248) == b"skinny_kernel<2, 1, 8, 3, true, 0, true>"
    assert kn(2, 3072, arr(9216, 9216), 2) == b"gemv_kernel<2, 8, 3, 0, false>"
    assert kn(3, 1280, arr(512), 1) == b"gemv_kernel<4, 8, 2, 0, false>"
    assert L.q4_0_linear_swiglu_kernel(1, 3072) == b"gemv_kernel<1, 8, 3, 6, true>"
    assert L.q4_0_linear_swiglu_kernel(2, 4096) == b"gemv_kernel<2, 8, 4, 0, true>"
    assert L.q4_0_linear_swiglu_kernel(1, 4096) == b"gemv_kernel<1, 16, 2, 0, true>"
    assert L.q4_0_linear_swiglu_kernel(32, 3072) == b"gemm_kernel<2, 1, 1, 8, 0, 2, true>"   # 17-32 rows
    assert L.q4_0_linear_swiglu_kernel(64, 3072) == b"gemm_kernel<4, 1, 1, 8, 0, 3, true>"   # 33-64 rows
    import torch
    if torch.cuda.is_available() and torch.cuda.get_device_properties(0).multi_processor_count != 256:
        return                                          # the tile counts below assume 256 CUs
    # 17-64 rows: the K-split decode kernel under 128 GEMM tiles, the GEMM from there
    assert kn(20, 3072, arr(3072), 1) == b"skinny_kernel<32, 1, 8, 2, false, 0, false>"
    assert kn(20, 3072, arr(4096, 1024, 1024), 3) == b"skinny_kernel<32, 2, 8, 2, false, 0, false>"
    assert kn(20, 256, arr(3072), 1) == b"skinny_kernel<32, 1, 8, 2, true, 0, false>"
    assert kn(40, 3072, arr(3072), 1) == b"skinny_kernel<64, 1, 8, 2, false, 0, false>"
    assert kn(20, 3072, arr(16384), 1) == b"gemm_kernel<2, 1, 1, 8, 0, 2>"
    assert kn(40, 3072, arr(131072), 1) == b"gemm_kernel<4, 1, 1, 8, 0, 3>"
    # one row: very tall weights take the stream kernel
    assert kn(1, 3072, arr(131072), 1) == b"skinny_stream_kernel<1, 8, 3, 6>"
    assert kn(1, 3072, arr(9216, 9216), 2) == b"gemv_kernel<1, 8, 3, 6, false>"
    assert kn(2048, 4096, arr(3072), 1) == b"gemm3_kernel<8, 1, 1, 12, 0, 4, false>"
    assert kn(1505, 5120, arr(3072), 1) == b"gemm3_kernel<6, 1, 1, 12, 0, 4, false>"   # 256 tiles of 96 x 192
    assert kn(2048, 3072, arr(3072, 3072, 3072), 3) == b"gemm3_kernel<8, 1, 1, 8, 4, 4, false>"
    assert kn(300, 3072, arr(3072), 1) == b"gemm3_kernel<4, 1, 1, 8, 4, 8, false>"


@pytest.mark.parametrize("fn", ["q4_0_embed", "q4_0_embed_gguf"])
def test_embed_validates_first(L, fn):
    em = getattr(L, fn)
    assert em(FAKE, 16, 48, FAKE, 4, FAKE, None) == SHAPE          # K % 32
    assert em(FAKE, 0, 64, FAKE, 4, FAKE, None) == SHAPE           # N < 1
    assert em(FAKE, 16, 64, FAKE, -1, FAKE, None) == SHAPE         # n_ids < 0
    assert em(FAKE, 16, 64, FAKE, 2**24 + 1, FAKE, None) == SHAPE
    assert em(None, 16, 64, FAKE, 4, FAKE, None) == NULL
    assert em(FAKE, 16, 64, None, 4, FAKE, None) == NULL
    assert em(FAKE, 16, 64, FAKE, 4, None, None) == NULL
    assert em(MISALIGNED, 16, 64, FAKE, 4, FAKE, None) == ALIGN
    assert em(FAKE, 16, 64, FAKE, 4, MISALIGNED, None) == ALIGN
    assert em(FAKE, 16, 64, FAKE + 2, 4, FAKE, None) == ALIGN        # ids need 4-byte alignment
    assert em(None, 16, 64, None, 0, None, None) == OK


def test_format_grids_beyond_the_limit_are_refused(L):
    """A matrix within the shape limits but needing more than 2^31 - 1
    workgroups is refused before any HIP call (Q4_ERR_HIP), not truncated."""
    HIP = 5
    n, k = 2**30, 2**20
    assert L.q4_0_quantize(FAKE, n, k, FAKE, None) == HIP
    assert L.q4_0_quantize_bf16(FAKE, n, k, FAKE, None) == HIP
    assert L.q4_0_pack(FAKE, n, k, FAKE, None) == HIP
    assert L.q4_0_unpack(FAKE, n, k, FAKE, None) == HIP
    assert L.q4_0_dequant(FAKE, n, k, FAKE, None) == HIP


def test_python_binding_raises_on_bad_status(L):
    with pytest.raises(q4.Q4Error) as ei:
        B._check(SHAPE, "q4_0_linear")
    assert ei.value.status == SHAPE and "Q4_ERR_SHAPE" in str(ei.value)


def test_product_path_has_no_oracle_dependency():
    """The package never imports the oracle (it is test infrastructure)."""
    pkg = os.path.dirname(q4.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(root, f), encoding="utf-8").read()
                assert "import oracle" not in src and "from oracle" not in src, f


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert p.returncode == 2
    assert "one GPU only" in p.stderr
    assert p.stdout == ""


def test_reference_read_validates_first(L):
    rr, words = L.q4_0_reference_read, L.q4_0_reference_read_words
    assert words(0) == 256                     # one workgroup (the launch alone), a word per thread
    assert words(16) == 256 and words(65536) == 256 and words(65552) == 512
    assert words(-16) == 0 and words(24) == 0 and words(2**40 + 16) == 0
    assert rr(FAKE, 24, FAKE, None) == SHAPE            # not a multiple of 16
    assert rr(FAKE, -16, FAKE, None) == SHAPE
    assert rr(None, 64, FAKE, None) == NULL
    assert rr(FAKE, 64, None, None) == NULL
    assert rr(MISALIGNED + 4, 64, FAKE, None) == ALIGN
    assert rr(FAKE, 64, FAKE + 2, None) == ALIGN


def test_reference_mfma_validates_first(L):
    rm = L.q4_0_reference_mfma
    assert rm(4, 10, FAKE, None) == SHAPE                # modes 0-3 only
    assert rm(-1, 10, FAKE, None) == SHAPE
    assert rm(0, 0, FAKE, None) == SHAPE                 # at least one iteration
    assert rm(2, 2**20 + 1, FAKE, None) == SHAPE
    assert rm(1, 10, None, None) == NULL
    assert rm(1, 10, FAKE + 2, None) == ALIGN


@pytest.mark.parametrize("n,k", [(4096, 3072), (40, 384), (1, 32), (17, 96)])
def test_q41_packed_bytes_matches_layout_definition(L, n, k):
    assert q4.q41_packed_bytes(n, k) == O.q41_packed_bytes(n, k)


def test_q41_entry_points_validate_first(L):
    for fn in (L.q4_1_quantize, L.q4_1_pack, L.q4_1_dequant):
        assert fn(FAKE, 16, 48, FAKE, None) == SHAPE
        assert fn(None, 16, 64, FAKE, None) == NULL
        assert fn(FAKE, 16, 64, MISALIGNED, None) == ALIGN
    lin = L.q4_1_linear
    assert lin(FAKE, 1, FAKE, 16, 48, FAKE, None) == SHAPE
    assert lin(FAKE, -1, FAKE, 16, 64, FAKE, None) == SHAPE
    assert lin(None, 1, FAKE, 16, 64, FAKE, None) == NULL
    assert lin(FAKE, 1, FAKE, 16, 64, MISALIGNED, None) == ALIGN
    assert lin(None, 0, None, 16, 64, None, None) == OK
    assert L.q4_1_packed_bytes(16, 48) == 0
    kn = L.q4_1_linear_kernel
    assert kn(0, 64, 16) == b""
    assert kn(1, 3072, 4096) == b"gemv_kernel<1, 8, 3, 6, false, true>"
    assert kn(1, 9216, 3072) == b"gemv_kernel<1, 12, 6, 0, false, true>"
    assert kn(2, 5120, 3072) == b"gemv_kernel<2, 12, 4, 0, false, true>"
    assert kn(1, 4096, 3072) == b"gemv_kernel<1, 16, 2, 0, false, true>"
    assert kn(1, 12288, 3072) == b"gemv_kernel<1, 16, 6, 0, false, true>"   # past 12 x 6 stages
    assert kn(3, 20480, 64) == b"gemm3_kernel<2, 1, 1, 8, 0, 8, false, true>"   # K past the decode kernel's reach
    assert kn(40, 3072, 3072) == b"gemm3_kernel<4, 1, 1, 8, 0, 8, false, true>"
