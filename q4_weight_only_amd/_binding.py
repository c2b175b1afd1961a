"""ctypes binding of libq4amd (include/q4_0.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  PyTorch provides device memory and the current stream.  If the
library has not been built the first call raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq4amd.so")
_lib = None
_lock = threading.Lock()

Q4_OK = 0
STATUS_NAMES = {0: "Q4_OK", 1: "Q4_ERR_NULL", 2: "Q4_ERR_SHAPE", 3: "Q4_ERR_ALIGN",
                4: "Q4_ERR_SEGMENTS", 5: "Q4_ERR_HIP"}
EXPORTS = ("q4_status_str", "q4_0_packed_bytes", "q4_0_quantize", "q4_0_quantize_bf16", "q4_0_pack", "q4_0_unpack",
           "q4_0_dequant", "q4_0_linear", "q4_0_linear_multi", "q4_0_time_next_launch",
           "q4_0_linear_kernel", "q4_0_linear_swiglu", "q4_0_linear_swiglu_kernel", "q4_0_embed",
           "q4_0_embed_gguf", "q4_0_reference_read", "q4_0_reference_read_words", "q4_0_reference_mfma",
           "q4_0_reference_mfma_threads", "q4_1_packed_bytes",
           "q4_1_quantize", "q4_1_pack", "q4_1_dequant", "q4_1_linear", "q4_1_linear_kernel")


class Q4Error(ValueError):
    """A nonzero q4_status from the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_str(status)})")


class Segment(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("N", ctypes.c_int64), ("y", ctypes.c_void_p)]


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libq4amd.so (once); raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    f"{_LIB_PATH} is not built; run `python -m q4_weight_only_amd.build` "
                    "(or __graft_entry__.build()) first")
            L = ctypes.CDLL(_LIB_PATH)
            vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
            L.q4_status_str.argtypes = [i32]
            L.q4_status_str.restype = ctypes.c_char_p
            L.q4_0_packed_bytes.argtypes = [i64, i64]
            L.q4_0_packed_bytes.restype = ctypes.c_size_t
            for name in ("q4_0_quantize", "q4_0_quantize_bf16", "q4_0_pack", "q4_0_unpack", "q4_0_dequant"):
                fn = getattr(L, name)
                fn.argtypes = [vp, i64, i64, vp, vp]
                fn.restype = i32
            for name in ("q4_0_embed", "q4_0_embed_gguf"):
                fn = getattr(L, name)
                fn.argtypes = [vp, i64, i64, vp, i64, vp, vp]
                fn.restype = i32
            L.q4_0_linear.argtypes = [vp, i64, vp, i64, i64, vp, vp]
            L.q4_0_linear.restype = i32
            L.q4_0_linear_multi.argtypes = [vp, i64, i64, ctypes.POINTER(Segment), i32, vp]
            L.q4_0_linear_multi.restype = i32
            L.q4_0_linear_kernel.argtypes = [i64, i64, ctypes.POINTER(i64), i32]
            L.q4_0_linear_kernel.restype = ctypes.c_char_p
            L.q4_0_linear_swiglu.argtypes = [vp, i64, i64, vp, vp, i64, vp, i32, vp]
            L.q4_0_linear_swiglu.restype = i32
            L.q4_0_linear_swiglu_kernel.argtypes = [i64, i64]
            L.q4_0_linear_swiglu_kernel.restype = ctypes.c_char_p
            L.q4_0_time_next_launch.argtypes = [vp, vp]
            L.q4_0_time_next_launch.restype = i32
            L.q4_0_reference_read.argtypes = [vp, i64, vp, vp]
            L.q4_0_reference_read.restype = i32
            L.q4_0_reference_read_words.argtypes = [i64]
            L.q4_0_reference_read_words.restype = i64
            L.q4_0_reference_mfma.argtypes = [i32, i64, vp, vp]
            L.q4_0_reference_mfma.restype = i32
            L.q4_0_reference_mfma_threads.argtypes = []
            L.q4_0_reference_mfma_threads.restype = i64
            L.q4_1_packed_bytes.argtypes = [i64, i64]
            L.q4_1_packed_bytes.restype = ctypes.c_size_t
            for fn in (L.q4_1_quantize, L.q4_1_pack, L.q4_1_dequant):
                fn.argtypes = [vp, i64, i64, vp, vp]
                fn.restype = i32
            L.q4_1_linear.argtypes = [vp, i64, vp, i64, i64, vp, vp]
            L.q4_1_linear.restype = i32
            L.q4_1_linear_kernel.argtypes = [i64, i64, i64]
            L.q4_1_linear_kernel.restype = ctypes.c_char_p
            _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().q4_status_str(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != Q4_OK:
        raise Q4Error(status, what)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA/HIP tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(t: torch.Tensor, other: torch.Tensor, name: str) -> None:
    if t.device != other.device:
        raise ValueError(f"{name} is on {other.device}, not {t.device}")


# ------------------------------------------------------------------ API
def packed_bytes(n: int, k: int) -> int:
    return int(lib().q4_0_packed_bytes(int(n), int(k)))


def gguf_bytes(n: int, k: int) -> int:
    return int(n) * (int(k) // 32) * 18


class PackedWeight:
    """A Q4_0 weight matrix [N, K] in the packed device layout."""

    __slots__ = ("data", "n", "k")

    def __init__(self, data: torch.Tensor, n: int, k: int):
        self.data, self.n, self.k = data, int(n), int(k)

    @property
    def device(self) -> torch.device:
        return self.data.device


def quantize(w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 or bf16 W [N, K] on the device -> GGUF Q4_0 bytes [N, K/32, 18]
    (uint8); bf16 values are widened to fp32 exactly first."""
    _dev(w, "w", torch.bfloat16 if w.dtype == torch.bfloat16 else torch.float32)
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    if out is None:
        out = torch.empty((n, max(k // 32, 0), 18), dtype=torch.uint8, device=w.device)
    _dev(out, "out", torch.uint8)
    if out.numel() != gguf_bytes(n, k):
        raise ValueError("out has the wrong size")
    _same_device(w, out, "out")
    fn = "q4_0_quantize_bf16" if w.dtype == torch.bfloat16 else "q4_0_quantize"
    with torch.cuda.device(w.device):
        _check(getattr(lib(), fn)(w.data_ptr(), n, k, out.data_ptr(), _stream(w.device)), fn)
    return out


def pack(blocks: torch.Tensor, n: int, k: int, out: torch.Tensor | None = None) -> PackedWeight:
    """GGUF Q4_0 bytes (uint8, N*K/32*18 elements, on the device) -> PackedWeight."""
    _dev(blocks, "blocks", torch.uint8)
    if blocks.numel() != gguf_bytes(n, k):
        raise ValueError(f"blocks must hold {gguf_bytes(n, k)} bytes for [{n}, {k}]")
    nbytes = packed_bytes(n, k)
    if nbytes == 0:
        raise ValueError(f"invalid shape [{n}, {k}]")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=blocks.device)
    _dev(out, "out", torch.uint8)
    if out.numel() != nbytes:
        raise ValueError("out has the wrong size")
    _same_device(blocks, out, "out")
    with torch.cuda.device(blocks.device):
        _check(lib().q4_0_pack(blocks.data_ptr(), n, k, out.data_ptr(), _stream(blocks.device)), "q4_0_pack")
    return PackedWeight(out, n, k)


def unpack(pw: PackedWeight) -> torch.Tensor:
    out = torch.empty((pw.n, pw.k // 32, 18), dtype=torch.uint8, device=pw.device)
    with torch.cuda.device(pw.device):
        _check(lib().q4_0_unpack(pw.data.data_ptr(), pw.n, pw.k, out.data_ptr(), _stream(pw.device)),
               "q4_0_unpack")
    return out


def dequant(pw: PackedWeight) -> torch.Tensor:
    out = torch.empty((pw.n, pw.k), dtype=torch.float32, device=pw.device)
    with torch.cuda.device(pw.device):
        _check(lib().q4_0_dequant(pw.data.data_ptr(), pw.n, pw.k, out.data_ptr(), _stream(pw.device)),
               "q4_0_dequant")
    return out


def embed(pw: PackedWeight, ids: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Rows ids of the packed table, dequantized: [len(ids), K] fp32 (NaN rows
    for ids outside [0, N))."""
    _dev(ids, "ids", torch.int32)
    if ids.dim() != 1:
        raise ValueError("ids must be 1-D")
    if out is None:
        out = torch.empty((ids.shape[0], pw.k), dtype=torch.float32, device=ids.device)
    _dev(out, "out", torch.float32)
    if tuple(out.shape) != (ids.shape[0], pw.k):
        raise ValueError("out has the wrong shape")
    _same_device(ids, pw.data, "the table")
    _same_device(ids, out, "out")
    with torch.cuda.device(ids.device):
        _check(lib().q4_0_embed(pw.data.data_ptr(), pw.n, pw.k, ids.data_ptr(), ids.shape[0], out.data_ptr(),
                                _stream(ids.device)), "q4_0_embed")
    return out


def embed_gguf(blocks: torch.Tensor, n: int, k: int, ids: torch.Tensor,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """Rows ids of a table kept as GGUF Q4_0 bytes (uint8, N*K/32*18 elements,
    on the device), dequantized: [len(ids), K] fp32, equal to embed() on the
    packed form of the same table."""
    _dev(blocks, "blocks", torch.uint8)
    if blocks.numel() != gguf_bytes(n, k):
        raise ValueError(f"blocks must hold {gguf_bytes(n, k)} bytes for [{n}, {k}]")
    _dev(ids, "ids", torch.int32)
    if ids.dim() != 1:
        raise ValueError("ids must be 1-D")
    if out is None:
        out = torch.empty((ids.shape[0], int(k)), dtype=torch.float32, device=ids.device)
    _dev(out, "out", torch.float32)
    if tuple(out.shape) != (ids.shape[0], int(k)):
        raise ValueError("out has the wrong shape")
    _same_device(ids, blocks, "the table")
    _same_device(ids, out, "out")
    with torch.cuda.device(ids.device):
        _check(lib().q4_0_embed_gguf(blocks.data_ptr(), int(n), int(k), ids.data_ptr(), ids.shape[0],
                                     out.data_ptr(), _stream(ids.device)), "q4_0_embed_gguf")
    return out


def linear(x: torch.Tensor, pw: PackedWeight, out: torch.Tensor | None = None) -> torch.Tensor:
    """y [M, N] fp32 = x [M, K] bf16 times W^T."""
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.shape[1] != pw.k:
        raise ValueError(f"x must be [M, {pw.k}]")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, pw.n), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if tuple(out.shape) != (m, pw.n):
        raise ValueError("out has the wrong shape")
    _same_device(x, pw.data, "the weights")
    _same_device(x, out, "out")
    with torch.cuda.device(x.device):
        _check(lib().q4_0_linear(x.data_ptr(), m, pw.data.data_ptr(), pw.n, pw.k, out.data_ptr(),
                                 _stream(x.device)), "q4_0_linear")
    return out


def linear_multi(x: torch.Tensor, weights, outs=None):
    """One launch over several weight matrices sharing x: returns [y_i]."""
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    weights = list(weights)
    if not 1 <= len(weights) <= 8:
        raise ValueError("need 1..8 weight matrices")
    k = x.shape[1]
    m = x.shape[0]
    if outs is None:
        outs = [torch.empty((m, w.n), dtype=torch.float32, device=x.device) for w in weights]
    outs = list(outs)
    if len(outs) != len(weights):
        raise ValueError(f"{len(weights)} weight matrices but {len(outs)} outputs")
    segs = (Segment * len(weights))()
    for i, (w, y) in enumerate(zip(weights, outs)):
        if w.k != k:
            raise ValueError("all segments must share K")
        _dev(y, f"outs[{i}]", torch.float32)
        if tuple(y.shape) != (m, w.n):
            raise ValueError(f"outs[{i}] has the wrong shape")
        _same_device(x, w.data, f"weights[{i}]")
        _same_device(x, y, f"outs[{i}]")
        segs[i] = Segment(w.data.data_ptr(), w.n, y.data_ptr())
    with torch.cuda.device(x.device):
        _check(lib().q4_0_linear_multi(x.data_ptr(), m, k, segs, len(weights), _stream(x.device)),
               "q4_0_linear_multi")
    return outs


def linear_swiglu(x: torch.Tensor, gate: PackedWeight, up: PackedWeight,
                  out: torch.Tensor | None = None, dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """h [M, N] = silu(x Wg^T) * (x Wu^T) in one launch (gate and up [N, K]);
    h is fp32, or bf16 (rounded to nearest even) with dtype=torch.bfloat16."""
    _dev(x, "x", torch.bfloat16)
    if dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dtype must be torch.float32 or torch.bfloat16")
    if gate.n != up.n or gate.k != up.k:
        raise ValueError("gate and up must have the same shape")
    if x.dim() != 2 or x.shape[1] != gate.k:
        raise ValueError(f"x must be [M, {gate.k}]")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, gate.n), dtype=dtype, device=x.device)
    _dev(out, "out", dtype)
    if tuple(out.shape) != (m, gate.n):
        raise ValueError("out has the wrong shape")
    _same_device(x, gate.data, "gate")
    _same_device(x, up.data, "up")
    _same_device(x, out, "out")
    with torch.cuda.device(x.device):
        _check(lib().q4_0_linear_swiglu(x.data_ptr(), m, gate.k, gate.data.data_ptr(), up.data.data_ptr(),
                                        gate.n, out.data_ptr(), int(dtype == torch.bfloat16), _stream(x.device)),
               "q4_0_linear_swiglu")
    return out


def reference_read(src: torch.Tensor, nbytes: int | None = None, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Measurement support: stream nbytes (default: all) of the device tensor
    src through the reference read kernel; returns the sink words (int32)."""
    if not src.is_cuda:
        raise ValueError("src must be a device tensor")
    total = src.numel() * src.element_size()
    nbytes = total if nbytes is None else int(nbytes)
    if nbytes > total:
        raise ValueError("nbytes exceeds the tensor")
    words = int(lib().q4_0_reference_read_words(nbytes))
    if words == 0:
        raise ValueError("nbytes must be a multiple of 16")
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device=src.device)
    if not sink.is_cuda or sink.dtype != torch.int32 or sink.numel() < words:
        raise ValueError(f"sink must be a device int32 tensor of at least {words} words")
    _same_device(src, sink, "sink")
    with torch.cuda.device(src.device):
        _check(lib().q4_0_reference_read(src.data_ptr(), nbytes, sink.data_ptr(), _stream(src.device)),
               "q4_0_reference_read")
    return sink


def reference_mfma(mode: int, iterations: int, device="cuda", sink: torch.Tensor | None = None) -> int:
    """Measurement support: one launch of the prefill GEMM's arithmetic
    alone (mode 0: MFMAs; 1: + the fp32 rescale; 2: + the decode; 3: MFMAs
    beside as many independent fp32 FMAs as the rescale) on the
    current stream of `device`; returns the number of 16x16x32 MFMAs it
    issues (each 16384 flops)."""
    device = torch.device(device)
    with torch.cuda.device(device):
        threads = int(lib().q4_0_reference_mfma_threads())   # from the current device's CU count
        if sink is None:
            sink = torch.empty(threads, dtype=torch.float32, device=device)
        if not sink.is_cuda or sink.dtype != torch.float32 or sink.numel() < threads:
            raise ValueError(f"sink must be a device float32 tensor of at least {threads} elements")
        _check(lib().q4_0_reference_mfma(int(mode), int(iterations), sink.data_ptr(), _stream(device)),
               "q4_0_reference_mfma")
    return threads // 64 * int(iterations) * 32


# ------------------------------------------------ the asymmetric variant
Q41_BLOCK_BYTES = 20


class PackedWeightQ41(PackedWeight):
    """An asymmetric 4-bit weight matrix [N, K] (w = q * d + m per 32-weight
    block) in the packed asymmetric layout."""

    __slots__ = ()


def q41_packed_bytes(n: int, k: int) -> int:
    return int(lib().q4_1_packed_bytes(int(n), int(k)))


def q41_quantize(w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 W [N, K] on the device -> asymmetric blocks [N, K/32, 20] (uint8)."""
    _dev(w, "w", torch.float32)
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    if out is None:
        out = torch.empty((n, max(k // 32, 0), Q41_BLOCK_BYTES), dtype=torch.uint8, device=w.device)
    _dev(out, "out", torch.uint8)
    if out.numel() != n * (k // 32) * Q41_BLOCK_BYTES:
        raise ValueError("out has the wrong size")
    _same_device(w, out, "out")
    with torch.cuda.device(w.device):
        _check(lib().q4_1_quantize(w.data_ptr(), n, k, out.data_ptr(), _stream(w.device)), "q4_1_quantize")
    return out


def q41_pack(blocks: torch.Tensor, n: int, k: int) -> PackedWeightQ41:
    """Asymmetric blocks (uint8, N*K/32*20 elements, on the device) -> PackedWeightQ41."""
    _dev(blocks, "blocks", torch.uint8)
    if blocks.numel() != int(n) * (int(k) // 32) * Q41_BLOCK_BYTES:
        raise ValueError(f"blocks must hold {int(n) * (int(k) // 32) * Q41_BLOCK_BYTES} bytes for [{n}, {k}]")
    nbytes = q41_packed_bytes(n, k)
    if nbytes == 0:
        raise ValueError(f"invalid shape [{n}, {k}]")
    out = torch.empty(nbytes, dtype=torch.uint8, device=blocks.device)
    with torch.cuda.device(blocks.device):
        _check(lib().q4_1_pack(blocks.data_ptr(), n, k, out.data_ptr(), _stream(blocks.device)), "q4_1_pack")
    return PackedWeightQ41(out, n, k)


def q41_dequant(pw: PackedWeightQ41) -> torch.Tensor:
    out = torch.empty((pw.n, pw.k), dtype=torch.float32, device=pw.device)
    with torch.cuda.device(pw.device):
        _check(lib().q4_1_dequant(pw.data.data_ptr(), pw.n, pw.k, out.data_ptr(), _stream(pw.device)),
               "q4_1_dequant")
    return out


def q41_linear(x: torch.Tensor, pw: PackedWeightQ41, out: torch.Tensor | None = None) -> torch.Tensor:
    """y [M, N] fp32 = x [M, K] bf16 times W^T for an asymmetric packed W."""
    if not isinstance(pw, PackedWeightQ41):
        raise ValueError("pw must be an asymmetric packed weight (q41_pack)")
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.shape[1] != pw.k:
        raise ValueError(f"x must be [M, {pw.k}]")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, pw.n), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if tuple(out.shape) != (m, pw.n):
        raise ValueError("out has the wrong shape")
    _same_device(x, pw.data, "pw")
    _same_device(x, out, "out")
    with torch.cuda.device(x.device):
        _check(lib().q4_1_linear(x.data_ptr(), m, pw.data.data_ptr(), pw.n, pw.k, out.data_ptr(), _stream(x.device)),
               "q4_1_linear")
    return out


def q41_linear_kernel(m: int, k: int, n: int) -> str:
    """Name of the kernel q4_1_linear runs for (M, K, N)."""
    return lib().q4_1_linear_kernel(int(m), int(k), int(n)).decode()


def time_next_launch(start: "torch.cuda.Event", stop: "torch.cuda.Event") -> None:
    """Arm this thread's next linear, SwiGLU or embedding (either table form) launch to record
    start/stop at its kernel's own start and end (events must already exist:
    record them once first)."""
    _check(lib().q4_0_time_next_launch(start.cuda_event, stop.cuda_event), "q4_0_time_next_launch")


def linear_kernel(m: int, k: int, n) -> str:
    """Name of the kernel q4_0_linear_multi runs for (M, K) over segments of
    n rows (an int for a single q4_0_linear, or a sequence of segment rows)."""
    ns = [int(n)] if isinstance(n, int) else [int(v) for v in n]
    arr = (ctypes.c_int64 * max(len(ns), 1))(*ns)
    return lib().q4_0_linear_kernel(int(m), int(k), arr, len(ns)).decode()


def linear_swiglu_kernel(m: int, k: int) -> str:
    """Name of the kernel q4_0_linear_swiglu runs for (M, K)."""
    return lib().q4_0_linear_swiglu_kernel(int(m), int(k)).decode()
