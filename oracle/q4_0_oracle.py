"""Plain CPU oracle for the Q4_0 weight-only linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

What the oracle computes, and where each step comes from:

* The weight format is GGUF Q4_0, the format named for the quantized Voxtral
  checkpoints ("Voxtral Mini 4B Realtime (Rust) -- Shannon-Prime Fork",
  section "RTF Benchmark Results", which lists the Q4_0 GGUF model; and the
  hakusoku summary page "Voxtral Mini 4B Realtime 概要", section "推論パス").
  A block holds 32 consecutive weights of one output row: an
  fp16 scale d followed by 16 bytes of 4-bit codes q, and a weight decodes as
  w = (q - 8) * d.  Byte j of the 16 holds element j in its low nibble and
  element j + 16 in its high nibble.  18 bytes per 32 weights is what the
  hakusoku page's section "線形演算・埋め込み" implies: the 131072 x 3072 Q4
  embedding is 216 MB there (131072 * 3072 / 32 * 18 B = 216 MiB).
* The layer is y = x W^T with W stored [N, K] (output rows, input columns)
  and x given as bf16, y returned in fp64 here (fp32 on the device).  The
  pages' engine folds the dequantization into a WGSL matmul shader (hakusoku,
  section "線形演算・埋め込み"); fusion changes no arithmetic, so the oracle is
  the unfused definition: dequantize, then multiply.
* Quantizer (host, off the timed path; the pages' counterpart is the offline
  script scripts/quantize_tts_gguf.py in "Model Preparation"): per block the
  signed element of largest magnitude (lowest index on ties) is amax,
  d = fp16(amax / -8), q = clamp(rint(w / d) + 8, 0, 15) with the division in
  fp32 and rint rounding half to even; a block whose fp16 d is zero stores
  d = +0 and q = 8.
* The gated MLP step after the fused gate/up projection (the Rust fork's
  "Architecture Summary" names SwiGLU right after the Q4 matmul; its "TTS"
  section fuses the gate and up projections).  The pages do not spell SwiGLU
  out; the reading taken is the usual one for this decoder family:
  h = silu(x Wg^T) * (x Wu^T) elementwise, silu(t) = t / (1 + e^-t).
* The Q4 embedding lookup: the 131072 x 3072 Q4 table stays on the GPU and
  token rows are looked up from it (hakusoku, "線形演算・埋め込み"; Rust fork,
  the browser constraints list: Q4 embeddings on the GPU with row lookups).
  A lookup returns the dequantized rows w[id, :] = (q - 8) * d, exact in
  fp32; an id outside [0, N) gives a row of NaN (a reading: the pages say
  nothing about bad ids, and NaN cannot be mistaken for a real row).
* The asymmetric variant.  The TTS card ("Voxtral-4B-TTS-2603-ExecuTorch-CUDA",
  opening paragraph) quantizes the same linears to group-wise asymmetric
  int4 but gives no group size, zero point or layout.  The reading taken is
  the asymmetric 4-bit block of the GGUF family the other pages use: 32
  consecutive k of one row share an fp16 scale d and an fp16 offset m, codes
  q are 4-bit unsigned and w = q * d + m.  A block is 20 bytes: d, then m
  (little-endian fp16), then the 16 code bytes in Q4_0's nibble order.  Its
  quantizer: mn, mx = min and max of the block, d = fp16((mx - mn) / 15),
  m = fp16(mn), q = clamp(rint((w - m) / d), 0, 15) with the stored fp16
  values and fp32 arithmetic (q = 0 where d is zero).  Its tolerance takes the
  magnitudes of both terms: 1e-3 * sum_k |x_k| (|q_k d| + |m|) + 1e-6.
* The packed device layout (the "CDNA4 tiled layout") is restated here from
  its definition in include/q4_0.h so the device repack can be checked byte
  for byte.  It is a permutation of the GGUF bytes, plus zero padding.

Everything here is NumPy on the CPU, in fp64 where it computes values.
"""

from __future__ import annotations

import numpy as np

QK = 32              # weights per Q4_0 block
BLOCK_BYTES = 18     # 2 bytes fp16 scale + 16 bytes of nibbles

# Device layout granularity (include/q4_0.h, "Packed layout").
TILE_ROWS = 16       # output rows per super-tile
TILE_BLOCKS = 4      # Q4_0 blocks (of 32 k) per super-tile
TILE_K = TILE_BLOCKS * QK          # 128
TILE_NIB_BYTES = 1024              # 16 rows * 4 blocks * 16 B
TILE_SCALE_BYTES = 128             # 16 rows * 4 blocks * 2 B


# ----------------------------------------------------------------- bf16 input
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp64 exactly.

    A bf16 value is the top half of an fp32 value, so shifting the 16 bits
    into the high half of a 32-bit word gives the fp32 value with the same
    number; fp32 -> fp64 is exact.
    """
    u16 = np.ascontiguousarray(bits).view(np.uint16)
    u32 = u16.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


# ------------------------------------------------------------ GGUF Q4_0 block
def gguf_decode(blocks: np.ndarray, n: int, k: int):
    """Split GGUF Q4_0 bytes [n, k/32, 18] into (d fp16 [n, k/32], q uint8 [n, k]).

    Bytes 0-1 of a block are d, little-endian fp16.  Of the 16 code bytes,
    byte j carries q[j] in bits 0-3 and q[j+16] in bits 4-7.
    """
    if k % QK:
        raise ValueError("K must be a multiple of 32")
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(n, k // QK, BLOCK_BYTES)
    d = b[:, :, 0:2].copy().view("<f2").reshape(n, k // QK)
    codes = b[:, :, 2:18]
    q = np.empty((n, k // QK, QK), dtype=np.uint8)
    q[:, :, 0:16] = codes & 0x0F
    q[:, :, 16:32] = codes >> 4
    return d, q.reshape(n, k)


def gguf_encode(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Inverse of gguf_decode: (d fp16 [n, k/32], q [n, k] in 0..15) -> bytes."""
    n, k = q.shape
    if k % QK:
        raise ValueError("K must be a multiple of 32")
    if q.max(initial=0) > 15:
        raise ValueError("codes must be 4-bit")
    qb = q.astype(np.uint8).reshape(n, k // QK, QK)
    out = np.empty((n, k // QK, BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = np.ascontiguousarray(d, dtype="<f2").reshape(n, k // QK, 1).view(np.uint8)
    out[:, :, 2:18] = qb[:, :, 0:16] | (qb[:, :, 16:32] << 4)
    return out


def gguf_bytes(n: int, k: int) -> int:
    """Size of an [n, k] Q4_0 matrix in GGUF form."""
    return n * (k // QK) * BLOCK_BYTES


# ------------------------------------------------------------------- dequant
def dequantize(blocks: np.ndarray, n: int, k: int) -> np.ndarray:
    """w = (q - 8) * d, evaluated in fp32 as the device does.

    The product is exact in fp32: |q - 8| <= 8 needs 4 significant bits and an
    fp16 d at most 11, so (q - 8) * d needs at most 15 of fp32's 24.
    """
    d, q = gguf_decode(blocks, n, k)
    qf = q.astype(np.float32) - np.float32(8)
    df = np.repeat(d.astype(np.float32), QK, axis=1)
    return qf * df


# --------------------------------------------------------------------- linear
def linear(x_bits: np.ndarray, blocks: np.ndarray, n: int, k: int,
           chunk_rows: int = 8192) -> np.ndarray:
    """y[m, j] = sum_k x[m, k] * w[j, k] in fp64; x given as bf16 bits [m, k].

    Every product of a bf16 x and a dequantized weight is exact in fp64; only
    the summation rounds.  Rows of W are processed in chunks to bound memory.
    """
    x = bf16_bits_to_f64(x_bits).reshape(-1, k)
    m = x.shape[0]
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(n, k // QK, BLOCK_BYTES)
    y = np.empty((m, n), dtype=np.float64)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        w = dequantize(b[r0:r1], r1 - r0, k).astype(np.float64)
        y[:, r0:r1] = x @ w.T
    return y


def error_bound(x_bits: np.ndarray, blocks: np.ndarray, n: int, k: int,
                chunk_rows: int = 8192) -> np.ndarray:
    """Per-output tolerance 1e-3 * sum_k |x_k * w_k| + 1e-6 (fp64)."""
    x = np.abs(bf16_bits_to_f64(x_bits).reshape(-1, k))
    m = x.shape[0]
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(n, k // QK, BLOCK_BYTES)
    out = np.empty((m, n), dtype=np.float64)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        w = np.abs(dequantize(b[r0:r1], r1 - r0, k).astype(np.float64))
        out[:, r0:r1] = x @ w.T
    return 1e-3 * out + 1e-6


def linear_with_bound(x_bits: np.ndarray, blocks: np.ndarray, n: int, k: int,
                      chunk_rows: int = 8192):
    """(linear(...), error_bound(...)) with each chunk of rows dequantized
    once: the same fp64 products and sums as the two functions, for checks
    of every output element of large matrices."""
    x = bf16_bits_to_f64(x_bits).reshape(-1, k)
    ax = np.abs(x)
    m = x.shape[0]
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(n, k // QK, BLOCK_BYTES)
    y = np.empty((m, n), dtype=np.float64)
    s = np.empty((m, n), dtype=np.float64)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        w = dequantize(b[r0:r1], r1 - r0, k).astype(np.float64)
        y[:, r0:r1] = x @ w.T
        s[:, r0:r1] = ax @ np.abs(w).T
    return y, 1e-3 * s + 1e-6


def linear_rows(x_bits: np.ndarray, blocks: np.ndarray, n: int, k: int,
                rows: np.ndarray):
    """(y, bound) restricted to the output columns `rows` (sampled checks)."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(n, k // QK, BLOCK_BYTES)
    sub = b[np.asarray(rows)]
    nr = sub.shape[0]
    return linear(x_bits, sub, nr, k), error_bound(x_bits, sub, nr, k)


# ------------------------------------------------------------------- SwiGLU
def silu(t) -> np.ndarray:
    """silu(t) = t * sigmoid(t) = t / (1 + e^-t) in fp64.

    Evaluated as t / (1 + e^-t) for t >= 0 and t * e^t / (1 + e^t) for t < 0,
    so that no exponential overflows.
    """
    t = np.asarray(t, dtype=np.float64)
    out = np.empty_like(t)
    pos = t >= 0
    out[pos] = t[pos] / (1.0 + np.exp(-t[pos]))
    e = np.exp(t[~pos])
    out[~pos] = t[~pos] * e / (1.0 + e)
    return out


SILU_SLOPE_MAX = 1.1   # sup |silu'(t)| = 1.0998... (at t near 2.4)


def swiglu(x_bits: np.ndarray, gate_blocks: np.ndarray, up_blocks: np.ndarray,
           n: int, k: int) -> np.ndarray:
    """h[m, j] = silu(g[m, j]) * u[m, j], g = x Wg^T, u = x Wu^T, in fp64."""
    g = linear(x_bits, gate_blocks, n, k)
    u = linear(x_bits, up_blocks, n, k)
    return silu(g) * u


def swiglu_bound(x_bits: np.ndarray, gate_blocks: np.ndarray, up_blocks: np.ndarray,
                 n: int, k: int) -> np.ndarray:
    """Tolerance on h when the device's g~ and u~ each meet the linear bound.

    With |g~ - g| <= bg and |u~ - u| <= bu (bg, bu from error_bound):
      |silu(g~) u~ - silu(g) u| <= |silu(g~) - silu(g)| |u~| + |silu(g)| |u~ - u|
                                <= 1.1 bg (|u| + bu) + |silu(g)| bu,
    since |silu'| <= 1.1 everywhere.  A relative 1e-5 of |h| covers the fp32
    evaluation of the exponential, the division and the product.
    """
    g = linear(x_bits, gate_blocks, n, k)
    u = linear(x_bits, up_blocks, n, k)
    bg = error_bound(x_bits, gate_blocks, n, k)
    bu = error_bound(x_bits, up_blocks, n, k)
    sg = silu(g)
    return SILU_SLOPE_MAX * bg * (np.abs(u) + bu) + np.abs(sg) * bu + 1e-5 * np.abs(sg * u)


def swiglu_rows(x_bits: np.ndarray, gate_blocks: np.ndarray, up_blocks: np.ndarray,
                n: int, k: int, rows: np.ndarray):
    """(h, bound) restricted to the output columns `rows` (sampled checks)."""
    gb = np.ascontiguousarray(gate_blocks, dtype=np.uint8).reshape(n, k // QK, BLOCK_BYTES)[np.asarray(rows)]
    ub = np.ascontiguousarray(up_blocks, dtype=np.uint8).reshape(n, k // QK, BLOCK_BYTES)[np.asarray(rows)]
    nr = gb.shape[0]
    return swiglu(x_bits, gb, ub, nr, k), swiglu_bound(x_bits, gb, ub, nr, k)


# ----------------------------------------------------------------- embedding
def embed(blocks: np.ndarray, n: int, k: int, ids) -> np.ndarray:
    """Rows ids[t] of the dequantized table (fp32, exact); NaN rows for ids
    outside [0, n)."""
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(n, k // QK, BLOCK_BYTES)
    ok = (ids >= 0) & (ids < n)
    out = np.full((ids.size, k), np.nan, dtype=np.float32)
    if ok.any():
        out[ok] = dequantize(b[ids[ok]], int(ok.sum()), k)
    return out


# ------------------------------------------------------------------ quantizer
def quantize(w: np.ndarray) -> np.ndarray:
    """fp32 W [n, k] -> GGUF Q4_0 bytes [n, k/32, 18] by the rule in the header."""
    w32 = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w32.shape
    if k % QK:
        raise ValueError("K must be a multiple of 32")
    wb = w32.reshape(n, k // QK, QK)
    idx = np.argmax(np.abs(wb), axis=2)                     # first maximum
    amax = np.take_along_axis(wb, idx[:, :, None], axis=2)[:, :, 0]
    d16 = (amax / np.float32(-8.0)).astype(np.float16)      # fp32 divide, RNE to fp16
    df = d16.astype(np.float32)
    zero = df == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(wb / df[:, :, None]) + np.float32(8.0)
    r = np.clip(r, np.float32(0.0), np.float32(15.0))
    r = np.where(zero[:, :, None], np.float32(8.0), r)
    q = r.astype(np.uint8).reshape(n, k)
    d16 = np.where(zero, np.float16(0.0), d16)
    return gguf_encode(d16, q)


# ---------------------------------------------- asymmetric variant (Q4_1)
Q41_BLOCK_BYTES = 20     # fp16 d, fp16 m, 16 bytes of nibbles


def q41_decode(blocks: np.ndarray, n: int, k: int):
    """Split asymmetric blocks [n, k/32, 20] into (d fp16, m fp16 [n, k/32],
    q uint8 [n, k]); code bytes are in Q4_0's nibble order."""
    if k % QK:
        raise ValueError("K must be a multiple of 32")
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(n, k // QK, Q41_BLOCK_BYTES)
    d = b[:, :, 0:2].copy().view("<f2").reshape(n, k // QK)
    m = b[:, :, 2:4].copy().view("<f2").reshape(n, k // QK)
    codes = b[:, :, 4:20]
    q = np.empty((n, k // QK, QK), dtype=np.uint8)
    q[:, :, 0:16] = codes & 0x0F
    q[:, :, 16:32] = codes >> 4
    return d, m, q.reshape(n, k)


def q41_encode(d: np.ndarray, m: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Inverse of q41_decode."""
    n, k = q.shape
    if k % QK:
        raise ValueError("K must be a multiple of 32")
    if q.max(initial=0) > 15:
        raise ValueError("codes must be 4-bit")
    qb = q.astype(np.uint8).reshape(n, k // QK, QK)
    out = np.empty((n, k // QK, Q41_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = np.ascontiguousarray(d, dtype="<f2").reshape(n, k // QK, 1).view(np.uint8)
    out[:, :, 2:4] = np.ascontiguousarray(m, dtype="<f2").reshape(n, k // QK, 1).view(np.uint8)
    out[:, :, 4:20] = qb[:, :, 0:16] | (qb[:, :, 16:32] << 4)
    return out


def q41_dequantize(blocks: np.ndarray, n: int, k: int) -> np.ndarray:
    """w = q * d + m in fp64 (exact: q * d needs 15 bits, and the sum of two
    values of fp16 origin fits the 53 bits of fp64)."""
    d, m, q = q41_decode(blocks, n, k)
    dd = np.repeat(d.astype(np.float64), QK, axis=1)
    mm = np.repeat(m.astype(np.float64), QK, axis=1)
    return q.astype(np.float64) * dd + mm


def q41_linear_with_bound(x_bits: np.ndarray, blocks: np.ndarray, n: int, k: int,
                          chunk_rows: int = 8192):
    """(y, bound) for the asymmetric format: y = x W^T in fp64 with
    W = q41_dequantize(...), bound = 1e-3 * sum_k |x_k| (|q_k d| + |m|) + 1e-6."""
    x = bf16_bits_to_f64(x_bits).reshape(-1, k)
    ax = np.abs(x)
    nrow = x.shape[0]
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(n, k // QK, Q41_BLOCK_BYTES)
    y = np.empty((nrow, n), dtype=np.float64)
    s = np.empty((nrow, n), dtype=np.float64)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        d, m, q = q41_decode(b[r0:r1], r1 - r0, k)
        dd = np.repeat(d.astype(np.float64), QK, axis=1)
        mm = np.repeat(m.astype(np.float64), QK, axis=1)
        qd = q.astype(np.float64) * dd
        y[:, r0:r1] = x @ (qd + mm).T
        s[:, r0:r1] = ax @ (np.abs(qd) + np.abs(mm)).T
    return y, 1e-3 * s + 1e-6


def q41_quantize(w: np.ndarray) -> np.ndarray:
    """fp32 W [n, k] -> asymmetric blocks by the rule in the module header."""
    w32 = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w32.shape
    if k % QK:
        raise ValueError("K must be a multiple of 32")
    wb = w32.reshape(n, k // QK, QK)
    mn = wb.min(axis=2)
    mx = wb.max(axis=2)
    d16 = ((mx - mn) / np.float32(15.0)).astype(np.float16)    # fp32 divide, RNE to fp16
    m16 = mn.astype(np.float16)
    df = d16.astype(np.float32)
    zero = df == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint((wb - m16.astype(np.float32)[:, :, None]) / df[:, :, None])
    r = np.clip(r, np.float32(0.0), np.float32(15.0))
    r = np.where(zero[:, :, None], np.float32(0.0), r)
    return q41_encode(d16, m16, r.astype(np.uint8).reshape(n, k))


# ----------------------------------------------------- device (packed) layout
def quantize_bf16(w_bits: np.ndarray) -> np.ndarray:
    """bf16 W (bit patterns [n, k]) -> GGUF Q4_0 bytes: each value widened to
    fp32 exactly (bf16 is the top half of an fp32), then the rule of
    quantize() unchanged."""
    return quantize(bf16_bits_to_f64(w_bits).astype(np.float32))


def padded_dims(n: int, k: int):
    """(Np, Kp): rows rounded up to 16, columns up to 128."""
    return -(-n // TILE_ROWS) * TILE_ROWS, -(-k // TILE_K) * TILE_K


def packed_bytes(n: int, k: int) -> int:
    np_, kp = padded_dims(n, k)
    return np_ * (kp // QK) * BLOCK_BYTES


def pack(blocks: np.ndarray, n: int, k: int) -> np.ndarray:
    """GGUF bytes -> packed device layout, following include/q4_0.h.

    Written as explicit index arithmetic over (row, block, k) so it can be
    compared with the header text by eye:

      nibble plane, super-tile (rt, kt) at byte ((rt * KT + kt) * 1024):
        row n = 16 rt + r, block b = 4 kt + i, element e (0..31) of the block,
        g = e // 8, j = e % 8:
        byte offset within the tile = g * 256 + r * 16 + i * 4 + j // 2,
        low nibble if j is even, high nibble if odd; stored value (q ^ 8).
      scale plane, starting at Np * Kp / 2:
        fp16 d of (n, b) at element index (rt * KT + kt) * 64 + r * 4 + i.
    """
    np_, kp = padded_dims(n, k)
    d, q = gguf_decode(blocks, n, k)
    qp = np.full((np_, kp), 8, dtype=np.uint8)
    qp[:n, :k] = q
    dp = np.zeros((np_, kp // QK), dtype=np.float16)
    dp[:n, :k // QK] = d
    kt_n = kp // TILE_K
    nib = np.zeros(np_ * kp // 2, dtype=np.uint8)
    sc = np.zeros(np_ * kp // QK, dtype=np.float16)
    code = (qp ^ 8).astype(np.uint8)
    # vectorised form of the loops described in the docstring
    rows = np.arange(np_)
    rt, r = rows // TILE_ROWS, rows % TILE_ROWS
    for b in range(kp // QK):
        kt, i = b // TILE_BLOCKS, b % TILE_BLOCKS
        tile_base = (rt * kt_n + kt) * TILE_NIB_BYTES
        for e in range(QK):
            g, j = e // 8, e % 8
            off = tile_base + g * 256 + r * 16 + i * 4 + j // 2
            val = code[:, b * QK + e]
            if j % 2 == 0:
                nib[off] |= val
            else:
                nib[off] |= val << 4
        sc[(rt * kt_n + kt) * 64 + r * 4 + i] = dp[:, b]
    return np.concatenate([nib, sc.view(np.uint8)])


def q41_packed_bytes(n: int, k: int) -> int:
    np_, kp = padded_dims(n, k)
    return np_ * (kp // QK) * Q41_BLOCK_BYTES


def q41_pack(blocks: np.ndarray, n: int, k: int) -> np.ndarray:
    """Asymmetric blocks -> packed device layout (include/q4_0.h, "Packed
    asymmetric layout"): pack()'s nibble and scale planes with the codes q
    themselves in the nibble slots (not q XOR 8) and d in the scale plane,
    then an offset plane with m at the same element index as d.  Padding
    blocks are all zero bytes (d = m = 0, q = 0)."""
    np_, kp = padded_dims(n, k)
    d, m, q = q41_decode(blocks, n, k)
    # pack() stores (code XOR 8) and pads with code 8: handing it q XOR 8 puts
    # q in every real slot and 0 in the padding
    front = pack(gguf_encode(d, q ^ 8), n, k)
    mp = np.zeros((np_, kp // QK), dtype=np.float16)
    mp[:n, :k // QK] = m
    kt_n = kp // TILE_K
    off = np.zeros(np_ * kp // QK, dtype=np.float16)
    rows = np.arange(np_)
    rt, r = rows // TILE_ROWS, rows % TILE_ROWS
    for b in range(kp // QK):
        kt, i = b // TILE_BLOCKS, b % TILE_BLOCKS
        off[(rt * kt_n + kt) * 64 + r * 4 + i] = mp[:, b]
    return np.concatenate([front, off.view(np.uint8)])
