/*
 * q4_0.h -- C ABI of libq4amd, a GGUF Q4_0 weight-only linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  The quantized Voxtral checkpoints store their linear
 * weights as GGUF Q4_0 ("Voxtral Mini 4B Realtime (Rust) -- Shannon-Prime
 * Fork", section "RTF Benchmark Results"; hakusoku summary "Voxtral Mini 4B
 * Realtime 概要", section "推論パス"), and
 * the Rust engine multiplies them with a shader that fuses dequantization into
 * the matmul (hakusoku summary, section "線形演算・埋め込み").  The format:
 * W is [N, K] (N outputs, K inputs, K a multiple of 32); each run of 32
 * consecutive k of one row is a block of 18 bytes -- an fp16 scale d
 * (little-endian) and 16 code bytes, byte j holding code q[j] in bits 0-3 and
 * q[j+16] in bits 4-7 -- and a weight is w = (q - 8) * d.  The layer computes
 *     y[m, n] = sum_k x[m, k] * w[n, k]
 * with x bf16 [M, K] row-major and y fp32 [M, N] row-major (overwritten, no
 * bias).  Fused QKV and fused gate/up projections (the Rust fork's TTS
 * section lists "fused QKV+gate/up projections") share x between several
 * weight matrices; q4_0_linear_multi does that in one launch.
 *
 * Conventions for every entry point.
 *   - Pointers named as device memory must be device (or managed) memory on
 *     the current HIP device; the caller owns every buffer.  The library
 *     allocates no device memory and keeps no data between calls: only
 *     per-device caches of the CU count and kernel occupancy, and the
 *     per-kernel LDS limits it raises once with hipFuncSetAttribute.
 *   - Output buffers must not overlap any input of the same call, nor each
 *     other; inputs may be shared freely, also by concurrent calls.
 *   - Entry points may be called from several host threads at once.  The
 *     timing hook (q4_0_time_next_launch) affects the calling thread only.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call that
 *     launches work is asynchronous on that stream; results are visible after
 *     the caller synchronizes it.
 *   - Every argument is checked before any HIP call.  On a bad argument the
 *     call returns a nonzero q4_status and launches nothing.  A failed launch
 *     returns Q4_ERR_HIP, and so does a shape inside the limits below whose
 *     launch would need more than 2^31 - 1 workgroups (only matrices far
 *     larger than any device memory).  A device fault surfaces at the
 *     caller's next synchronization.  Nothing aborts.
 *   - Device pointers to x, y, packed, GGUF blocks and fp32 weights must be
 *     16-byte aligned (any torch allocation is).  GGUF block buffers are
 *     N * K/32 * 18 bytes, contiguous.
 *   - Sizes: 1 <= N <= 2^30, 32 <= K <= 2^20, K % 32 == 0, 0 <= M <= 2^20.
 *     M == 0 is a successful no-op.
 *   - NaN or +-inf in x or in a scale d: an output is non-finite exactly
 *     where sum_k x[m,k] * ((q-8) * d) is (inf rather than NaN is possible
 *     when d is infinite, since d scales each 32-block's sum).
 */
#ifndef Q4_0_H
#define Q4_0_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    Q4_OK = 0,
    Q4_ERR_NULL = 1,      /* a required pointer is NULL                       */
    Q4_ERR_SHAPE = 2,     /* M, N or K out of range, or K % 32 != 0           */
    Q4_ERR_ALIGN = 3,     /* a device pointer is not 16-byte aligned          */
    Q4_ERR_SEGMENTS = 4,  /* nseg outside 1..8, or a bad segment entry        */
    Q4_ERR_HIP = 5        /* the HIP runtime reported an error at launch      */
} q4_status;

/* Static English text for a status code (never NULL). */
const char *q4_status_str(int status);

/*
 * Packed layout ("CDNA4 tiled Q4_0").  q4_0_pack rewrites GGUF blocks into
 * this layout once, at load time; q4_0_linear reads only this layout.
 *
 *   Np = N rounded up to 16, Kp = K rounded up to 128, KT = Kp / 128.
 *   Padding blocks have d = 0 and q = 8 (all their bytes are zero).
 *   A super-tile covers 16 rows x 4 blocks (128 k).  Super-tile (rt, kt),
 *   rt = n / 16, kt = b / 4 (b = k / 32), is stored at tile index
 *   T = rt * KT + kt.
 *
 *   Nibble plane, bytes [0, Np * Kp / 2):
 *     for row n = 16 rt + r, block b = 4 kt + i, element e = 8 g + j of the
 *     block (g = 0..3, j = 0..7), the code (q XOR 8) -- the 4-bit two's
 *     complement of q - 8 -- is at byte
 *         T * 1024 + g * 256 + r * 16 + i * 4 + j / 2,
 *     in the low nibble when j is even, the high nibble when j is odd.
 *     So lane (16 g + r) of a 64-lane wave reading 16 bytes at lane * 16
 *     receives, for blocks 4kt..4kt+3, elements 8g..8g+7 of row n, which is
 *     the B-operand slice of a 16x16x32 bf16 MFMA for that row and k range.
 *   Scale plane, bytes [Np * Kp / 2, Np * Kp / 2 + Np * Kp / 16):
 *     fp16 d of (n, b) at element index T * 64 + r * 4 + i.
 *
 *   Total size: Np * (Kp / 32) * 18 bytes (equal to the GGUF size when no
 *   padding is needed).
 */
size_t q4_0_packed_bytes(int64_t N, int64_t K);   /* 0 if N or K is invalid */

/*
 * Host-side quantizer counterpart, run on the device: fp32 W [N, K]
 * (row-major, device) -> GGUF Q4_0 blocks (device, N * K/32 * 18 bytes).
 * Per block: amax is the element of largest magnitude, keeping its sign
 * (lowest index on ties); d = fp16(amax / -8) rounded to nearest even;
 * q = clamp(rint(w / d) + 8, 0, 15), the division in fp32 and rint rounding
 * half to even; if the fp16 d is zero the block stores d = +0 and q = 8.
 * The pages quantize offline with scripts/quantize_tts_gguf.py (Rust fork,
 * "Model Preparation"); the rule above is the GGUF Q4_0 reading of it.
 * Inputs must be finite.  Bit-for-bit reproducible.
 */
q4_status q4_0_quantize(const float *w, int64_t N, int64_t K, void *gguf_blocks, void *stream);

/*
 * The same quantizer for bf16 weights (bit patterns, row-major [N, K] on the
 * device, 16-byte aligned): each value is widened to fp32 exactly (its bits
 * shifted into the top half) and the fp32 rule above applies unchanged, so
 * the result equals q4_0_quantize of the widened matrix byte for byte.
 * Validation and errors as for q4_0_quantize.
 */
q4_status q4_0_quantize_bf16(const void *w_bf16, int64_t N, int64_t K, void *gguf_blocks, void *stream);

/* GGUF Q4_0 blocks (device) -> packed layout (device, q4_0_packed_bytes). */
q4_status q4_0_pack(const void *gguf_blocks, int64_t N, int64_t K, void *packed, void *stream);

/* Exact inverse of q4_0_pack (padding dropped); for tests and export. */
q4_status q4_0_unpack(const void *packed, int64_t N, int64_t K, void *gguf_blocks, void *stream);

/* Dequantize a packed matrix to fp32 W [N, K] (device): w = (q - 8) * d,
 * exact in fp32.  For tests. */
q4_status q4_0_dequant(const void *packed, int64_t N, int64_t K, float *w, void *stream);

/*
 * Q4 embedding lookup (the Q4 table stays on the GPU and token rows are
 * looked up from it: hakusoku, "線形演算・埋め込み"; Rust fork, the browser
 * constraints list).  out[t, :] (fp32, device, [n_ids, K] row-major) = row
 * ids[t] of the packed table [N, K] dequantized, w = (q - 8) * d, exact (the
 * same values q4_0_dequant gives for that row).  ids: device int32[n_ids].
 * An id outside [0, N) yields a row of NaN (nothing is read for it).  The
 * table can be the one a linear uses (a tied LM head).  Sizes as for the
 * other calls, 0 <= n_ids <= 2^24; n_ids == 0 is a no-op.
 */
q4_status q4_0_embed(const void *packed, int64_t N, int64_t K, const int32_t *ids, int64_t n_ids,
                     float *out, void *stream);

/*
 * The same lookup on a table kept as GGUF Q4_0 blocks ([N, K/32, 18] bytes,
 * device, 16-byte aligned), where one row's blocks are contiguous.  A lookup
 * then reads only its rows' K/32 * 18 bytes; in the packed layout a row is
 * 16-byte pieces 256 bytes apart, and each piece costs a whole cache line
 * (about 9x the row's bytes measured from HBM).  Same result as q4_0_embed
 * on the packed form of the same table, bit for bit (NaN rows for bad ids);
 * same validation and limits.
 */
q4_status q4_0_embed_gguf(const void *gguf_blocks, int64_t N, int64_t K, const int32_t *ids, int64_t n_ids,
                          float *out, void *stream);

/*
 * y[M, N] (fp32, device) = x[M, K] (bf16, device) times W^T, W packed.
 * Accuracy: every product (q - 8) * x is formed exactly and scaled by d in
 * fp32; y is within 1e-3 * sum_k |x_k * w_k| + 1e-6 of the exact result for
 * any finite input whose result does not overflow fp32.  Deterministic:
 * the same inputs give the same bits on every call (no atomics).
 */
q4_status q4_0_linear(const void *x_bf16, int64_t M, const void *packed, int64_t N, int64_t K,
                      float *y, void *stream);

/* One weight matrix of a fused launch: packed weights [N, K], output y [M, N]. */
typedef struct {
    const void *packed;
    int64_t N;
    float *y;
} q4_0_segment;

/*
 * Several weight matrices sharing x and K in one launch (fused QKV: three
 * segments 4096/1024/1024; fused gate/up: two of 9216).  `segs` is host
 * memory with nseg entries, 1 <= nseg <= 8; each segment is validated like a
 * q4_0_linear call.  Each segment's result meets the q4_0_linear bound, and
 * equals a separate q4_0_linear call bit for bit whenever both run the same
 * kernel family (see q4_0_linear_kernel: the choice can depend on the total
 * tile count at M = 1 for very tall weights and at 17 rows and more).
 */
q4_status q4_0_linear_multi(const void *x_bf16, int64_t M, int64_t K, const q4_0_segment *segs,
                            int nseg, void *stream);

/*
 * Fused gate/up projection with the SwiGLU epilogue (the gated MLP of the
 * decoder: the Rust fork's "Architecture Summary" puts SwiGLU right after
 * the Q4 matmul, and its "TTS" section fuses the gate and up projections):
 *
 *   h[m, n] = silu(g[m, n]) * u[m, n],   g = x Wg^T,  u = x Wu^T,
 *   silu(t) = t / (1 + e^-t),
 *
 * with gate_packed (Wg) and up_packed (Wu) packed [N, K] matrices of the same
 * shape and h [M, N] (device, row-major): fp32 when h_bf16 == 0, bf16 (the
 * fp32 value rounded to nearest even, ready to be the x of the down
 * projection) when h_bf16 == 1; other values are Q4_ERR_SHAPE.  One launch;
 * g and u never reach memory, so the output is at most half the bytes of a
 * gate/up q4_0_linear_multi.  g and u are computed exactly as q4_0_linear
 * computes them, and silu and the product in fp32, so the fp32 h is within
 * 1.1 bg (|u| + bu) + |silu(g)| bu + 1e-5 |h| of the exact value, where bg
 * and bu are the q4_0_linear bounds of g and u (bf16: plus 2^-9 |h|).
 * Arguments are validated as for q4_0_linear (both weight pointers);
 * deterministic.
 */
q4_status q4_0_linear_swiglu(const void *x_bf16, int64_t M, int64_t K, const void *gate_packed,
                             const void *up_packed, int64_t N, void *h, int h_bf16, void *stream);

/* Name of the kernel instantiation q4_0_linear_swiglu runs for M and K
 * (static string; "" for an invalid M or K). */
const char *q4_0_linear_swiglu_kernel(int64_t M, int64_t K);

/*
 * Name of the kernel instantiation q4_0_linear_multi runs for M, K and the
 * segments' row counts N[0 .. nseg-1] (host array; q4_0_linear is nseg = 1).
 * The choice depends on M and K, and also on how many work tiles the segments
 * make against the current device's compute-unit count (256 is assumed when
 * no device answers): at M = 1 for very tall weights (a fixed-grid walk of
 * the same per-tile arithmetic), at 17-64 rows (the K-split decode kernel for
 * short weights, the GEMM for tall ones) and above 64 rows (the GEMM tile
 * shape).  A fused launch and separate launches of its segments give bitwise
 * equal results when they run the same kernel family (the tile shapes of the
 * GEMM add an output's block results in the same order, and so do the decode
 * kernels for one M); across families they agree within the stated bound.
 * Static string; "" for an invalid argument.  For reports that match timings
 * to kernel names.
 */
const char *q4_0_linear_kernel(int64_t M, int64_t K, const int64_t *N, int nseg);

/*
 * The asymmetric variant.  The TTS card ("Voxtral-4B-TTS-2603-ExecuTorch-CUDA",
 * opening paragraph) quantizes the same linears to group-wise asymmetric
 * int4 without giving the group size, zero point or layout; the reading
 * taken is the asymmetric block of the GGUF family: 32 consecutive k of one
 * row share an fp16 scale d and an fp16 offset m, codes q are 4-bit unsigned,
 * and w = q * d + m.  A block is 20 bytes: d, then m (little-endian fp16),
 * then 16 code bytes in the Q4_0 nibble order (byte j: q[j] in bits 0-3,
 * q[j+16] in bits 4-7).  Block buffers are N * K/32 * 20 bytes.
 *
 * Packed asymmetric layout: the Q4_0 packed layout's nibble plane with the
 * code q itself in each slot (not q XOR 8; padding slots 0), its scale plane
 * holding d, then an offset plane of the same size holding m at the same
 * element index as d.  Padding blocks are all zero bytes.  Total size
 * Np * (Kp / 32) * 20 bytes.
 *
 * q4_1_quantize: fp32 W [N, K] (device) -> blocks; per block mn and mx are
 * the smallest and largest w, d = fp16((mx - mn) / 15) and m = fp16(mn), both
 * rounded to nearest even, q = clamp(rint((w - m) / d), 0, 15) with the
 * stored values, fp32 arithmetic and ties to even (q = 0 where d is zero).
 * Inputs must be finite; bit-for-bit reproducible.
 * q4_1_pack / q4_1_dequant: as their Q4_0 counterparts (w = q * d + m rounded
 * once to fp32).
 * q4_1_linear: y[M, N] (fp32) = x[M, K] (bf16) times W^T, computed as
 * sum over blocks of d * (sum x q) + m * (sum x): each block's sum of x * q
 * and sum of x are formed by MFMAs; up to 4 rows each block then adds both
 * terms in fp32, above 4 rows the offsets' share of each run of 8 blocks is
 * one more MFMA over bf16 hi / lo parts of m (exact) and of the sums of x
 * (within 2^-16).  y is within 1e-3 * sum_k |x_k| (|q_k d| + |m|) + 1e-6 of
 * the exact result for finite inputs (both terms' magnitudes: q d and m may
 * cancel in w).  Deterministic; above 4 rows an output's bits do not depend
 * on M.  Sizes, validation and errors as for q4_0_linear.
 */
size_t q4_1_packed_bytes(int64_t N, int64_t K);   /* 0 if N or K is invalid */
q4_status q4_1_quantize(const float *w, int64_t N, int64_t K, void *blocks, void *stream);
q4_status q4_1_pack(const void *blocks, int64_t N, int64_t K, void *packed, void *stream);
q4_status q4_1_dequant(const void *packed, int64_t N, int64_t K, float *w, void *stream);
q4_status q4_1_linear(const void *x_bf16, int64_t M, const void *packed, int64_t N, int64_t K, float *y,
                      void *stream);
/* Name of the kernel q4_1_linear runs for M, K and N (static; "" if invalid). */
const char *q4_1_linear_kernel(int64_t M, int64_t K, int64_t N);

/*
 * Measurement support: a reference streaming read.  Reads `bytes` bytes at
 * src (device, 16-byte aligned, bytes a multiple of 16, 0 <= bytes <= 2^40)
 * with the 16-byte nontemporal loads the linear kernels use for weights, and
 * does nothing else with them: workgroup b (256 threads) reads the 64 KiB
 * from byte 65536 b, thread t the 16-byte chunks 4096 b + 256 p + t
 * (p = 0 .. 15), and writes the XOR of their 32-bit words (zero past
 * `bytes`) to sink word 256 b + t, so the reads cannot be elided; no
 * cross-lane work, barrier or other step follows the loads.  With
 * bytes == 0 it launches one workgroup that reads nothing: the cost of a
 * launch alone.  sink is device memory of q4_0_reference_read_words(bytes)
 * 32-bit words, 4-byte aligned.  Not a step of the method: the pages weigh
 * per-dispatch overheads against the work of short launches (Rust fork,
 * "Why L0 Is Faster"), and a benchmark uses this to put each linear launch
 * next to a launch that only moves the same bytes.  Asynchronous on stream;
 * q4_0_time_next_launch applies to it.  Errors as for the other calls.
 */
q4_status q4_0_reference_read(const void *src, int64_t bytes, void *sink, void *stream);

/* 32-bit words of sink a q4_0_reference_read of `bytes` writes (0 if bytes
 * is invalid). */
int64_t q4_0_reference_read_words(int64_t bytes);

/*
 * Measurement support: the prefill GEMM's arithmetic alone.  Each wave runs
 * `iterations` rounds of the 128-row GEMM tiles' inner loop on operands held
 * in registers -- 4 blocks, each 8 v_mfma_f32_16x16x32_bf16 sharing one B
 * fragment -- with no loads, stores or barriers, at 4 waves per SIMD:
 *   mode 0: the MFMAs alone, accumulating in the matrix pipe;
 *   mode 1: each MFMA's result rescaled into the fp32 accumulators by the
 *           block's scale (four FMAs per MFMA), as the exact method needs;
 *   mode 2: mode 1 plus the decode of each block's B fragment from its codes;
 *   mode 3: mode 0 plus four fp32 FMAs per MFMA on registers the MFMAs do not
 *           touch (mode 1's VALU work without its dependence on the MFMAs).
 * A launch runs q4_0_reference_mfma_threads() threads (4 workgroups of 256
 * per compute unit) and issues threads / 64 * iterations * 32 MFMAs of
 * 16 * 16 * 32 multiply-adds each; each thread writes one float to sink
 * (device memory of that many floats, 4-byte aligned).  1 <= iterations <=
 * 2^20 (one iteration takes about a microsecond on MI355X), 0 <= mode <= 3.
 * Not a step of the method: a benchmark uses it to
 * put the GEMM next to what its arithmetic allows apart from memory (the
 * pages weigh compute against bandwidth for this layer: Rust fork, "Why L0
 * Is Faster").  Asynchronous on stream; q4_0_time_next_launch applies to it.
 */
q4_status q4_0_reference_mfma(int mode, int64_t iterations, float *sink, void *stream);
int64_t q4_0_reference_mfma_threads(void);

/*
 * Measurement hook for benchmarks.  Arms the calling thread's next
 * q4_0_linear / q4_0_linear_multi / q4_0_linear_swiglu / q4_0_embed / q4_0_embed_gguf /
 * q4_1_linear / q4_0_reference_read / q4_0_reference_mfma launch so that
 * its kernel records
 * `start_event` when it starts executing and `stop_event` when it finishes
 * (hipExtLaunchKernelGGL); hipEventElapsedTime on the pair is then that
 * kernel's own duration, without launch gaps -- the quantity a kernel trace
 * reports.  Events are hipEvent_t created by the caller; either may be NULL.
 * One-shot: the arming is consumed by the next launch (or by a validation
 * failure of that call it is kept).  Not for use under stream capture.
 */
q4_status q4_0_time_next_launch(void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* Q4_0_H */
