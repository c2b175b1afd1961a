// Internal declarations shared by the host-side ABI and the kernel files.
// Not part of the public ABI (that is include/q4_0.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

// Layout constants of the packed ("CDNA4 tiled") Q4_0 format.
constexpr int kQK = 32;            // weights per block
constexpr int kBlockBytes = 18;    // fp16 d + 16 code bytes (GGUF)
constexpr int kTileRows = 16;      // rows per super-tile
constexpr int kTileBlocks = 4;     // blocks per super-tile
constexpr int kTileK = 128;        // k per super-tile
constexpr int kTileNibBytes = 1024;
constexpr int kTileScales = 64;    // fp16 scales per super-tile
constexpr int kMaxSegments = 8;
constexpr int kQ41BlockBytes = 20; // asymmetric block: fp16 d, fp16 m + 16 code bytes

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

struct PackedDims {
    int64_t N, K, Np, Kp, KT, RT;
    explicit PackedDims(int64_t n, int64_t k)
        : N(n), K(k), Np(round_up(n, kTileRows)), Kp(round_up(k, kTileK)),
          KT(round_up(k, kTileK) / kTileK), RT(round_up(n, kTileRows) / kTileRows) {}
    int64_t nib_bytes() const { return Np * Kp / 2; }
    int64_t total_bytes() const { return Np * (Kp / kQK) * kBlockBytes; }
    int64_t q41_total_bytes() const { return Np * (Kp / kQK) * kQ41BlockBytes; }
};

// One weight matrix of a (possibly fused) launch, as the kernels see it.
struct Segment {
    const uint8_t *nib;      // nibble plane
    const uint16_t *scales;  // scale plane (fp16 bits)
    const uint16_t *offsets; // offset plane (fp16 bits; asymmetric layout only)
    float *y;                // [M, N] row-major
    int32_t N;               // true rows of W (= columns of y)
    int32_t RT;              // padded rows / 16
    int32_t tile_begin;      // first work tile of this segment in the launch
};

struct LinearArgs {
    const uint16_t *x;       // bf16 bits [M, K]
    int32_t M;
    int32_t K;               // true K (multiple of 32)
    int32_t KT;              // padded K / 128
    int32_t nseg;
    int32_t y_bf16;          // gated launches: store h as bf16 (RNE) instead of fp32
    Segment seg[kMaxSegments];
};

// Launchers (return hipError_t from the launch).
hipError_t launch_quantize(const float *w, int64_t N, int64_t K, uint8_t *out, hipStream_t s);
hipError_t launch_quantize_bf16(const uint16_t *w, int64_t N, int64_t K, uint8_t *out, hipStream_t s);
hipError_t launch_pack(const uint8_t *gguf, int64_t N, int64_t K, uint8_t *packed, hipStream_t s);
hipError_t launch_unpack(const uint8_t *packed, int64_t N, int64_t K, uint8_t *gguf, hipStream_t s);
hipError_t launch_dequant(const uint8_t *packed, int64_t N, int64_t K, float *w, hipStream_t s);
hipError_t launch_q41_quantize(const float *w, int64_t N, int64_t K, uint8_t *out, hipStream_t s);
hipError_t launch_q41_pack(const uint8_t *blocks, int64_t N, int64_t K, uint8_t *packed, hipStream_t s);
hipError_t launch_q41_dequant(const uint8_t *packed, int64_t N, int64_t K, float *w, hipStream_t s);
hipError_t launch_embed(const uint8_t *packed, int64_t N, int64_t K, const int32_t *ids, int64_t n_ids,
                        float *out, hipStream_t s);
hipError_t launch_embed_gguf(const uint8_t *gguf, int64_t N, int64_t K, const int32_t *ids, int64_t n_ids,
                             float *out, hipStream_t s);

// Runs the fused linear over all segments of `a` (segments' tile_begin is
// filled in by the launcher).
hipError_t launch_linear(LinearArgs a, hipStream_t s);

// Name of the kernel instantiation launch_linear picks for a launch (M, K
// and, above 64 rows, the segments' RT and the current device's CU count).
const char *linear_config_name(const LinearArgs &a);

// The asymmetric layout's linear (one segment, offsets set).
hipError_t launch_linear_q41(LinearArgs a, hipStream_t s);
const char *linear_q41_config_name(const LinearArgs &a);

// The gated launch: segment 0 is gate (its y receives silu(gate) * up),
// segment 1 is up, of the same shape; tile_begin is filled in here too.
hipError_t launch_linear_glu(LinearArgs a, hipStream_t s);
const char *linear_glu_config_name(int64_t M, int64_t K);

// Reference streaming read (measurement support): workgroups a read of
// `bytes` launches, and the launch (sink holds one word per workgroup).
int64_t reference_read_workgroups(int64_t bytes);
int64_t reference_read_sink_words(int64_t bytes);   // one word per thread: 256 per workgroup
hipError_t launch_reference_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s);

// The prefill GEMM's arithmetic alone (measurement support): threads of a
// launch (sink holds one float per thread) and the launch, mode 0-2.
int64_t reference_mfma_threads();
hipError_t launch_reference_mfma(int mode, int iters, float *sink, hipStream_t s);

// Makes the calling thread's next linear, gated or embedding launch record
// `start` / `stop` at its kernel's start and end.
void arm_launch_events(hipEvent_t start, hipEvent_t stop);
// Takes (and disarms) the calling thread's armed events; false if none.
bool take_launch_events(hipEvent_t &start, hipEvent_t &stop);

}  // namespace q4
