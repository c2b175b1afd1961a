// extern "C" entry points of libq4amd (declared in include/q4_0.h).
// Every argument is validated here, before any HIP call, so the error paths
// are testable without a GPU.

#include "q4_0.h"

#include "q4_0_internal.h"

namespace {

constexpr int64_t kMaxN = int64_t(1) << 30;
constexpr int64_t kMaxK = int64_t(1) << 20;
constexpr int64_t kMaxM = int64_t(1) << 20;

bool shape_ok(int64_t N, int64_t K) {
    return N >= 1 && N <= kMaxN && K >= q4::kQK && K <= kMaxK && K % q4::kQK == 0;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

q4_status from_hip(hipError_t e) { return e == hipSuccess ? Q4_OK : Q4_ERR_HIP; }

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

q4::Segment make_segment(const void *packed, int64_t N, int64_t K, float *y) {
    const q4::PackedDims pd(N, K);
    q4::Segment sg;
    sg.nib = static_cast<const uint8_t *>(packed);
    sg.scales = reinterpret_cast<const uint16_t *>(static_cast<const uint8_t *>(packed) + pd.nib_bytes());
    sg.offsets = nullptr;
    sg.y = y;
    sg.N = static_cast<int32_t>(N);
    sg.RT = static_cast<int32_t>(pd.RT);
    sg.tile_begin = 0;
    return sg;
}

}  // namespace

extern "C" {

const char *q4_status_str(int status) {
    switch (status) {
        case Q4_OK: return "ok";
        case Q4_ERR_NULL: return "a required pointer is NULL";
        case Q4_ERR_SHAPE: return "shape out of range (need 1<=N<=2^30, 32<=K<=2^20, K%32==0, 0<=M<=2^20)";
        case Q4_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
        case Q4_ERR_SEGMENTS: return "bad segment list (need 1<=nseg<=8 and valid entries)";
        case Q4_ERR_HIP: return "HIP runtime error at launch";
        default: return "unknown status";
    }
}

size_t q4_0_packed_bytes(int64_t N, int64_t K) {
    if (!shape_ok(N, K)) return 0;
    return static_cast<size_t>(q4::PackedDims(N, K).total_bytes());
}

q4_status q4_0_quantize(const float *w, int64_t N, int64_t K, void *gguf_blocks, void *stream) {
    if (!shape_ok(N, K)) return Q4_ERR_SHAPE;
    if (!w || !gguf_blocks) return Q4_ERR_NULL;
    if (!aligned16(w) || !aligned16(gguf_blocks)) return Q4_ERR_ALIGN;
    return from_hip(q4::launch_quantize(w, N, K, static_cast<uint8_t *>(gguf_blocks), as_stream(stream)));
}

q4_status q4_0_quantize_bf16(const void *w_bf16, int64_t N, int64_t K, void *gguf_blocks, void *stream) {
    if (!shape_ok(N, K)) return Q4_ERR_SHAPE;
    if (!w_bf16 || !gguf_blocks) return Q4_ERR_NULL;
    if (!aligned16(w_bf16) || !aligned16(gguf_blocks)) return Q4_ERR_ALIGN;
    return from_hip(q4::launch_quantize_bf16(static_cast<const uint16_t *>(w_bf16), N, K,
                                             static_cast<uint8_t *>(gguf_blocks), as_stream(stream)));
}

q4_status q4_0_pack(const void *gguf_blocks, int64_t N, int64_t K, void *packed, void *stream) {
    if (!shape_ok(N, K)) return Q4_ERR_SHAPE;
    if (!gguf_blocks || !packed) return Q4_ERR_NULL;
    if (!aligned16(gguf_blocks) || !aligned16(packed)) return Q4_ERR_ALIGN;
    return from_hip(q4::launch_pack(static_cast<const uint8_t *>(gguf_blocks), N, K,
                                    static_cast<uint8_t *>(packed), as_stream(stream)));
}

q4_status q4_0_unpack(const void *packed, int64_t N, int64_t K, void *gguf_blocks, void *stream) {
    if (!shape_ok(N, K)) return Q4_ERR_SHAPE;
    if (!gguf_blocks || !packed) return Q4_ERR_NULL;
    if (!aligned16(gguf_blocks) || !aligned16(packed)) return Q4_ERR_ALIGN;
    return from_hip(q4::launch_unpack(static_cast<const uint8_t *>(packed), N, K,
                                      static_cast<uint8_t *>(gguf_blocks), as_stream(stream)));
}

q4_status q4_0_dequant(const void *packed, int64_t N, int64_t K, float *w, void *stream) {
    if (!shape_ok(N, K)) return Q4_ERR_SHAPE;
    if (!w || !packed) return Q4_ERR_NULL;
    if (!aligned16(w) || !aligned16(packed)) return Q4_ERR_ALIGN;
    return from_hip(q4::launch_dequant(static_cast<const uint8_t *>(packed), N, K, w, as_stream(stream)));
}

q4_status q4_0_embed(const void *packed, int64_t N, int64_t K, const int32_t *ids, int64_t n_ids,
                     float *out, void *stream) {
    if (!shape_ok(N, K) || n_ids < 0 || n_ids > (int64_t(1) << 24)) return Q4_ERR_SHAPE;
    if (n_ids == 0) return Q4_OK;
    if (!packed || !ids || !out) return Q4_ERR_NULL;
    if (!aligned16(packed) || !aligned16(out) || (reinterpret_cast<uintptr_t>(ids) & 3u)) return Q4_ERR_ALIGN;
    return from_hip(q4::launch_embed(static_cast<const uint8_t *>(packed), N, K, ids, n_ids, out,
                                     as_stream(stream)));
}

q4_status q4_0_embed_gguf(const void *gguf_blocks, int64_t N, int64_t K, const int32_t *ids, int64_t n_ids,
                          float *out, void *stream) {
    if (!shape_ok(N, K) || n_ids < 0 || n_ids > (int64_t(1) << 24)) return Q4_ERR_SHAPE;
    if (n_ids == 0) return Q4_OK;
    if (!gguf_blocks || !ids || !out) return Q4_ERR_NULL;
    if (!aligned16(gguf_blocks) || !aligned16(out) || (reinterpret_cast<uintptr_t>(ids) & 3u)) return Q4_ERR_ALIGN;
    return from_hip(q4::launch_embed_gguf(static_cast<const uint8_t *>(gguf_blocks), N, K, ids, n_ids, out,
                                          as_stream(stream)));
}

q4_status q4_0_linear(const void *x_bf16, int64_t M, const void *packed, int64_t N, int64_t K, float *y,
                      void *stream) {
    q4_0_segment seg;
    seg.packed = packed;
    seg.N = N;
    seg.y = y;
    return q4_0_linear_multi(x_bf16, M, K, &seg, 1, stream);
}

q4_status q4_0_linear_multi(const void *x_bf16, int64_t M, int64_t K, const q4_0_segment *segs, int nseg,
                            void *stream) {
    if (!segs) return Q4_ERR_NULL;
    if (nseg < 1 || nseg > q4::kMaxSegments) return Q4_ERR_SEGMENTS;
    if (M < 0 || M > kMaxM) return Q4_ERR_SHAPE;
    for (int i = 0; i < nseg; ++i)
        if (!shape_ok(segs[i].N, K)) return Q4_ERR_SHAPE;
    if (M == 0) return Q4_OK;
    if (!x_bf16) return Q4_ERR_NULL;
    if (!aligned16(x_bf16)) return Q4_ERR_ALIGN;
    for (int i = 0; i < nseg; ++i) {
        if (!segs[i].packed || !segs[i].y) return Q4_ERR_NULL;
        if (!aligned16(segs[i].packed) || !aligned16(segs[i].y)) return Q4_ERR_ALIGN;
    }
    q4::LinearArgs a;
    a.x = static_cast<const uint16_t *>(x_bf16);
    a.M = static_cast<int32_t>(M);
    a.K = static_cast<int32_t>(K);
    a.KT = static_cast<int32_t>(q4::round_up(K, q4::kTileK) / q4::kTileK);
    a.nseg = nseg;
    a.y_bf16 = 0;
    for (int i = 0; i < q4::kMaxSegments; ++i) a.seg[i] = q4::Segment{};
    for (int i = 0; i < nseg; ++i) a.seg[i] = make_segment(segs[i].packed, segs[i].N, K, segs[i].y);
    return from_hip(q4::launch_linear(a, as_stream(stream)));
}

q4_status q4_0_linear_swiglu(const void *x_bf16, int64_t M, int64_t K, const void *gate_packed,
                             const void *up_packed, int64_t N, void *h, int h_bf16, void *stream) {
    if (h_bf16 != 0 && h_bf16 != 1) return Q4_ERR_SHAPE;
    if (M < 0 || M > kMaxM || !shape_ok(N, K)) return Q4_ERR_SHAPE;
    if (M == 0) return Q4_OK;
    if (!x_bf16 || !gate_packed || !up_packed || !h) return Q4_ERR_NULL;
    if (!aligned16(x_bf16) || !aligned16(gate_packed) || !aligned16(up_packed) || !aligned16(h))
        return Q4_ERR_ALIGN;
    q4::LinearArgs a;
    a.x = static_cast<const uint16_t *>(x_bf16);
    a.M = static_cast<int32_t>(M);
    a.K = static_cast<int32_t>(K);
    a.KT = static_cast<int32_t>(q4::round_up(K, q4::kTileK) / q4::kTileK);
    a.nseg = 2;
    a.y_bf16 = h_bf16;
    for (int i = 0; i < q4::kMaxSegments; ++i) a.seg[i] = q4::Segment{};
    a.seg[0] = make_segment(gate_packed, N, K, static_cast<float *>(h));
    a.seg[1] = make_segment(up_packed, N, K, nullptr);
    return from_hip(q4::launch_linear_glu(a, as_stream(stream)));
}

const char *q4_0_linear_swiglu_kernel(int64_t M, int64_t K) {
    if (M < 1 || M > kMaxM || !shape_ok(1, K)) return "";
    return q4::linear_glu_config_name(M, K);
}

const char *q4_0_linear_kernel(int64_t M, int64_t K, const int64_t *N, int nseg) {
    if (!N || nseg < 1 || nseg > q4::kMaxSegments || M < 1 || M > kMaxM) return "";
    q4::LinearArgs a;
    a.x = nullptr;
    a.M = static_cast<int32_t>(M);
    a.K = static_cast<int32_t>(K);
    a.nseg = nseg;
    a.y_bf16 = 0;
    for (int i = 0; i < q4::kMaxSegments; ++i) a.seg[i] = q4::Segment{};
    for (int i = 0; i < nseg; ++i) {
        if (!shape_ok(N[i], K)) return "";
        a.seg[i].N = static_cast<int32_t>(N[i]);
        a.seg[i].RT = static_cast<int32_t>(q4::PackedDims(N[i], K).RT);
    }
    a.KT = static_cast<int32_t>(q4::round_up(K, q4::kTileK) / q4::kTileK);
    return q4::linear_config_name(a);
}

size_t q4_1_packed_bytes(int64_t N, int64_t K) {
    if (!shape_ok(N, K)) return 0;
    return static_cast<size_t>(q4::PackedDims(N, K).q41_total_bytes());
}

q4_status q4_1_quantize(const float *w, int64_t N, int64_t K, void *blocks, void *stream) {
    if (!shape_ok(N, K)) return Q4_ERR_SHAPE;
    if (!w || !blocks) return Q4_ERR_NULL;
    if (!aligned16(w) || !aligned16(blocks)) return Q4_ERR_ALIGN;
    return from_hip(q4::launch_q41_quantize(w, N, K, static_cast<uint8_t *>(blocks), as_stream(stream)));
}

q4_status q4_1_pack(const void *blocks, int64_t N, int64_t K, void *packed, void *stream) {
    if (!shape_ok(N, K)) return Q4_ERR_SHAPE;
    if (!blocks || !packed) return Q4_ERR_NULL;
    if (!aligned16(blocks) || !aligned16(packed)) return Q4_ERR_ALIGN;
    return from_hip(q4::launch_q41_pack(static_cast<const uint8_t *>(blocks), N, K, static_cast<uint8_t *>(packed),
                                        as_stream(stream)));
}

q4_status q4_1_dequant(const void *packed, int64_t N, int64_t K, float *w, void *stream) {
    if (!shape_ok(N, K)) return Q4_ERR_SHAPE;
    if (!w || !packed) return Q4_ERR_NULL;
    if (!aligned16(w) || !aligned16(packed)) return Q4_ERR_ALIGN;
    return from_hip(q4::launch_q41_dequant(static_cast<const uint8_t *>(packed), N, K, w, as_stream(stream)));
}

namespace {
q4::LinearArgs q41_args(const void *x_bf16, int64_t M, const void *packed, int64_t N, int64_t K, float *y) {
    q4::LinearArgs a;
    a.x = static_cast<const uint16_t *>(x_bf16);
    a.M = static_cast<int32_t>(M);
    a.K = static_cast<int32_t>(K);
    a.KT = static_cast<int32_t>(q4::round_up(K, q4::kTileK) / q4::kTileK);
    a.nseg = 1;
    a.y_bf16 = 0;
    for (int i = 0; i < q4::kMaxSegments; ++i) a.seg[i] = q4::Segment{};
    const q4::PackedDims pd(N, K);
    a.seg[0] = make_segment(packed, N, K, y);
    a.seg[0].offsets = reinterpret_cast<const uint16_t *>(static_cast<const uint8_t *>(packed) + pd.nib_bytes() +
                                                          pd.RT * pd.KT * q4::kTileScales * 2);
    return a;
}
}  // namespace

q4_status q4_1_linear(const void *x_bf16, int64_t M, const void *packed, int64_t N, int64_t K, float *y,
                      void *stream) {
    if (M < 0 || M > kMaxM || !shape_ok(N, K)) return Q4_ERR_SHAPE;
    if (M == 0) return Q4_OK;
    if (!x_bf16 || !packed || !y) return Q4_ERR_NULL;
    if (!aligned16(x_bf16) || !aligned16(packed) || !aligned16(y)) return Q4_ERR_ALIGN;
    return from_hip(q4::launch_linear_q41(q41_args(x_bf16, M, packed, N, K, y), as_stream(stream)));
}

const char *q4_1_linear_kernel(int64_t M, int64_t K, int64_t N) {
    if (M < 1 || M > kMaxM || !shape_ok(N, K)) return "";
    q4::LinearArgs a = q41_args(nullptr, M, nullptr, N, K, nullptr);
    return q4::linear_q41_config_name(a);
}

int64_t q4_0_reference_read_words(int64_t bytes) {
    if (bytes < 0 || bytes > (int64_t(1) << 40) || bytes % 16) return 0;
    return q4::reference_read_sink_words(bytes);
}

q4_status q4_0_reference_read(const void *src, int64_t bytes, void *sink, void *stream) {
    if (bytes < 0 || bytes > (int64_t(1) << 40) || bytes % 16) return Q4_ERR_SHAPE;
    if ((bytes > 0 && !src) || !sink) return Q4_ERR_NULL;
    if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return Q4_ERR_ALIGN;
    return from_hip(q4::launch_reference_read(src, bytes, static_cast<uint32_t *>(sink), as_stream(stream)));
}

int64_t q4_0_reference_mfma_threads(void) { return q4::reference_mfma_threads(); }

q4_status q4_0_reference_mfma(int mode, int64_t iterations, float *sink, void *stream) {
    if (mode < 0 || mode > 3 || iterations < 1 || iterations > (int64_t(1) << 20)) return Q4_ERR_SHAPE;
    if (!sink) return Q4_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(sink) & 3u) return Q4_ERR_ALIGN;
    return from_hip(q4::launch_reference_mfma(mode, static_cast<int>(iterations), sink, as_stream(stream)));
}

q4_status q4_0_time_next_launch(void *start_event, void *stop_event) {
    q4::arm_launch_events(reinterpret_cast<hipEvent_t>(start_event), reinterpret_cast<hipEvent_t>(stop_event));
    return Q4_OK;
}

}  // extern "C"
