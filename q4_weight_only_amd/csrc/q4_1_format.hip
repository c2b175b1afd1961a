// Format kernels of the asymmetric 4-bit variant: 32 consecutive k of one
// row share an fp16 scale d and an fp16 offset m, w = q * d + m with 4-bit
// unsigned codes q (the TTS card's group-wise asymmetric int4, read as the
// GGUF asymmetric block: d, m, then 16 code bytes in Q4_0's nibble order, 20
// bytes per block).  Quantize (fp32 -> blocks), pack (blocks -> the packed
// asymmetric layout of include/q4_0.h) and dequantize (packed -> fp32).  One
// thread per block; one-time or test-only steps.

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "q4_0_internal.h"

namespace q4 {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kMaxGrid = 0x7fffffff;

inline bool grid_for(int64_t n, dim3 &grid) {
    const int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks > kMaxGrid) return false;
    grid = dim3(static_cast<unsigned>(blocks));
    return true;
}

// A 20-byte block is 4-byte aligned: word 0 = d | m << 16, words 1-4 the
// code bytes (byte j: q[j] in bits 0-3, q[j + 16] in bits 4-7).
__device__ inline void load_block(const uint8_t *p, uint16_t &d, uint16_t &m, uint8_t q[32]) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(p);
    d = static_cast<uint16_t>(w[0] & 0xFFFF);
    m = static_cast<uint16_t>(w[0] >> 16);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t v = w[1 + t];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t b = (v >> (8 * c)) & 0xFF;
            q[4 * t + c] = b & 0xF;
            q[4 * t + c + 16] = b >> 4;
        }
    }
}

__device__ inline void store_block(uint8_t *p, uint16_t d, uint16_t m, const uint8_t q[32]) {
    uint32_t *w = reinterpret_cast<uint32_t *>(p);
    w[0] = static_cast<uint32_t>(d) | (static_cast<uint32_t>(m) << 16);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t v = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) v |= static_cast<uint32_t>(q[4 * t + c] | (q[4 * t + c + 16] << 4)) << (8 * c);
        w[1 + t] = v;
    }
}

// mn, mx = min and max of the block; d = fp16((mx - mn) / 15), m = fp16(mn)
// (both rounded to nearest even); q = clamp(rint((w - m) / d), 0, 15) with the
// stored values, fp32 arithmetic and ties to even; q = 0 where d is zero.
__global__ __launch_bounds__(kThreads) void q41_quantize_kernel(const float *__restrict__ w, int64_t nblocks,
                                                                uint8_t *__restrict__ out) {
    const int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x;
    if (idx >= nblocks) return;
    float v[32];
    const float4 *src = reinterpret_cast<const float4 *>(w + idx * kQK);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float4 f = src[t];
        v[4 * t] = f.x;
        v[4 * t + 1] = f.y;
        v[4 * t + 2] = f.z;
        v[4 * t + 3] = f.w;
    }
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) {
        mn = fminf(mn, v[j]);
        mx = fmaxf(mx, v[j]);
    }
    const __half d16 = __float2half_rn((mx - mn) / 15.0f);
    const __half m16 = __float2half_rn(mn);
    const float df = __half2float(d16), mf = __half2float(m16);
    uint8_t q[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        float r = df == 0.0f ? 0.0f : rintf((v[j] - mf) / df);
        r = fminf(fmaxf(r, 0.0f), 15.0f);
        q[j] = static_cast<uint8_t>(r);
    }
    store_block(out + idx * kQ41BlockBytes, __half_as_ushort(d16), __half_as_ushort(m16), q);
}

// One thread per (row, block) of the padded matrix, as the Q4_0 pack: entry
// e = 4 r + i of super-tile T writes its four 4-byte code pieces to
// T * 1024 + g * 256 + e * 4 (the codes q themselves), d to the scale plane
// and m to the offset plane at element T * 64 + e.
__global__ __launch_bounds__(kThreads) void q41_pack_kernel(const uint8_t *__restrict__ blocks, int32_t N, int32_t K,
                                                            int32_t KT, int64_t nentries, uint8_t *__restrict__ nib,
                                                            uint16_t *__restrict__ scales,
                                                            uint16_t *__restrict__ offsets) {
    const int64_t t = blockIdx.x * (int64_t)kThreads + threadIdx.x;
    if (t >= nentries) return;
    const int64_t T = t >> 6;
    const int e = static_cast<int>(t & 63);
    const int r = e >> 2, i = e & 3;
    const int64_t rt = T / KT, kt = T % KT;
    const int64_t n = rt * kTileRows + r;
    const int64_t b = kt * kTileBlocks + i;
    uint16_t d = 0, m = 0;
    uint8_t q[32];
    if (n < N && b < K / kQK) {
        load_block(blocks + (n * (K / kQK) + b) * kQ41BlockBytes, d, m, q);
    } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) q[j] = 0;
    }
    uint32_t *dst = reinterpret_cast<uint32_t *>(nib + T * kTileNibBytes);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t piece = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) piece |= static_cast<uint32_t>(q[8 * g + j]) << (4 * j);
        dst[g * 64 + e] = piece;
    }
    scales[T * kTileScales + e] = d;
    offsets[T * kTileScales + e] = m;
}

// w[n, 32 b + k] = q * d + m, one rounding to fp32 (an fma of exact inputs).
__global__ __launch_bounds__(kThreads) void q41_dequant_kernel(const uint8_t *__restrict__ nib,
                                                               const uint16_t *__restrict__ scales,
                                                               const uint16_t *__restrict__ offsets, int32_t N,
                                                               int32_t K, int32_t KT, int64_t nentries,
                                                               float *__restrict__ w) {
    const int64_t t = blockIdx.x * (int64_t)kThreads + threadIdx.x;
    if (t >= nentries) return;
    const int64_t T = t >> 6;
    const int e = static_cast<int>(t & 63);
    const int r = e >> 2, i = e & 3;
    const int64_t rt = T / KT, kt = T % KT;
    const int64_t n = rt * kTileRows + r;
    const int64_t b = kt * kTileBlocks + i;
    if (n >= N || b >= K / kQK) return;
    const uint32_t *src = reinterpret_cast<const uint32_t *>(nib + T * kTileNibBytes);
    const float d = __half2float(__ushort_as_half(scales[T * kTileScales + e]));
    const float m = __half2float(__ushort_as_half(offsets[T * kTileScales + e]));
    float4 *dst = reinterpret_cast<float4 *>(w + n * K + b * kQK);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t piece = src[g * 64 + e];
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = fmaf(static_cast<float>((piece >> (4 * j)) & 0xF), d, m);
        dst[2 * g] = make_float4(v[0], v[1], v[2], v[3]);
        dst[2 * g + 1] = make_float4(v[4], v[5], v[6], v[7]);
    }
}

}  // namespace

hipError_t launch_q41_quantize(const float *w, int64_t N, int64_t K, uint8_t *out, hipStream_t s) {
    const int64_t nblocks = N * (K / kQK);
    dim3 grid;
    if (!grid_for(nblocks, grid)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(q41_quantize_kernel, grid, dim3(kThreads), 0, s, w, nblocks, out);
    return hipGetLastError();
}

hipError_t launch_q41_pack(const uint8_t *blocks, int64_t N, int64_t K, uint8_t *packed, hipStream_t s) {
    const PackedDims pd(N, K);
    const int64_t nentries = pd.RT * pd.KT * 64;
    dim3 grid;
    if (!grid_for(nentries, grid)) return hipErrorInvalidValue;
    uint16_t *scales = reinterpret_cast<uint16_t *>(packed + pd.nib_bytes());
    hipLaunchKernelGGL(q41_pack_kernel, grid, dim3(kThreads), 0, s, blocks, (int32_t)N, (int32_t)K, (int32_t)pd.KT,
                       nentries, packed, scales, scales + pd.RT * pd.KT * kTileScales);
    return hipGetLastError();
}

hipError_t launch_q41_dequant(const uint8_t *packed, int64_t N, int64_t K, float *w, hipStream_t s) {
    const PackedDims pd(N, K);
    const int64_t nentries = pd.RT * pd.KT * 64;
    dim3 grid;
    if (!grid_for(nentries, grid)) return hipErrorInvalidValue;
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(packed + pd.nib_bytes());
    hipLaunchKernelGGL(q41_dequant_kernel, grid, dim3(kThreads), 0, s, packed, scales,
                       scales + pd.RT * pd.KT * kTileScales, (int32_t)N, (int32_t)K, (int32_t)pd.KT, nentries, w);
    return hipGetLastError();
}

}  // namespace q4
