// Format kernels: quantize (fp32 -> GGUF Q4_0), pack (GGUF -> CDNA4 tiled
// layout), unpack (inverse) and dequant (packed -> fp32).  All are one-time or
// test-only steps outside the linear's hot loop; they are written for
// straightforward coalescing rather than peak bandwidth.
//
// GGUF Q4_0 block (the format of the quantized Voxtral checkpoints, named in
// the Rust fork's "RTF Benchmark Results"): 2 bytes fp16 d, then 16 bytes;
// byte j holds code q[j] (bits 0-3) and q[j+16] (bits 4-7); w = (q - 8) * d.
// The packed layout is defined in include/q4_0.h.

#include <hip/hip_fp16.h>

#include <hip/hip_ext.h>

#include "q4_0_internal.h"

namespace q4 {
namespace {

constexpr int kThreads = 256;

// Read one 18-byte GGUF block (2-byte aligned) as 9 halfwords.
__device__ inline void load_gguf_block(const uint8_t *p, uint16_t &d, uint8_t q[32]) {
    const uint16_t *h = reinterpret_cast<const uint16_t *>(p);
    d = h[0];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint16_t v = h[1 + t];
        const uint8_t b0 = v & 0xFF, b1 = v >> 8;     // code bytes 2t and 2t+1
        q[2 * t] = b0 & 0xF;
        q[2 * t + 16] = b0 >> 4;
        q[2 * t + 1] = b1 & 0xF;
        q[2 * t + 17] = b1 >> 4;
    }
}

__device__ inline void store_gguf_block(uint8_t *p, uint16_t d, const uint8_t q[32]) {
    uint16_t *h = reinterpret_cast<uint16_t *>(p);
    h[0] = d;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t b0 = q[2 * t] | (q[2 * t + 16] << 4);
        const uint32_t b1 = q[2 * t + 1] | (q[2 * t + 17] << 4);
        h[1 + t] = static_cast<uint16_t>(b0 | (b1 << 8));
    }
}

// --------------------------------------------------------------- quantize
// One thread per GGUF block (row n, block b); the block's 32 floats are
// contiguous at w + (n * K + 32 b), i.e. at w + 32 * (n * K/32 + b).
// T is float (fp32 weights) or uint16_t (bf16 bit patterns, widened to fp32
// exactly by a 16-bit shift before the same rule).
template <typename T>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const T *__restrict__ w,
                                                            int64_t nblocks,
                                                            uint8_t *__restrict__ out) {
    const int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x;
    if (idx >= nblocks) return;
    float v[32];
    if constexpr (sizeof(T) == 4) {
        const float4 *src = reinterpret_cast<const float4 *>(w + idx * kQK);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float4 f = src[t];
            v[4 * t] = f.x;
            v[4 * t + 1] = f.y;
            v[4 * t + 2] = f.z;
            v[4 * t + 3] = f.w;
        }
    } else {
        const uint4 *src = reinterpret_cast<const uint4 *>(w + idx * kQK);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint4 u = src[t];
            const uint32_t words[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[8 * t + 2 * h] = __uint_as_float(words[h] << 16);
                v[8 * t + 2 * h + 1] = __uint_as_float(words[h] & 0xFFFF0000u);
            }
        }
    }
    // signed element of largest magnitude; strict '>' keeps the first one
    float amax = v[0];
#pragma unroll
    for (int j = 1; j < 32; ++j)
        if (fabsf(v[j]) > fabsf(amax)) amax = v[j];
    const __half d16 = __float2half_rn(amax / -8.0f);
    const float df = __half2float(d16);
    uint8_t q[32];
    uint16_t dbits;
    if (df == 0.0f) {
        dbits = 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) q[j] = 8;
    } else {
        dbits = __half_as_ushort(d16);
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            float r = rintf(v[j] / df) + 8.0f;   // IEEE fp32 divide, ties to even
            r = fminf(fmaxf(r, 0.0f), 15.0f);
            q[j] = static_cast<uint8_t>(r);
        }
    }
    store_gguf_block(out + idx * kBlockBytes, dbits, q);
}

// ------------------------------------------------------------------- pack
// One thread per (row, block) of the padded matrix.  Thread t works on
// super-tile T = t / 64 and entry e = t % 64 = 4 r + i (row r, block i of the
// tile); for each k-group g its 4-byte piece goes to
// T * 1024 + g * 256 + e * 4, so a wave writes four contiguous 256-byte runs.
__global__ __launch_bounds__(kThreads) void pack_kernel(const uint8_t *__restrict__ gguf, int32_t N,
                                                        int32_t K, int32_t KT, int64_t nentries,
                                                        uint8_t *__restrict__ nib,
                                                        uint16_t *__restrict__ scales) {
    const int64_t t = blockIdx.x * (int64_t)kThreads + threadIdx.x;
    if (t >= nentries) return;
    const int64_t T = t >> 6;
    const int e = static_cast<int>(t & 63);
    const int r = e >> 2, i = e & 3;
    const int64_t rt = T / KT, kt = T % KT;
    const int64_t n = rt * kTileRows + r;
    const int64_t b = kt * kTileBlocks + i;
    uint16_t d = 0;
    uint8_t q[32];
    if (n < N && b < K / kQK) {
        load_gguf_block(gguf + (n * (K / kQK) + b) * kBlockBytes, d, q);
    } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) q[j] = 8;
    }
    uint32_t *dst = reinterpret_cast<uint32_t *>(nib + T * kTileNibBytes);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t piece = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) piece |= static_cast<uint32_t>(q[8 * g + j] ^ 8) << (4 * j);
        dst[g * 64 + e] = piece;
    }
    scales[T * kTileScales + e] = d;
}

// ----------------------------------------------------------------- unpack
__global__ __launch_bounds__(kThreads) void unpack_kernel(const uint8_t *__restrict__ nib,
                                                          const uint16_t *__restrict__ scales,
                                                          int32_t N, int32_t K, int32_t KT,
                                                          int64_t nentries,
                                                          uint8_t *__restrict__ gguf) {
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
    uint8_t q[32];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t piece = src[g * 64 + e];
#pragma unroll
        for (int j = 0; j < 8; ++j) q[8 * g + j] = ((piece >> (4 * j)) & 0xF) ^ 8;
    }
    store_gguf_block(gguf + (n * (K / kQK) + b) * kBlockBytes, scales[T * kTileScales + e], q);
}

// ---------------------------------------------------------------- dequant
// One thread per real (row, block); writes 32 floats w[n, 32 b .. 32 b + 31].
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t *__restrict__ nib,
                                                           const uint16_t *__restrict__ scales,
                                                           int32_t N, int32_t K, int32_t KT,
                                                           int64_t nentries,
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
    float4 *dst = reinterpret_cast<float4 *>(w + n * K + b * kQK);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t piece = src[g * 64 + e];
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // sign-extend the 4-bit code: it is q - 8 in two's complement
            const int s = static_cast<int>(piece << (28 - 4 * j)) >> 28;
            v[j] = static_cast<float>(s) * d;
        }
        dst[2 * g] = make_float4(v[0], v[1], v[2], v[3]);
        dst[2 * g + 1] = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// One thread per item; a count needing more than 2^31 - 1 workgroups (far
// beyond any matrix that fits in memory) is refused rather than truncated.
constexpr int64_t kMaxGrid = 0x7fffffff;
inline bool grid_for(int64_t n, dim3 &grid) {
    const int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks > kMaxGrid) return false;
    grid = dim3(static_cast<unsigned>(blocks));
    return true;
}

// ---------------------------------------------------------------- embed
// Row lookup in a packed table: thread t of a looked-up row writes that row's
// columns 8t .. 8t+7, one 4-byte piece of codes (super-tile kt = t / 16,
// block i = (t % 16) / 4, lane group g = t % 4) times the block's d.  Row
// `id` of the table lies at rows id % 16 of its super-tiles.  Consecutive
// threads write consecutive 32-byte runs of the output row; a grid-stride
// loop covers any number of ids.  An id outside [0, N) gets a row of NaN
// and reads nothing.
__global__ __launch_bounds__(kThreads) void embed_kernel(const uint8_t *__restrict__ nib,
                                                         const uint16_t *__restrict__ scales,
                                                         int32_t N, int32_t K, int32_t KT,
                                                         const int32_t *__restrict__ ids, int64_t total,
                                                         float *__restrict__ out) {
    const int per_row = K / 8;
    for (int64_t t = blockIdx.x * (int64_t)kThreads + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * kThreads) {
        const int64_t row = t / per_row;
        const int p = static_cast<int>(t - row * per_row);
        const int32_t id = ids[row];
        float v[8];
        if (id < 0 || id >= N) {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = __builtin_nanf("");
        } else {
            const int kt = p >> 4, i = (p >> 2) & 3, g = p & 3, r = id & 15;
            const int64_t T = static_cast<int64_t>(id >> 4) * KT + kt;
            const uint32_t piece =
                *reinterpret_cast<const uint32_t *>(nib + T * kTileNibBytes + g * 256 + r * 16 + i * 4);
            const float d = __half2float(__ushort_as_half(scales[T * kTileScales + r * 4 + i]));
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // sign-extend the 4-bit code: it is q - 8 in two's complement
                const int c = static_cast<int>(piece << (28 - 4 * j)) >> 28;
                v[j] = static_cast<float>(c) * d;
            }
        }
        float4 *dst = reinterpret_cast<float4 *>(out + row * K + p * 8);
        dst[0] = make_float4(v[0], v[1], v[2], v[3]);
        dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// ---------------------------------------------------------- embed (GGUF)
// The same lookup on a table kept in GGUF block order, where one row's
// blocks are contiguous (K/32 * 18 bytes): a lookup reads only the bytes of
// its rows, whereas in the tiled layout a row is 16-byte pieces 256 bytes
// apart and every piece costs a whole cache line.  A work unit is (id, run
// of up to kEmbedRunBlocks blocks).  A workgroup takes units blockIdx.x,
// blockIdx.x + gridDim.x, ...: it holds the next unit's bytes in registers
// (coalesced 2-byte loads: a row starts on any even byte) while it writes
// the current unit's outputs from LDS as consecutive float4 stores, which
// are nontemporal (the rows are written once and not read back here).  Two
// LDS buffers alternate, so one barrier per unit suffices.
constexpr int kEmbedRunBlocks = 256;
constexpr int kEmbedPerThread = kEmbedRunBlocks * 9 / kThreads;   // halfwords of a run per thread
static_assert(kEmbedRunBlocks * 9 % kThreads == 0, "a run splits evenly over the threads");
typedef float float4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void embed_gguf_kernel(const uint16_t *__restrict__ table, int32_t N,
                                                              int32_t K, const int32_t *__restrict__ ids,
                                                              int64_t units, int32_t runs,
                                                              float *__restrict__ out) {
    __shared__ uint16_t buf[2][kEmbedRunBlocks * 9];
    const int nb = K / kQK;
    struct Unit {
        const uint16_t *src;
        int64_t row;
        int b0, nbr;
        bool ok;
    };
    auto unit_of = [&](int64_t u) {
        Unit w;
        w.row = u / runs;
        w.b0 = static_cast<int>(u - w.row * runs) * kEmbedRunBlocks;
        w.nbr = nb - w.b0 < kEmbedRunBlocks ? nb - w.b0 : kEmbedRunBlocks;
        const int32_t id = ids[w.row];
        w.ok = id >= 0 && id < N;   // uniform over the workgroup
        w.src = table + (static_cast<int64_t>(w.ok ? id : 0) * nb + w.b0) * 9;
        return w;
    };
    uint16_t R[kEmbedPerThread];
    auto load = [&](const Unit &w) {
#pragma unroll
        for (int j = 0; j < kEmbedPerThread; ++j) {
            const int idx = threadIdx.x + kThreads * j;
            R[j] = (w.ok && idx < w.nbr * 9) ? w.src[idx] : 0;
        }
    };
    int64_t u = blockIdx.x;
    if (u >= units) return;
    Unit cur = unit_of(u);
    load(cur);
    int parity = 0;
    for (;;) {
        uint16_t *sb = buf[parity];
#pragma unroll
        for (int j = 0; j < kEmbedPerThread; ++j) {
            const int idx = threadIdx.x + kThreads * j;
            if (idx < cur.nbr * 9) sb[idx] = R[j];
        }
        __syncthreads();
        const int64_t un = u + gridDim.x;
        Unit nxt = cur;
        if (un < units) {
            nxt = unit_of(un);
            load(nxt);
        }
        float4v *dst = reinterpret_cast<float4v *>(out + cur.row * K + static_cast<int64_t>(cur.b0) * kQK);
        for (int q = threadIdx.x; q < cur.nbr * 8; q += kThreads) {
            const int b = q >> 3, e = (q & 7) * 4;   // elements e .. e+3 of block b
            float4v v;
            if (cur.ok) {
                const float d = __half2float(__ushort_as_half(sb[b * 9]));
                // code bytes 2 + (e mod 16) .. +3: elements e < 16 in the low
                // nibbles, e >= 16 in the high nibbles of the same bytes
                const int h = b * 9 + 1 + ((e & 15) >> 1);
                const uint32_t bytes = sb[h] | (static_cast<uint32_t>(sb[h + 1]) << 16);
                const int sh = e < 16 ? 0 : 4;
                v.x = static_cast<float>(static_cast<int>((bytes >> sh) & 15u) - 8) * d;
                v.y = static_cast<float>(static_cast<int>((bytes >> (8 + sh)) & 15u) - 8) * d;
                v.z = static_cast<float>(static_cast<int>((bytes >> (16 + sh)) & 15u) - 8) * d;
                v.w = static_cast<float>(static_cast<int>((bytes >> (24 + sh)) & 15u) - 8) * d;
            } else {
                const float nan = __builtin_nanf("");
                v = (float4v){nan, nan, nan, nan};
            }
            __builtin_nontemporal_store(v, dst + q);
        }
        if (un >= units) break;
        u = un;
        cur = nxt;
        parity ^= 1;
    }
}

}  // namespace

hipError_t launch_quantize(const float *w, int64_t N, int64_t K, uint8_t *out, hipStream_t s) {
    const int64_t nblocks = N * (K / kQK);
    dim3 grid;
    if (!grid_for(nblocks, grid)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_kernel<float>, grid, dim3(kThreads), 0, s, w, nblocks, out);
    return hipGetLastError();
}

hipError_t launch_quantize_bf16(const uint16_t *w, int64_t N, int64_t K, uint8_t *out, hipStream_t s) {
    const int64_t nblocks = N * (K / kQK);
    dim3 grid;
    if (!grid_for(nblocks, grid)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_kernel<uint16_t>, grid, dim3(kThreads), 0, s, w, nblocks, out);
    return hipGetLastError();
}

hipError_t launch_pack(const uint8_t *gguf, int64_t N, int64_t K, uint8_t *packed, hipStream_t s) {
    const PackedDims pd(N, K);
    const int64_t nentries = pd.RT * pd.KT * 64;
    dim3 grid;
    if (!grid_for(nentries, grid)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_kernel, grid, dim3(kThreads), 0, s, gguf, (int32_t)N,
                       (int32_t)K, (int32_t)pd.KT, nentries, packed,
                       reinterpret_cast<uint16_t *>(packed + pd.nib_bytes()));
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int64_t N, int64_t K, uint8_t *gguf, hipStream_t s) {
    const PackedDims pd(N, K);
    const int64_t nentries = pd.RT * pd.KT * 64;
    dim3 grid;
    if (!grid_for(nentries, grid)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(unpack_kernel, grid, dim3(kThreads), 0, s, packed,
                       reinterpret_cast<const uint16_t *>(packed + pd.nib_bytes()), (int32_t)N,
                       (int32_t)K, (int32_t)pd.KT, nentries, gguf);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t *packed, int64_t N, int64_t K, float *w, hipStream_t s) {
    const PackedDims pd(N, K);
    const int64_t nentries = pd.RT * pd.KT * 64;
    dim3 grid;
    if (!grid_for(nentries, grid)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dequant_kernel, grid, dim3(kThreads), 0, s, packed,
                       reinterpret_cast<const uint16_t *>(packed + pd.nib_bytes()), (int32_t)N,
                       (int32_t)K, (int32_t)pd.KT, nentries, w);
    return hipGetLastError();
}

hipError_t launch_embed(const uint8_t *packed, int64_t N, int64_t K, const int32_t *ids, int64_t n_ids,
                        float *out, hipStream_t s) {
    const PackedDims pd(N, K);
    const int64_t total = n_ids * (K / 8);
    // enough workgroups to fill the chip several times over; the kernel loops
    const int64_t want = (total + kThreads - 1) / kThreads;
    const dim3 grid(static_cast<uint32_t>(want < 65536 ? want : 65536));
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(packed + pd.nib_bytes());
    hipEvent_t start = nullptr, stop = nullptr;
    if (take_launch_events(start, stop))
        hipExtLaunchKernelGGL(embed_kernel, grid, dim3(kThreads), 0, s, start, stop, 0, packed, scales, (int32_t)N,
                              (int32_t)K, (int32_t)pd.KT, ids, total, out);
    else
        hipLaunchKernelGGL(embed_kernel, grid, dim3(kThreads), 0, s, packed, scales, (int32_t)N, (int32_t)K,
                           (int32_t)pd.KT, ids, total, out);
    return hipGetLastError();
}

hipError_t launch_embed_gguf(const uint8_t *gguf, int64_t N, int64_t K, const int32_t *ids, int64_t n_ids,
                             float *out, hipStream_t s) {
    const int32_t runs = static_cast<int32_t>((K / kQK + kEmbedRunBlocks - 1) / kEmbedRunBlocks);
    const int64_t units = n_ids * runs;
    // two units or more per workgroup, so the second one's loads overlap the
    // first one's stores (16384 ids: 50 -> 45 us; 2048 ids unchanged)
    const int64_t want = (units + 1) / 2;
    const dim3 grid(static_cast<uint32_t>(want < 65536 ? want : 65536));
    const uint16_t *table = reinterpret_cast<const uint16_t *>(gguf);
    hipEvent_t start = nullptr, stop = nullptr;
    if (take_launch_events(start, stop))
        hipExtLaunchKernelGGL(embed_gguf_kernel, grid, dim3(kThreads), 0, s, start, stop, 0, table, (int32_t)N,
                              (int32_t)K, ids, units, runs, out);
    else
        hipLaunchKernelGGL(embed_gguf_kernel, grid, dim3(kThreads), 0, s, table, (int32_t)N, (int32_t)K, ids, units,
                           runs, out);
    return hipGetLastError();
}

}  // namespace q4
