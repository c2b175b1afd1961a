// The fused Q4_0 linear: y = x * W^T with W in the packed layout of
// include/q4_0.h, x bf16, y fp32.
//
// Arithmetic (identical in both kernels).  A 16x16x32 bf16 MFMA covers one
// Q4_0 block (32 k) for 16 output rows x 16 weight rows.  Its B operand is
// the block's codes decoded exactly to bf16 (q - 8) / 16 -- v_cvt_off_f32_i4
// turns a 4-bit two's-complement code c into c / 16, which is why the packed
// layout stores q XOR 8 -- and its A operand is x itself, so every product is
// exact and the MFMA sums the block in fp32.  The block result is then scaled
// by the block's fp16 d in fp32 (one FMA per output element per block) and
// the final sum is multiplied by 16.  This is the pages' fused
// dequant + matmul (hakusoku summary, "線形演算・埋め込み") with the
// dequantization split so that no weight is ever rounded.
//
// Kernels.
//   skinny_kernel  (M <= 32, decode-sized batches): a wave owns all M rows,
//                  NT 16-row weight tiles and every WK-th super-tile along K;
//                  weights go straight from HBM into MFMA B registers (each
//                  lane's 16-byte load is exactly its B slice for 4 blocks),
//                  x comes from global memory (L2-resident), and the WK waves
//                  of a workgroup are summed through LDS in a fixed order.
//   gemm_kernel    (M > 32, prefill / encoder sizes): a workgroup tile of
//                  BM x BN outputs; the x tile of each 128-k step is staged in
//                  LDS (double-buffered, XOR-swizzled 16-byte chunks) and
//                  shared by the WN waves; weights again go HBM -> registers.
// Neither kernel uses atomics: results are bitwise reproducible.

#include <hip/hip_fp16.h>

#include "q4_0_internal.h"

namespace q4 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// c / 16 for the 4-bit two's-complement code in bits [3:0] of byte B of w.
// Written as a byte extract so the compiler folds it into the SDWA source
// select of v_cvt_off_f32_i4 (one instruction per code, no shifts).
template <int B>
__device__ __forceinline__ float code_of_byte(uint32_t w) {
    if constexpr (B == 0) return __builtin_amdgcn_cvt_off_f32_i4(w);
    else if constexpr (B == 3) return __builtin_amdgcn_cvt_off_f32_i4(w >> 24);
    else return __builtin_amdgcn_cvt_off_f32_i4((w >> (8 * B)) & 0xFFu);
}

// 8 codes (one 4-byte piece: element 2p in the low nibble of byte p, 2p+1 in
// the high nibble) -> bf16x8 of (q - 8) / 16 in element order.  Exact.
__device__ __forceinline__ bf16x8 decode_piece(uint32_t w) {
    uint32_t h = w >> 4;
    // keep h as one shifted word so every high-nibble code is a byte select
    // of it (an empty asm emits no instruction; it only hides the shift from
    // the combiner, which would otherwise fold it into per-code bit extracts)
    asm("" : "+v"(h));
    const bf16x2 p0 = __builtin_convertvector((floatx2){code_of_byte<0>(w), code_of_byte<0>(h)}, bf16x2);
    const bf16x2 p1 = __builtin_convertvector((floatx2){code_of_byte<1>(w), code_of_byte<1>(h)}, bf16x2);
    const bf16x2 p2 = __builtin_convertvector((floatx2){code_of_byte<2>(w), code_of_byte<2>(h)}, bf16x2);
    const bf16x2 p3 = __builtin_convertvector((floatx2){code_of_byte<3>(w), code_of_byte<3>(h)}, bf16x2);
    const bf16x4 lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
    const bf16x4 hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(bits16)));
}

__device__ __forceinline__ uint32_t piece_of(const u32x4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float scale_of(const u32x2 &v, int i) {
    const uint32_t w = (i < 2) ? v.x : v.y;
    return half_bits_to_float((i & 1) ? (w >> 16) : (w & 0xFFFF));
}

__device__ __forceinline__ floatx4 mfma_block(const bf16x8 &a, const bf16x8 &b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, (floatx4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

// Segment lookup: the segments' work tiles are laid end to end.
__device__ __forceinline__ int find_segment(const LinearArgs &a, int tile) {
    int s = 0;
#pragma unroll
    for (int t = 1; t < kMaxSegments; ++t)
        if (t < a.nseg && tile >= a.seg[t].tile_begin) s = t;
    return s;
}

// ------------------------------------------------------------------ skinny
template <int MROWS, int NT, int WK, int P>
struct SkinnyCfg {
    static constexpr int MT = MROWS > 16 ? 2 : 1;        // 16-row m-tiles
    static constexpr int REGS = MROWS < 4 ? MROWS : 4;   // live accumulator rows per lane
    static constexpr int kThreads = 64 * WK;
};

template <int MROWS, int NT, int WK, int P>
__global__ __launch_bounds__(64 * WK) void skinny_kernel(const LinearArgs a) {
    using C = SkinnyCfg<MROWS, NT, WK, P>;
    constexpr int MT = C::MT, REGS = C::REGS;
    const int lane = threadIdx.x & 63;
    const int wk = threadIdx.x >> 6;
    const int nl = lane & 15, g = lane >> 4;

    const int s = find_segment(a, blockIdx.x);
    const Segment sg = a.seg[s];
    const int rt0 = (static_cast<int>(blockIdx.x) - sg.tile_begin) * NT;
    const int KT = a.KT;
    const int nblk = a.K / kQK;

    struct Stage {
        u32x4 nib[NT];
        u32x2 sc[NT];
        u32x4 xa[MT][kTileBlocks];
    };

    auto load = [&](Stage &S, int kt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int rt = rt0 + nt;
            if (rt < sg.RT) {
                const int64_t T = static_cast<int64_t>(rt) * KT + kt;
                S.nib[nt] = *reinterpret_cast<const u32x4 *>(sg.nib + T * kTileNibBytes + lane * 16);
                S.sc[nt] = *reinterpret_cast<const u32x2 *>(sg.scales + T * kTileScales + nl * 4);
            } else {
                S.nib[nt] = (u32x4){0u, 0u, 0u, 0u};
                S.sc[nt] = (u32x2){0u, 0u};
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mt * 16 + nl;
#pragma unroll
            for (int i = 0; i < kTileBlocks; ++i) {
                const int b = kt * kTileBlocks + i;
                if (m < a.M && b < nblk)
                    S.xa[mt][i] = *reinterpret_cast<const u32x4 *>(
                        a.x + static_cast<int64_t>(m) * a.K + b * kQK + g * 8);
                else
                    S.xa[mt][i] = (u32x4){0u, 0u, 0u, 0u};
            }
        }
    };

    floatx4 acc[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = (floatx4){0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Stage &S) {
#pragma unroll
        for (int i = 0; i < kTileBlocks; ++i) {
            bf16x8 A[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) A[mt] = __builtin_bit_cast(bf16x8, S.xa[mt][i]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16x8 B = decode_piece(piece_of(S.nib[nt], i));
                const float d = scale_of(S.sc[nt], i);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const floatx4 D = mfma_block(A[mt], B);
#pragma unroll
                    for (int r = 0; r < REGS; ++r) acc[nt][mt][r] = fmaf(d, D[r], acc[nt][mt][r]);
                }
            }
        }
    };

    Stage st[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int kt = wk + p * WK;
        if (kt < KT) load(st[p], kt);
    }
    for (int base = wk; base < KT; base += P * WK) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int kt = base + p * WK;
            if (kt < KT) {
                compute(st[p]);
                const int ktn = kt + P * WK;
                if (ktn < KT) load(st[p], ktn);
            }
        }
    }

    // Sum the WK partial results in wave order through LDS.
    if constexpr (WK > 1) {
        __shared__ float red[WK - 1][NT][MT][REGS][64];
        if (wk > 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < REGS; ++r) red[wk - 1][nt][mt][r][lane] = acc[nt][mt][r];
        }
        __syncthreads();
        if (wk != 0) return;
#pragma unroll
        for (int w = 0; w < WK - 1; ++w)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < REGS; ++r) acc[nt][mt][r] += red[w][nt][mt][r][lane];
    }

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int rt = rt0 + nt;
        const int n = rt * 16 + nl;
        if (rt >= sg.RT || n >= sg.N) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < REGS; ++r) {
                const int m = mt * 16 + 4 * g + r;
                if (m < a.M) sg.y[static_cast<int64_t>(m) * sg.N + n] = acc[nt][mt][r] * 16.0f;
            }
    }
}

// -------------------------------------------------------------------- gemm
template <int MT, int NT, int WM, int WN>
struct GemmCfg {
    static constexpr int BM = 16 * MT * WM;
    static constexpr int BN = 16 * NT * WN;
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int kAChunks = BM * 16;                   // 16-byte chunks per A tile
    static constexpr int kAPerThread = kAChunks / kThreads;
    static_assert(kAChunks % kThreads == 0, "A tile must split evenly over the threads");
};

// Byte offset of 16-byte chunk c (0..15) of row m in a swizzled A tile.
__device__ __forceinline__ int a_tile_offset(int m, int c) { return (m * 16 + (c ^ (m & 7))) * 16; }

template <int MT, int NT, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(const LinearArgs a) {
    using C = GemmCfg<MT, NT, WM, WN>;
    constexpr int BM = C::BM, NPT = C::kAPerThread;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * 256];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int nl = lane & 15, g = lane >> 4;

    const int s = find_segment(a, blockIdx.x);
    const Segment sg = a.seg[s];
    const int rt_base = (static_cast<int>(blockIdx.x) - sg.tile_begin) * (NT * WN) + wn * NT;
    const int m0 = blockIdx.y * BM;
    const int KT = a.KT;
    const int nblk = a.K / kQK;

    // ---- A staging: thread owns chunks q = tid + kThreads * j of the tile
    u32x4 a_regs[NPT];
    auto load_a = [&](int kt) {
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
            const int q = tid + C::kThreads * j;
            const int m = q >> 4, c = q & 15;
            const int b = kt * kTileBlocks + (c >> 2);
            if (m0 + m < a.M && b < nblk)
                a_regs[j] = *reinterpret_cast<const u32x4 *>(
                    a.x + static_cast<int64_t>(m0 + m) * a.K + kt * kTileK + c * 8);
            else
                a_regs[j] = (u32x4){0u, 0u, 0u, 0u};
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
            const int q = tid + C::kThreads * j;
            const int m = q >> 4, c = q & 15;
            *reinterpret_cast<u32x4 *>(&lds_a[buf][a_tile_offset(m, c)]) = a_regs[j];
        }
    };

    // ---- B: this wave's NT weight tiles, straight into registers
    struct BStage {
        u32x4 nib[NT];
        u32x2 sc[NT];
    };
    auto load_b = [&](BStage &S, int kt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int rt = rt_base + nt;
            if (rt < sg.RT) {
                const int64_t T = static_cast<int64_t>(rt) * KT + kt;
                S.nib[nt] = *reinterpret_cast<const u32x4 *>(sg.nib + T * kTileNibBytes + lane * 16);
                S.sc[nt] = *reinterpret_cast<const u32x2 *>(sg.scales + T * kTileScales + nl * 4);
            } else {
                S.nib[nt] = (u32x4){0u, 0u, 0u, 0u};
                S.sc[nt] = (u32x2){0u, 0u};
            }
        }
    };

    floatx4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (floatx4){0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf, const BStage &S) {
        const uint8_t *tile = lds_a[buf];
#pragma unroll
        for (int i = 0; i < kTileBlocks; ++i) {
            bf16x8 A[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = (wm * MT + mt) * 16 + nl;
                A[mt] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(tile + a_tile_offset(m, 4 * i + g)));
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16x8 B = decode_piece(piece_of(S.nib[nt], i));
                const float d = scale_of(S.sc[nt], i);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const floatx4 D = mfma_block(A[mt], B);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[mt][nt][r] = fmaf(d, D[r], acc[mt][nt][r]);
                }
            }
        }
    };

    BStage b0, b1;
    load_a(0);
    load_b(b0, 0);
    store_a(0);
    __syncthreads();
    int kt = 0;
    for (;;) {
        // even step: compute kt from buffer 0 / b0, prefetch kt+1 into buffer 1 / b1
        if (kt + 1 < KT) {
            load_a(kt + 1);
            load_b(b1, kt + 1);
        }
        compute(0, b0);
        if (kt + 1 >= KT) break;
        store_a(1);
        __syncthreads();
        ++kt;
        // odd step
        if (kt + 1 < KT) {
            load_a(kt + 1);
            load_b(b0, kt + 1);
        }
        compute(1, b1);
        if (kt + 1 >= KT) break;
        store_a(0);
        __syncthreads();
        ++kt;
    }

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int rt = rt_base + nt;
        const int n = rt * 16 + nl;
        if (rt >= sg.RT || n >= sg.N) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + (wm * MT + mt) * 16 + 4 * g + r;
                if (m < a.M) sg.y[static_cast<int64_t>(m) * sg.N + n] = acc[mt][nt][r] * 16.0f;
            }
    }
}

// ---------------------------------------------------------------- launch
// Tile configurations depend on M only, so a fused multi-segment launch and
// separate single launches run the same arithmetic in the same order.
template <int MROWS, int NT, int WK, int P>
hipError_t run_skinny(LinearArgs a, hipStream_t s) {
    int tiles = 0;
    for (int i = 0; i < a.nseg; ++i) {
        a.seg[i].tile_begin = tiles;
        tiles += (a.seg[i].RT + NT - 1) / NT;
    }
    hipLaunchKernelGGL((skinny_kernel<MROWS, NT, WK, P>), dim3(tiles), dim3(64 * WK), 0, s, a);
    return hipGetLastError();
}

template <int MT, int NT, int WM, int WN>
hipError_t run_gemm(LinearArgs a, hipStream_t s) {
    using C = GemmCfg<MT, NT, WM, WN>;
    int tiles = 0;
    for (int i = 0; i < a.nseg; ++i) {
        a.seg[i].tile_begin = tiles;
        tiles += (a.seg[i].RT + NT * WN - 1) / (NT * WN);
    }
    const int mtiles = (a.M + C::BM - 1) / C::BM;
    hipLaunchKernelGGL((gemm_kernel<MT, NT, WM, WN>), dim3(tiles, mtiles), dim3(C::kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(LinearArgs a, hipStream_t s) {
    if (a.M == 1) return run_skinny<1, 1, 8, 4>(a, s);
    if (a.M == 2) return run_skinny<2, 1, 8, 4>(a, s);
    if (a.M <= 4) return run_skinny<4, 1, 8, 4>(a, s);
    if (a.M <= 16) return run_skinny<16, 1, 8, 4>(a, s);
    if (a.M <= 32) return run_skinny<32, 4, 4, 2>(a, s);
    return run_gemm<4, 4, 2, 2>(a, s);
}

}  // namespace q4
