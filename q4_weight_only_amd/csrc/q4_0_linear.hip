// The fused Q4_0 linear: y = x * W^T with W in the packed layout of
// include/q4_0.h, x bf16, y fp32; the gated (SwiGLU) launch; the asymmetric
// variant (w = q d + m); and the arithmetic-only measurement loop.
//
// Arithmetic (identical in every linear kernel).  A 16x16x32 bf16 MFMA covers
// one Q4_0 block (32 k) for 16 output rows x 16 weight rows.  Its B operand
// is the block's codes decoded exactly to bf16 (q - 8) / 16 --
// v_cvt_off_f32_i4 turns a 4-bit two's-complement code c into c / 16, which
// is why the packed layout stores q XOR 8 -- and its A operand is x itself,
// so every product is exact and the MFMA sums the block in fp32.  The block
// result is then scaled by the block's fp16 d in fp32 (one FMA per output
// element per block) and the final sum is multiplied by 16.  This is the
// pages' fused dequant + matmul (hakusoku summary, "線形演算・埋め込み") with
// the dequantization split so that no weight is ever rounded.
//
// Kernels.
//   gemv_kernel    (M <= 4 with K <= 9216: every launch of the decode step;
//                  gated launches of 3-4 rows only to K = 4096): a workgroup owns one 16-row
//                  weight tile and all M rows, its WK waves split K; each wave
//                  issues its own x chunks and then every one of its weight
//                  stages at once, and consumes them as they land.
//   skinny_kernel  (other M <= 16, and 17-64 rows when the weights are
//                  short): the same work split with a P-deep refill of each
//                  wave's stages; x from LDS (staged once) or global memory.
//   skinny_stream_kernel (M = 1, very tall weights): the same per tile, with
//                  a fixed grid walking the tiles.
//   gemm_kernel    (17 <= M <= 64, tall weights): a workgroup tile of BM x BN
//                  outputs; the x tile of each 128-k step is staged in LDS
//                  (double-buffered, XOR-swizzled 16-byte chunks) and shared
//                  by the WN waves; weights go HBM -> registers.
//   gemm3_kernel   (M > 64, prefill / encoder sizes): the same arithmetic with
//                  MT x NT register tiles per wave, x staged a quarter per
//                  block step through bounds-checked buffer loads, and an
//                  XCD-aware workgroup -> tile order.
// In every kernel the weights go straight from HBM into MFMA B registers
// (each lane's 16-byte load is exactly its B slice for 4 blocks) and the
// partial sums of a K split are added through LDS in a fixed order.
// gemm_kernel and gemm3_kernel add the block results of an output in the same
// order, so they give bitwise equal results for any tiling.  No kernel uses
// atomics: results are bitwise reproducible.

#include <atomic>
#include <string>
#include <vector>

#include <hip/hip_ext.h>
#include <hip/hip_bf16.h>
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

// 8 unsigned codes (the asymmetric layout: element 2p in the low nibble of
// byte p, 2p+1 in the high nibble) -> bf16x8 of q in element order.  Exact.
__device__ __forceinline__ bf16x8 decode_piece_u(uint32_t w) {
    uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    // hide the masks from the combiner, so each code is one byte-select
    // conversion (v_cvt_f32_ubyte0..3) of a masked word, not a bit-field
    // extract followed by a conversion
    asm("" : "+v"(lo), "+v"(hi));
    bf16x2 p[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        p[b] = __builtin_convertvector((floatx2){static_cast<float>((lo >> (8 * b)) & 0xFFu),
                                                 static_cast<float>((hi >> (8 * b)) & 0xFFu)}, bf16x2);
    const bf16x4 l = __builtin_shufflevector(p[0], p[1], 0, 1, 2, 3);
    const bf16x4 h = __builtin_shufflevector(p[2], p[3], 0, 1, 2, 3);
    return __builtin_shufflevector(l, h, 0, 1, 2, 3, 4, 5, 6, 7);
}

// An MFMA B operand of ones: the product is the block's sum of x per row.
__device__ __forceinline__ bf16x8 bf16_ones() {
    const __bf16 one = static_cast<__bf16>(1.0f);
    return (bf16x8){one, one, one, one, one, one, one, one};
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

// An fp32 value as two bf16 (bit patterns in the low 16 bits): hi is v with
// its low 16 bits cleared, lo the remainder v - hi (exact in fp32) rounded
// to nearest even, so hi + lo is v within 2^-16 |v|, and exactly v when v
// has at most 16 significant bits (an fp16 value has 11).
__device__ __forceinline__ void split_bf16(float v, uint32_t &hi, uint32_t &lo) {
    const uint32_t vb = __builtin_bit_cast(uint32_t, v);
    hi = vb >> 16;
    const float r = v - __builtin_bit_cast(float, vb & 0xFFFF0000u);
    lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(r));
}

// silu(g) = g / (1 + e^-g), as g * rcp(1 + 2^(-g log2 e)) with the hardware
// exp2 and reciprocal (about 1 ulp each).  The rounding of -g log2 e adds a
// relative error of at most |g| 2^-24 log2 e ln 2, under 6e-6 while e^-g is
// finite (g > -88).  Below that e^-g overflows and the result is -0 (the
// exact value is under 1e-36 in magnitude); g = -inf gives NaN, as the
// quotient does.
__device__ __forceinline__ float silu_f32(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504f));
}

// Epilogue store of one output: fp32, or for a gated launch that asks for it
// bf16 rounded to nearest even (the y pointer then addresses bf16 elements).
__device__ __forceinline__ void store_out(const LinearArgs &a, const Segment &sg, int64_t idx, float v) {
    if (a.y_bf16)
        reinterpret_cast<__hip_bfloat16 *>(sg.y)[idx] = __float2bfloat16(v);
    else
        sg.y[idx] = v;
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
// x staged in LDS: row m of the (padded) x tile starts at m * row_bytes; rows
// are padded by 16 bytes so the 16 rows read by one MFMA A fragment fall in
// different LDS banks.
__device__ __forceinline__ int x_row_bytes(int KT) { return KT * kTileK * 2 + 16; }

template <int MROWS, int NT, int WK, int P, bool XLDS, int WPE, bool GLU>
struct SkinnyCfg {
    static constexpr int MT = (MROWS + 15) / 16;         // 16-row m-tiles
    static constexpr int REGS = MROWS < 4 ? MROWS : 4;   // live accumulator rows per lane
    static constexpr int kWaves = GLU ? 2 * WK : WK;     // waves per workgroup
    static constexpr int kThreads = 64 * kWaves;
};

// Decode-sized batches.  Every wave owns all M rows, NT weight row-tiles
// (16 rows each) and the super-tiles kt = wk, wk + WK, ... along K.  All of a
// wave's weight loads (up to P super-tiles) are issued before anything else,
// so a launch puts its whole weight stream in flight at once; x is staged
// once per workgroup (in LDS when XLDS) while those loads are outstanding.
//
// GLU: the launch has two segments of the same shape, gate (seg 0, whose y
// receives the result) and up (seg 1).  A workgroup then has 2 WK waves: the
// first WK run the gate rows, the last WK the same rows of up, each exactly
// as a plain launch would; the reduction through LDS sums both in the same
// wave order and the epilogue stores silu(gate) * up.
template <int MROWS, int NT, int WK, int P, bool XLDS, int WPE, bool GLU>
__global__ __launch_bounds__(64 * WK * (GLU ? 2 : 1)) __attribute__((amdgpu_waves_per_eu(WPE > 0 ? WPE : 1, 8)))
void skinny_kernel(const LinearArgs a) {
    using C = SkinnyCfg<MROWS, NT, WK, P, XLDS, WPE, GLU>;
    constexpr int MT = C::MT, REGS = C::REGS;
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
    const int lane = threadIdx.x & 63;
    // wave index as a scalar: every loop bound and branch below is uniform
    // across the wave, so the compiler emits scalar branches and keeps exact
    // per-stage load counters (no drain of the prefetch queue)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wk = GLU ? wave % WK : wave;             // K-slice of this wave
    const bool up_wave = GLU && wave >= WK;            // runs the up rows
    const int nl = lane & 15, g = lane >> 4;

    const int s = GLU ? 0 : find_segment(a, blockIdx.x);
    const Segment sg = a.seg[s];
    const Segment &src = up_wave ? a.seg[1] : sg;      // the matrix this wave streams
    const int rt0 = (static_cast<int>(blockIdx.x) - sg.tile_begin) * NT;
    const int KT = a.KT;
    const int nblk = a.K / kQK;
    const int mrows = a.M < 16 * MT ? a.M : 16 * MT;   // staged x rows
    const int row_bytes = x_row_bytes(KT);
    const int nkt = (KT - wk + WK - 1) / WK;            // super-tiles of this wave: wk + j * WK

    // Weight tiles past the segment's end are read from its last tile (their
    // results are never stored), so loads need no branches.
    const uint8_t *nib_base[NT];
    const uint16_t *sc_base[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int rt = rt0 + nt < src.RT ? rt0 + nt : src.RT - 1;
        const int64_t T0 = static_cast<int64_t>(rt) * KT + wk;
        nib_base[nt] = src.nib + T0 * kTileNibBytes + lane * 16;
        sc_base[nt] = src.scales + T0 * kTileScales + nl * 4;
    }

    struct WStage {
        u32x4 nib[NT];
        u32x2 sc[NT];
    };
    auto load_w = [&](WStage &S, int j) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            S.nib[nt] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(nib_base[nt] + static_cast<int64_t>(j) * WK * kTileNibBytes));
            S.sc[nt] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(sc_base[nt] + static_cast<int64_t>(j) * WK * kTileScales));
        }
    };

    // A fragment of m-tile mt for block b: x[m][32 b + 8 g .. + 8].  Rows at
    // or beyond M only feed output rows that are never stored, so they read
    // row M - 1 (from LDS) or zeros (from global memory).
    int a_row[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + nl;
        a_row[mt] = XLDS ? (m < mrows ? m : mrows - 1) : m;
    }
    auto load_a = [&](int mt, int b) -> bf16x8 {
        if constexpr (XLDS) {
            return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                                                  xs + a_row[mt] * row_bytes + (b * kQK + g * 8) * 2));
        } else {
            u32x4 v = (u32x4){0u, 0u, 0u, 0u};
            if (a_row[mt] < a.M && b < nblk)
                v = *reinterpret_cast<const u32x4 *>(a.x + static_cast<int64_t>(a_row[mt]) * a.K + b * kQK + g * 8);
            return __builtin_bit_cast(bf16x8, v);
        }
    };

    floatx4 acc[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = (floatx4){0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const WStage &S, int j) {
        const int kt = wk + j * WK;
#pragma unroll
        for (int i = 0; i < kTileBlocks; ++i) {
            const int b = kt * kTileBlocks + i;
            bf16x8 A[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) A[mt] = load_a(mt, b);
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

    // 1. weight loads for the first P super-tiles of this wave
    WStage st[P];
#pragma unroll
    for (int p = 0; p < P; ++p)
        if (p < nkt) load_w(st[p], p);
    // 2. stage x (zero beyond K) while they are in flight
    if constexpr (XLDS) {
        const int chunks_per_row = KT * (kTileK / 8);          // 16-byte chunks
        const int total = mrows * chunks_per_row;
        for (int c = threadIdx.x; c < total; c += C::kThreads) {
            // a one-row launch has no row index to divide out
            const int m = MROWS == 1 ? 0 : c / chunks_per_row, kc = c - m * chunks_per_row;
            u32x4 v = (u32x4){0u, 0u, 0u, 0u};
            if (kc * 8 < a.K) v = *reinterpret_cast<const u32x4 *>(a.x + static_cast<int64_t>(m) * a.K + kc * 8);
            *reinterpret_cast<u32x4 *>(xs + m * row_bytes + kc * 16) = v;
        }
        __syncthreads();
    }
    // 3. steady state: P computes, each followed by the refill of its stage
    //    P super-tiles ahead; no conditions inside
    int j = 0;
    for (; j + 2 * P <= nkt; j += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            compute(st[p], j + p);
            load_w(st[p], j + p + P);
        }
    }
    // 4. drain: at most 2P - 1 super-tiles remain
#pragma unroll
    for (int p = 0; p < P; ++p) {
        if (j + p < nkt) {
            compute(st[p], j + p);
            if (j + p + P < nkt) load_w(st[p], j + p + P);
        }
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
        if (j + P + p < nkt) compute(st[p], j + P + p);

    // Sum the WK partial results in wave order through LDS (gate and up
    // separately in a gated launch: waves 1 .. WK-1, then WK .. 2WK-1).
    floatx4 up[NT][MT];
    if constexpr (C::kWaves > 1) {
        __shared__ float red[C::kWaves - 1][NT][MT][REGS][64];
        if (wave > 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < REGS; ++r) red[wave - 1][nt][mt][r][lane] = acc[nt][mt][r];
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w = 0; w < WK - 1; ++w)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < REGS; ++r) acc[nt][mt][r] += red[w][nt][mt][r][lane];
        if constexpr (GLU) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < REGS; ++r) {
                        up[nt][mt][r] = red[WK - 1][nt][mt][r][lane];
#pragma unroll
                        for (int w = WK; w < 2 * WK - 1; ++w) up[nt][mt][r] += red[w][nt][mt][r][lane];
                    }
        }
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
                if (m >= a.M) continue;
                const float v = acc[nt][mt][r] * 16.0f;
                if constexpr (GLU)
                    store_out(a, sg, static_cast<int64_t>(m) * sg.N + n, silu_f32(v) * (up[nt][mt][r] * 16.0f));
                else
                    sg.y[static_cast<int64_t>(m) * sg.N + n] = v;
            }
    }
}

// ------------------------------------------------------------------- gemv
// Word 3 of a raw buffer resource on gfx9: 32-bit data format, so untyped
// loads are bounds-checked against the resource's byte size and read zero
// past it.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kOutOfRange = 0x40000000;   // a byte offset beyond every x resource (at most 2^29 bytes)
constexpr int kNonTemporal = 2;           // cache-policy bit of a buffer load: streaming (nt)

// Decode batches (up to 16 rows, short K): skinny_kernel<MROWS, 1, WK, P>'s
// work split and arithmetic -- wave wk owns super-tiles wk, wk + WK, ... of
// one 16-row weight tile, blocks are added in k order and the WK partial sums
// through LDS in wave order, so both give the same bits -- with a different
// issue order.  The x loads go out first, then every one of the wave's NS
// weight stages (NS = ceil(KT / WK), fixed at compile time, so the code is
// straight-line and each wait names an exact count).  Loads complete in issue
// order for the wait counter: the x store to LDS waits for x alone, and the
// MFMAs of stage j wait for stage j alone, so blocks are decoded and
// multiplied while the later stages are still arriving.  A stage past the
// last super-tile (when WK does not divide KT) reads the last tile with its
// scales forced to zero, which adds nothing (and x is read from that tile's
// columns, zero past K).  Weights are read through buffer resources, whose
// base and size sit in scalar registers, at one per-lane offset.
//
// GLU: the launch has two segments of the same shape, gate (seg 0, whose y
// receives the result) and up (seg 1).  Workgroup 2 rt + h covers the eight
// rows 16 rt + 8 h .. + 7 of both: MFMA columns 0-7 are those gate rows and
// columns 8-15 the same up rows (each lane reads its 16 bytes from the gate
// or the up tile), so a gated launch has the plain launch's workgroups,
// waves and bytes per wave.  A column's result does not depend on its
// neighbours, so g and u are the plain launch's values; after the reduction
// lane c < 8 takes u from lane c + 8 and stores silu(g) * u.
//
// ASYM: the asymmetric layout (codes q, scale d, offset m; w = q d + m).  The
// codes are decoded as q itself, a second MFMA against ones gives the
// block's sum S of x, and each block adds d * D + m * S (no final * 16).
template <int MROWS, int WK, int NS, int WPE, bool GLU, bool ASYM = false>
__global__ __launch_bounds__(64 * WK) __attribute__((amdgpu_waves_per_eu(WPE > 0 ? WPE : 1, 8)))
void gemv_kernel(const uint16_t *__restrict__ ax, const int aM, const int aK, const int aKT, const int anseg,
                 const int tb1, const int tb2, const int tb3, const int tb4, const int tb5, const int tb6,
                 const int tb7, const LinearArgs a) {
    static_assert(MROWS >= 1 && MROWS <= 16, "one 16-row m-tile");
    static_assert(!(GLU && ASYM), "no gated launch of the asymmetric layout");
    constexpr int REGS = MROWS < 4 ? MROWS : 4;
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
    const int lane = threadIdx.x & 63;
    const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nl = lane & 15, g = lane >> 4;

    // the segment from the start tiles passed as scalar arguments: with them
    // preloaded into SGPRs the segment is known without a load, and only its
    // pointers are fetched before the weight loads
    int s = 0;
    if constexpr (!GLU) {
        const int tbs[kMaxSegments - 1] = {tb1, tb2, tb3, tb4, tb5, tb6, tb7};
#pragma unroll
        for (int t = 1; t < kMaxSegments; ++t)
            if (t < anseg && static_cast<int>(blockIdx.x) >= tbs[t - 1]) s = t;
    }
    const Segment sg = a.seg[s];
    // plain: 16-row tile rt0; gated: tile rt0, rows 8 h .. 8 h + 7 of it.
    // Gated workgroups come in groups of 16: b and b + 8 take the two halves
    // of one tile, so that under round-robin dispatch over the 8 XCDs both
    // halves of each 256-byte code piece are fetched through one XCD at about
    // the same time (adjacent b would split every piece across two XCDs)
    const int b = static_cast<int>(blockIdx.x);
    const int rt0 = GLU ? ((b >> 4) << 3) + (b & 7) : b - sg.tile_begin;
    const int half = GLU ? (b >> 3) & 1 : 0;
    const int KT = aKT;
    const int mrows = aM < MROWS ? aM : MROWS;

    // x: each wave stages only the chunks (16 bytes) its own super-tiles
    // read, [row][stage][chunk], into an LDS region of its own, so no wave
    // waits for another's x; lane L takes chunks L, L + 64, ...
    constexpr int kWaveChunks = MROWS * NS * (kTileK / 8);
    constexpr int kXPer = (kWaveChunks + 63) / 64;
    // with a pad slot for each lane past the chunks, so that every lane stores
    // (a conditional store lets the compiler sink the x loads below the
    // weight loads, and the first stage then waits for all of them)
    uint8_t *const xw = xs + wk * (kXPer * 64 * 16);
    // weights: past the segment's end the last tile is read (its outputs are
    // never stored)
    const int rt = rt0 < sg.RT ? rt0 : sg.RT - 1;
    const int64_t T0 = static_cast<int64_t>(rt) * KT;
    __amdgpu_buffer_rsrc_t nib_rsrc, sc_rsrc, off_rsrc;
    const uint8_t *nib_lane = nullptr;
    const uint8_t *sc_lane = nullptr;
    if constexpr (GLU) {
        // row r of the tile for this lane's column: gate rows in columns 0-7,
        // the same up rows in columns 8-15
        const Segment &src = a.seg[nl < 8 ? 0 : 1];
        const int r = 8 * half + (nl & 7);
        nib_lane = src.nib + T0 * kTileNibBytes + g * 256 + r * 16;
        sc_lane = reinterpret_cast<const uint8_t *>(src.scales + T0 * kTileScales + r * 4);
    } else {
        nib_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(sg.nib + T0 * kTileNibBytes), 0,
                                                     KT * kTileNibBytes, kBufferRsrcWord3);
        sc_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(sg.scales + T0 * kTileScales), 0,
                                                    KT * kTileScales * 2, kBufferRsrcWord3);
        if constexpr (ASYM)
            off_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(sg.offsets + T0 * kTileScales), 0,
                                                         KT * kTileScales * 2, kBufferRsrcWord3);
    }

    // 1. x first: every chunk of this thread, zero past K (a chunk past the
    //    row's K, or a thread without a chunk, reads beyond the resource)
    const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(ax), 0, mrows * aK * 2, kBufferRsrcWord3);
    u32x4 xv[kXPer];
#pragma unroll
    for (int q = 0; q < kXPer; ++q) {
        const int c = lane + 64 * q;                       // [row][stage][chunk] of this wave
        const int m = c / (NS * 16), st = (c / 16) % NS, cc = c % 16;
        const int kt = wk + st * WK, kc = kt * 16 + cc;    // 16-byte chunk of the row
        const bool in = c < kWaveChunks && m < mrows && kt < KT && kc * 8 < aK;
        xv[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              xrsrc, in ? (m * aK + kc * 8) * 2 : kOutOfRange, 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the x loads ahead of the weights

    // 2. then every weight stage of this wave, each one's codes then scales
    u32x4 nib[NS];
    u32x2 sc[NS];
    u32x2 mo[ASYM ? NS : 1];
    int ktj[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int kt = wk + j * WK;
        ktj[j] = kt < KT ? kt : KT - 1;
        if constexpr (GLU) {
            nib[j] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(nib_lane + static_cast<int64_t>(ktj[j]) * kTileNibBytes));
            sc[j] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x2 *>(sc_lane + static_cast<int64_t>(ktj[j]) * kTileScales * 2));
        } else {
            nib[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   nib_rsrc, lane * 16, ktj[j] * kTileNibBytes, kNonTemporal));
            sc[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                  sc_rsrc, nl * 8, ktj[j] * kTileScales * 2, kNonTemporal));
            if constexpr (ASYM)
                mo[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                      off_rsrc, nl * 8, ktj[j] * kTileScales * 2, kNonTemporal));
        }
        __builtin_amdgcn_sched_barrier(0);   // stages go out in order
    }
    // 3. this wave's x into its LDS region (waits for the x loads only);
    //    the region is the wave's alone, so a wave-scope fence stands in for
    //    a workgroup barrier
#pragma unroll
    for (int q = 0; q < kXPer; ++q)
        *reinterpret_cast<u32x4 *>(xw + (lane + 64 * q) * 16) = xv[q];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // 4. stage j's MFMAs wait for stage j's weights only
    const int a_off = (nl < mrows ? nl : mrows - 1) * (NS * 256) + g * 16;
    floatx4 acc = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const bool live = wk + j * WK < KT;
        // a stage past K adds zeros: its scales (and offsets) are zeroed once per stage
        const u32x2 scj = live ? sc[j] : (u32x2){0u, 0u};
        u32x2 moj = (u32x2){0u, 0u};
        if constexpr (ASYM) moj = live ? mo[j] : (u32x2){0u, 0u};
#pragma unroll
        for (int i = 0; i < kTileBlocks; ++i) {
            const bf16x8 A = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(xw + a_off + j * 256 + i * 64));
            const bf16x8 B = ASYM ? decode_piece_u(piece_of(nib[j], i)) : decode_piece(piece_of(nib[j], i));
            const float d = scale_of(scj, i);
            const floatx4 D = mfma_block(A, B);
#pragma unroll
            for (int r = 0; r < REGS; ++r) acc[r] = fmaf(d, D[r], acc[r]);
            if constexpr (ASYM) {
                const float m = scale_of(moj, i);
                const floatx4 S = mfma_block(A, bf16_ones());
#pragma unroll
                for (int r = 0; r < REGS; ++r) acc[r] = fmaf(m, S[r], acc[r]);
            }
        }
    }

    // wave-ordered sum of the K slices
    if constexpr (WK > 1) {
        __shared__ float red[WK - 1][REGS][64];
        if (wk > 0) {
#pragma unroll
            for (int r = 0; r < REGS; ++r) red[wk - 1][r][lane] = acc[r];
        }
        __syncthreads();
        if (wk != 0) return;
#pragma unroll
        for (int w = 0; w < WK - 1; ++w)
#pragma unroll
            for (int r = 0; r < REGS; ++r) acc[r] += red[w][r][lane];
    }
    if constexpr (GLU) {
        float u[REGS];
#pragma unroll
        for (int r = 0; r < REGS; ++r) u[r] = __shfl_xor(acc[r], 8, 64);   // column c + 8: the up row of c
        const int n = rt0 * 16 + 8 * half + nl;
        if (nl >= 8 || rt0 >= sg.RT || n >= sg.N) return;
#pragma unroll
        for (int r = 0; r < REGS; ++r) {
            const int m = 4 * g + r;
            if (m < aM) store_out(a, sg, static_cast<int64_t>(m) * sg.N + n, silu_f32(acc[r] * 16.0f) * (u[r] * 16.0f));
        }
    } else {
        const int n = rt0 * 16 + nl;
        if (rt0 >= sg.RT || n >= sg.N) return;
#pragma unroll
        for (int r = 0; r < REGS; ++r) {
            const int m = 4 * g + r;
            if (m < aM) sg.y[static_cast<int64_t>(m) * sg.N + n] = ASYM ? acc[r] : acc[r] * 16.0f;
        }
    }
}

// ----------------------------------------------------------- skinny stream
// Very tall weights (the LM head: thousands of 16-row tiles in one launch).
// A grid of as many workgroups as the device holds at once, each walking the
// tiles blockIdx.x, blockIdx.x + gridDim.x, ...  Per tile the arithmetic is
// that of skinny_kernel<MROWS, 1, WK, P, true, WPE, false> (the same
// super-tiles per wave, added in the same order, the same wave-ordered
// reduction), so the results are bitwise equal to it.  x is staged in LDS
// once per workgroup instead of once per tile, and a wave issues the load of
// its next stage -- the next tile's, across the boundary -- as soon as a
// stage is consumed, so the weight stream keeps running through each tile's
// reduction.  Every wave owns KT / WK super-tiles of every tile (the
// launcher requires KT % WK == 0), so all waves meet each tile's barrier.
template <int MROWS, int WK, int P, int WPE>
__global__ __launch_bounds__(64 * WK) __attribute__((amdgpu_waves_per_eu(WPE > 0 ? WPE : 1, 8)))
void skinny_stream_kernel(const LinearArgs a, const int tiles) {
    static_assert(MROWS <= 16 && WK > 1, "one 16-row m-tile, K split over the waves");
    constexpr int REGS = MROWS < 4 ? MROWS : 4;
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
    // wave-ordered partial sums, double-buffered by tile parity so that one
    // barrier per tile suffices
    __shared__ float red[2][WK - 1][REGS][64];
    const int lane = threadIdx.x & 63;
    const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nl = lane & 15, g = lane >> 4;
    const int KT = a.KT;
    const int mrows = a.M < 16 ? a.M : 16;
    const int row_bytes = x_row_bytes(KT);
    const int nkt = KT / WK;
    const int stride = gridDim.x;
    const int my_tiles = (tiles - static_cast<int>(blockIdx.x) + stride - 1) / stride;
    const int total = my_tiles * nkt;   // stages of this wave

    // the next stage to load: super-tile wk + ld_j * WK of tile ld_tile
    int ld_tile = blockIdx.x, ld_j = 0;
    const uint8_t *ld_nib = nullptr;
    const uint16_t *ld_sc = nullptr;
    auto aim = [&](int tile) {
        const Segment &sg = a.seg[find_segment(a, tile)];
        const int64_t T0 = static_cast<int64_t>(tile - sg.tile_begin) * KT + wk;
        ld_nib = sg.nib + T0 * kTileNibBytes + lane * 16;
        ld_sc = sg.scales + T0 * kTileScales + nl * 4;
    };
    struct WStage {
        u32x4 nib;
        u32x2 sc;
    };
    auto load_next = [&](WStage &S) {
        S.nib = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ld_nib + static_cast<int64_t>(ld_j) * WK * kTileNibBytes));
        S.sc = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(ld_sc + static_cast<int64_t>(ld_j) * WK * kTileScales));
        if (++ld_j == nkt) {
            ld_j = 0;
            ld_tile += stride;
            if (ld_tile < tiles) aim(ld_tile);
        }
    };

    const int a_row = nl < mrows ? nl : mrows - 1;
    floatx4 acc = (floatx4){0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const WStage &S, int kt) {
#pragma unroll
        for (int i = 0; i < kTileBlocks; ++i) {
            const int b = kt * kTileBlocks + i;
            const bf16x8 A = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(xs + a_row * row_bytes + (b * kQK + g * 8) * 2));
            const bf16x8 B = decode_piece(piece_of(S.nib, i));
            const float d = scale_of(S.sc, i);
            const floatx4 D = mfma_block(A, B);
#pragma unroll
            for (int r = 0; r < REGS; ++r) acc[r] = fmaf(d, D[r], acc[r]);
        }
    };

    // 1. the first P stages, then x (zero beyond K) while they are in flight
    aim(ld_tile);
    WStage st[P];
#pragma unroll
    for (int p = 0; p < P; ++p)
        if (p < total) load_next(st[p]);
    {
        const int chunks_per_row = KT * (kTileK / 8);
        const int all = mrows * chunks_per_row;
        for (int c = threadIdx.x; c < all; c += 64 * WK) {
            const int m = c / chunks_per_row, kc = c - m * chunks_per_row;
            u32x4 v = (u32x4){0u, 0u, 0u, 0u};
            if (kc * 8 < a.K) v = *reinterpret_cast<const u32x4 *>(a.x + static_cast<int64_t>(m) * a.K + kc * 8);
            *reinterpret_cast<u32x4 *>(xs + m * row_bytes + kc * 16) = v;
        }
        __syncthreads();
    }

    // 2. every stage: compute, refill P stages ahead, and at a tile's last
    //    super-tile reduce over the waves and store
    int cj = 0, out_tile = blockIdx.x, parity = 0;
    for (int q0 = 0; q0 < total; q0 += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int q = q0 + p;
            if (q >= total) break;
            compute(st[p], wk + cj * WK);
            if (q + P < total) load_next(st[p]);
            if (++cj < nkt) continue;
            cj = 0;
            if (wk > 0) {
#pragma unroll
                for (int r = 0; r < REGS; ++r) red[parity][wk - 1][r][lane] = acc[r];
            }
            __syncthreads();
            if (wk == 0) {
#pragma unroll
                for (int w = 0; w < WK - 1; ++w)
#pragma unroll
                    for (int r = 0; r < REGS; ++r) acc[r] += red[parity][w][r][lane];
                const Segment &sg = a.seg[find_segment(a, out_tile)];
                const int n = (out_tile - sg.tile_begin) * 16 + nl;
                if (n < sg.N) {
#pragma unroll
                    for (int r = 0; r < REGS; ++r) {
                        const int m = 4 * g + r;
                        if (m < a.M) sg.y[static_cast<int64_t>(m) * sg.N + n] = acc[r] * 16.0f;
                    }
                }
            }
            acc = (floatx4){0.f, 0.f, 0.f, 0.f};
            out_tile += stride;
            parity ^= 1;
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

// Byte offset of 16-byte chunk c (0..15) of row m in a swizzled A tile: the
// chunk index is XORed with the row's low 4 bits, so the 16 rows read by one
// MFMA A fragment (same chunk) land in 16 different chunk slots.
__device__ __forceinline__ int a_tile_offset(int m, int c) { return (m * 16 + (c ^ (m & 15))) * 16; }

// PB weight stages per wave: the loads for step kt + PB - 1 are issued while
// step kt computes (the x tile is double-buffered in LDS either way).  Each
// weight tile is read by one workgroup per 64 rows of x, so the weight loads
// are nontemporal.
//
// GLU: as in gemm3_kernel, the first WN / 2 waves of a workgroup row run
// gate rows and the last WN / 2 the same rows of up, each exactly as a plain
// launch would, and the up waves hand their results to the gate waves
// through LDS for the silu(gate) * up epilogue.
template <int MT, int NT, int WM, int WN, int WPE, int PB, bool GLU = false>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(WPE > 0 ? WPE : 1, 8)))
void gemm_kernel(const LinearArgs a) {
    static_assert(PB >= 2, "at least one step of weights in flight");
    static_assert(!GLU || (WN % 2 == 0 && (WN / 2) * NT <= 8), "gate / up waves and their LDS hand-off");
    using C = GemmCfg<MT, NT, WM, WN>;
    constexpr int BM = C::BM, NPT = C::kAPerThread;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * 256];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: uniform branches
    const int wm = wave / WN, wn = wave % WN;
    const int nl = lane & 15, g = lane >> 4;

    constexpr int WNO = GLU ? WN / 2 : WN;   // waves per workgroup row with distinct output rows
    const bool up_wave = GLU && wn >= WNO;
    const int wno = GLU ? wn % WNO : wn;
    const int s = GLU ? 0 : find_segment(a, blockIdx.x);
    const Segment sg = a.seg[s];
    const Segment &src = up_wave ? a.seg[1] : sg;   // the matrix this wave streams
    const int rt_base = (static_cast<int>(blockIdx.x) - sg.tile_begin) * (NT * WNO) + wno * NT;
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
            a_regs[j] = (u32x4){0u, 0u, 0u, 0u};
            if (m0 + m < a.M && b < nblk)
                a_regs[j] = *reinterpret_cast<const u32x4 *>(
                    a.x + static_cast<int64_t>(m0 + m) * a.K + kt * kTileK + c * 8);
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

    // ---- B: this wave's NT weight tiles, straight into registers.  Tiles
    // past the segment's end read its last tile (never stored).
    const uint8_t *nib_base[NT];
    const uint16_t *sc_base[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int rt = rt_base + nt < src.RT ? rt_base + nt : src.RT - 1;
        const int64_t T0 = static_cast<int64_t>(rt) * KT;
        nib_base[nt] = src.nib + T0 * kTileNibBytes + lane * 16;
        sc_base[nt] = src.scales + T0 * kTileScales + nl * 4;
    }
    struct BStage {
        u32x4 nib[NT];
        u32x2 sc[NT];
    };
    auto load_b = [&](BStage &S, int kt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            S.nib[nt] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(nib_base[nt] + static_cast<int64_t>(kt) * kTileNibBytes));
            S.sc[nt] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(sc_base[nt] + static_cast<int64_t>(kt) * kTileScales));
        }
    };

    floatx4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (floatx4){0.f, 0.f, 0.f, 0.f};

    int a_off[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a_off[mt] = ((wm * MT + mt) * 16 + nl) * 256;

    auto compute = [&](int buf, const BStage &S) {
        const uint8_t *tile = lds_a[buf];
#pragma unroll
        for (int i = 0; i < kTileBlocks; ++i) {
            bf16x8 A[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = (wm * MT + mt) * 16 + nl;
                A[mt] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(tile + a_off[mt] + (((4 * i + g) ^ (m & 15)) * 16)));
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
                // keep one weight tile's MFMAs and rescales together: bounds
                // the live MFMA results (register pressure -> occupancy)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // step kt: x from LDS buffer kt % 2, weights from stage kt % PB; the loop
    // is unrolled so both indices are static.  Loads past the last step are
    // clamped to it (their stages are never used).
    constexpr int U = PB % 2 == 0 ? PB : 2 * PB;
    BStage W[PB];
    const int kt_last = KT - 1;
#pragma unroll
    for (int p = 0; p < PB - 1; ++p) load_b(W[p], p < kt_last ? p : kt_last);
    load_a(0);
    store_a(0);
    __syncthreads();
    for (int kt0 = 0;; kt0 += U) {
        bool done = false;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kt = kt0 + u;
            const int kp = kt + PB - 1;
            load_b(W[(u + PB - 1) % PB], kp < kt_last ? kp : kt_last);
            const bool more = kt < kt_last;
            if (more) load_a(kt + 1);
            // always true here; as a branch it keeps the compiler from
            // interleaving the surrounding loads into the compute block, which
            // took 32-row launches from 80 to 56 VGPRs (6 -> 8 waves per SIMD;
            // 8% faster on the 32-row LM head) and 64-row ones from 126 to 90
            if (kt < KT) compute(u % 2, W[u % PB]);
            if (!more) {
                done = true;
                break;
            }
            store_a((u + 1) % 2);
            __syncthreads();
        }
        if (done) break;
    }

    // gated: once every wave is past its last step's x reads, the up waves
    // leave their results in the x buffers for the matching gate wave
    float *xch = reinterpret_cast<float *>(&lds_a[0][0]) + (wm * WNO + wno) * (MT * NT * 4 * 64);
    if constexpr (GLU) {
        __syncthreads();
        if (up_wave) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) xch[((mt * NT + nt) * 4 + r) * 64 + lane] = acc[mt][nt][r];
        }
        __syncthreads();
        if (up_wave) return;
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
                if (m >= a.M) continue;
                if constexpr (GLU)
                    store_out(a, sg, static_cast<int64_t>(m) * sg.N + n,
                              silu_f32(acc[mt][nt][r] * 16.0f) * (xch[((mt * NT + nt) * 4 + r) * 64 + lane] * 16.0f));
                else
                    sg.y[static_cast<int64_t>(m) * sg.N + n] = acc[mt][nt][r] * 16.0f;
            }
    }
}

// ------------------------------------------------------------------- gemm3
// Prefill-sized M with register tiles of MT x NT MFMA tiles per wave.  The
// x tile of the next 128-k step is staged a quarter per block step (so the
// staging registers stay few) into the other LDS buffer; the rescale of
// each group of MFMA results is issued after the next group's MFMAs, so the
// FMAs never wait on a result still in flight.  Work tiles are mapped to
// workgroups so that each of the 8 XCDs owns a contiguous range of them, in
// an order where GM consecutive tiles share one weight tile.  128-row tiles
// take GM = 4: an XCD's resident workgroups then cover 4 x tiles (3 MiB of x
// at K = 3072, within its 4 MiB L2) and 16 weight tiles; at M = 2048 that
// read 31-35% fewer bytes from beyond L2 than groups of 8, in the same time.
template <int MT, int NT, int WM, int WN>
struct Gemm3Cfg {
    static constexpr int BM = 16 * MT * WM;
    static constexpr int BN = 16 * NT * WN;
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int kAStep = BM * 16 / kTileBlocks;   // 16-byte x chunks staged per block step
    // Threads per staged chunk set: the largest whole number of waves that
    // divides the chunks of a step (all threads when they do); the other
    // waves then load and store the same chunks again (the same bytes to the
    // same place), which keeps the loop free of branches.
    static constexpr int stagers() {
        int t = kThreads < kAStep ? kThreads : kAStep;
        while (t > 64 && kAStep % t != 0) t -= 64;
        return t;
    }
    static constexpr int kStagers = stagers();
    static constexpr int kAPerThread = kAStep / kStagers;
    static_assert(kAStep % kStagers == 0 && kStagers % 64 == 0, "x staging must split evenly over whole waves");
};

// GLU: gate / up as in skinny_kernel: the first WN / 2 waves of a workgroup
// row run gate rows, the last WN / 2 the same rows of up, each exactly as a
// plain launch would; each gate wave and its up wave trade half of their
// results through LDS and form silu(gate) * up for half the m-tiles each.
//
// ASYM: the asymmetric layout (w = q d + m).  The codes are decoded as q and
// each block's product D is rescaled by d as in the symmetric kernel; the
// offsets' share, sum over blocks b of m[n, b] S[row, b] with S the block
// sums of x, is itself a small product, taken on the matrix cores once per
// 8 blocks.  Per 128-k step, wave w computes S for m-tile w % MT (four MFMAs
// against its x fragments -- block i with A rows 4i .. 4i + 3 set to ones --
// leave S[row r, block g] in lane 16 g + r) and stores S split into bf16
// hi + lo in LDS; per 8 blocks every wave builds MFMA A fragments from them
// and multiplies by its rows' offsets, split the same way (exactly: fp16 has
// 11 significant bits), accumulating into acc with k = 4 b + t running over
// the pairs (S_hi, m_hi), (S_hi, m_lo), (S_lo, m_hi), (S_lo, m_lo).
template <int MT, int NT, int WM, int WN, int WPE, int GM, bool GLU, bool ASYM = false>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(WPE > 0 ? WPE : 1, 8)))
void gemm3_kernel(const LinearArgs a, const int mtiles, const int ntiles) {
    static_assert(!(GLU && ASYM), "no gated launch of the asymmetric layout");
    static_assert(!ASYM || (WM == 1 && WN >= MT), "asymmetric: one wave per m-tile computes its block sums");
    using C = Gemm3Cfg<MT, NT, WM, WN>;
    constexpr int BM = C::BM, NPT = C::kAPerThread;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * 256];
    // asymmetric: S of two 8-block windows, the one being read and the one
    // being written, as (hi, lo) bf16 pairs [m-tile][row][block]
    __shared__ __attribute__((aligned(16))) uint32_t lds_s[ASYM ? 2 : 1][ASYM ? MT * 16 * 8 : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int nl = lane & 15, g = lane >> 4;

    // workgroup -> tile: XCD x (dispatch round-robins workgroups over the 8
    // XCDs) takes the x-th contiguous share of the tile order
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int q8 = nwg >> 3, r8 = nwg & 7, xcd = bid & 7, local = bid >> 3;
    const int t = (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + local;
    const int per_group = GM * ntiles;
    const int first_m = (t / per_group) * GM;
    const int gsize = mtiles - first_m < GM ? mtiles - first_m : GM;
    const int within = t - (t / per_group) * per_group;
    const int mtile = first_m + within % gsize;
    const int ntile = within / gsize;

    static_assert(!GLU || (WN % 2 == 0 && (WN / 2) * NT <= 8), "gate / up waves and their LDS hand-off");
    constexpr int WNO = GLU ? WN / 2 : WN;   // waves per workgroup row with distinct output rows
    const bool up_wave = GLU && wn >= WNO;
    const int wno = GLU ? wn % WNO : wn;
    const int s = GLU ? 0 : find_segment(a, ntile);
    const Segment sg = a.seg[s];
    const Segment &src = up_wave ? a.seg[1] : sg;   // the matrix this wave streams
    const int rt_base = (ntile - sg.tile_begin) * (NT * WNO) + wno * NT;
    const int m0 = mtile * BM;
    const int KT = a.KT;
    const int nblk = a.K / kQK;

    // ---- x staging: part p of a tile is chunks p * kAStep + tid % kStagers + kStagers * j,
    // i.e. chunk c = tid % 16 of rows p * kAStep / 16 + (tid % kStagers) / 16 + j * kStagers / 16
    // (both steps are multiples of 16 rows, so every chunk of a thread has the same c).
    // Loads go through a buffer resource over this tile's rows: a row past M
    // lies beyond the resource's size and reads zeros (its outputs are never
    // stored), and a chunk past K gets an offset beyond every resource, so
    // the loop has no branch.
    const int rows = a.M - m0 < BM ? a.M - m0 : BM;
    const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.x + static_cast<int64_t>(m0) * a.K), 0, rows * a.K * 2, kBufferRsrcWord3);
    const int x_st = tid % C::kStagers, x_c = x_st & 15;
    const int x_base = (x_st >> 4) * a.K * 2 + x_c * 16;                  // byte offset at k-step 0, part 0, j 0
    const int x_kt_end = (nblk - (x_c >> 2) + kTileBlocks - 1) / kTileBlocks;   // first k-step past K
    auto load_part = [&](u32x4 (&R)[NPT], int kt, int part) {
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
            const int row = part * (C::kAStep / 16) + j * (C::kStagers / 16);
            const int off = kt < x_kt_end ? x_base + row * a.K * 2 : kOutOfRange;
            R[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, off, kt * kTileK * 2, 0));
        }
    };
    auto store_part = [&](const u32x4 (&R)[NPT], int buf, int part) {
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
            const int qc = part * C::kAStep + tid % C::kStagers + C::kStagers * j;
            const int m = qc >> 4, c = qc & 15;
            *reinterpret_cast<u32x4 *>(&lds_a[buf][a_tile_offset(m, c)]) = R[j];
        }
    };

    // ---- weights: this wave's NT tiles, straight into registers.  Each tile
    // row's planes are a buffer resource (wave-uniform, in SGPRs) read at a
    // per-lane offset shared by all tiles, so the addresses cost no VGPRs.
    __amdgpu_buffer_rsrc_t nib_rsrc[NT], sc_rsrc[NT], off_rsrc[ASYM ? NT : 1];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int rt = rt_base + nt < src.RT ? rt_base + nt : src.RT - 1;
        const int64_t T0 = static_cast<int64_t>(rt) * KT;
        nib_rsrc[nt] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(src.nib + T0 * kTileNibBytes), 0,
                                                         KT * kTileNibBytes, kBufferRsrcWord3);
        sc_rsrc[nt] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(src.scales + T0 * kTileScales), 0,
                                                        KT * kTileScales * 2, kBufferRsrcWord3);
        if constexpr (ASYM)
            off_rsrc[nt] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(src.offsets + T0 * kTileScales),
                                                             0, KT * kTileScales * 2, kBufferRsrcWord3);
    }
    const int nib_lane = lane * 16, sc_lane = nl * 8;
    struct BStage {
        u32x4 nib[NT];
        u32x2 sc[NT];
    };
    auto load_b = [&](BStage &S, int kt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            S.nib[nt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(nib_rsrc[nt], nib_lane, kt * kTileNibBytes, 0));
            S.sc[nt] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(sc_rsrc[nt], sc_lane, kt * kTileScales * 2, 0));
        }
    };

    floatx4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (floatx4){0.f, 0.f, 0.f, 0.f};

    const int a_row0 = (wm * MT) * 16 + nl;   // LDS row of m-tile 0 for this lane; m-tile mt adds 16 mt
    // asymmetric: this step's block sums (of m-tile wave % MT), and per
    // n-tile the two offsets (an fp16 pair) of this lane's blocks 2g, 2g + 1
    // of an 8-block window: row nl of super-tile 2 win + g / 2, blocks
    // 2 (g & 1), + 1.  The whole offset is in the per-lane (range-checked)
    // part, so a super-tile past K reads zeros.
    floatx4 ssum = (floatx4){0.f, 0.f, 0.f, 0.f};
    uint32_t mpair[NT];
    const int m_lane = nl * 8 + (g & 1) * 4 + (g >> 1) * kTileScales * 2;
    auto load_offsets = [&](int win) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            mpair[nt] = __builtin_amdgcn_raw_buffer_load_b32(off_rsrc[nt], m_lane + 2 * win * kTileScales * 2, 0, 0);
    };

    auto compute_block = [&](int buf, const BStage &S, int i) {
        const uint8_t *tile = lds_a[buf];
        const int sw = ((4 * i + g) ^ nl) * 16;   // swizzled chunk of block i (row & 15 == nl)
        bf16x8 A[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            A[mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(tile + (a_row0 + 16 * mt) * 256 + sw));
        if constexpr (ASYM) {
            // block sums of x for m-tile wave % MT (waves past MT repeat
            // one, without a branch): A rows 4i .. 4i + 3 are ones, so after
            // the step's four blocks lane 16 g + r holds S[row r, block g]
            const bf16x8 X = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4 *>(tile + ((wave % MT) * 16 + nl) * 256 + sw));
            const uint32_t ones = (nl >> 2) == i ? 0x3F803F80u : 0u;   // two bf16 1.0
            ssum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, (u32x4){ones, ones, ones, ones}),
                                                           X, i == 0 ? (floatx4){0.f, 0.f, 0.f, 0.f} : ssum, 0, 0, 0);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const bf16x8 B = ASYM ? decode_piece_u(piece_of(S.nib[nt], i)) : decode_piece(piece_of(S.nib[nt], i));
            const float d = scale_of(S.sc[nt], i);
            // each MFMA's rescale is issued after the next MFMA, so the FMAs
            // never wait on a result still in the matrix pipe
            floatx4 D[MT];
            D[0] = mfma_block(A[0], B);
#pragma unroll
            for (int mt = 1; mt < MT; ++mt) {
                D[mt] = mfma_block(A[mt], B);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mt - 1][nt][r] = fmaf(d, D[mt - 1][r], acc[mt - 1][nt][r]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[MT - 1][nt][r] = fmaf(d, D[MT - 1][r], acc[MT - 1][nt][r]);
        }
        // blocks in groups: within a group the compiler may pull a block's x
        // reads up among the previous block's MFMAs (hiding their LDS
        // latency); the barrier between groups bounds the live MFMA results
        // and operands.  Groups of 2 blocks for 8 m-tiles, of 4 (a whole
        // step) for 4 m-tiles.  Against a barrier after every block: +3-4%
        // at M = 2048 and +5-6% at M = 1505 (128-row tiles, 113 VGPRs either
        // way), +3-9% at M = 130 and 300 (64-row tiles).
        if ((i + 1) % (MT >= 8 ? 2 : 4) == 0) __builtin_amdgcn_sched_barrier(0);
    };

    u32x4 R0[NPT], R1[NPT];
    BStage b0, b1;
    load_b(b0, 0);
#pragma unroll
    for (int p = 0; p < kTileBlocks; ++p) {
        load_part(R0, 0, p);
        store_part(R0, 0, p);
    }
    __syncthreads();

    // asymmetric: the offsets' share of 8-block window `win` (steps 2 win and
    // 2 win + 1) into acc.  `half`: the window's second step lies past K, and
    // lanes g >= 2 (its blocks) add zeros.
    auto offset_term = [&](int win, bool half) {
        const bool zero = half && g >= 2;
        bf16x8 MB[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            uint32_t h0, l0, h1, l1;
            split_bf16(half_bits_to_float(mpair[nt] & 0xFFFFu), h0, l0);
            split_bf16(half_bits_to_float(mpair[nt] >> 16), h1, l1);
            const uint32_t w0 = zero ? 0u : h0 | (l0 << 16), w1 = zero ? 0u : h1 | (l1 << 16);
            MB[nt] = __builtin_bit_cast(bf16x8, (u32x4){w0, w0, w1, w1});
        }
        const uint32_t *sb = lds_s[win & 1] + nl * 8 + 2 * g;   // row nl, blocks 2g, 2g + 1
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const u32x2 p = zero ? (u32x2){0u, 0u} : *reinterpret_cast<const u32x2 *>(sb + mt * 128);
            // (hi, hi), (lo, lo) of each block: byte selects of its pair
            const u32x4 sa = (u32x4){__builtin_amdgcn_perm(p.x, p.x, 0x01000100u), __builtin_amdgcn_perm(p.x, p.x, 0x03020302u),
                                     __builtin_amdgcn_perm(p.y, p.y, 0x01000100u), __builtin_amdgcn_perm(p.y, p.y, 0x03020302u)};
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, sa), MB[nt],
                                                                      acc[mt][nt], 0, 0, 0);
        }
    };
    // asymmetric, after the blocks of step kt (parity cur): lane (r, g)
    // stores S of row r, block g of the step, for m-tile wave % MT (waves
    // past MT store the same bytes as wave % MT).  No store here depends on
    // the lane: as a branch it cost some 70 more registers.
    auto window_part = [&](int kt, int cur) {
        uint32_t h, l;
        split_bf16(ssum[0], h, l);
        lds_s[(kt >> 1) & 1][(wave % MT) * 128 + nl * 8 + 4 * cur + g] = h | (l << 16);
    };

    // One 128-k step with no branches: the loads for step kt + 1 are clamped
    // to the last step (the extra loads and stores of the final step go to
    // the buffer nobody reads any more).  Loads complete in issue order for
    // the wait counter, so the next step's weights go out after the first two
    // x parts: storing part 0 then waits for x alone, and the weights have
    // until part 2's store (two blocks of compute) to arrive.  Issued ahead
    // of the x parts instead, they had one block, which cost 2-4% at
    // M = 2048 and 7-14% at M = 130.
    auto step = [&](int kt, int cur, BStage &bc, BStage &bn) {
        const int kn = kt + 1 < KT ? kt + 1 : KT - 1;
        load_part(R0, kn, 0);
        load_part(R1, kn, 1);
        load_b(bn, kn);
        if constexpr (ASYM) {
            if (cur == 0 && kt > 0) offset_term((kt >> 1) - 1, false);   // the window that ended
            if (cur == 0) load_offsets(kt >> 1);                        // the window that starts
        }
        compute_block(cur, bc, 0);
        store_part(R0, cur ^ 1, 0);
        load_part(R0, kn, 2);
        compute_block(cur, bc, 1);
        store_part(R1, cur ^ 1, 1);
        load_part(R1, kn, 3);
        compute_block(cur, bc, 2);
        store_part(R0, cur ^ 1, 2);
        compute_block(cur, bc, 3);
        store_part(R1, cur ^ 1, 3);
        if constexpr (ASYM) window_part(kt, cur);
        __syncthreads();
    };
    for (int kt = 0;;) {
        step(kt, 0, b0, b1);
        if (++kt == KT) break;
        step(kt, 1, b1, b0);
        if (++kt == KT) break;
    }
    if constexpr (ASYM) offset_term((KT - 1) >> 1, (KT & 1) != 0);   // the last window (one step if KT is odd)

    // gated: a gate wave and its up wave split the epilogue. The gate wave
    // leaves g of its last MT / 2 m-tiles in LDS, the up wave u of its first
    // MT / 2 (the x buffers are free once the last step's barrier has passed);
    // each then forms silu(g) * u for its own half of the m-tiles.
    static_assert(!GLU || MT % 2 == 0, "the gated epilogue splits the m-tiles in halves");
    float *xch = reinterpret_cast<float *>(&lds_a[0][0]) + (wm * WNO + wno) * (MT * NT * 4 * 64);
    if constexpr (GLU) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            if ((mt < MT / 2) == up_wave)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) xch[((mt * NT + nt) * 4 + r) * 64 + lane] = acc[mt][nt][r];
        __syncthreads();
    }

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int rt = rt_base + nt;
        const int n = rt * 16 + nl;
        if (rt >= sg.RT || n >= sg.N) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (GLU && (mt < MT / 2) == up_wave) continue;   // the other wave of the pair stores these
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + (wm * MT + mt) * 16 + 4 * g + r;
                if (m >= a.M) continue;
                const float v = ASYM ? acc[mt][nt][r] : acc[mt][nt][r] * 16.0f;
                if constexpr (GLU) {
                    const float other = xch[((mt * NT + nt) * 4 + r) * 64 + lane] * 16.0f;
                    store_out(a, sg, static_cast<int64_t>(m) * sg.N + n,
                              up_wave ? silu_f32(other) * v : silu_f32(v) * other);
                } else {
                    sg.y[static_cast<int64_t>(m) * sg.N + n] = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------- launch
// Events armed by q4_0_time_next_launch for this thread's next linear launch.
thread_local hipEvent_t t_start_event = nullptr;
thread_local hipEvent_t t_stop_event = nullptr;

template <typename Kernel, typename... Args>
hipError_t launch_kernel(Kernel kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                         const Args &...a) {
    if (t_start_event || t_stop_event) {
        hipEvent_t start = t_start_event, stop = t_stop_event;
        t_start_event = t_stop_event = nullptr;
        // records the events at the kernel's own start and end
        hipExtLaunchKernelGGL(kernel, grid, block, lds, s, start, stop, 0, a...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, lds, s, a...);
    }
    return hipGetLastError();
}

// Tile configurations depend on M and K only, so a fused multi-segment launch
// and separate single launches run the same arithmetic in the same order.

// x is staged in LDS when it fits a budget that keeps several workgroups on
// a CU: up to 4 rows it may take 128 KiB (x is small next to the weights);
// for more rows 48 KiB, since a 16-row x of 3072 columns (98 KiB) would leave
// room for one workgroup per CU, and those rows then read x from L2 instead.
constexpr uint32_t kMaxXLds = 128 * 1024;
constexpr uint64_t xlds_budget(int mrows_max) { return mrows_max <= 4 ? kMaxXLds : 48 * 1024; }
inline uint64_t skinny_x_bytes(int64_t M, int64_t K, int mrows_max) {
    const int64_t mrows = M < mrows_max ? M : mrows_max;
    return static_cast<uint64_t>(mrows) * static_cast<uint64_t>((K + kTileK - 1) / kTileK * kTileK * 2 + 16);
}

// hipFuncSetAttribute (the dynamic LDS limit) is applied once per device
// and kernel instantiation.
template <typename Kernel>
hipError_t allow_dynamic_lds(Kernel kernel, std::atomic<uint64_t> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = uint64_t(1) << (dev & 63);
    if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, kMaxXLds);
    if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

// Work tiles of a launch: the segments' tiles laid end to end, each tile
// covering `rows_per_tile` 16-row tiles; a gated launch tiles the gate rows
// only (the up rows ride along in the same workgroups).
template <bool GLU>
int assign_tiles(LinearArgs &a, int rows_per_tile) {
    if (GLU) {
        a.seg[0].tile_begin = 0;
        a.seg[1].tile_begin = 0;
        return (a.seg[0].RT + rows_per_tile - 1) / rows_per_tile;
    }
    int tiles = 0;
    for (int i = 0; i < a.nseg; ++i) {
        a.seg[i].tile_begin = tiles;
        tiles += (a.seg[i].RT + rows_per_tile - 1) / rows_per_tile;
    }
    return tiles;
}

// Compute units of the current device, queried once per device (256 on
// MI355X; also the answer when there is no device to ask).
int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = 256;
    }
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Workgroups of a stream kernel resident per CU at this dynamic LDS size,
// cached per device for the last size asked (1 if the runtime cannot say).
template <typename Kernel>
int resident_per_cu(Kernel kernel, int threads, uint32_t lds, std::atomic<uint64_t> (&cache)[64]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 1;
    }
    const uint64_t v = cache[dev].load(std::memory_order_relaxed);
    if (v != 0 && (v >> 16) == lds) return static_cast<int>(v & 0xffff);
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void *>(kernel), threads, lds) !=
            hipSuccess || occ < 1) {
        (void)hipGetLastError();
        occ = 1;
    }
    if (occ > 0xffff) occ = 0xffff;
    cache[dev].store((static_cast<uint64_t>(lds) << 16) | static_cast<uint64_t>(occ), std::memory_order_relaxed);
    return occ;
}

// The stream launch: x must fit the LDS budget and KT be a multiple of WK
// (the dispatch checks both).
template <int MROWS, int WK, int P, int WPE>
hipError_t run_skinny_stream(LinearArgs a, hipStream_t s) {
    const int tiles = assign_tiles<false>(a, 1);
    const uint32_t lds = static_cast<uint32_t>(skinny_x_bytes(a.M, a.K, MROWS));
    auto kernel = skinny_stream_kernel<MROWS, WK, P, WPE>;
    static std::atomic<uint64_t> lds_allowed{0};
    const hipError_t e = allow_dynamic_lds(kernel, lds_allowed);
    if (e != hipSuccess) return e;
    static std::atomic<uint64_t> occ_cache[64];
    const int64_t resident = static_cast<int64_t>(device_cus()) * resident_per_cu(kernel, 64 * WK, lds, occ_cache);
    const int grid = static_cast<int>(tiles < resident ? tiles : resident);
    if (t_start_event || t_stop_event) {
        hipEvent_t start = t_start_event, stop = t_stop_event;
        t_start_event = t_stop_event = nullptr;
        hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(64 * WK), lds, s, start, stop, 0, a, tiles);
    } else {
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(64 * WK), lds, s, a, tiles);
    }
    return hipGetLastError();
}

template <int MROWS, int NT, int WK, int P, int WPE = 0, bool GLU = false>
hipError_t run_skinny(LinearArgs a, hipStream_t s) {
    const int tiles = assign_tiles<GLU>(a, NT);
    constexpr int kThreads = 64 * WK * (GLU ? 2 : 1);
    static_assert(MROWS <= 64, "at most four 16-row m-tiles per wave");
    const uint64_t lds = skinny_x_bytes(a.M, a.K, MROWS);
    if (lds <= xlds_budget(MROWS)) {
        auto kernel = skinny_kernel<MROWS, NT, WK, P, true, WPE, GLU>;
        static std::atomic<uint64_t> lds_allowed{0};
        const hipError_t e = allow_dynamic_lds(kernel, lds_allowed);
        if (e != hipSuccess) return e;
        return launch_kernel(kernel, dim3(tiles), dim3(kThreads), static_cast<uint32_t>(lds), s, a);
    }
    return launch_kernel(skinny_kernel<MROWS, NT, WK, P, false, WPE, GLU>, dim3(tiles), dim3(kThreads), 0, s, a);
}

// The decode kernel with all NS = ceil(KT / WK) weight stages of a wave in
// flight at once: up to kGemvMaxStages stages, so the dispatch takes it for
// KT <= 6 WK (K <= 4096 with 8 or 16 K-slices, K <= 9216 with 12).  Each wave stages its own x chunks (at most 4 rows x 6 stages x
// 256 bytes); the launcher instantiates one kernel per NS.
constexpr int kGemvMaxStages = 6;
inline int gemv_stages(const LinearArgs &a, int wk) { return (a.KT + wk - 1) / wk; }

template <int MROWS, int WK, int NS, int WPE, bool GLU, bool ASYM>
hipError_t launch_gemv_ns(const LinearArgs &a, int tiles, uint32_t lds, hipStream_t s) {
    auto kernel = gemv_kernel<MROWS, WK, NS, WPE, GLU, ASYM>;
    static std::atomic<uint64_t> lds_allowed{0};
    const hipError_t e = allow_dynamic_lds(kernel, lds_allowed);
    if (e != hipSuccess) return e;
    // x, the sizes and the segments' start tiles go ahead of the segment table
    // as scalar arguments (preloaded into SGPRs where the firmware supports it)
    return launch_kernel(kernel, dim3(tiles), dim3(64 * WK), lds, s, a.x, a.M, a.K, a.KT, a.nseg, a.seg[1].tile_begin,
                         a.seg[2].tile_begin, a.seg[3].tile_begin, a.seg[4].tile_begin, a.seg[5].tile_begin,
                         a.seg[6].tile_begin, a.seg[7].tile_begin, a);
}

// NSMAX: the most stages the dispatch can ask of this configuration (only
// those stage counts are instantiated).
template <int MROWS, int WK, int WPE, bool GLU, int NSMAX, bool ASYM = false>
hipError_t run_gemv(LinearArgs a, hipStream_t s) {
    static_assert(NSMAX >= 1 && NSMAX <= kGemvMaxStages, "stage count");
    // gated: two 8-row halves per tile, in groups of 8 tiles (the groups past
    // the last tile read it again and store nothing)
    const int tiles = GLU ? (assign_tiles<GLU>(a, 1) + 7) / 8 * 16 : assign_tiles<GLU>(a, 1);
    const int ns = gemv_stages(a, WK);
    // each wave's x chunks, rounded up to whole 64-lane stores
    const uint32_t lds = static_cast<uint32_t>(WK * ((MROWS * ns * 16 + 63) / 64) * 64 * 16);
    switch (ns) {
        case 1: return launch_gemv_ns<MROWS, WK, 1, WPE, GLU, ASYM>(a, tiles, lds, s);
        case 2: if constexpr (NSMAX >= 2) return launch_gemv_ns<MROWS, WK, 2, WPE, GLU, ASYM>(a, tiles, lds, s); break;
        case 3: if constexpr (NSMAX >= 3) return launch_gemv_ns<MROWS, WK, 3, WPE, GLU, ASYM>(a, tiles, lds, s); break;
        case 4: if constexpr (NSMAX >= 4) return launch_gemv_ns<MROWS, WK, 4, WPE, GLU, ASYM>(a, tiles, lds, s); break;
        case 5: if constexpr (NSMAX >= 5) return launch_gemv_ns<MROWS, WK, 5, WPE, GLU, ASYM>(a, tiles, lds, s); break;
        case 6: if constexpr (NSMAX >= 6) return launch_gemv_ns<MROWS, WK, 6, WPE, GLU, ASYM>(a, tiles, lds, s); break;
        default: break;
    }
    return hipErrorInvalidValue;   // the dispatch never asks for more than NSMAX stages
}

template <int MT, int NT, int WM, int WN, int WPE = 0, int PB = 2, bool GLU = false>
hipError_t run_gemm(LinearArgs a, hipStream_t s) {
    using C = GemmCfg<MT, NT, WM, WN>;
    const int tiles = assign_tiles<GLU>(a, NT * (GLU ? WN / 2 : WN));
    const int mtiles = (a.M + C::BM - 1) / C::BM;
    return launch_kernel(gemm_kernel<MT, NT, WM, WN, WPE, PB, GLU>, dim3(tiles, mtiles), dim3(C::kThreads), 0, s, a);
}

template <int MT, int NT, int WM, int WN, int WPE = 0, int GM = 8, bool GLU = false, bool ASYM = false>
hipError_t run_gemm3(LinearArgs a, hipStream_t s) {
    using C = Gemm3Cfg<MT, NT, WM, WN>;
    const int ntiles = assign_tiles<GLU>(a, NT * (GLU ? WN / 2 : WN));
    const int mtiles = static_cast<int>((a.M + C::BM - 1) / C::BM);
    const int64_t total = static_cast<int64_t>(ntiles) * mtiles;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    auto kernel = gemm3_kernel<MT, NT, WM, WN, WPE, GM, GLU, ASYM>;
    const dim3 grid(static_cast<uint32_t>(total)), block(C::kThreads);
    if (t_start_event || t_stop_event) {
        hipEvent_t start = t_start_event, stop = t_stop_event;
        t_start_event = t_stop_event = nullptr;
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, start, stop, 0, a, mtiles, ntiles);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, 0, s, a, mtiles, ntiles);
    }
    return hipGetLastError();
}

}  // namespace

void arm_launch_events(hipEvent_t start, hipEvent_t stop) {
    t_start_event = start;
    t_stop_event = stop;
}

bool take_launch_events(hipEvent_t &start, hipEvent_t &stop) {
    if (!t_start_event && !t_stop_event) return false;
    start = t_start_event;
    stop = t_stop_event;
    t_start_event = t_stop_event = nullptr;
    return true;
}

// The dispatch table.  Decode sizes (M <= 16) pick by M and K: skinny
// kernels split K over the waves of a workgroup with a short prefetch, so
// that many waves stay resident (the launches are latency-bound); long rows
// (K > 3072) split K wider; one row over very tall weights walks the tiles
// with a fixed grid.  17-64 rows choose between the K-split kernel and the
// GEMM by tile count (pick_17_64).  Above 64 rows four GEMM tile shapes compete
// on how evenly their work tiles spread over the device's compute units:
//   gemm3 64 x 128   (two workgroups per CU),
//   gemm3 128 x 128  (two workgroups per CU),
//   gemm3 128 x 192  (12 waves, one workgroup per CU),
//   gemm3 96 x 192   (12 waves, one workgroup per CU).
// A launch costs about ceil(tiles / CUs) x the time of one tile on a fully
// occupied CU; measured on MI355X at M = 1505, 2048 and 6020 over the decoder,
// adapter and encoder shapes, those per-tile times are 0.30 : 0.50 : 0.85 :
// 0.79 (the 128-row tiles' unit; 96 x 192 from the M = 1505 adapter shapes,
// where its 256 tiles ran 6-7% faster than 192 tiles of 128 x 192), and the
// smallest estimate wins (a tie goes to 128 x 128, then to 64 x 128, then to
// 128 x 192).  This puts N = 3072 at M = 2048 (384 tiles of 128 x 128 on 256
// CUs, a last round half empty) on exactly 256 tiles of 128 x 192, and at
// M = 1505 on 256 tiles of 96 x 192.  Every GEMM tile shape adds the block
// results of an output in the same order, so the choice never changes a
// result.
namespace {
enum class Cfg { G1, G1K, G2, G2K, G4, G4K, G1L, G2L, G4L, M1Stream, M1Long, M2Long, M4Long, M16, M16Long, M32, M32Split, M32Split2,
                 M64, M64Split,
                 Gemm64, Gemm128, Gemm128W, Gemm96W };

// Configuration by M and K alone: the decode sizes, and the gated launch's
// GEMM split at 2048 rows.
Cfg pick_mk(int64_t M, int64_t K) {
    // up to 4 rows: the decode kernel with every stage in flight for K up to
    // 4096 (3 or 4 stages per wave)
    if (M <= 4 && K <= 4096) {
        const bool k3 = K <= 3072;
        if (M == 1) return k3 ? Cfg::G1 : Cfg::G1K;
        if (M == 2) return k3 ? Cfg::G2 : Cfg::G2K;
        return k3 ? Cfg::G4 : Cfg::G4K;
    }
    // up to K = 9216: 12 K-slices of up to 6 stages, all in flight (down
    // 9216 -> 3072: 7.0-7.1 us against 7.2-7.6 with the 2-stage refill of the
    // K-split kernel at one row, 7.4-7.5 against 8.2-8.8 at three and four)
    if (M <= 4 && K <= 12 * kGemvMaxStages * kTileK) return M == 1 ? Cfg::G1L : M == 2 ? Cfg::G2L : Cfg::G4L;
    if (M == 1) return Cfg::M1Long;
    if (M == 2) return Cfg::M2Long;
    if (M <= 4) return Cfg::M4Long;
    const bool long_k = K > 3072;
    if (M <= 16) return long_k ? Cfg::M16Long : Cfg::M16;
    if (M <= 32) return Cfg::M32;
    if (M <= 64) return Cfg::M64;
    return M < 2048 ? Cfg::Gemm64 : Cfg::Gemm128;
}

// Work tiles of a BM x BN GEMM tiling over all segments of a launch.
int64_t gemm_tiles(const LinearArgs &a, int bm, int bn) {
    const int rows_per_tile = bn / kTileRows;
    int64_t ntiles = 0;
    for (int i = 0; i < a.nseg; ++i) ntiles += (a.seg[i].RT + rows_per_tile - 1) / rows_per_tile;
    return ntiles * ((a.M + bm - 1) / bm);
}

// One row of x and at least 8 row tiles per CU (the LM head: 8192 tiles on
// 256 CUs): the stream kernel, when x fits in LDS and K splits evenly over
// its 8 waves.
bool stream_m1(const LinearArgs &a) {
    int64_t rts = 0;
    for (int i = 0; i < a.nseg; ++i) rts += a.seg[i].RT;
    return a.KT % 8 == 0 && skinny_x_bytes(a.M, a.K, 1) <= xlds_budget(1) && rts >= 8 * static_cast<int64_t>(device_cus());
}

// 17-64 rows: the GEMM's 128-column tiles number under half the CUs (every
// N of a few thousand rows: 24 tiles for N = 3072) leave most of the chip
// idle, and the decode kernel's K split over 8 waves runs 2-3x faster there
// (measured at M = 32 and 64); tall weights (gate/up, the LM head) keep the
// GEMM.  32 rows: two row tiles per wave once the row tiles outnumber the CUs.
Cfg pick_17_64(const LinearArgs &a, Cfg gemm) {
    int64_t rts = 0, tiles = 0;
    for (int i = 0; i < a.nseg; ++i) {
        rts += a.seg[i].RT;
        tiles += (a.seg[i].RT + 7) / 8;
    }
    const int64_t cus = device_cus();
    if (2 * tiles >= cus) return gemm;
    if (gemm == Cfg::M64) return Cfg::M64Split;
    return rts >= cus ? Cfg::M32Split2 : Cfg::M32Split;
}

// GEMM tile shape above 64 rows by wave quantization (see the table above).
Cfg gemm_shape(const LinearArgs &a) {
    const int64_t cus = device_cus();
    auto cost = [&](int bm, int bn, int64_t unit) { return (gemm_tiles(a, bm, bn) + cus - 1) / cus * unit; };
    const int64_t c64 = cost(64, 128, 30), c128 = cost(128, 128, 50), c128w = cost(128, 192, 85),
                  c96w = cost(96, 192, 79);
    if (c128 <= c64 && c128 <= c128w && c128 <= c96w) return Cfg::Gemm128;
    if (c64 <= c128w && c64 <= c96w) return Cfg::Gemm64;
    return c128w <= c96w ? Cfg::Gemm128W : Cfg::Gemm96W;
}

Cfg pick(const LinearArgs &a) {
    if (a.M <= 64) {
        const Cfg c = pick_mk(a.M, a.K);
        if (c == Cfg::M32 || c == Cfg::M64) return pick_17_64(a, c);
        return c == Cfg::G1 && stream_m1(a) ? Cfg::M1Stream : c;
    }
    return gemm_shape(a);
}

// Name of a skinny_kernel instantiation, with the x staging the launch picks.
const char *skinny_name(int64_t M, int64_t K, int mrows_max, const char *lds_name, const char *l2_name) {
    return skinny_x_bytes(M, K, mrows_max) <= xlds_budget(mrows_max) ? lds_name : l2_name;
}
}  // namespace

// Name of a gemv_kernel instantiation (static string): the stage count
// follows from K, so the names come from a table built once.
const char *gemv_name(int mrows, int wk, int ns, int wpe, bool glu, bool asym = false) {
    static const std::vector<std::string> table = [] {
        std::vector<std::string> t;
        for (int m : {1, 2, 4})
            for (int w : {4, 8, 12, 16})
                for (int n = 1; n <= kGemvMaxStages; ++n)
                    for (int e : {0, 6})
                        for (int gl : {0, 1})
                            for (int as : {0, 1})
                                t.push_back("gemv_kernel<" + std::to_string(m) + ", " + std::to_string(w) + ", " +
                                            std::to_string(n) + ", " + std::to_string(e) + ", " +
                                            (gl ? "true" : "false") + (as ? ", true>" : ">"));
        return t;
    }();
    const int mi = mrows == 1 ? 0 : mrows == 2 ? 1 : 2, wi = wk == 4 ? 0 : wk == 8 ? 1 : wk == 12 ? 2 : 3;
    if (ns < 1 || ns > kGemvMaxStages) return "";
    return table[(((((mi * 4 + wi) * kGemvMaxStages + ns - 1) * 2 + (wpe ? 1 : 0)) * 2 + (glu ? 1 : 0)) * 2 +
                  (asym ? 1 : 0))].c_str();
}

// The decode configurations: rows, K-slices and waves-per-EU hint by M and K.
struct GemvCfg {
    int mrows, wk, wpe;
};
GemvCfg gemv_cfg(Cfg c) {
    switch (c) {
        case Cfg::G1: return {1, 8, 6};
        case Cfg::G1K: return {1, 16, 0};
        case Cfg::G2: return {2, 8, 0};
        case Cfg::G2K: return {2, 8, 0};
        case Cfg::G4: return {4, 8, 0};
        case Cfg::G1L: return {1, 12, 0};
        case Cfg::G2L: return {2, 12, 0};
        case Cfg::G4L: return {4, 12, 0};
        default: return {4, 16, 0};   // G4K
    }
}
bool is_gemv(Cfg c) {
    return c == Cfg::G1 || c == Cfg::G1K || c == Cfg::G2 || c == Cfg::G2K || c == Cfg::G4 || c == Cfg::G4K ||
           c == Cfg::G1L || c == Cfg::G2L || c == Cfg::G4L;
}

const char *linear_config_name(const LinearArgs &a) {
    const int64_t M = a.M, K = a.K;
    const Cfg c = pick(a);
    if (is_gemv(c)) {
        const GemvCfg g = gemv_cfg(c);
        return gemv_name(g.mrows, g.wk, gemv_stages(a, g.wk), g.wpe, false);
    }
    switch (c) {
        case Cfg::M1Stream: return "skinny_stream_kernel<1, 8, 3, 6>";
        case Cfg::M1Long: return skinny_name(M, K, 1, "skinny_kernel<1, 1, 16, 2, true, 0, false>", "skinny_kernel<1, 1, 16, 2, false, 0, false>");
        case Cfg::M2Long: return skinny_name(M, K, 2, "skinny_kernel<2, 1, 16, 2, true, 0, false>", "skinny_kernel<2, 1, 16, 2, false, 0, false>");
        case Cfg::M4Long: return skinny_name(M, K, 4, "skinny_kernel<4, 1, 16, 2, true, 0, false>", "skinny_kernel<4, 1, 16, 2, false, 0, false>");
        case Cfg::M16: return skinny_name(M, K, 16, "skinny_kernel<16, 1, 4, 2, true, 0, false>", "skinny_kernel<16, 1, 4, 2, false, 0, false>");
        case Cfg::M16Long: return skinny_name(M, K, 16, "skinny_kernel<16, 1, 16, 2, true, 0, false>", "skinny_kernel<16, 1, 16, 2, false, 0, false>");
        case Cfg::M32: return "gemm_kernel<2, 1, 1, 8, 0, 2>";
        case Cfg::M32Split: return skinny_name(M, K, 32, "skinny_kernel<32, 1, 8, 2, true, 0, false>", "skinny_kernel<32, 1, 8, 2, false, 0, false>");
        case Cfg::M32Split2: return skinny_name(M, K, 32, "skinny_kernel<32, 2, 8, 2, true, 0, false>", "skinny_kernel<32, 2, 8, 2, false, 0, false>");
        case Cfg::M64: return "gemm_kernel<4, 1, 1, 8, 0, 3>";
        case Cfg::M64Split: return skinny_name(M, K, 64, "skinny_kernel<64, 1, 8, 2, true, 0, false>", "skinny_kernel<64, 1, 8, 2, false, 0, false>");
        case Cfg::Gemm64: return "gemm3_kernel<4, 1, 1, 8, 4, 8, false>";
        case Cfg::Gemm128W: return "gemm3_kernel<8, 1, 1, 12, 0, 4, false>";
        case Cfg::Gemm96W: return "gemm3_kernel<6, 1, 1, 12, 0, 4, false>";
        default: return "gemm3_kernel<8, 1, 1, 8, 4, 4, false>";
    }
}

hipError_t launch_linear(LinearArgs a, hipStream_t s) {
    switch (pick(a)) {
        case Cfg::G1: return run_gemv<1, 8, 6, false, 3>(a, s);
        case Cfg::G1K: return run_gemv<1, 16, 0, false, 2>(a, s);
        case Cfg::G2: return run_gemv<2, 8, 0, false, 3>(a, s);
        case Cfg::G2K: return run_gemv<2, 8, 0, false, 4>(a, s);
        case Cfg::G4: return run_gemv<4, 8, 0, false, 3>(a, s);
        case Cfg::G4K: return run_gemv<4, 16, 0, false, 2>(a, s);
        case Cfg::G1L: return run_gemv<1, 12, 0, false, 6>(a, s);
        case Cfg::G2L: return run_gemv<2, 12, 0, false, 6>(a, s);
        case Cfg::G4L: return run_gemv<4, 12, 0, false, 6>(a, s);
        case Cfg::M1Long: return run_skinny<1, 1, 16, 2, 0>(a, s);
        case Cfg::M2Long: return run_skinny<2, 1, 16, 2, 0>(a, s);
        case Cfg::M4Long: return run_skinny<4, 1, 16, 2, 0>(a, s);
        case Cfg::M1Stream: return run_skinny_stream<1, 8, 3, 6>(a, s);
        case Cfg::M16: return run_skinny<16, 1, 4, 2, 0>(a, s);
        case Cfg::M16Long: return run_skinny<16, 1, 16, 2, 0>(a, s);
        case Cfg::M32: return run_gemm<2, 1, 1, 8, 0, 2>(a, s);
        case Cfg::M32Split: return run_skinny<32, 1, 8, 2, 0>(a, s);
        case Cfg::M32Split2: return run_skinny<32, 2, 8, 2, 0>(a, s);
        case Cfg::M64: return run_gemm<4, 1, 1, 8, 0, 3>(a, s);
        case Cfg::M64Split: return run_skinny<64, 1, 8, 2, 0>(a, s);
        case Cfg::Gemm64: return run_gemm3<4, 1, 1, 8, 4, 8>(a, s);
        case Cfg::Gemm128W: return run_gemm3<8, 1, 1, 12, 0, 4>(a, s);
        case Cfg::Gemm96W: return run_gemm3<6, 1, 1, 12, 0, 4>(a, s);
        default: return run_gemm3<8, 1, 1, 8, 4, 4>(a, s);
    }
}

// The gated (SwiGLU) launch: the plain configurations with the gate and up
// rows of a tile on separate waves (skinny: 2 WK waves, at most 8 K-slices
// so a workgroup stays within 1024 threads; gemm and gemm3: WN / 2 gate and
// WN / 2 up waves), so every wave runs the plain arithmetic.
// The gated launch's decode configurations are the plain ones (its
// workgroups cover 8 gate and 8 up rows: the plain wave count per workgroup).
GemvCfg gemv_glu_cfg(Cfg c) { return gemv_cfg(c); }

const char *linear_glu_config_name(int64_t M, int64_t K) {
    const Cfg c = pick_mk(M, K);
    if (c == Cfg::G4L)
        return skinny_name(M, K, 4, "skinny_kernel<4, 1, 8, 3, true, 0, true>", "skinny_kernel<4, 1, 8, 3, false, 0, true>");
    if (is_gemv(c)) {
        const GemvCfg g = gemv_glu_cfg(c);
        return gemv_name(g.mrows, g.wk, static_cast<int>((round_up(K, kTileK) / kTileK + g.wk - 1) / g.wk), g.wpe, true);
    }
    switch (c) {
        case Cfg::M1Long: return skinny_name(M, K, 1, "skinny_kernel<1, 1, 8, 3, true, 0, true>", "skinny_kernel<1, 1, 8, 3, false, 0, true>");
        case Cfg::M2Long: return skinny_name(M, K, 2, "skinny_kernel<2, 1, 8, 3, true, 0, true>", "skinny_kernel<2, 1, 8, 3, false, 0, true>");
        case Cfg::M4Long: return skinny_name(M, K, 4, "skinny_kernel<4, 1, 8, 3, true, 0, true>", "skinny_kernel<4, 1, 8, 3, false, 0, true>");
        case Cfg::M16: return skinny_name(M, K, 16, "skinny_kernel<16, 1, 4, 2, true, 0, true>", "skinny_kernel<16, 1, 4, 2, false, 0, true>");
        case Cfg::M16Long: return skinny_name(M, K, 16, "skinny_kernel<16, 1, 8, 3, true, 0, true>", "skinny_kernel<16, 1, 8, 3, false, 0, true>");
        case Cfg::M32: return "gemm_kernel<2, 1, 1, 8, 0, 2, true>";
        case Cfg::M64: return "gemm_kernel<4, 1, 1, 8, 0, 3, true>";
        case Cfg::Gemm64: return "gemm3_kernel<4, 1, 1, 8, 4, 8, true>";
        default: return "gemm3_kernel<8, 1, 1, 8, 4, 4, true>";
    }
}

hipError_t launch_linear_glu(LinearArgs a, hipStream_t s) {
    switch (pick_mk(a.M, a.K)) {
        case Cfg::G1: return run_gemv<1, 8, 6, true, 3>(a, s);
        case Cfg::G1K: return run_gemv<1, 16, 0, true, 2>(a, s);
        case Cfg::G2: return run_gemv<2, 8, 0, true, 3>(a, s);
        case Cfg::G2K: return run_gemv<2, 8, 0, true, 4>(a, s);
        case Cfg::G4: return run_gemv<4, 8, 0, true, 3>(a, s);
        case Cfg::G4K: return run_gemv<4, 16, 0, true, 2>(a, s);
        case Cfg::G1L: return run_gemv<1, 12, 0, true, 6>(a, s);
        case Cfg::G2L: return run_gemv<2, 12, 0, true, 6>(a, s);
        case Cfg::G4L: return run_skinny<4, 1, 8, 3, 0, true>(a, s);   // 13.6 against 12.8 us as a 12-slice gemv
        case Cfg::M1Long: return run_skinny<1, 1, 8, 3, 0, true>(a, s);
        case Cfg::M2Long: return run_skinny<2, 1, 8, 3, 0, true>(a, s);
        case Cfg::M4Long: return run_skinny<4, 1, 8, 3, 0, true>(a, s);
        case Cfg::M16: return run_skinny<16, 1, 4, 2, 0, true>(a, s);
        case Cfg::M16Long: return run_skinny<16, 1, 8, 3, 0, true>(a, s);
        case Cfg::M32: return run_gemm<2, 1, 1, 8, 0, 2, true>(a, s);
        case Cfg::M64: return run_gemm<4, 1, 1, 8, 0, 3, true>(a, s);
        case Cfg::Gemm64: return run_gemm3<4, 1, 1, 8, 4, 8, true>(a, s);
        default: return run_gemm3<8, 1, 1, 8, 4, 4, true>(a, s);
    }
}

// The asymmetric layout (one segment): up to 4 rows and K up to 12288 the
// decode kernel (8 K-slices up to K = 3072 at one row and 4096 at two; 12 of
// up to 6 stages from there to K = 9216 at one and two rows, which took the
// 9216 -> 3072 launch from 6.9-7.0 to 6.5 us at one row; 16 otherwise),
// otherwise the GEMM (32- or 64-row tiles up to 64 rows, the tile
// model above that).
namespace {
enum class Q41 { G1, G1K, G2, G2K, G4, G1L, G2L, Gemm32, Gemm64r, Gemm64, Gemm128, Gemm128W };
Q41 pick_q41(const LinearArgs &a) {
    if (a.M <= 4 && a.KT <= 96) {
        if (a.M == 1) return a.KT <= 24 ? Q41::G1 : a.KT <= 32 ? Q41::G1K : a.KT <= 72 ? Q41::G1L : Q41::G1K;
        if (a.M == 2) return a.KT <= 32 ? Q41::G2 : a.KT <= 72 ? Q41::G2L : Q41::G2K;
        return Q41::G4;
    }
    if (a.M <= 32) return Q41::Gemm32;
    if (a.M <= 64) return Q41::Gemm64r;
    switch (gemm_shape(a)) {
        case Cfg::Gemm64: return Q41::Gemm64;
        case Cfg::Gemm128W:
        case Cfg::Gemm96W: return Q41::Gemm128W;
        default: return Q41::Gemm128;
    }
}
}  // namespace

const char *linear_q41_config_name(const LinearArgs &a) {
    const int ns16 = (a.KT + 15) / 16;
    switch (pick_q41(a)) {
        case Q41::G1: return gemv_name(1, 8, (a.KT + 7) / 8, 6, false, true);
        case Q41::G1K: return gemv_name(1, 16, ns16, 0, false, true);
        case Q41::G2: return gemv_name(2, 8, (a.KT + 7) / 8, 0, false, true);
        case Q41::G2K: return gemv_name(2, 16, ns16, 0, false, true);
        case Q41::G4: return gemv_name(4, 16, ns16, 0, false, true);
        case Q41::G1L: return gemv_name(1, 12, (a.KT + 11) / 12, 0, false, true);
        case Q41::G2L: return gemv_name(2, 12, (a.KT + 11) / 12, 0, false, true);
        case Q41::Gemm32: return "gemm3_kernel<2, 1, 1, 8, 0, 8, false, true>";
        case Q41::Gemm64r: return "gemm3_kernel<4, 1, 1, 8, 0, 8, false, true>";
        case Q41::Gemm64: return "gemm3_kernel<4, 1, 1, 8, 0, 8, false, true>";
        case Q41::Gemm128W: return "gemm3_kernel<8, 1, 1, 12, 0, 8, false, true>";
        default: return "gemm3_kernel<8, 1, 1, 8, 0, 8, false, true>";
    }
}

hipError_t launch_linear_q41(LinearArgs a, hipStream_t s) {
    switch (pick_q41(a)) {
        case Q41::G1: return run_gemv<1, 8, 6, false, 3, true>(a, s);
        case Q41::G1K: return run_gemv<1, 16, 0, false, 6, true>(a, s);
        case Q41::G2: return run_gemv<2, 8, 0, false, 4, true>(a, s);
        case Q41::G2K: return run_gemv<2, 16, 0, false, 6, true>(a, s);
        case Q41::G4: return run_gemv<4, 16, 0, false, 6, true>(a, s);
        case Q41::G1L: return run_gemv<1, 12, 0, false, 6, true>(a, s);
        case Q41::G2L: return run_gemv<2, 12, 0, false, 6, true>(a, s);
        case Q41::Gemm32: return run_gemm3<2, 1, 1, 8, 0, 8, false, true>(a, s);
        case Q41::Gemm64r: return run_gemm3<4, 1, 1, 8, 0, 8, false, true>(a, s);
        case Q41::Gemm64: return run_gemm3<4, 1, 1, 8, 0, 8, false, true>(a, s);
        case Q41::Gemm128W: return run_gemm3<8, 1, 1, 12, 0, 8, false, true>(a, s);
        default: return run_gemm3<8, 1, 1, 8, 0, 8, false, true>(a, s);
    }
}

// ------------------------------------------------------------- measurement
// The prefill GEMM's arithmetic and nothing else: per wave the 128-row
// tiles' 8 x 1 register tile (8 m-tiles sharing one B fragment per block),
// operands in registers, no loads, stores or barriers, 4 waves per SIMD as in
// the GEMM.  MODE 0: the MFMAs alone, accumulating in the matrix pipe;
// MODE 1: each MFMA's result rescaled into acc by the block's scale in fp32
// (four FMAs, issued after the next MFMA, as in gemm3_kernel); MODE 2: MODE 1
// plus the decode of each block's B fragment from its codes; MODE 3: MODE 0
// with four fp32 FMAs per MFMA beside it on registers no MFMA reads or
// writes (the same VALU work as MODE 1's rescale, with no dependence on the
// matrix pipe).  The operands pass through an empty asm statement each
// iteration, so no MFMA, FMA or decode is loop-invariant.  What it shows: the
// rate the exact arithmetic allows on this chip, apart from memory, and
// whether its VALU work could hide under the MFMAs.
namespace {
constexpr int kCeilThreads = 256;
constexpr int kCeilPerCU = 4;   // 256-thread workgroups per CU: 4 waves per SIMD

template <int MODE>
__global__ __launch_bounds__(kCeilThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void ceiling_kernel(float *sink, int iters) {
    const uint32_t t = threadIdx.x + blockIdx.x * kCeilThreads;
    bf16x8 A[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int e = 0; e < 8; ++e) A[mt][e] = static_cast<__bf16>(static_cast<float>(static_cast<int>((t + 3 * mt + e) & 7) - 3));
    bf16x8 Bfix[kTileBlocks];   // modes 0 and 1: a distinct fragment per block
#pragma unroll
    for (int i = 0; i < kTileBlocks; ++i) Bfix[i] = A[(t + i) & 7];
    u32x4 nib = (u32x4){t * 2654435761u, t * 40503u + 1u, t ^ 0x5bd1e995u, t * 7u + 3u};
    u32x2 sc = (u32x2){0x3C003800u, 0x34003000u};   // fp16 1, 0.5, 0.25, 0.125
    floatx4 acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = (floatx4){0.f, 0.f, 0.f, 0.f};
    float side[4] = {1.f, 2.f, 3.f, 4.f};   // mode 3's FMA chains
    for (int it = 0; it < iters; ++it) {
        asm volatile("" : "+v"(nib), "+v"(sc), "+v"(Bfix[0]), "+v"(Bfix[1]), "+v"(Bfix[2]), "+v"(Bfix[3]));
#pragma unroll
        for (int i = 0; i < kTileBlocks; ++i) {
            const bf16x8 B = MODE == 2 ? decode_piece(piece_of(nib, i)) : Bfix[i];
            if constexpr (MODE == 0) {
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt], B, acc[mt], 0, 0, 0);
            } else if constexpr (MODE == 3) {
                const float d = scale_of(sc, i);
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt], B, acc[mt], 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) side[r] = fmaf(d, side[r], static_cast<float>(r));
                }
            } else {
                const float d = scale_of(sc, i);
                floatx4 D[8];
                D[0] = mfma_block(A[0], B);
#pragma unroll
                for (int mt = 1; mt < 8; ++mt) {
                    D[mt] = mfma_block(A[mt], B);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[mt - 1][r] = fmaf(d, D[mt - 1][r], acc[mt - 1][r]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[7][r] = fmaf(d, D[7][r], acc[7][r]);
            }
            if (i % 2 == 1) __builtin_amdgcn_sched_barrier(0);
        }
    }
    float f = side[0] + side[1] + side[2] + side[3];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) f += acc[mt][0] + acc[mt][1] + acc[mt][2] + acc[mt][3];
    sink[t] = f;
}
}  // namespace

int64_t reference_mfma_threads() { return static_cast<int64_t>(device_cus()) * kCeilPerCU * kCeilThreads; }

hipError_t launch_reference_mfma(int mode, int iters, float *sink, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(device_cus() * kCeilPerCU)), block(kCeilThreads);
    auto kernel = mode == 0   ? ceiling_kernel<0>
                  : mode == 1 ? ceiling_kernel<1>
                  : mode == 2 ? ceiling_kernel<2>
                              : ceiling_kernel<3>;
    hipEvent_t start = nullptr, stop = nullptr;
    if (take_launch_events(start, stop))
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, start, stop, 0, sink, iters);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, s, sink, iters);
    return hipGetLastError();
}

}  // namespace q4
