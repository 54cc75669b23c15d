// Device kernels of libswiglu: the fused SwiGLU GEMM, its split-K form, the
// weight pack, and the unfused baseline's GEMM and element-wise SwiGLU.
//
// Citations name the pages about "Tile-Level Activation Overlap for Efficient
// LLM Inference": [Abstract] is the paper's abstract (paper-with-me page);
// [Summary: X] is section X of the gist.science technical summary.
//
// What is computed ([Summary: Problem Statement]):
//     Y = SiLU(A x W1) (.) (A x W2)
// Gate = A x W1 and Up = A x W2 are accumulated in fp32 registers, side by
// side, for the SAME output positions of the same lanes, so SiLU(Gate) * Up is
// a lane-local epilogue and neither intermediate is ever stored ([Abstract]:
// tile-level fusion; [Summary: Key Contributions]: the four Gate/Up memory
// operations disappear).
//
// gfx950 mapping (CDNA4, 64-wide wavefronts):
//  * Matrix core op: v_mfma_f32_32x32x16_bf16.  The weight fragment is the
//    first operand and the activation fragment the second, so the 32x32 fp32
//    result holds rows = output columns n and columns = tokens m; each lane
//    then owns four consecutive n of one token, which makes the Y store a
//    single 8-byte write.
//  * One LDS-staged A tile [BM x 64] is shared by the Gate and the Up weight
//    tiles of the same K step (the Kernel-2 idea of one GEMM over a fused
//    weight, [Summary: Methodology]); two LDS stages are double-buffered with
//    a register prefetch of the next K step issued before the MFMAs of the
//    current one.
//  * LDS rows are 128 bytes (64 bf16 of K); 16-byte chunks are XOR-swizzled
//    by swz(row) so the 16-byte-per-lane fragment reads of 8 or 16
//    consecutive rows hit distinct banks.
//  * Workgroup ids are remapped so each XCD (own L2) gets a contiguous run of
//    output tiles, grouped along M so neighbours share weight panels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace swk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;             // K depth of one LDS stage (one 128-byte row)
constexpr int PACK_BN = 128;       // output columns per packed weight tile
constexpr int PACK_BK = 64;        // K depth per packed block
constexpr int PACK_ROWS = 2 * PACK_BN;   // Gate rows then Up rows
constexpr int NUM_XCD = 8;
constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// element offset of 16-byte chunk c (0..7) of row r in an LDS tile [rows][64]
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ swz(r)) << 3); }

// Packed weights, within one 64-deep block of a 128-column tile: packed row
// p (0..127 Gate columns, 128..255 Up columns) and depth k (0..63).  Each
// 16-row group x 32-deep half is one 1 KiB fragment in MFMA lane order:
// lane (k % 32) / 8 * 16 + p % 16 holds the 8 consecutive k of its 16 bytes,
// so a wave reads a whole fragment with one fully coalesced load.
__host__ __device__ __forceinline__ int packed_off(int p, int k) {
    return ((((p >> 4) * 2 + (k >> 5)) * 64 + ((k & 31) >> 3) * 16 + (p & 15)) << 3) + (k & 7);
}

// LDS stage of packed weights in the direct-load kernel: groups of 8 rows,
// chunk-major inside a group (16-byte unit (row & 7) of chunk slot s), slots
// XOR-ed with the group's parity.  A direct load of one group then has lanes
// 8s..8s+7 reading 128 contiguous bytes of one packed fragment line, and the
// 16 rows of a fragment read fall in two groups 1 KiB +- 128 B apart (disjoint
// banks).  Element offset of chunk c of row r:
__device__ __forceinline__ int wlds_off(int r, int c) {
    return (((r >> 3) << 6) + ((c ^ ((r >> 3) & 1)) << 3) + (r & 7)) << 3;
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
// Non-temporal 16-byte load, for weight bytes that exactly one wave of the
// grid reads (the decode kernels' weight stream): the lines stream through
// L2 instead of displacing the activations that every workgroup re-reads
// (measured: 72B-width M=32 decode 160 -> 145 us, 7B-width M=1 45.8 -> 42.5 us)
__device__ __forceinline__ u32x4 ld16_stream(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// SiLU(g) = g * sigmoid(g) = g / (1 + 2^(-g log2 e)); v_exp_f32 and v_rcp_f32.
// g -> -inf: the exponential overflows to +inf, rcp gives 0, result -0.
// g >= 17: the exponential is below 2^-24, 1 + e rounds to 1, result g.
__device__ __forceinline__ float silu_f(float g) {
    const float e = __builtin_amdgcn_exp2f(-g * LOG2E);
    return g * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ unsigned bf16_bits(float x) {
    __bf16 h = (__bf16)x;   // v_cvt_pk_bf16_f32: round to nearest even
    return (unsigned)__builtin_bit_cast(unsigned short, h);
}

// Two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32;
// `lo` lands in the low half.
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 h2 __attribute__((ext_vector_type(2)));
    const h2 h = __builtin_convertvector((f2){lo, hi}, h2);
    return __builtin_bit_cast(unsigned, h);
}

// Map the hardware workgroup id to a logical id such that XCD x (which gets
// ids x, x+8, x+16, ...) owns one contiguous range of logical ids.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int q = total / NUM_XCD, r = total % NUM_XCD;
    const int x = bid % NUM_XCD, j = bid / NUM_XCD;
    return x * q + (x < r ? x : r) + j;
}

// 8x8 bf16 transpose: in[i] holds W[k+i][n..n+7]; out[j] gets W[k..k+7][n+j].
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int d = j >> 1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const unsigned lo = in[2 * q][d], hi = in[2 * q + 1][d];
            out[j][q] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u))
                                : ((lo & 0xFFFFu) | (hi << 16));
        }
    }
}

struct FusedArgs {
    const uint16_t* A;    // [M,K]
    const uint16_t* W1;   // [K,N] row-major, or the packed weights
    const uint16_t* W2;   // [K,N] row-major (unused when packed)
    uint16_t* Y;          // [M,N]
    float* part;          // split-K partials (fp32, [split][M][2N])
    int M, K, N;
    int tiles_m, tiles_n;
    int n_tile0;          // first output-column tile this launch covers (in tiles of BN)
    int splits;           // number of K splits (1 = none)
    int kb_per_split;     // K blocks (of 64) per split
    int KB;               // ceil(K / 64)
    int panels;           // > 0: panel schedule over this many 32-column weight panels
                          // (streaming kernel, one row tile): work item w takes
                          // panels [w*panels/total, (w+1)*panels/total), one per wave
    float sg, su;         // FP8 operands: scale products applied to the Gate and Up sums
};

// ---------------------------------------------------------------------------
// Split-K partials.  Layout [split][M][2N] fp32: the Gate sum of (m, n) at
// column n, the Up sum at column N + n.  Each lane owns four consecutive
// columns of one token per 32x32 accumulator block, so it writes 16 bytes of
// Gate and 16 bytes of Up per block.  Rows >= M and columns >= N are skipped.
// ---------------------------------------------------------------------------
template <int TM, int TN>
__device__ __forceinline__ void store_partials(const f32x16 (&acc)[2][TM][TN], float* part, int split,
                                               int M, int N, int row0, int col0, int lane) {
    float* base = part + (size_t)split * M * (2 * (size_t)N);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int m = row0 + i * 32 + (lane & 31);
        if (m >= M) continue;
        float* prow = base + (size_t)m * (2 * (size_t)N);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = col0 + j * 32 + 8 * q + 4 * (lane >> 5);
                if (n >= N) continue;
                f32x4 g, u;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    g[e] = acc[0][i][j][4 * q + e];
                    u[e] = acc[1][i][j][4 * q + e];
                }
                *reinterpret_cast<f32x4*>(prow + n) = g;
                *reinterpret_cast<f32x4*>(prow + N + n) = u;
            }
    }
}

// Y[m, n..n+3] = bf16(SiLU(sum_s G_s) * sum_s U_s), splits added in order
// 0..S-1 (so the result does not depend on which workgroup finished first).
// One thread per 4 outputs, grid-stride.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            uint16_t* __restrict__ Y, int M, int N,
                                                            int S) {
    const long long groups = (long long)M * (N / 4);
    const size_t split_stride = (size_t)M * 2 * (size_t)N;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < groups;
         t += (long long)gridDim.x * blockDim.x) {
        const int m = (int)(t / (N / 4));
        const int n = (int)(t % (N / 4)) * 4;
        const float* src = part + (size_t)m * 2 * (size_t)N + n;
        f32x4 g = *reinterpret_cast<const f32x4*>(src);
        f32x4 u = *reinterpret_cast<const f32x4*>(src + N);
        for (int s2 = 1; s2 < S; ++s2) {
            g += *reinterpret_cast<const f32x4*>(src + s2 * split_stride);
            u += *reinterpret_cast<const f32x4*>(src + s2 * split_stride + N);
        }
        u32x2 out;
        out[0] = pack2(silu_f(g[0]) * u[0], silu_f(g[1]) * u[1]);
        out[1] = pack2(silu_f(g[2]) * u[2], silu_f(g[3]) * u[3]);
        *reinterpret_cast<u32x2*>(Y + (size_t)m * N + n) = out;
    }
}

// The single-weight GEMM's split-K reduction: partials [split][M][2*NT] over
// the NT tiled columns of the pack (the "Gate" sum of tiled column n is output
// column (n / 128) * 256 + n % 128, the "Up" sum that column + 128), added in
// split order 0..S-1 and stored as bf16; output columns >= N are skipped.
__global__ __launch_bounds__(256) void splitk_gemm_reduce_kernel(const float* __restrict__ part,
                                                                 uint16_t* __restrict__ C, int M, int N, int NT,
                                                                 int S) {
    const long long groups = (long long)M * (NT / 4);
    const size_t split_stride = (size_t)M * 2 * (size_t)NT;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < groups;
         t += (long long)gridDim.x * blockDim.x) {
        const int m = (int)(t / (NT / 4));
        const int n = (int)(t % (NT / 4)) * 4;
        const float* src = part + (size_t)m * 2 * (size_t)NT + n;
        f32x4 g = *reinterpret_cast<const f32x4*>(src);
        f32x4 u = *reinterpret_cast<const f32x4*>(src + NT);
        for (int s2 = 1; s2 < S; ++s2) {
            g += *reinterpret_cast<const f32x4*>(src + s2 * split_stride);
            u += *reinterpret_cast<const f32x4*>(src + s2 * split_stride + NT);
        }
        const int col = (n / PACK_BN) * PACK_ROWS + n % PACK_BN;
        if (col < N) {
            u32x2 out;
            out[0] = pack2(g[0], g[1]);
            out[1] = pack2(g[2], g[3]);
            *reinterpret_cast<u32x2*>(C + (size_t)m * N + col) = out;
        }
        if (col + PACK_BN < N) {
            u32x2 out;
            out[0] = pack2(u[0], u[1]);
            out[1] = pack2(u[2], u[3]);
            *reinterpret_cast<u32x2*>(C + (size_t)m * N + col + PACK_BN) = out;
        }
    }
}

// ---------------------------------------------------------------------------
// The fused (DUAL) / single-GEMM (!DUAL) tile kernel.
//   BM x BN output tile per workgroup, WM x WN waves, each wave owning a
//   (BM/WM) x (BN/WN) sub-tile as (BM/WM/32) x (BN/WN/32) MFMA 32x32 blocks,
//   for Gate and for Up when DUAL.
//   PACKED: weights come from the packed layout (K-contiguous rows), else from
//   row-major [K,N] W1/W2 and are transposed in registers on the way to LDS.
//   SPLIT: the workgroup covers kb_per_split K blocks and writes its fp32
//   partial Gate/Up sums to `part`; splitk_reduce_kernel, launched after it,
//   adds the partials in split order 0..S-1 (before SiLU) and runs the
//   epilogue.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, bool DUAL, bool PACKED, bool SPLIT>
__global__ __launch_bounds__(64 * WM * WN) void fused_tile_kernel(FusedArgs p) {
    constexpr int NT = 64 * WM * WN;
    constexpr int NG = DUAL ? 2 : 1;          // accumulator groups (Gate, Up)
    constexpr int NB = NG * BN;               // weight rows (n) per stage
    constexpr int TM = BM / WM / 32;
    constexpr int TN = BN / WN / 32;
    constexpr int A_LD = BM * 8 / NT;         // 16-byte A chunks per thread per stage
    constexpr int B_LD = NB * 8 / NT;         // 16-byte packed-weight chunks per thread
    constexpr int B_BLK = NB / NT;            // 8x8 row-major weight blocks per thread
    constexpr int GROUP_M = 8;
    static_assert(TM >= 1 && TN >= 1, "tile too small for the wave grid");
    static_assert(BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "tile/wave mismatch");
    static_assert(A_LD >= 1 && (BM * 8) % NT == 0, "A tile not evenly split");
    static_assert(!PACKED || ((NB * 8) % NT == 0 && B_LD >= 1), "B tile not evenly split");
    static_assert(PACKED || (NB % NT == 0 && B_BLK >= 1), "B tile not evenly split");
    static_assert(!PACKED || DUAL, "packed weights hold a Gate/Up pair");
    static_assert(!PACKED || (PACK_BN % BN == 0), "tile must divide the packed tile");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + NB) * BK];
    uint16_t* const sA0 = smem;
    uint16_t* const sB0 = smem + BM * BK;
    constexpr int STAGE = (BM + NB) * BK;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int wrow0 = wm * (BM / WM);
    const int wcol0 = wn * (BN / WN);

    // ---- which tile / split -----------------------------------------------
    const int S = SPLIT ? p.splits : 1;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = logical / S;
    const int split = logical - tile * S;
    int tm, tn;
    {
        const int per_group = GROUP_M * p.tiles_n;
        const int group = tile / per_group;
        const int first_m = group * GROUP_M;
        const int gsize = min(p.tiles_m - first_m, GROUP_M);
        const int in_group = tile - group * per_group;
        tm = first_m + in_group % gsize;
        tn = in_group / gsize;
    }
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int M = p.M, K = p.K, N = p.N;
    const int kb_begin = SPLIT ? split * p.kb_per_split : 0;
    const int kb_end = SPLIT ? min(p.KB, kb_begin + p.kb_per_split) : p.KB;

    // ---- global -> register loaders ------------------------------------------
    u32x4 ra[A_LD];
    u32x4 rb[PACKED ? B_LD : 8 * B_BLK];

    auto load_stage = [&](int kb) {
        const int k0 = kb * BK;
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int q = tid + i * NT;
            const int row = q >> 3, c = q & 7;
            const int grow = min(m0 + row, M - 1);
            const int gk = k0 + c * 8;
            ra[i] = gk < K ? ld16(p.A + (size_t)grow * K + gk) : u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (PACKED) {
            const int jp = n0 / PACK_BN, ro = n0 % PACK_BN;
            const uint16_t* blk = p.W1 + ((size_t)jp * p.KB + kb) * (PACK_ROWS * PACK_BK);
#pragma unroll
            for (int i = 0; i < B_LD; ++i) {
                const int q = tid + i * NT;
                const int row = q >> 3, c = q & 7;
                const int prow = row < BN ? ro + row : PACK_BN + ro + (row - BN);
                rb[i] = ld16(blk + packed_off(prow, c * 8));
            }
        } else {
            constexpr int NGRP = NB / 8;
#pragma unroll
            for (int b = 0; b < B_BLK; ++b) {
                const int blkid = tid + b * NT;
                const int ng = blkid % NGRP, kc = blkid / NGRP;
                const int nl = ng * 8;
                const bool up = DUAL && nl >= BN;
                const uint16_t* W = up ? p.W2 : p.W1;
                const int ncol = min(n0 + (up ? nl - BN : nl), N - 8);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int gk = k0 + kc * 8 + i;
                    rb[b * 8 + i] = gk < K ? ld16(W + (size_t)gk * N + ncol) : u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    };

    auto store_stage = [&](int buf) {
        uint16_t* sA = sA0 + buf * STAGE;
        uint16_t* sB = sB0 + buf * STAGE;
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int q = tid + i * NT;
            *reinterpret_cast<u32x4*>(sA + lds_off(q >> 3, q & 7)) = ra[i];
        }
        if constexpr (PACKED) {
#pragma unroll
            for (int i = 0; i < B_LD; ++i) {
                const int q = tid + i * NT;
                *reinterpret_cast<u32x4*>(sB + lds_off(q >> 3, q & 7)) = rb[i];
            }
        } else {
            constexpr int NGRP = NB / 8;
#pragma unroll
            for (int b = 0; b < B_BLK; ++b) {
                const int blkid = tid + b * NT;
                const int ng = blkid % NGRP, kc = blkid / NGRP;
                u32x4 in[8], out[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) in[i] = rb[b * 8 + i];
                transpose8x8(in, out);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    *reinterpret_cast<u32x4*>(sB + lds_off(ng * 8 + j, kc)) = out[j];
            }
        }
    };

    // ---- accumulators -----------------------------------------------------------
    f32x16 acc[NG][TM][TN];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[g][i][j][r] = 0.0f;

    auto compute_stage = [&](int buf) {
        const uint16_t* sA = sA0 + buf * STAGE;
        const uint16_t* sB = sB0 + buf * STAGE;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            bf16x8 af[TM];
            bf16x8 bfr[NG][TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(sA + lds_off(wrow0 + i * 32 + (lane & 31), c));
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bfr[g][j] = *reinterpret_cast<const bf16x8*>(
                        sB + lds_off(g * BN + wcol0 + j * 32 + (lane & 31), c));
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[g][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[g][j], af[i],
                                                                               acc[g][i][j], 0, 0, 0);
        }
    };

    // ---- main loop: double-buffered LDS, register prefetch ------------------------
    if (kb_begin < kb_end) {
        load_stage(kb_begin);
        store_stage(0);
        __syncthreads();
        for (int kb = kb_begin; kb < kb_end; ++kb) {
            const int buf = (kb - kb_begin) & 1;
            const bool more = kb + 1 < kb_end;
            if (more) load_stage(kb + 1);
            compute_stage(buf);
            if (more) store_stage(buf ^ 1);
            __syncthreads();
        }
    }

    // ---- split-K: fp32 partials to the workspace, reduced by splitk_reduce_kernel ---
    if constexpr (SPLIT) {
        store_partials<TM, TN>(acc, p.part, split, M, N, m0 + wrow0, n0 + wcol0, lane);
        return;
    }

    // ---- epilogue: SiLU(Gate) * Up (or the plain GEMM value), bf16, store ---------
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int m = m0 + wrow0 + i * 32 + (lane & 31);
        if (m >= M) continue;
        uint16_t* yrow = p.Y + (size_t)m * N;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wcol0 + j * 32 + 8 * q + 4 * (lane >> 5);
                if (n >= N) continue;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float g = acc[0][i][j][4 * q + e];
                    if constexpr (DUAL) {
                        const float u = acc[NG - 1][i][j][4 * q + e];
                        v[e] = silu_f(g) * u;
                    } else {
                        v[e] = g;
                    }
                }
                u32x2 out;
                out[0] = pack2(v[0], v[1]);
                out[1] = pack2(v[2], v[3]);
                *reinterpret_cast<u32x2*>(yrow + n) = out;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill (large M) fused kernel on packed weights.
//   Same math and lane layout as fused_tile_kernel, but the global -> LDS copy
//   uses the direct LDS load (global_load_lds_dwordx4): each wave instruction
//   writes 64 x 16 bytes to consecutive LDS chunks, so the bank swizzle is
//   applied by choosing which global chunk each lane fetches.  No staging
//   registers and no LDS-write instructions: the next K step streams into the
//   other LDS stage while the MFMAs run on this one, and the only wait per
//   step is the final vmcnt + barrier.  Fragments are double-buffered in
//   registers across the four 16-deep K sub-steps.
//   A ragged last K block (K % 64 != 0) goes through registers so the
//   activation columns beyond K are zero-filled (the packed weights are
//   already zero there).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// 16-byte global store of an output tile, written through: device scope
// (sc1) with the non-temporal hint (nt), so the line goes out to memory now
// instead of sitting dirty in this XCD's L2 until the end-of-kernel
// writeback, and the output does not displace operand lines (measured: the
// 0.5B prefill launch ends about 6 us sooner).
// The compiler does not track the store: the streaming kernel leaves its Y
// stores in flight across the next tile's K loop, and a tracked store would
// make the compiler's own waits for later register loads conservative (it
// treats loads and stores as completing in any order relative to each
// other).  The kernel's explicit waits only ever rely on loads completing in
// order among themselves, which extra stores in the count cannot break.  The
// s_nop covers the store-data read of the VGPRs.
__device__ __forceinline__ void store16_untracked(uint16_t* gdst, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 1" ::"v"(gdst), "v"(v) : "memory");
}

__device__ __forceinline__ void dma16(const uint16_t* gsrc, uint16_t* lds_dst) {
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(gsrc),
                                     (lds_void_ptr)(lds_dst), 16, 0, 0);
}

// Weight sources of the direct-load kernel.
enum WeightSource : int {
    W_PACKED = 0,      // packed [W1|W2] tiles, rows K-contiguous; dual Gate/Up
    W_ROW_DUAL = 1,    // row-major W1 and W2 [K,N]; dual Gate/Up
    W_ROW_SINGLE = 2   // row-major W [K,N]; plain GEMM, bf16 output
};

// Row-major weight stage in LDS: 64 K-rows of NB columns (N-contiguous); the
// 16-byte chunks of row k are XOR-swizzled by (k & 3) << 2, which keeps the
// transposing fragment reads below free of bank conflicts (each 16-lane group
// reads 4 consecutive rows x 32 bytes, two groups read 16 columns apart).
template <int NB>
__device__ __forceinline__ int rm_off(int k, int col) {
    return k * NB + ((((col >> 3) ^ ((k & 3) << 2))) << 3) + (col & 7);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i & 3) of the 8-byte pieces addressed by lanes 4e + (i >> 2), e = 0..3.
__device__ __forceinline__ s16x4 ds_read_tr16(const uint16_t* lds) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_ptr)((__attribute__((address_space(3))) uint16_t*)(lds)));
}

template <int BM, int BN, int WM, int WN, bool SPLIT, int WSRC>
__global__ __launch_bounds__(64 * WM * WN) void fused_prefill_kernel(FusedArgs p) {
    constexpr bool PACKED_W = WSRC == W_PACKED;
    constexpr int NG = WSRC == W_ROW_SINGLE ? 1 : 2;   // accumulator groups (Gate, Up)
    constexpr int NW = WM * WN;
    constexpr int NB = NG * BN;               // weight columns (or packed rows) per stage
    constexpr int TM = BM / WM / 32;
    constexpr int TN = BN / WN / 32;
    constexpr int A_INS = BM / 8 / NW;        // 1 KiB direct loads per wave per stage (A)
    constexpr int B_INS = NB / 8 / NW;        // ... (weights)
    constexpr int STAGE = (BM + NB) * BK;     // elements per LDS stage
    constexpr int CPRB = NB / 8;              // row-major weights: 16-byte chunks per K-row
    constexpr int RPIB = 64 / CPRB;           // ... K-rows per wave-wide direct load
    constexpr int GROUP_M = 8;
    static_assert(TM >= 1 && TN >= 1, "tile too small for the wave grid");
    static_assert(A_INS >= 1 && B_INS >= 1 && (BM / 8) % NW == 0 && (NB / 8) % NW == 0, "load split");
    static_assert(!PACKED_W || PACK_BN % BN == 0, "tile must divide the packed tile");
    static_assert(PACKED_W || (CPRB >= 16 && CPRB <= 64), "row-major weight rows of 128..512 columns");
    static_assert(!SPLIT || NG == 2, "split-K is a fused schedule");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = wave % WM, wn = wave / WM;
    const int wrow0 = wm * (BM / WM);
    const int wcol0 = wn * (BN / WN);

    // logical id -> (output tile, K split); the splits of a tile are
    // consecutive, so they stay on one XCD
    const int S = SPLIT ? p.splits : 1;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = SPLIT ? logical / S : logical;
    const int split = SPLIT ? logical - tile * S : 0;
    int tm, tn;
    {
        const int per_group = GROUP_M * p.tiles_n;
        const int group = tile / per_group;
        const int first_m = group * GROUP_M;
        const int gsize = min(p.tiles_m - first_m, GROUP_M);
        const int in_group = tile - group * per_group;
        tm = first_m + in_group % gsize;
        tn = in_group / gsize;
    }
    const int m0 = tm * BM;
    const int n0 = (p.n_tile0 + tn) * BN;
    const int M = p.M, K = p.K, N = p.N, KB = p.KB;
    const bool ragged_k = (K % BK) != 0;
    // this workgroup's K blocks [kb_first, kb_last]; the host never makes an
    // empty split
    const int kb_first = SPLIT ? split * p.kb_per_split : 0;
    const int kb_last = SPLIT ? min(KB, kb_first + p.kb_per_split) - 1 : KB - 1;

    // per-lane source addresses, constant over K steps
    const int lrow = lane >> 3, lpc = lane & 7;
    const uint16_t* a_src[A_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        const int r = (wave * A_INS + i) * 8 + lrow;
        const int grow = min(m0 + r, M - 1);
        a_src[i] = p.A + (size_t)grow * K + 8 * (lpc ^ swz(r));
    }
    // packed: element offset within a 64-deep block; row-major: pointer to the
    // lane's 16 bytes in K-row r of the tile (advanced by k0 rows per stage)
    int b_off[PACKED_W ? B_INS : 1];
    const uint16_t* b_src[PACKED_W ? 1 : B_INS];
    const uint16_t* wtile = p.W1;
    if constexpr (PACKED_W) {
        const int jp = n0 / PACK_BN, ro = n0 % PACK_BN;
#pragma unroll
        for (int i = 0; i < B_INS; ++i) {
            const int g8 = wave * B_INS + i;                  // 8-row group = one direct load
            const int r = g8 * 8 + (lane & 7);
            const int c = (lane >> 3) ^ (g8 & 1);
            const int prow = r < BN ? ro + r : PACK_BN + ro + (r - BN);
            b_off[i] = packed_off(prow, 8 * c);
        }
        wtile = p.W1 + (size_t)jp * KB * (PACK_ROWS * PACK_BK);
    } else {
#pragma unroll
        for (int i = 0; i < B_INS; ++i) {
            const int r = (wave * B_INS + i) * RPIB + lane / CPRB;   // K-row within the stage
            const int c = 8 * ((lane % CPRB) ^ ((r & 3) << 2));      // logical column in the stage
            const bool up = NG == 2 && c >= BN;
            const int col = min(n0 + (up ? c - BN : c), N - 8);
            b_src[i] = (up ? p.W2 : p.W1) + (size_t)r * N + col;
        }
    }

    // activation columns beyond K (ragged last block) are zero-filled through
    // registers; every other stage is a direct load
    auto issue_a_regs = [&](int kb, int buf) {
        uint16_t* sA = smem + buf * STAGE;
        const int k0 = kb * BK;
#pragma unroll
        for (int i = 0; i < A_INS; ++i) {
            const int r = (wave * A_INS + i) * 8 + lrow;
            const int kc = k0 + 8 * (lpc ^ swz(r));
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (kc < K) v = ld16(a_src[i] + k0);
            *reinterpret_cast<u32x4*>(sA + ((wave * A_INS + i) * 64 + lane) * 8) = v;
        }
    };
    auto issue_a = [&](int kb, int buf) {
        uint16_t* sA = smem + buf * STAGE;
        const int k0 = kb * BK;
#pragma unroll
        for (int i = 0; i < A_INS; ++i) dma16(a_src[i] + k0, sA + (wave * A_INS + i) * 512);
    };
    auto issue_b = [&](int kb, int buf) {
        uint16_t* sB = smem + buf * STAGE + BM * BK;
        if constexpr (PACKED_W) {
            const uint16_t* blk = wtile + (size_t)kb * (PACK_ROWS * PACK_BK);
#pragma unroll
            for (int i = 0; i < B_INS; ++i) dma16(blk + b_off[i], sB + (wave * B_INS + i) * 512);
        } else {
            const size_t k0N = (size_t)kb * BK * N;
#pragma unroll
            for (int i = 0; i < B_INS; ++i) dma16(b_src[i] + k0N, sB + (wave * B_INS + i) * 512);
        }
    };
    // row-major weights, ragged last block: K-rows beyond K are zero-filled
    // through registers (packed weights are already zero there)
    auto issue_b_regs = [&](int kb, int buf) {
        if constexpr (!PACKED_W) {
            uint16_t* sB = smem + buf * STAGE + BM * BK;
            const size_t k0N = (size_t)kb * BK * N;
#pragma unroll
            for (int i = 0; i < B_INS; ++i) {
                const int r = (wave * B_INS + i) * RPIB + lane / CPRB;
                u32x4 v = u32x4{0u, 0u, 0u, 0u};
                if (kb * BK + r < K) v = ld16(b_src[i] + k0N);
                *reinterpret_cast<u32x4*>(sB + ((wave * B_INS + i) * 64 + lane) * 8) = v;
            }
        } else {
            issue_b(kb, buf);
        }
    };

    f32x16 acc[NG][TM][TN];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[g][i][j][r] = 0.0f;

    bf16x8 fa[2][TM], fb[2][NG][TN];
    auto read_frags = [&](int buf, int kk, int set) {
        const uint16_t* sA = smem + buf * STAGE;
        const uint16_t* sB = sA + BM * BK;
        const int c = 2 * kk + (lane >> 5);
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa[set][i] = *reinterpret_cast<const bf16x8*>(sA + lds_off(wrow0 + i * 32 + (lane & 31), c));
        if constexpr (PACKED_W) {
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    fb[set][g][j] = *reinterpret_cast<const bf16x8*>(
                        sB + wlds_off(g * BN + wcol0 + j * 32 + (lane & 31), c));
        } else {
            // two transposing reads give lane l the 8 K-consecutive values
            // W[16kk + 8(l>>5) + 0..7][column l & 31 of the fragment]
            const int kr = kk * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
            const int cl = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = g * BN + wcol0 + j * 32 + cl;
                    const s16x4 lo = ds_read_tr16(sB + rm_off<NB>(kr, col));
                    const s16x4 hi = ds_read_tr16(sB + rm_off<NB>(kr + 4, col));
                    const s16x4 both[2] = {lo, hi};
                    fb[set][g][j] = __builtin_bit_cast(bf16x8, both);
                }
        }
    };
    auto mfmas = [&](int set) {
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[g][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][g][j], fa[set][i],
                                                                           acc[g][i][j], 0, 0, 0);
    };

    // Software pipeline over the four 16-deep sub-steps of a 64-deep stage:
    // the fragments of sub-step kk+1 are read while the MFMAs of kk run
    // (each read slotted between MFMAs), and the one barrier per stage sits
    // before the last sub-step's MFMAs, so the first reads of the next stage
    // overlap those MFMAs instead of stalling the matrix pipe.
    constexpr int NFRAG = TM + (PACKED_W ? 1 : 2) * NG * TN;   // LDS reads per sub-step
    constexpr int NMFMA = NG * TM * TN;                          // MFMAs per sub-step
    constexpr int NSLOT = NMFMA > NFRAG ? NMFMA : NFRAG;
    // [MFMA, LDS read (, direct load)] pairs, then whatever is left: the
    // sub-step opens with an MFMA (its operands were read a whole sub-step
    // earlier) and its reads are issued early enough for the next sub-step.
    auto interleave = [&](auto ndma) {
        constexpr int ND = decltype(ndma)::value;
#pragma unroll
        for (int t = 0; t < NSLOT; ++t) {
            if (t < NMFMA) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            if (t < NFRAG) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            if (t < ND) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // direct load
        }
    };
    using Z = std::integral_constant<int, 0>;
    using NL = std::integral_constant<int, (A_INS + B_INS < NSLOT ? A_INS + B_INS : NSLOT)>;

    // One 64-deep stage.  PREFETCH: stage kb+1 is loaded into the other LDS
    // buffer during this one (through registers when RAGGED_NEXT, i.e. stage
    // kb+1 is a ragged last block).  Both operands' loads go out in the first
    // sub-step, so they have three sub-steps to land before the barrier
    // (with the weights' loads in the second sub-step: 72B-width M=4096
    // 4212 -> 3846 us, M=256 494 -> 410 us, bitwise equal).
    auto stage = [&](auto prefetch, auto ragged_next, int kb) {
        constexpr bool PF = decltype(prefetch)::value;
        constexpr bool RN = decltype(ragged_next)::value;
        const int buf = (kb - kb_first) & 1;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PF) {
            if constexpr (RN) issue_a_regs(kb + 1, buf ^ 1);
            else issue_a(kb + 1, buf ^ 1);
            if constexpr (RN && !PACKED_W) issue_b_regs(kb + 1, buf ^ 1);
            else issue_b(kb + 1, buf ^ 1);
        }
        read_frags(buf, 1, 1);
        mfmas(0);
        if constexpr (PF && !RN) interleave(NL{});
        else interleave(Z{});
        __builtin_amdgcn_sched_barrier(0);
        read_frags(buf, 2, 0);
        mfmas(1);
        interleave(Z{});
        __builtin_amdgcn_sched_barrier(0);
        read_frags(buf, 3, 1);
        mfmas(0);
        interleave(Z{});
        __builtin_amdgcn_sched_barrier(0);
        // stage kb+1 has landed in LDS for every wave, and every wave is done
        // reading stage kb (its last fragments are in registers)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if constexpr (PF) {
            read_frags(buf ^ 1, 0, 0);
            mfmas(1);
            interleave(Z{});
        } else {
            mfmas(1);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    const bool last_ragged = ragged_k && kb_last == KB - 1;
    if (last_ragged && kb_first == kb_last) {
        issue_a_regs(kb_first, 0);
        issue_b_regs(kb_first, 0);
    } else {
        issue_a(kb_first, 0);
        issue_b(kb_first, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    read_frags(0, 0, 0);
    const bool rn = last_ragged && kb_last > kb_first;
    const int steady_end = kb_last - (rn ? 1 : 0);
    for (int kb = kb_first; kb < steady_end; ++kb) stage(std::true_type{}, std::false_type{}, kb);
    if (rn) stage(std::true_type{}, std::true_type{}, kb_last - 1);
    stage(std::false_type{}, std::false_type{}, kb_last);

    // Split-K: this split's fp32 Gate/Up partial sums go to the workspace
    // ([split][M][2N]: Gate at column n, Up at column N + n); splitk_reduce_kernel
    // adds the splits in order 0..S-1 and applies the epilogue.
    if constexpr (SPLIT) {
        store_partials<TM, TN>(acc, p.part, split, M, N, m0 + wrow0, n0 + wcol0, lane);
        return;
    }

    // Epilogue: SiLU(Gate) * Up (or the plain GEMM value) -> bf16, staged
    // through LDS so the global stores are 16 bytes per lane over whole row
    // segments of the wave's sub-tile.  Every wave is done with the operand
    // stages (the last barrier came before the final sub-step, whose operands
    // were in registers), so the stage buffers hold the Y tile: each wave owns
    // a disjoint (BM/WM) x CW region; rows of up to 64 columns are padded by
    // 16 bytes, 128-column rows have their chunks XOR-swizzled by row.
    constexpr int CW = BN / WN;                 // columns per wave
    constexpr int PY = CW == 128 ? CW : CW + 8; // row pitch (elements)
    constexpr int CPR = CW / 8;                 // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;               // rows per wave-wide store
    static_assert(CW == 32 || CW == 64 || CW == 128, "epilogue handles 32, 64 or 128 columns per wave");
    static_assert(NW * (BM / WM) * PY <= 2 * STAGE, "epilogue staging fits the stage buffers");
    auto y_off = [&](int r, int chunk) {
        return r * PY + 8 * (CW == 128 ? (chunk ^ (r & 15)) : chunk);
    };
    __syncthreads();
    uint16_t* sY = smem + wave * (BM / WM) * PY;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (NG == 2)
                        v[e] = silu_f(acc[0][i][j][4 * q + e]) * acc[NG - 1][i][j][4 * q + e];
                    else
                        v[e] = acc[0][i][j][4 * q + e];
                }
                u32x2 out;
                out[0] = pack2(v[0], v[1]);
                out[1] = pack2(v[2], v[3]);
                *reinterpret_cast<u32x2*>(sY + y_off(r, 4 * j + q) + 4 * (lane >> 5)) = out;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < (BM / WM) / RPI; ++t) {
        const int r = t * RPI + lane / CPR;
        const int c = lane % CPR;
        const int m = m0 + wrow0 + r;
        const int n = n0 + wcol0 + 8 * c;
        const u32x4 v = *reinterpret_cast<const u32x4*>(sY + y_off(r, c));
        if (m < M && n < N) *reinterpret_cast<u32x4*>(p.Y + (size_t)m * N + n) = v;
    }
}

// ---------------------------------------------------------------------------
// Prefill on packed weights with the weights streamed to registers.
//   The direct global->LDS path moves far more bytes per CU with two 64-deep
//   stages in flight than with one, but with both operands in LDS only one
//   stage fits beside the stage being read (2 x 64 KiB of 160 KiB).  So only
//   the activation tile, the operand all four waves share, goes through LDS:
//   a ring of three BM x 64 stages (32 KiB each at BM = 256), loaded two
//   stages ahead.  The weights skip LDS.  The four waves sit side by side and
//   own 32 output columns each (Gate and Up), so every packed weight fragment
//   is needed by exactly one wave, which loads it straight into registers,
//   also two stages ahead (three register sets of 8 x 16 bytes per lane).  In
//   the packed fragment order each such load is two contiguous 512-byte runs.
//   Per wave and 16-deep sub-step: 2 x TM MFMA 32x32x16, TM fragment reads
//   (double-buffered: the next sub-step's, issued in the first half) and a
//   quarter of the stage's A_INS direct loads + 8 weight loads.  One barrier
//   per stage, before the last sub-step's MFMAs: it publishes the next
//   stage's activation tile and frees the ring slot just read.  Wait counts
//   are explicit (vmcnt counts vector-memory instructions in issue order):
//   at that barrier only loads of the stage two ahead may be in flight.
//   Activation columns beyond K (ragged last block, RAGGED) are fetched from
//   a 16-byte zero chunk, so the ragged stage stays on the direct path; the
//   packed weights are already zero there.
//   Each output sums the same MFMAs in the same order (k ascending, weight
//   fragment as first operand) as fused_prefill_kernel, so the two agree
//   bitwise.
// ---------------------------------------------------------------------------
__device__ __attribute__((aligned(16))) uint16_t g_zero_chunk[8];

// s_waitcnt immediate: vector-memory count vm, LDS/scalar count lgkm (no
// export wait)
constexpr int waitcnt_imm(int vm, int lgkm) {
    return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// LDS elements of the streaming kernel: three ring slots of BM x 64
// activations, then the BM x 128 Y tile of the epilogue (kept apart from the
// ring so that the next tile's first stages can stream in meanwhile)
template <int BM>
constexpr int stream_smem_elems() {
    return 3 * BM * BK + BM * PACK_BN;
}

// Output tiles (or K splits) w = first, first + stride, ... < total of the
// streaming kernel, one after another in one workgroup; LDS at smem
// (stream_smem_elems<BM>() elements, 16-byte aligned).  Between two tiles the
// next tile's first two stages are issued before the epilogue of the
// current one, and its Y stores are left in flight while the next tile's K
// loop starts.
// F8: FP8 E4M3 activations and packed weights (per-tensor scale products
// p.sg, p.su applied to the fp32 sums): a stage is 128 k (the same 128-byte
// activation rows), each 32-row block takes one v_mfma_f32_32x32x64_f8f6f4
// per 64 k, and a sub-step covers one 64-k step for half of the row blocks.
// SEQ: the sequential order (Gate first, then Up): each tile is two K loops
// over the same activations, the first on the Gate half of every packed
// block, the second on the Up half, each with one MFMA per 32-row block into
// the one accumulator set acc[0].  Between the two, the Up loop's first two
// stages are issued and SiLU(Gate) is computed into acc[1] while they land;
// the epilogue is then acc[1] * acc[0].  The Gate and Up sums take the same
// MFMAs in the same order as the dual loop, so the two agree bitwise.
// GEMM: a plain product C = bf16(A x W) on a single-weight pack (packed tile
// jt holds W's columns jt*256 + 0..255): the "Gate" accumulators are output
// columns jt*256 + c, the "Up" ones jt*256 + 128 + c; p.N is C's width.  The
// Y tile in LDS holds 128 columns, so the epilogue runs in two passes (Gate
// half, then Up half), each staged, synchronised and stored.  With SPLIT the
// partial sums go out over the pack's p.tiles_n * 128 tiled columns instead.
// With PANELS each wave takes half a panel -- 32 tiled columns of one weight
// half, one accumulator set -- so the units are twice the fused product's
// panels and the CUs share them as evenly (p.panels counts half-panels; the
// single Y-tile pass maps each wave's 32 columns to its half).
template <int BM, bool SPLIT, bool RAGGED, bool PANELS = false, bool IL = false, bool F8 = false,
          bool SEQ = false, bool GEMM = false>
__device__ __forceinline__ void stream_prefill_tiles(const FusedArgs& p, uint16_t* smem, int first, int stride,
                                                     int total) {
    static_assert(!(GEMM && (IL || F8 || SEQ)), "plain GEMM: bf16 single-weight pack");
    static_assert(!(IL && SPLIT), "the interleaved layout has no split-K schedule");
    static_assert(!(F8 && (IL || SPLIT)), "FP8 operands: per-tile layout, data-parallel only");
    static_assert(!(SEQ && (SPLIT || PANELS || IL || F8)), "sequential order: bf16 per-tile tiles only");
    constexpr int EB = F8 ? 1 : 2;              // bytes per operand element
    constexpr int KSTAGE = F8 ? 128 : BK;       // k per stage (128-byte activation rows)
    constexpr int CE = 16 / EB;                 // elements per 16-byte chunk
    constexpr int NW = 4;                       // waves, 32 output columns each
    constexpr int TM = BM / 32;                 // 32-row MFMA tiles per wave
    constexpr int A_INS = BM / 8 / NW;          // 1 KiB direct loads per wave per stage
    constexpr int ASTAGE = BM * BK;             // elements per activation stage
    constexpr int NBUF = 3;                     // ring slots == weight register sets
    // GEMM on the panel schedule: a wave's unit is half a panel (32 columns of
    // one weight half), twice the units of the fused product's panels
    constexpr bool GH = GEMM && PANELS;
    constexpr int WT = (SEQ || GH) ? 1 : 2;     // weight halves per stage (Gate and Up, or one)
    constexpr int LOADS = A_INS + 4 * WT;       // vector-memory instructions per wave per stage
    constexpr int NST = BM / 16;                // Y stores per wave per tile
    constexpr int GROUP_M = 8;
    static_assert(TM >= 1 && A_INS >= 1 && (BM / 8) % NW == 0, "tile");
    static_assert(LOADS + NST <= 63, "vmcnt range");
    uint16_t* const sY = smem + NBUF * ASTAGE;  // the Y tile

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = p.M, K = p.K, N = p.N, KB = p.KB;
    const int S = SPLIT ? p.splits : 1;

    // work item w -> output tile (m0, n0), K blocks [kb_first, kb_first + ns)
    // and the number np of waves with weights (32-column panels from n0 on)
    struct Item {
        int m0, n0, kb_first, ns, split, np, up;
    };
    auto item_of = [&](int w) {
        if constexpr (PANELS) {
            // Panel schedule: when the row tile has fewer 128-column tiles
            // than there are CUs, the 32-column panels (one wave's share of a
            // tile) are spread evenly over `total` workgroups, so every CU
            // streams weights: adjacent panels, possibly from two packed
            // tiles, all sharing the one activation tile in LDS.
            {
                const int q0 = (int)((long long)w * p.panels / total);
                const int q1 = (int)((long long)(w + 1) * p.panels / total);
                Item it;
                it.m0 = 0;
                it.n0 = q0 * 32;
                it.kb_first = 0;
                it.ns = KB;
                it.split = 0;
                it.np = q1 - q0;
                it.up = 0;
                return it;
            }
        }
        const int logical = xcd_remap(w, total);
        const int tile = SPLIT ? logical / S : logical;
        const int split = SPLIT ? logical - tile * S : 0;
        const int per_group = GROUP_M * p.tiles_n;
        const int group = tile / per_group;
        const int first_m = group * GROUP_M;
        const int gsize = min(p.tiles_m - first_m, GROUP_M);
        const int in_group = tile - group * per_group;
        Item it;
        it.m0 = (first_m + in_group % gsize) * BM;
        it.n0 = (p.n_tile0 + in_group / gsize) * PACK_BN;
        it.kb_first = SPLIT ? split * p.kb_per_split : 0;
        it.ns = (SPLIT ? min(KB, it.kb_first + p.kb_per_split) : KB) - it.kb_first;   // >= 1
        it.split = split;
        it.np = 4;
        it.up = 0;
        return it;
    };

    // activation: lane l of direct load i fetches row (wave*A_INS+i)*8 + l/8,
    // logical chunk (l%8) ^ swz(row), so LDS holds the tile in lds_off order;
    // byte offsets from A (the host splits products whose activations reach
    // 2 GiB into row chunks) so the uniform part of the address stays scalar
    uint32_t a_off[A_INS];
    // lane l's logical chunk in direct load i is (l%8) ^ swz(row) with
    // row = (wave*A_INS + i)*8 + l/8, i.e. chunk_x ^ ((wave*A_INS + i) & 7)
    // with chunk_x = ((l & 7) ^ (l >> 3)) & 7 (only the ragged K stage needs it)
    int chunk_x = 0;
    // weights: the wave's 32 columns are panel wq = n0/32 + wave, i.e.
    // columns 32(wq & 3) + (l & 31) of packed tile wq >> 2; lane l needs the
    // 8 k at chunk c = 2kk + (l >> 5) of each 64-deep block, i.e. packed
    // group t*8 + (wq & 3)*2 + ((l >> 4) & 1), half kk >> 1, fragment lane
    // (2(kk & 1) + (l >> 5))*16 + (l & 15): a lane byte offset plus a
    // constant per (t, kk).  Interleaved layout (IL): the wave's 64 packed
    // rows (its 32 columns' Gate and Up, alternating) are groups
    // 4(wq & 3) + 2t + ((l >> 4) & 1), so register set t holds Gate and Up
    // of the columns 16t .. 16t + 15, each pair in two adjacent rows
    uint32_t w_off = 0;
    const char* w_tile = nullptr;
    // the item whose stages the loads below fetch (ld_ns = 0: none, every
    // load reads the zero chunk; ld_ns_w: the same for this wave's weights,
    // 0 for a wave without a panel)
    int ld_kb_first = 0, ld_ns = 0, ld_ns_w = 0;
    auto load_item = [&](const Item& it, bool valid) {
        // lane index behind an opaque copy: recomputed per item rather than
        // hoisted out of the tile loop (see the epilogue)
        int ll = lane;
        asm volatile("" : "+v"(ll));
#pragma unroll
        for (int i = 0; i < A_INS; ++i) {
            const int r = (wave * A_INS + i) * 8 + (ll >> 3);
            const int c = (ll & 7) ^ swz(r);
            a_off[i] = (uint32_t)((size_t)min(it.m0 + r, M - 1) * K * EB + 16 * c);
        }
        chunk_x = ((ll & 7) ^ (ll >> 3)) & 7;
        const int wu = it.n0 / 32 + wave;       // the wave's panel (GH: half-panel)
        const int wq = GH ? (wu >> 1) : wu;
        if constexpr (F8)
            // FP8 block: [32-row block rb][64-k step][half][lane][16 bytes];
            // Gate block wq & 3, Up block 4 + (wq & 3)
            w_off = (uint32_t)((wq & 3) * 4096 + ll * 16);
        else
            w_off = (uint32_t)((((wq & 3) * (IL ? 4 : 2) + ((ll >> 4) & 1)) * 1024 + (ll >> 5) * 128 +
                                (ll & 15) * 8) * 2);
        w_tile = reinterpret_cast<const char*>(p.W1) + (size_t)(wq >> 2) * KB * (PACK_ROWS * PACK_BK * 2) +
                 (SEQ && it.up ? 16384 : 0) +   // SEQ: the Up half of each packed block
                 (GH ? (wu & 1) * 16384 : 0);   // GH: the wave's half
        ld_kb_first = it.kb_first;
        ld_ns = valid ? it.ns : 0;
        ld_ns_w = (!PANELS || wave < it.np) ? ld_ns : 0;
    };
    // fragment reads: lane l reads row i*32 + (l & 31), logical chunk
    // 2kk + (l >> 5).  swz(i*32 + r) = swz(r) ^ 4(i & 1) for r < 32, so the
    // physical chunk is ((l >> 5) ^ swz(l & 31)) ^ 2(kk ^ 2(i & 1)): four lane
    // base offsets (x = kk ^ 2(i & 1)) plus i*4096 bytes plus the ring slot
    uint32_t rd_base[4];
    // formed per item from an opaque lane copy (not held across epilogues)
    auto set_rd_base = [&]() {
        int lr = lane;
        asm volatile("" : "+v"(lr));
        const int lrow = lr & 31;
        const int hs = (lr >> 5) ^ swz(lrow);
        if constexpr (F8) {
            // a 32-byte fragment is logical chunks 4ks + 2(l >> 5) + e, e = 0, 1:
            // physical chunk (2(l >> 5) ^ swz) ^ x with x = 4(ks ^ (i & 1)) + e
            const int hs8 = (2 * (lr >> 5)) ^ swz(lrow);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                rd_base[j] = (uint32_t)(lrow * 128 + ((hs8 ^ (4 * (j >> 1) + (j & 1))) << 4));
        } else {
#pragma unroll
            for (int x = 0; x < 4; ++x) rd_base[x] = (uint32_t)((lrow * BK + ((hs ^ (2 * x)) << 3)) * 2);
        }
    };

    f32x16 acc[2][TM][1];
    auto zero_acc = [&]() {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[g][i][0][r] = 0.0f;
    };
    zero_acc();
    bf16x8 fa[2][TM];
    i32x8 fa8[2][TM / 2 > 0 ? TM / 2 : 1];
    bf16x8 wf[NBUF][WT][4];
    // every register set defined on every path into the stage loop
#pragma unroll
    for (int q = 0; q < NBUF; ++q)
#pragma unroll
        for (int t = 0; t < WT; ++t)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) wf[q][t][kk] = bf16x8{};

    // byte offset of ring slot b, kept opaque so the fragment addresses are
    // formed per stage from the four lane bases instead of being precomputed
    // for every (slot, sub-step, tile)
    auto slot_off = [&](int b) {
        uint32_t so = (uint32_t)(b * ASTAGE * 2);
        asm volatile("" : "+s"(so));
        return so;
    };
    auto read_a = [&](uint32_t so, int kk, int i, int set) {
        fa[set][i] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(smem) + so + i * 4096 +
                                                      rd_base[kk ^ (2 * (i & 1))]);
    };
    // FP8: the fragment of sub-step q (64-k step q >> 1, row blocks
    // (q & 1) * TM/2 + ii) into fa8[set][ii]
    auto read_a8 = [&](uint32_t so, int q, int ii, int set) {
        const int i = (q & 1) * (TM / 2) + ii;
        const char* b = reinterpret_cast<const char*>(smem) + so + i * 4096;
        const int j = 2 * ((q >> 1) ^ (i & 1));
        const i32x4 lo = *reinterpret_cast<const i32x4*>(b + rd_base[j]);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(b + rd_base[j + 1]);
        fa8[set][ii] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // Stages past the last (ls >= ld_ns) are issued like any other, but every
    // lane then reads the 16-byte zero chunk (a single cache line): the
    // stage code stays the same for every stage, with no tail variants.
    // Their weight registers are consumed (without instructions) at the end,
    // so those loads are not dropped as dead code and every stage issues
    // exactly LOADS vector-memory instructions, which the wait counts rely on.
    // load j of stage ls: j < A_INS the activation direct load j into slot
    // buf, else weight fragment (t, kk) = ((j - A_INS) / 4, (j - A_INS) % 4)
    // into register set SET
    auto issue_one = [&](int j, int ls, int buf, auto setc) {
        constexpr int SET = decltype(setc)::value;
        const bool valid = ls < (j < A_INS ? ld_ns : ld_ns_w);
        const uint32_t keep = valid ? 0xffffffffu : 0u;
        if (j < A_INS) {
            const int k0 = (ld_kb_first + ls) * KSTAGE;
            const char* base = valid ? reinterpret_cast<const char*>(p.A) + (size_t)k0 * EB
                                     : reinterpret_cast<const char*>(g_zero_chunk);
            const uint16_t* src = reinterpret_cast<const uint16_t*>(base + (a_off[j] & keep));
            if constexpr (RAGGED) {
                if (k0 + CE * (chunk_x ^ ((wave * A_INS + j) & 7)) >= K) src = g_zero_chunk;
            }
            dma16(src, smem + buf * ASTAGE + (wave * A_INS + j) * 512);
        } else {
            const int t = (j - A_INS) >> 2, kk = (j - A_INS) & 3;
            const char* base = valid ? w_tile + (size_t)(ld_kb_first + ls) * (PACK_ROWS * PACK_BK * 2) +
                                           t * (IL ? 4096 : 16384) +
                                           (kk >> 1) * (F8 ? 2048 : 1024) + (kk & 1) * (F8 ? 1024 : 512)
                                     : reinterpret_cast<const char*>(g_zero_chunk);
            const bf16x8* wsrc = reinterpret_cast<const bf16x8*>(base + (w_off & keep));
            // panel schedule: each weight byte is read by one wave of the
            // whole grid, so it streams through L2 non-temporally
            wf[SET][t][kk] = PANELS ? __builtin_nontemporal_load(wsrc) : *wsrc;
        }
    };
    constexpr int LPS = LOADS / 4;                // loads per sub-step
    static_assert(LOADS % 4 == 0, "loads split over four sub-steps");
    constexpr int RPI = TM >= 2 ? 2 : 1;          // next-sub-step reads per step
    // One 16-deep sub-step on fragment set CUR, in a fixed order (each step
    // fenced): for each 32-row tile, its Gate and Up MFMAs, then the next
    // sub-step's fragments (RD: from slot offset rso, sub-step rkk; two per
    // step, so they are all issued in the first half), then (LD) its share of
    // the sub-step's loads of stage ls (LPS of them, or all LOADS with ALL).
    // The reads go to the other fragment set, so any wait for
    // them lands at the start of the next sub-step, long after they were
    // issued.
    auto substep = [&](auto wsetc, int kk, int cur, auto rdc, uint32_t rso, int rkk, auto ldc, int ls, int lbuf,
                       auto lsetc, int lq, auto allc) {
        constexpr int WS = decltype(wsetc)::value;
        constexpr bool RD = decltype(rdc)::value;
        constexpr bool LD = decltype(ldc)::value;
        constexpr bool ALL = decltype(allc)::value;   // all LOADS loads of the stage in this sub-step
        constexpr int NLD = ALL ? LOADS : LPS;
        constexpr int LPIX = (NLD + TM - 1) / TM;
        // this sub-step's fragments were all read during the first half of
        // the previous one: wait for them here, before any new read, so no
        // later wait in this sub-step has to cover the new reads
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
        if constexpr (F8) {
            // sub-step kk: 64-k step kk >> 1 on row blocks (kk & 1) * TM/2 + ii;
            // the weight fragment is the register pieces 2ks, 2ks + 1
            constexpr int TH = TM / 2;
            constexpr int LPI8 = (LPS + TH - 1) / TH;
            const int ks = kk >> 1;
#pragma unroll
            for (int ii = 0; ii < TH; ++ii) {
                const int i = (kk & 1) * TH + ii;
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const i32x8 wv = __builtin_shufflevector(__builtin_bit_cast(i32x4, wf[WS][g][2 * ks]),
                                                             __builtin_bit_cast(i32x4, wf[WS][g][2 * ks + 1]),
                                                             0, 1, 2, 3, 4, 5, 6, 7);
                    acc[g][i][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, fa8[cur][ii], acc[g][i][0],
                                                                                   0, 0, 0, 0, 0, 0);
                }
                if constexpr (RD) read_a8(rso, rkk, ii, cur ^ 1);
                if constexpr (LD) {
                    // the weights' loads first, as in the bf16 panel schedule
                    // below (FP8 7B-width M=48 29.1 -> 27.7 us; FP8 prefill
                    // about 1 % faster: 72B-width M=4096 1397 -> 1383 us)
#pragma unroll
                    for (int j = ii * LPI8; j < (ii + 1) * LPI8; ++j)
                        if (j < LPS) issue_one((lq * LPS + j + A_INS) % LOADS, ls, lbuf, lsetc);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            acc[0][i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[WS][0][kk], fa[cur][i], acc[0][i][0], 0, 0, 0);
            if constexpr (WT == 2)
                acc[1][i][0] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[WS][WT - 1][kk], fa[cur][i], acc[1][i][0], 0, 0, 0);
            if constexpr (RD) {
#pragma unroll
                for (int q = i * RPI; q < (i + 1) * RPI; ++q)
                    if (q < TM) read_a(rso, rkk, q, cur ^ 1);
            }
            if constexpr (LD) {
#pragma unroll
                for (int j = i * LPIX; j < (i + 1) * LPIX; ++j)
                    if (j < NLD) {
                        // the fused product's panel schedule issues the
                        // weights' loads (from HBM) before the activations'
                        // (L2 hits): 7B-width M=64 54.2 -> 51.4 us, 0.5B-width
                        // M=128 15.4 -> 14.8 us, the other panel shapes alike
                        constexpr bool WFIRST = PANELS && !GEMM && !F8;
                        const int x = ALL ? j : lq * LPS + j;
                        issue_one(WFIRST ? (x + A_INS) % LOADS : x, ls, lbuf, lsetc);
                    }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using T = std::true_type;
    using F = std::false_type;

    // One 64-deep stage s in ring slot / register set P = s % 3: issues
    // stage s+2's loads (slot and set (P+2) % 3, freed by the previous
    // stage's barrier), LPS per sub-step, and reads stage s+1's first
    // fragments during its last sub-step.  The single-weight GEMM's panel
    // schedule (one accumulator set, half-panels) issues all of them in the
    // first sub-step instead (7B-width M=128 GEMM 43.8 -> 39.8 us, M=64
    // 42.0 -> 34.9 us, 0.5B-width M=128 12.5 -> 11.1 us; the fused product's
    // panels were slower that way, 7B-width M=128 56.7 -> 58.5 us).
    auto stage = [&](auto pc, int s) {
        constexpr int P = decltype(pc)::value;
        constexpr int PN = (P + 1) % NBUF, PL = (P + 2) % NBUF;
        using WP = std::integral_constant<int, P>;
        using WL = std::integral_constant<int, PL>;
        const uint32_t so = slot_off(P);
        __builtin_amdgcn_sched_barrier(0);
        constexpr bool EARLY = PANELS && GEMM && !F8;
        using EA = std::integral_constant<bool, EARLY>;
        using LR = std::integral_constant<bool, !EARLY>;
        substep(WP{}, 0, 0, T{}, so, 1, T{}, s + 2, PL, WL{}, 0, EA{});
        substep(WP{}, 1, 1, T{}, so, 2, LR{}, s + 2, PL, WL{}, 1, F{});
        substep(WP{}, 2, 0, T{}, so, 3, LR{}, s + 2, PL, WL{}, 2, F{});
        const uint32_t son = slot_off(PN);
        // stage s+1 (activations and this wave's weights) has landed once at
        // most the loads of stage s+2 issued so far (3*LPS, or all LOADS when
        // EARLY) are in flight (every stage issues all LOADS loads, also past
        // the end: see below); after the barrier every wave is done reading
        // slot P
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(EARLY ? LOADS : 3 * LPS, 0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        substep(WP{}, 3, 1, T{}, son, 0, LR{}, s + 2, PL, WL{}, 3, F{});
        __builtin_amdgcn_sched_barrier(0);
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;


    // stages 0 and 1 of an item into slots 0 and 1 and register sets 0 and 1
    auto issue_first_w = [&]() {
#pragma unroll
        for (int j = A_INS; j < LOADS; ++j) issue_one(j, 0, 0, I0{});
#pragma unroll
        for (int j = A_INS; j < LOADS; ++j) issue_one(j, 1, 1, I1{});
    };
    auto issue_first_a = [&]() {
#pragma unroll
        for (int j = 0; j < A_INS; ++j) issue_one(j, 0, 0, I0{});
#pragma unroll
        for (int j = 0; j < A_INS; ++j) issue_one(j, 1, 1, I1{});
    };

    // first item: weights of both stages first, so that waiting for stage 0
    // leaves only stage 1's direct loads in flight, no register load pending
    // into the loop
    Item cur = item_of(first);
    load_item(cur, true);
    issue_first_w();
    issue_first_a();
    set_rd_base();
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(A_INS, 0));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int i = 0; i < (F8 ? TM / 2 : TM); ++i) {
        if constexpr (F8) read_a8(0u, 0, i, 0);
        else read_a(0u, 0, i, 0);
    }

    for (int w = first;;) {
        const int ns = cur.ns;
        // periods of three stages and a remainder of one or two (slots 0, 1)
        int s = 0;
        for (; s + 3 <= ns; s += 3) {
            stage(I0{}, s);
            stage(I1{}, s + 1);
            stage(I2{}, s + 2);
        }
        if (ns - s >= 1) stage(I0{}, s);
        if (ns - s >= 2) stage(I1{}, s + 1);
        // the zero-chunk loads of the two stages past the end are still in
        // flight (their weight registers are consumed here, without
        // instructions, so the loads are not dropped); after the barrier no
        // wave reads the ring any more
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
#pragma unroll
        for (int q = 0; q < NBUF; ++q)
#pragma unroll
            for (int t = 0; t < WT; ++t)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) asm volatile("" ::"v"(wf[q][t][kk]));
        __builtin_amdgcn_s_barrier();

        if constexpr (SPLIT) {
            // GEMM: the partials cover the pack's tiled columns (both halves
            // of each packed tile), reduced by splitk_gemm_reduce_kernel
            store_partials<TM, 1>(acc, p.part, cur.split, M, GEMM ? p.tiles_n * PACK_BN : N, cur.m0,
                                  cur.n0 + wave * 32, lane);
            break;   // one item per workgroup
        }

        if constexpr (SEQ) {
            if (!cur.up) {
                // Gate done: the Up loop's first two stages stream in while
                // SiLU(Gate) goes to acc[1] and acc[0] is cleared for Up
                Item upi = cur;
                upi.up = 1;
                load_item(upi, true);
                issue_first_w();
                issue_first_a();
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        acc[1][i][0][r] = silu_f(acc[0][i][0][r]);
                        acc[0][i][0][r] = 0.0f;
                    }
                __builtin_amdgcn_sched_barrier(0);
                set_rd_base();
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(A_INS, 0));
                __builtin_amdgcn_s_barrier();
#pragma unroll
                for (int i = 0; i < TM; ++i) read_a(0u, 0, i, 0);
                cur = upi;
                continue;
            }
        }

        // the next item's first two stages stream in during this epilogue
        // (past the last item they read the zero chunk): activations and
        // stage 0's weights now, stage 1's weights once the accumulators are
        // consumed
        const int wn = w + stride;
        const bool more = wn < total;
        const Item nxt = item_of(more ? wn : w);
        load_item(nxt, more);
        issue_first_a();
#pragma unroll
        for (int j = A_INS; j < LOADS; ++j) issue_one(j, 0, 0, I0{});

        // Epilogue: SiLU(Gate) * Up -> bf16 into the LDS Y tile (16-byte chunk
        // index XOR row & 15, and the two 8-byte halves swapped on rows with
        // bit 4 set, so each 32-lane write pass covers all banks), then whole
        // 256-byte row segments to HBM, left in flight.
        // (one 32-row step at a time, so the accumulators are not all moved
        // to VGPRs at once).  `el` is the lane index behind an opaque copy:
        // the epilogue's many lane-dependent addresses are then formed here,
        // per tile, instead of being hoisted out of the tile loop and held
        // in registers across every K loop.
        int el = lane;
        asm volatile("" : "+v"(el));
        __builtin_amdgcn_sched_barrier(0);
        // GEMM pass gh: bf16 of accumulator set gh (no SiLU) into the Y tile
        auto fill_gemm = [&](int gh) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = i * 32 + (el & 31);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    u32x2 out;
                    out[0] = pack2(acc[gh][i][0][4 * q], acc[gh][i][0][4 * q + 1]);
                    out[1] = pack2(acc[gh][i][0][4 * q + 2], acc[gh][i][0][4 * q + 3]);
                    const int chunk = wave * 4 + q;
                    *reinterpret_cast<u32x2*>(sY + r * PACK_BN + 8 * (chunk ^ (r & 15)) +
                                              4 * ((el >> 5) ^ ((r >> 4) & 1))) = out;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if constexpr (GEMM) fill_gemm(0);
#pragma unroll
        for (int i = 0; i < (GEMM ? 0 : TM); ++i) {
            const int r = i * 32 + (el & 31);
            if constexpr (IL) {
                // accumulator register 4q + 2e + g of set t is packed row
                // 32t + 8q + 4(l >> 5) + 2e + g: Gate (g = 0) and Up (g = 1)
                // of column 16t + 4q + 2(l >> 5) + e, so each lane pairs
                // adjacent registers and writes two columns (4 bytes) per (t, q)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const unsigned out =
                            pack2(silu_f(acc[t][i][0][4 * q]) * acc[t][i][0][4 * q + 1],
                                  silu_f(acc[t][i][0][4 * q + 2]) * acc[t][i][0][4 * q + 3]);
                        const int chunk = wave * 4 + 2 * t + (q >> 1);
                        *reinterpret_cast<unsigned*>(sY + r * PACK_BN + 8 * (chunk ^ (r & 15)) +
                                                     4 * ((q & 1) ^ ((r >> 4) & 1)) + 2 * (el >> 5)) = out;
                    }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float gv = acc[0][i][0][4 * q + e], uv = acc[1][i][0][4 * q + e];
                        if constexpr (F8) {
                            gv *= p.sg;
                            uv *= p.su;
                        }
                        // SEQ: acc[1] holds SiLU(Gate), acc[0] Up
                        v[e] = SEQ ? uv * gv : silu_f(gv) * uv;
                    }
                    u32x2 out;
                    out[0] = pack2(v[0], v[1]);
                    out[1] = pack2(v[2], v[3]);
                    const int chunk = wave * 4 + q;
                    *reinterpret_cast<u32x2*>(sY + r * PACK_BN + 8 * (chunk ^ (r & 15)) +
                                              4 * ((el >> 5) ^ ((r >> 4) & 1))) = out;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // the offsets are formed again rather than held through the epilogue
        load_item(nxt, more);
#pragma unroll
        for (int j = A_INS; j < LOADS; ++j) issue_one(j, 1, 1, I1{});
        // the next item's stage 0 (and stage 1's activations) has landed once
        // at most stage 1's weight loads are in flight; the Y tile is in LDS
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(LOADS - A_INS, 0));
        __builtin_amdgcn_s_barrier();
        // wave w stores rows w*BM/4 + 4t + l/16, 16 bytes at tile column
        // 8(l%16); GEMM pass gh: output column (f / 128) * 256 + 128 gh +
        // f % 128 of tile column f
        auto store_tile = [&](int gh) {
            const int r0 = wave * (BM / 4) + (el >> 4);
            const int c = el & 15;
            const int f = cur.n0 + 8 * c;
            int n;
            bool col_ok;
            if constexpr (GH) {
                // tile columns 32w .. 32w + 31 are wave w's half-panel
                // u = n0/32 + w: tiled columns 32(u >> 1) + 0..31 of half u & 1
                const int u = cur.n0 / 32 + (c >> 2);
                const int tc = (u >> 1) * 32 + 8 * (c & 3);
                n = (tc >> 7) * PACK_ROWS + PACK_BN * (u & 1) + (tc & (PACK_BN - 1));
                col_ok = (c >> 2) < cur.np && n < N;
            } else {
                n = GEMM ? (f >> 7) * PACK_ROWS + PACK_BN * gh + (f & (PACK_BN - 1)) : f;
                col_ok = GEMM ? (n < N && (!PANELS || f < cur.n0 + 32 * cur.np))
                              : (n < (PANELS ? min(N, cur.n0 + 32 * cur.np) : N));
            }
            const int rows_left = M - cur.m0 - r0;   // rows r0 + 4t < M - m0
            uint16_t* yp = p.Y + (size_t)(cur.m0 + r0) * N + n;
#pragma unroll
            for (int t = 0; t < NST; ++t) {
                const int r = r0 + t * 4;
                u32x4 v = *reinterpret_cast<const u32x4*>(sY + r * PACK_BN + 8 * (c ^ (r & 15)));
                if ((r >> 4) & 1) v = u32x4{v[2], v[3], v[0], v[1]};
                if (4 * t < rows_left && col_ok) store16_untracked(yp + (size_t)t * 4 * N, v);
            }
        };
        store_tile(0);
        if constexpr (GEMM && !GH) {
            // every wave has read the Gate half out of the Y tile (its reads
            // fed the stores above); then the Up half goes through it
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            fill_gemm(1);
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            store_tile(1);
        }
        if (!more) break;

        // next item: the Y stores stay in flight into its K loop
        zero_acc();
        cur = nxt;
        w = wn;
        set_rd_base();
#pragma unroll
        for (int i = 0; i < (F8 ? TM / 2 : TM); ++i) {
            if constexpr (F8) read_a8(0u, 0, i, 0);
            else read_a(0u, 0, i, 0);
        }
    }
    // the zero-chunk loads of the stages past the last item are in flight
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int t = 0; t < WT; ++t)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) asm volatile("" ::"v"(wf[q][t][kk]));
}

template <int BM, bool SPLIT, bool RAGGED, bool PANELS = false, bool IL = false, bool F8 = false,
          bool SEQ = false, bool GEMM = false>
__global__ __launch_bounds__(256) void stream_prefill_kernel(FusedArgs p, int total) {
    static_assert(!PANELS || !SPLIT, "panel schedule: one row tile, data-parallel");
    __shared__ __attribute__((aligned(16))) uint16_t smem[stream_smem_elems<BM>()];
    stream_prefill_tiles<BM, SPLIT, RAGGED, PANELS, IL, F8, SEQ, GEMM>(p, smem, blockIdx.x, gridDim.x, total);
}

// The 256-row tiles and the 128-row tail column tiles in one launch: blocks
// 0 .. n_pers-1 work through the n_big 256-row tiles of `big` (block b takes
// tiles b, b + n_pers, ...), the remaining blocks take one 128-row tile of
// `tail` each and start on CUs as the 256-row work drains.
template <bool RAGGED, bool IL = false, bool F8 = false, bool SEQ = false, bool GEMM = false>
__global__ __launch_bounds__(256) void stream_prefill_mixed_kernel(FusedArgs big, FusedArgs tail, int n_pers,
                                                                   int n_big) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[stream_smem_elems<256>()];
    static_assert(stream_smem_elems<256>() >= stream_smem_elems<128>(), "one LDS block serves both tiles");
    const int b = blockIdx.x;
    if (b < n_pers) {
        stream_prefill_tiles<256, false, RAGGED, false, IL, F8, SEQ, GEMM>(big, smem, b, n_pers, n_big);
    } else {
        const int n_tail = gridDim.x - n_pers;
        stream_prefill_tiles<128, false, RAGGED, false, IL, F8, SEQ, GEMM>(tail, smem, b - n_pers, n_tail, n_tail);
    }
}

// ---------------------------------------------------------------------------
// Decode (small M): weight streaming.
//   The product is bound by reading the packed weights once from HBM, so the
//   kernel is shaped around keeping many 16-byte loads in flight, not around
//   the matrix cores: each workgroup owns a group of 16 output columns (its 16
//   Gate rows and 16 Up rows of every packed block), and its 4 waves take the
//   K blocks round-robin (wave w: kb = w, w+4, ...).  Weight fragments go
//   straight from HBM to registers with non-temporal loads -- every weight
//   element is used once, so there is nothing to share through LDS or keep in
//   L2 -- and an MFMA 16x16x32 per
//   (Gate|Up, 16-token tile) does the dot products (its cost is negligible
//   next to the loads).  The four per-wave fp32 partial sums of Gate and Up
//   are then added in LDS in wave order 0..3 (fixed order, BEFORE SiLU) and
//   the epilogue applies SiLU(Gate) * Up.
//   MT 16-token tiles cover M <= 16 * MT.
// ---------------------------------------------------------------------------
struct DecodeArgs {
    const uint16_t* A;    // [M,K]
    const uint16_t* Wp;   // packed weights
    uint16_t* Y;          // [M,N]
    int M, K, N;
    int KB;               // ceil(K / 64)
};

// GEMM: a plain product C = bf16(A x W) on a single-weight pack (packed tile
// jt holds W's columns jt*256 + 0..255); the "Gate" sums of tile column c are
// output column jt*256 + c, the "Up" sums jt*256 + 128 + c; p.N is C's width
// (the grid covers the packed tiles' 128 columns each).
// HALF (GEMM only): each workgroup takes one of the two halves of its column
// groups (blockIdx.x & 1: the "Gate" rows, i.e. output columns jt*256 + c, or
// the "Up" rows, jt*256 + 128 + c), so a single-weight product has as many
// workgroups, each streaming half the bytes, as the fused product on weights
// of the same width -- finer work units for the CUs to balance.
// LDSA: each wave stages its K blocks' activations (16*MT rows x 64 k) in its
// own LDS slots with full-line direct loads (8 rows x 128 bytes per
// instruction; the 16-byte chunks of row r XOR-ed with r & 7) and reads the
// MFMA fragments from there, instead of loading each fragment (16 rows x 64
// bytes, half lines) from global memory.
template <int MT, int CG, int UNROLL, bool GEMM = false, bool HALF = false, bool LDSA = false>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs p) {
    static_assert(GEMM || !HALF, "HALF splits the single-weight product only");
    constexpr int WAVES = 4;
    constexpr int NH = HALF ? 1 : 2;    // weight halves per workgroup
    constexpr int AROWS = 16 * MT;      // activation rows per K block
    __shared__ f32x4 red[WAVES][MT][CG][NH][64];
    __shared__ __attribute__((aligned(16))) uint16_t sA[LDSA ? WAVES * UNROLL * AROWS * PACK_BK : 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15;          // weight row within a group / token within a tile
    const int kq = lane >> 4;           // which 8-wide K slice of a 32-deep step
    const int half = HALF ? (int)(blockIdx.x & 1) : 0;
    const int n0 = (HALF ? (int)(blockIdx.x >> 1) : (int)blockIdx.x) * (16 * CG);
    const int jt = n0 / PACK_BN, ro = n0 % PACK_BN;
    const int M = p.M, K = p.K, N = p.N, KB = p.KB;

    // Gate rows of group c are packed rows ro + 16c + (0..15), Up rows the
    // same + 128; each (16-row group, 32-deep half) is one 1 KiB fragment in
    // lane order, so lane l's 16 bytes sit at l * 8 in it.  16*CG columns never
    // straddle a packed tile (128 is a multiple of 16*CG).
    const uint16_t* wtile = p.Wp + (size_t)jt * KB * (PACK_ROWS * PACK_BK);
    const int grp0 = ro >> 4;
    const uint16_t* a_row[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) a_row[t] = p.A + (size_t)min(t * 16 + r16, M - 1) * K + 8 * kq;
    // LDSA: direct load i of a block brings rows 8i + (lane >> 3), lane l's
    // logical chunk (l & 7) ^ (row & 7), to physical chunk l & 7
    const uint16_t* a_dma[LDSA ? 2 * MT : 1];
    int a_chunk[LDSA ? 2 * MT : 1];
    if constexpr (LDSA) {
#pragma unroll
        for (int i = 0; i < 2 * MT; ++i) {
            const int r = 8 * i + (lane >> 3);
            a_chunk[i] = (lane & 7) ^ (r & 7);
            a_dma[i] = p.A + (size_t)min(r, M - 1) * K + 8 * a_chunk[i];
        }
    }
    uint16_t* const sAw = sA + (LDSA ? wave * UNROLL * AROWS * PACK_BK : 0);

    f32x4 accg[MT][CG], accu[MT][CG];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int c = 0; c < CG; ++c) {
            accg[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
            accu[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
            // opaque zeros: with one shared zero register as every sum's
            // start, the allocator gave the loop-carried sums different
            // registers at the loop's entry and back edge and copied them at
            // every step (80 copies per 32 MFMAs at 64 rows; tiny-width
            // M=64 9.4 -> 8.8 us, bitwise equal)
            asm volatile("" : "+a"(accg[t][c]), "+a"(accu[t][c]));
        }

    for (int kb0 = wave; kb0 < KB; kb0 += WAVES * UNROLL) {
        u32x4 wg[UNROLL][2][CG], wu[UNROLL][2][CG], av[UNROLL][2][MT];
        if constexpr (LDSA) {
            // this wave's fragment reads of its slots (previous blocks) are done
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
            asm volatile("" ::: "memory");
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int kb = kb0 + u * WAVES;
                if (kb < KB) {
#pragma unroll
                    for (int i = 0; i < 2 * MT; ++i) {
                        const uint16_t* src = kb * PACK_BK + 8 * a_chunk[i] < K ? a_dma[i] + (size_t)kb * PACK_BK
                                                                                : g_zero_chunk;
                        dma16(src, sAw + (u * AROWS + 8 * i) * PACK_BK);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kb = kb0 + u * WAVES;
            if (kb < KB) {
                const size_t boff = (size_t)kb * (PACK_ROWS * PACK_BK);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int c = 0; c < CG; ++c) {
                        wg[u][h][c] = ld16_stream(wtile + boff + (((grp0 + c + 8 * half) * 2 + h) * 64 + lane) * 8);
                        if constexpr (!HALF)
                            wu[u][h][c] = ld16_stream(wtile + boff + (((grp0 + c + 8) * 2 + h) * 64 + lane) * 8);
                    }
                    if constexpr (!LDSA) {
                        const int k = kb * PACK_BK + 32 * h + 8 * kq;
#pragma unroll
                        for (int t = 0; t < MT; ++t)
                            av[u][h][t] = k < K ? ld16(a_row[t] + (size_t)kb * PACK_BK + 32 * h)
                                                : u32x4{0u, 0u, 0u, 0u};
                    }
                }
            }
        }
        if constexpr (LDSA) {
            // the activations have landed in this wave's slots (the weight
            // loads issued after them too)
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 63));
            asm volatile("" ::: "memory");
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        const int r = t * 16 + r16;
                        av[u][h][t] = *reinterpret_cast<const u32x4*>(
                            sAw + (u * AROWS + r) * PACK_BK + 8 * ((4 * h + kq) ^ (r & 7)));
                    }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kb = kb0 + u * WAVES;
            if (kb < KB) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        const bf16x8 a8 = __builtin_bit_cast(bf16x8, av[u][h][t]);
#pragma unroll
                        for (int c = 0; c < CG; ++c) {
                            accg[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, wg[u][h][c]), a8, accg[t][c], 0, 0, 0);
                            if constexpr (!HALF)
                                accu[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, wu[u][h][c]), a8, accu[t][c], 0, 0, 0);
                        }
                    }
            }
        }
    }

#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int c = 0; c < CG; ++c) {
            red[wave][t][c][0][lane] = accg[t][c];
            if constexpr (!HALF) red[wave][t][c][NH - 1][lane] = accu[t][c];
        }
    __syncthreads();
    // epilogue: wave w finishes (token tile, column group) pairs w, w+4, ...
    for (int tc = wave; tc < MT * CG; tc += WAVES) {
        const int t = tc / CG, c = tc % CG;
        f32x4 g = red[0][t][c][0][lane], u = red[0][t][c][NH - 1][lane];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) {
            g += red[w][t][c][0][lane];
            if constexpr (!HALF) u += red[w][t][c][NH - 1][lane];
        }
        const int m = t * 16 + r16;
        const int n = n0 + 16 * c + 4 * kq;
        if constexpr (HALF) {
            const int col = (n / PACK_BN) * PACK_ROWS + n % PACK_BN + PACK_BN * half;
            if (m < M && col < N) {
                u32x2 out;
                out[0] = pack2(g[0], g[1]);
                out[1] = pack2(g[2], g[3]);
                *reinterpret_cast<u32x2*>(p.Y + (size_t)m * N + col) = out;
            }
        } else if constexpr (GEMM) {
            const int col = (n / PACK_BN) * PACK_ROWS + n % PACK_BN;
            if (m < M && col < N) {
                u32x2 out;
                out[0] = pack2(g[0], g[1]);
                out[1] = pack2(g[2], g[3]);
                *reinterpret_cast<u32x2*>(p.Y + (size_t)m * N + col) = out;
            }
            if (m < M && col + PACK_BN < N) {
                u32x2 out;
                out[0] = pack2(u[0], u[1]);
                out[1] = pack2(u[2], u[3]);
                *reinterpret_cast<u32x2*>(p.Y + (size_t)m * N + col + PACK_BN) = out;
            }
        } else if (m < M && n < N) {
            u32x2 out;
            out[0] = pack2(silu_f(g[0]) * u[0], silu_f(g[1]) * u[1]);
            out[1] = pack2(silu_f(g[2]) * u[2], silu_f(g[3]) * u[3]);
            *reinterpret_cast<u32x2*>(p.Y + (size_t)m * N + n) = out;
        }
    }
}

// ---------------------------------------------------------------------------
// FP8 decode (M <= 32): weight streaming on the FP8 pack.  Each workgroup owns
// CG groups of 32 output columns (32-row blocks rb of the packed tile for
// Gate, 4 + rb for Up); its 4 waves take the 128-k blocks round-robin,
// UNROLL blocks in flight, and each 64-k step is one
// v_mfma_f32_32x32x64_f8f6f4 per (group, Gate|Up) with the weight fragment
// as src0 (lane l: packed row l & 31, k 32(l >> 5) + 0..31, its two 16-byte
// halves read with non-temporal loads from the pack's two 1 KiB runs) and the
// activations as src1 (lane l: token l & 31, the same k, two 16-byte loads).  The four per-wave fp32 sums are added in LDS in wave
// order 0..3, scaled (p.sg, p.su), and SiLU(Gate) * Up is stored as bf16.
// ---------------------------------------------------------------------------
// LDSA: the 32 token rows of each 128-k block go through the wave's own LDS
// slots (one full-line direct load per 8 rows, chunks XOR-ed with row & 7)
// instead of four half-filled 16-byte loads per row.
template <int CG, int UNROLL, bool LDSA = false>
__global__ __launch_bounds__(256) void decode_fp8_kernel(FusedArgs p) {
    constexpr int WAVES = 4;
    // per-wave sums in 16-byte quarters, lane-contiguous (conflict-free LDS
    // stores and loads: 64 lanes x 16 bytes per instruction)
    __shared__ f32x4 red[WAVES][CG][2][4][64];
    __shared__ __attribute__((aligned(16))) uint8_t sA8[LDSA ? WAVES * UNROLL * 32 * 128 : 16];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int M = p.M, K = p.K, N = p.N, KB = p.KB;
    const int n0 = blockIdx.x * (32 * CG);
    const int jt = n0 / PACK_BN, rb0 = (n0 % PACK_BN) / 32;
    const char* wtile = reinterpret_cast<const char*>(p.W1) + (size_t)jt * KB * 32768 + lane * 16;
    const char* arow = reinterpret_cast<const char*>(p.A) + (size_t)min(lane & 31, M - 1) * K + 32 * (lane >> 5);
    // LDSA: direct load i of a block brings row 8i + (lane >> 3), logical
    // 16-byte chunk (lane & 7) ^ (lane >> 3), to physical chunk lane & 7
    const int a_chunk = (lane & 7) ^ (lane >> 3);
    uint8_t* const sAw = sA8 + (LDSA ? wave * UNROLL * 32 * 128 : 0);

    f32x16 acc[CG][2];
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[c][g][r] = 0.0f;

    for (int kb0 = wave; kb0 < KB; kb0 += WAVES * UNROLL) {
        i32x4 wv[UNROLL][CG][2][2][2], av[UNROLL][2][2];
        if constexpr (LDSA) {
            // this wave's fragment reads of its slots (previous blocks) are done
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
            asm volatile("" ::: "memory");
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int kb = kb0 + u * WAVES;
                if (kb < KB) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 8 * i + (lane >> 3);
                        const char* src = kb * 128 + 16 * a_chunk < K
                                              ? reinterpret_cast<const char*>(p.A) + (size_t)min(r, M - 1) * K +
                                                    (size_t)kb * 128 + 16 * a_chunk
                                              : reinterpret_cast<const char*>(g_zero_chunk);
                        dma16(reinterpret_cast<const uint16_t*>(src),
                              reinterpret_cast<uint16_t*>(sAw + (u * 32 + 8 * i) * 128));
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kb = kb0 + u * WAVES;
            if (kb < KB) {
                const char* blk = wtile + (size_t)kb * 32768;
#pragma unroll
                for (int c = 0; c < CG; ++c)
#pragma unroll
                    for (int g = 0; g < 2; ++g)
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                            for (int h = 0; h < 2; ++h)
                                wv[u][c][g][ks][h] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(
                                    blk + ((4 * g + rb0 + c) * 2 + ks) * 2048 + 1024 * h));
                if constexpr (!LDSA) {
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int k = kb * 128 + 64 * ks + 32 * (lane >> 5) + 16 * h;
                            av[u][ks][h] = k < K ? *reinterpret_cast<const i32x4*>(arow + (size_t)kb * 128 + 64 * ks +
                                                                                   16 * h)
                                                 : i32x4{0, 0, 0, 0};
                        }
                }
            }
        }
        if constexpr (LDSA) {
            // the activations have landed (the weight loads issued after them too)
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 63));
            asm volatile("" ::: "memory");
            const int r = lane & 31;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        av[u][ks][h] = *reinterpret_cast<const i32x4*>(
                            sAw + (u * 32 + r) * 128 + 16 * ((4 * ks + 2 * (lane >> 5) + h) ^ (r & 7)));
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kb = kb0 + u * WAVES;
            if (kb < KB) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const i32x8 a8 = __builtin_shufflevector(av[u][ks][0], av[u][ks][1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int c = 0; c < CG; ++c)
#pragma unroll
                        for (int g = 0; g < 2; ++g) {
                            const i32x8 w8 = __builtin_shufflevector(wv[u][c][g][ks][0], wv[u][c][g][ks][1],
                                                                     0, 1, 2, 3, 4, 5, 6, 7);
                            acc[c][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w8, a8, acc[c][g], 0, 0,
                                                                                        0, 0, 0, 0);
                        }
                }
            }
        }
    }

#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                red[wave][c][g][j][lane] =
                    f32x4{acc[c][g][4 * j], acc[c][g][4 * j + 1], acc[c][g][4 * j + 2], acc[c][g][4 * j + 3]};
    __syncthreads();
    // epilogue: wave w finishes groups w, w + 4, ...; lane l holds token
    // m = l & 31 and columns n0 + 32c + 8(r/4) + 4(l >> 5) + r%4
    for (int c = wave; c < CG; c += WAVES) {
        const int m = lane & 31;
        if (m < M) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f32x4 g = red[0][c][0][q][lane], u = red[0][c][1][q][lane];
#pragma unroll
                for (int w = 1; w < WAVES; ++w) {
                    g += red[w][c][0][q][lane];
                    u += red[w][c][1][q][lane];
                }
                const int n = n0 + 32 * c + 8 * q + 4 * (lane >> 5);
                if (n < N) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = silu_f(g[e] * p.sg) * (u[e] * p.su);
                    u32x2 out;
                    out[0] = pack2(v[0], v[1]);
                    out[1] = pack2(v[2], v[3]);
                    *reinterpret_cast<u32x2*>(p.Y + (size_t)m * N + n) = out;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Row-major decode (swiglu_fused, M <= 64): the weight-streaming shape of
// decode_kernel on W1, W2 as they lie in memory ([K,N], N-contiguous).  Each
// workgroup owns CW output columns (64 or 32); its 4 waves take the 64-deep K
// blocks round-robin, UNROLL blocks at a time.  A wave brings each block's 64
// rows of its CW W1 and CW W2 columns into its own LDS slot with direct
// loads -- slot row k holds 2*CW columns, W1's then W2's, its 16-byte chunks
// XOR-swizzled by rmd_swz(k) -- and reads the MFMA weight fragments back with
// the transposing LDS read (8 K-consecutive values of one column per lane).
// The activations (MT tiles of 32 token rows, rows past M repeating row
// M - 1) are 16-byte loads straight to registers.  One
// v_mfma_f32_32x32x16_bf16 per (Gate|Up, 32-column piece, token tile, 16-deep
// step); the four per-wave fp32 sums are
// added in LDS in wave order 0..3, then SiLU(Gate) * Up in fp32 and bf16
// stores.  With CW = 32 a row of W1 (or W2) per block is half a cache line,
// the other half belonging to the neighbouring workgroup, which the XCD-aware
// block order places on the same XCD.
// ---------------------------------------------------------------------------
template <int CW>
__device__ __forceinline__ int rmd_swz(int k) {
    return CW == 64 ? ((k & 3) << 2) : ((k & 1) << 2);
}
template <int CW>
__device__ __forceinline__ int rmd_off(int k, int col) {
    return k * (2 * CW) + ((((col >> 3) ^ rmd_swz<CW>(k))) << 3) + (col & 7);
}

template <int CW, int UNROLL, int MT>
__global__ __launch_bounds__(256) void rowmajor_decode_kernel(FusedArgs p) {
    static_assert(CW == 64 || CW == 32, "64 or 32 columns per workgroup");
    static_assert(MT == 1 || MT == 2, "one or two 32-token tiles");
    constexpr int WAVES = 4;
    constexpr int NB = 2 * CW;               // LDS row: CW W1 columns, then CW W2 columns
    constexpr int CH = NB / 8;               // 16-byte chunks per LDS row
    constexpr int RPL = 64 / CH;             // LDS rows per 1 KiB direct load
    constexpr int KBLK = 64;                 // K rows per block
    constexpr int SLOT = KBLK * NB;          // elements per block slot
    constexpr int NJ = CW / 32;              // 32-column pieces per weight
    constexpr int RED = WAVES * 2 * NJ * MT * 4 * 64 * 4;   // floats of the per-wave sums
    constexpr int SW = WAVES * UNROLL * SLOT > 2 * RED ? WAVES * UNROLL * SLOT : 2 * RED;
    __shared__ __attribute__((aligned(16))) uint16_t sW[SW];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int M = p.M, K = p.K, N = p.N;
    const int n0 = xcd_remap(blockIdx.x, gridDim.x) * CW;
    const int KB = (K + KBLK - 1) / KBLK;
    uint16_t* const sWw = sW + wave * UNROLL * SLOT;

    // direct load i of a block writes slot rows RPL*i + lane / CH, physical
    // chunk lane % CH, i.e. logical chunk (lane % CH) ^ rmd_swz(row) (the row's
    // low bits are those of lane / CH): chunks below CH/2 are W1 columns
    // n0 + 8c, the rest W2 columns n0 + 8(c - CH/2)
    const int prow = lane / CH;
    const int lchunk = (lane % CH) ^ rmd_swz<CW>(prow);
    const int ncol = n0 + 8 * (lchunk % (CH / 2));
    const bool col_ok = ncol < N;
    const uint16_t* const wsrc = (lchunk >= CH / 2 ? p.W2 : p.W1) + (col_ok ? ncol : 0);
    // activation rows: token lane & 31 (rows past M repeat row M - 1), the
    // 8 k at 8 (lane >> 5) of each 16-deep step
    const uint16_t* arow[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) arow[t] = p.A + (size_t)min(t * 32 + (lane & 31), M - 1) * K + 8 * (lane >> 5);
    // transposing reads: lane l gets W[16kk + 8(l >> 5) + 0..7][column l & 31
    // of the 32-column piece]
    const int kr0 = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int cl = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    f32x16 acc[2][NJ][MT];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int t = 0; t < MT; ++t) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[g][j][t][r] = 0.0f;
                asm volatile("" : "+a"(acc[g][j][t]));   // opaque zeros, as in decode_kernel
            }

    for (int kb0 = wave; kb0 < KB; kb0 += WAVES * UNROLL) {
        // this wave's fragment reads of its slots (previous blocks) are done
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
        asm volatile("" ::: "memory");
        u32x4 av[UNROLL][4][MT];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kb = kb0 + u * WAVES;
            if (kb < KB) {
#pragma unroll
                for (int i = 0; i < KBLK / RPL; ++i) {
                    const int k = kb * KBLK + RPL * i + prow;
                    const uint16_t* src = (k < K && col_ok) ? wsrc + (size_t)k * N : g_zero_chunk;
                    dma16(src, sWw + u * SLOT + i * 512);
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int k = kb * KBLK + 16 * kk + 8 * (lane >> 5);
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        av[u][kk][t] = k < K ? ld16(arow[t] + (size_t)kb * KBLK + 16 * kk) : u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
        // the direct loads have landed in this wave's slots, and the activations
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 63));
        asm volatile("" ::: "memory");
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kb = kb0 + u * WAVES;
            if (kb < KB) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                    for (int g = 0; g < 2; ++g)
#pragma unroll
                        for (int j = 0; j < NJ; ++j) {
                            const int col = g * CW + j * 32 + cl;
                            const s16x4 lo = ds_read_tr16(sWw + u * SLOT + rmd_off<CW>(16 * kk + kr0, col));
                            const s16x4 hi = ds_read_tr16(sWw + u * SLOT + rmd_off<CW>(16 * kk + kr0 + 4, col));
                            const s16x4 both[2] = {lo, hi};
                            const bf16x8 w8 = __builtin_bit_cast(bf16x8, both);
#pragma unroll
                            for (int t = 0; t < MT; ++t)
                                acc[g][j][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                    w8, __builtin_bit_cast(bf16x8, av[u][kk][t]), acc[g][j][t], 0, 0, 0);
                        }
                }
            }
        }
    }

    // per-wave sums in 16-byte quarters, lane-contiguous, in the slots' LDS
    // once every wave is done with them: red[wave][g][j][t][q][lane]
    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(sW);
    auto ridx = [&](int w, int g, int j, int t, int q) {
        return ((((w * 2 + g) * NJ + j) * MT + t) * 4 + q) * 64 + lane;
    };
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    red[ridx(wave, g, j, t, q)] = f32x4{acc[g][j][t][4 * q], acc[g][j][t][4 * q + 1],
                                                        acc[g][j][t][4 * q + 2], acc[g][j][t][4 * q + 3]};
    __syncthreads();
    // wave w finishes the (32-column piece j, token tile t, row quad q)
    // pieces (j * MT + t) * 4 + q = w, w + 4, ...
#pragma unroll
    for (int x = 0; x < NJ * MT; ++x) {
        const int jtq = wave + 4 * x;
        const int q = jtq & 3, t = (jtq >> 2) % MT, j = (jtq >> 2) / MT;
        f32x4 g = red[ridx(0, 0, j, t, q)], u = red[ridx(0, 1, j, t, q)];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) {
            g += red[ridx(w, 0, j, t, q)];
            u += red[ridx(w, 1, j, t, q)];
        }
        const int m = t * 32 + (lane & 31);
        const int n = n0 + 32 * j + 8 * q + 4 * (lane >> 5);
        if (m < M && n < N) {
            u32x2 out;
            out[0] = pack2(silu_f(g[0]) * u[0], silu_f(g[1]) * u[1]);
            out[1] = pack2(silu_f(g[2]) * u[2], silu_f(g[3]) * u[3]);
            *reinterpret_cast<u32x2*>(p.Y + (size_t)m * N + n) = out;
        }
    }
}

// ---------------------------------------------------------------------------
// Weight pack / unpack (one-time transforms; see the packed layout in swiglu.h
// and packed_off above).  One thread per 16-byte packed chunk: 8 consecutive
// k of one packed row, at chunk index q = block * 2048 + ((group * 2 + half)
// * 64 + lane), where the chunk's row is group * 16 + lane % 16 and its first
// k is half * 32 + (lane / 16) * 8.
// ---------------------------------------------------------------------------
struct PackChunk {
    int n;          // output column (may be >= N: padding)
    bool up;        // Up weight (W2) rather than Gate (W1)
    int k0;         // first of the chunk's 8 consecutive k (may be >= K: padding)
};

// IL = false: per-tile [W1 | W2] (packed rows 0-127 the tile's W1 columns,
// 128-255 its W2 columns).  IL = true: column-granular interleave (packed row
// 2c the tile's W1 column c, row 2c + 1 its W2 column c).  SINGLE: one
// weight W (passed as W1) for a plain GEMM, 256 of its columns per packed
// tile: packed row p of tile jt is column jt*256 + p, so the dual kernels'
// "Gate" half of a tile holds columns jt*256 + 0..127 and the "Up" half
// jt*256 + 128..255.
template <bool IL, bool SINGLE = false>
__device__ __forceinline__ PackChunk pack_chunk(long long q, int KB) {
    const long long blk = q >> 11;                  // jt * KB + kb
    const int within = (int)(q & 2047);
    const int grp = within >> 7;
    const int half = (within >> 6) & 1;
    const int lane = within & 63;
    const int prow = grp * 16 + (lane & 15);
    const int kb = (int)(blk % KB);
    const int jt = (int)(blk / KB);
    PackChunk c;
    if constexpr (SINGLE) {
        c.up = false;
        c.n = jt * PACK_ROWS + prow;
    } else if constexpr (IL) {
        c.up = (prow & 1) != 0;
        c.n = jt * PACK_BN + (prow >> 1);
    } else {
        c.up = prow >= PACK_BN;
        c.n = jt * PACK_BN + (c.up ? prow - PACK_BN : prow);
    }
    c.k0 = kb * PACK_BK + half * 32 + (lane >> 4) * 8;
    return c;
}

template <bool IL, bool SINGLE = false>
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ W1,
                                                   const uint16_t* __restrict__ W2,
                                                   uint16_t* __restrict__ Wp, int K, int N,
                                                   int KB, long long nchunks) {
    const long long q = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= nchunks) return;
    const PackChunk c = pack_chunk<IL, SINGLE>(q, KB);
    const uint16_t* W = c.up ? W2 : W1;
    unsigned short v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int k = c.k0 + i;
        v[i] = (c.n < N && k < K) ? W[(size_t)k * N + c.n] : (unsigned short)0;
    }
    u32x4 out;
#pragma unroll
    for (int d = 0; d < 4; ++d) out[d] = (unsigned)v[2 * d] | ((unsigned)v[2 * d + 1] << 16);
    *reinterpret_cast<u32x4*>(Wp + q * 8) = out;
}

template <bool IL>
__global__ __launch_bounds__(256) void unpack_kernel(const uint16_t* __restrict__ Wp,
                                                     uint16_t* __restrict__ W1,
                                                     uint16_t* __restrict__ W2, int K, int N,
                                                     int KB, long long nchunks) {
    const long long q = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= nchunks) return;
    const PackChunk c = pack_chunk<IL>(q, KB);
    if (c.n >= N) return;
    uint16_t* W = c.up ? W2 : W1;
    const u32x4 in = *reinterpret_cast<const u32x4*>(Wp + q * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int k = c.k0 + i;
        if (k < K) W[(size_t)k * N + c.n] = (uint16_t)((in[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
    }
}

// ---------------------------------------------------------------------------
// FP8 weight pack: per (128-column tile jt, 128-k block kb) one 32 KiB block
// [32-row block rb][64-k step ks][half h][lane][16 bytes], holding packed row
// rb*32 + (lane & 31) (rows 0-127: W1 column jt*128 + row, 128-255: W2 column
// jt*128 + row - 128) at k = kb*128 + ks*64 + 32*(lane >> 5) + 16*h + 0..15:
// the lane order of a v_mfma_f32_32x32x64_f8f6f4 operand, each half of a
// lane's 32 bytes in its own 1 KiB run so that one wave load reads 1 KiB
// contiguous.  Padding is zero.  One thread per 16-byte piece (piece index =
// byte offset / 16).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_fp8_kernel(const uint8_t* __restrict__ W1,
                                                       const uint8_t* __restrict__ W2,
                                                       uint8_t* __restrict__ Wp, int K, int N, int KB,
                                                       long long npieces) {
    const long long q = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= npieces) return;
    const long long blk = q >> 11;
    const int within = (int)(q & 2047);
    const int rb = within >> 8, ks = (within >> 7) & 1, half = (within >> 6) & 1, lane = within & 63;
    const int kb = (int)(blk % KB), jt = (int)(blk / KB);
    const int prow = rb * 32 + (lane & 31);
    const bool up = prow >= PACK_BN;
    const int n = jt * PACK_BN + (up ? prow - PACK_BN : prow);
    const int k0 = kb * 128 + ks * 64 + 32 * (lane >> 5) + 16 * half;
    const uint8_t* W = up ? W2 : W1;
    u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const unsigned v = (n < N && k0 + i < K) ? W[(size_t)(k0 + i) * N + n] : 0u;
        out[i >> 2] |= v << (8 * (i & 3));
    }
    *reinterpret_cast<u32x4*>(Wp + q * 16) = out;
}

// ---------------------------------------------------------------------------
// Element-wise SwiGLU of the unfused pipeline: Y = bf16(SiLU(G) * U), fp32 math.
// 8 elements (16 bytes) per thread per step, grid-stride; scalar tail.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void silu_mul_kernel(const uint16_t* __restrict__ G,
                                                       const uint16_t* __restrict__ U,
                                                       uint16_t* __restrict__ Y, long long count) {
    const long long nvec = count / 8;
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long v = (long long)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
        const u32x4 g = *reinterpret_cast<const u32x4*>(G + v * 8);
        const u32x4 u = *reinterpret_cast<const u32x4*>(U + v * 8);
        u32x4 y;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float g0 = __builtin_bit_cast(float, g[d] << 16);
            const float g1 = __builtin_bit_cast(float, g[d] & 0xFFFF0000u);
            const float u0 = __builtin_bit_cast(float, u[d] << 16);
            const float u1 = __builtin_bit_cast(float, u[d] & 0xFFFF0000u);
            y[d] = pack2(silu_f(g0) * u0, silu_f(g1) * u1);
        }
        *reinterpret_cast<u32x4*>(Y + v * 8) = y;
    }
    const long long t = nvec * 8 + (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < count && blockIdx.x == 0 && (long long)threadIdx.x < count - nvec * 8) {
        const float g0 = __builtin_bit_cast(float, (unsigned)G[t] << 16);
        const float u0 = __builtin_bit_cast(float, (unsigned)U[t] << 16);
        Y[t] = (uint16_t)bf16_bits(silu_f(g0) * u0);
    }
}

}  // namespace swk
