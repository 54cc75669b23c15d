// Host side of libswiglu: argument validation, schedule choice and kernel
// launches behind the C ABI declared in include/swiglu.h.
//
// Every argument check runs before the first HIP call, so a rejected call has
// no effect on the device and the checks work on a machine without a GPU.
#include "swiglu.h"
#include "swiglu_probe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "fused_kernels.hpp"
#include "probe_kernels.hpp"

// Device scratch of swiglu_fused_packed_noalloc: the split-K partial sums of
// callers that cannot allocate.  One copy per device, held from the
// library's load until the process ends; every no-allocation call on a
// device shares it.  Host code never uses this name as an address: the
// device address comes from hipGetSymbolAddress (scratch_device_ptr below).
static __device__ __align__(256) unsigned char scratch[SWIGLU_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

swiglu_status hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return SWIGLU_ERR_HIP;
}

constexpr int64_t kMaxDim = (int64_t)1 << 30;   // every dimension fits int32 with room
constexpr int64_t kMaxK = (int64_t)1 << 22;     // 256 rows of activations stay below 2 GiB

bool log_enabled() {
    static int on = -1;
    if (on < 0) {
        const char* s = std::getenv("SWIGLU_LOG");
        on = (s && s[0] && s[0] != '0') ? 1 : 0;
    }
    return on == 1;
}

// ---------------------------------------------------------------------------
// argument checks (host only, no HIP calls)
// ---------------------------------------------------------------------------
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
    return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes};
}

bool overlap(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

swiglu_status check_shape(int64_t M, int64_t K, int64_t N) {
    if (M < 0 || K <= 0 || N <= 0) return SWIGLU_ERR_BAD_SHAPE;
    if (M > kMaxDim || K > kMaxDim || N > kMaxDim) return SWIGLU_ERR_BAD_SHAPE;
    if (M * N > ((int64_t)1 << 40) || K * N > ((int64_t)1 << 40) || M * K > ((int64_t)1 << 40))
        return SWIGLU_ERR_BAD_SHAPE;
    if ((K % 8) != 0 || (N % 8) != 0) return SWIGLU_ERR_UNSUPPORTED_SHAPE;
    if (K > kMaxK) return SWIGLU_ERR_UNSUPPORTED_SHAPE;
    return SWIGLU_OK;
}

// The streaming kernel keeps each activation address as a 32-bit byte offset
// from the stage base (row * K * bytes).  Calls whose activation slice would
// reach 2 GiB are split into row chunks of at most this many rows (a multiple
// of 256), each with A and Y advanced to its first row.
int64_t stream_rows_limit(int64_t K, int elem_bytes) {
    const int64_t rows = (((int64_t)1 << 31) / (K * elem_bytes)) / 256 * 256;
    return rows >= 256 ? rows : 256;
}

// Equal chunks (multiples of 256 rows) of at most `limit` rows covering M.
int64_t balanced_chunk(int64_t M, int64_t limit) {
    const int64_t n = (M + limit - 1) / limit;
    const int64_t per = (M + n - 1) / n;
    return std::min(limit, (per + 255) / 256 * 256);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// FP8 operands: K a multiple of 16 (16-byte activation rows), packed weights
// in 32 KiB blocks per (128 columns, 128 k)
swiglu_status check_shape_fp8(int64_t M, int64_t K, int64_t N) {
    const swiglu_status st = check_shape(M, K, N);
    if (st != SWIGLU_OK) return st;
    return (K % 16) != 0 ? SWIGLU_ERR_UNSUPPORTED_SHAPE : SWIGLU_OK;
}

int64_t packed_bytes_fp8(int64_t K, int64_t N) { return ceil_div(N, swk::PACK_BN) * ceil_div(K, 128) * 32768; }

int64_t packed_elems(int64_t K, int64_t N) {
    return ceil_div(N, swk::PACK_BN) * ceil_div(K, swk::PACK_BK) * swk::PACK_ROWS * swk::PACK_BK;
}

// Single-weight pack of W [K,N] for the plain GEMM: 256 columns per packed
// tile (the dual kernels' Gate and Up halves), so ceil(N/256) tiles whose
// 128-column "output" width n_tiled the dual schedules are planned on.
int64_t gemm_packed_elems(int64_t K, int64_t N) {
    return ceil_div(N, swk::PACK_ROWS) * ceil_div(K, swk::PACK_BK) * swk::PACK_ROWS * swk::PACK_BK;
}
int64_t gemm_tiled_cols(int64_t N) { return ceil_div(N, swk::PACK_ROWS) * swk::PACK_BN; }

// ---------------------------------------------------------------------------
// device facts
// ---------------------------------------------------------------------------
int cu_count_now() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}

// Device address of `scratch` on the current device: looked up once per
// device (with that device current) and kept; each device holds its own copy
// of the array at its own address.
hipError_t scratch_device_ptr(void** out) {
    static std::mutex mu;
    static void* ptrs[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// kernel configurations
// ---------------------------------------------------------------------------
// Output tile for a token count and schedule.  M <= 64 (forced data-parallel
// or split-K; AUTO uses the decode kernel there): 32/64-row register-path
// tiles.  Split-K above that: 128 x 64 tiles (two workgroups fit a CU, and a
// narrow tile gives more tiles to split).  Data-parallel: 128 x 128 up to
// 2048 tokens, then 256 x 128 (each wave 128 rows x 64 columns of Gate and Up).
struct TileCfg {
    int BM, BN;
};

// Split-K keeps small row tiles for small M; the data-parallel schedule is
// the streaming kernel at every M (one row of 128-row tiles for M <= 128, on
// the panel schedule when its column tiles leave CUs idle).
// Data-parallel tiles: 256 x 128 (persistent, with the 128-row tail of the
// mixed launch) above 512 rows, and from 385 rows when the last row tile is
// at least three quarters full and the 256-row grid fills the CUs; else
// 128 x 128 (measured against 128-row tiles everywhere up to 2048 rows:
// 7B width M=512 152 -> 141 us, M=768 201 -> 178 us, M=2048 479 -> 422 us,
// 72B width M=1024 865 -> 751 us; 0.5B width M=1024 29.4 -> 25.0 us).
TileCfg packed_tile_for(int64_t M, int variant, int64_t N, int cus) {
    if (variant == SWIGLU_VARIANT_SPLIT_K) {
        if (M <= 32) return {32, 128};
        if (M <= 64) return {64, 128};
        return {128, 128};
    }
    if (M <= 512) {
        if (M > 384 && (M % 256 == 0 || M % 256 >= 192) && ceil_div(M, 256) * ceil_div(N, 128) >= cus)
            return {256, 128};
        return {128, 128};
    }
    return {256, 128};
}

// workgroups per CU the split count aims for
constexpr int kSplitWavesPerCu = 2;

// Split-K above this many output tiles is pointless (the tiles alone fill
// the device many times over).
constexpr int kMaxSplitTiles = 16384;

struct Plan {
    TileCfg t;
    int tiles_m, tiles_n, tiles;
    int tail_ntiles;   // data-parallel 256-row tiles: last column tiles run as 128x128 tiles
    int panels;        // data-parallel, one 128-row tile: 32-column panels spread over the CUs
    int splits, kb_per_split, KB;
    int variant;   // resolved: DATA_PARALLEL, SPLIT_K or DECODE
    int decode_mt; // DECODE: 16-token tiles per workgroup
    int cus;       // compute units the plan was made for
};

constexpr int kDecodeMaxM = 64;
bool variant_known(int v) { return v >= SWIGLU_VARIANT_AUTO && v <= SWIGLU_VARIANT_SEQUENTIAL; }

Plan make_plan(int64_t M, int64_t K, int64_t N, int variant, int cus) {
    Plan p{};
    if (cus <= 0) cus = 256;
    p.cus = cus;
    p.KB = (int)ceil_div(K, swk::BK);
    int v = variant;
    int auto_split_cap = 0;   // AUTO's split-K: most splits worth their partial-sum traffic
    if (v == SWIGLU_VARIANT_AUTO) {
        // Decode up to 32 rows; from 33 to 64 rows only while the weight
        // panels cannot fill the CUs (a small product, where the decode
        // kernel's single pass wins), otherwise the panel schedule streams
        // the weights faster (measured: 7B M=64 57 us against 76 us).
        const int64_t panels = 4 * ceil_div(N, swk::PACK_BN);
        if (M <= 32 || (M <= kDecodeMaxM && panels < cus)) {
            v = SWIGLU_VARIANT_DECODE;
        } else if (M <= kDecodeMaxM) {
            v = SWIGLU_VARIANT_DATA_PARALLEL;
        } else {
            // Split-K writes and re-reads S fp32 partial sums of Gate and Up,
            // 16*S*M*N bytes against the 4*K*N bytes of weights: worth it only
            // while the data-parallel tiles leave most CUs idle, and with at
            // most K / (16 M) splits (extra traffic <= a quarter of the
            // weights).  A data-parallel grid that fills half the CUs streams
            // the weights faster than split-K does.
            const TileCfg dp = packed_tile_for(M, SWIGLU_VARIANT_DATA_PARALLEL, N, cus);
            const int64_t dp_tiles = ceil_div(M, dp.BM) * ceil_div(N, dp.BN);
            auto_split_cap = (int)std::min<int64_t>(K / (16 * M), 1 << 20);
            v = (2 * dp_tiles >= cus || p.KB < 4 || auto_split_cap < 2) ? SWIGLU_VARIANT_DATA_PARALLEL
                                                                         : SWIGLU_VARIANT_SPLIT_K;
        }
    }
    p.variant = v;
    p.decode_mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    // the sequential order runs on the data-parallel tiles (no panel schedule)
    const bool dp_tiles = v == SWIGLU_VARIANT_DATA_PARALLEL || v == SWIGLU_VARIANT_SEQUENTIAL;
    p.t = packed_tile_for(M, dp_tiles ? SWIGLU_VARIANT_DATA_PARALLEL : v, N, cus);
    p.tiles_m = (int)ceil_div(M, p.t.BM);
    p.tiles_n = (int)ceil_div(N, p.t.BN);
    p.tiles = p.tiles_m * p.tiles_n;
    // Wave quantisation of the 256 x 128 schedule: when the last round of
    // tiles would leave most CUs idle, the column tiles that make up that round
    // run afterwards as 128 x 128 tiles (twice as many, half the work each).
    p.tail_ntiles = 0;
    if (dp_tiles && p.t.BM == 256 && p.tiles > cus) {
        const int rem = p.tiles % cus;
        if (rem > 0 && rem * 10 <= cus * 6) {
            const int nt = (int)ceil_div(rem, p.tiles_m);
            if (nt < p.tiles_n) p.tail_ntiles = nt;
        }
    }
    // One row of 128-row tiles that leaves CUs idle: the 32-column weight
    // panels (four per tile) are spread evenly over the CUs instead, so every
    // CU streams weights.
    p.panels = 0;
    if (v == SWIGLU_VARIANT_DATA_PARALLEL && p.t.BM == 128 && p.tiles_m == 1 && p.tiles_n < cus)
        p.panels = 4 * p.tiles_n;
    if (v == SWIGLU_VARIANT_SPLIT_K && p.tiles <= kMaxSplitTiles) {
        // about kSplitWavesPerCu workgroups per CU, at least two K blocks per split
        int s = (int)ceil_div((int64_t)kSplitWavesPerCu * cus, p.tiles);
        if (auto_split_cap > 0) s = std::min(s, auto_split_cap);
        s = std::max(1, std::min(s, p.KB / 2 > 0 ? p.KB / 2 : 1));
        p.kb_per_split = (int)ceil_div(p.KB, s);
        p.splits = (int)ceil_div(p.KB, p.kb_per_split);
    } else {
        p.splits = 1;
        p.kb_per_split = p.KB;
    }
    return p;
}

// Split-K workspace: fp32 Gate and Up partial sums, [split][M][2N].
size_t split_workspace_bytes(const Plan& p, int64_t M, int64_t N) {
    if (p.variant != SWIGLU_VARIANT_SPLIT_K || p.splits <= 1) return 0;
    return (size_t)p.splits * (size_t)M * 2 * (size_t)N * sizeof(float);
}

template <int BM, int BN, int WM, int WN, bool DUAL, bool PACKED, bool SPLIT>
hipError_t launch_tile(const swk::FusedArgs& a, int grid, hipStream_t s) {
    const void* fn = reinterpret_cast<const void*>(&swk::fused_tile_kernel<BM, BN, WM, WN, DUAL, PACKED, SPLIT>);
    swk::FusedArgs args = a;
    void* kargs[] = {&args};
    return hipLaunchKernel(fn, dim3(grid), dim3(64 * WM * WN), kargs, 0, s);
}

// n_tiled: the packed weights' output columns (N for the fused product; 128
// per packed tile for the single-weight GEMM).  HALF: one workgroup per
// (column groups, weight half), twice the grid.
template <int MT, int CG, int UNROLL, bool GEMM = false, bool HALF = false, bool LDSA = false>
hipError_t launch_decode(const swk::DecodeArgs& a, int64_t n_tiled, hipStream_t s) {
    const void* fn = reinterpret_cast<const void*>(&swk::decode_kernel<MT, CG, UNROLL, GEMM, HALF, LDSA>);
    swk::DecodeArgs args = a;
    void* kargs[] = {&args};
    return hipLaunchKernel(fn, dim3((unsigned)(ceil_div(n_tiled, 16 * CG) * (HALF ? 2 : 1))), dim3(256), kargs, 0,
                           s);
}

template <int BM, int BN, int WM, int WN, bool SPLIT, int WSRC = swk::W_PACKED>
hipError_t launch_prefill(const swk::FusedArgs& a, int grid, hipStream_t s) {
    const void* fn = reinterpret_cast<const void*>(&swk::fused_prefill_kernel<BM, BN, WM, WN, SPLIT, WSRC>);
    swk::FusedArgs args = a;
    void* kargs[] = {&args};
    return hipLaunchKernel(fn, dim3(grid), dim3(64 * WM * WN), kargs, 0, s);
}

// `total` work items (tiles, or tile x K split) on `grid` <= total workgroups;
// each workgroup takes items b, b + grid, ...
template <int BM, bool SPLIT, bool PANELS = false, bool IL = false, bool F8 = false, bool SEQ = false,
          bool GEMM = false>
hipError_t launch_stream(const swk::FusedArgs& a, int total, int grid, hipStream_t s) {
    const bool ragged = (a.K % (F8 ? 128 : swk::BK)) != 0;
    const void* fn =
        ragged ? reinterpret_cast<const void*>(&swk::stream_prefill_kernel<BM, SPLIT, true, PANELS, IL, F8, SEQ, GEMM>)
               : reinterpret_cast<const void*>(&swk::stream_prefill_kernel<BM, SPLIT, false, PANELS, IL, F8, SEQ, GEMM>);
    swk::FusedArgs args = a;
    void* kargs[] = {&args, &total};
    return hipLaunchKernel(fn, dim3(grid), dim3(256), kargs, 0, s);
}

// The data-parallel streaming schedules (128- or 256-row tiles, the panel
// schedule, the mixed 256/128-row launch) on either weight layout; SEQ: the
// sequential Gate-then-Up order (per-tile layout, no panel schedule).
template <bool IL, bool F8 = false, bool SEQ = false, bool GEMM = false>
hipError_t launch_stream_dp(const swk::FusedArgs& a, const Plan& p, hipStream_t s) {
    const int grid = p.tiles;
    if (p.t.BM == 128) {
        if constexpr (SEQ) return launch_stream<128, false, false, false, false, true>(a, grid, grid, s);
        if constexpr (!GEMM && !IL) {
            // two rows of 128-row tiles that leave CUs idle on a wide product:
            // one row of 256-row tiles on the panel schedule instead, the
            // weights streamed once (7B width M=192 98.6 -> 84.2 us, 72B width
            // M=256 259 -> 226 us; FP8 72B width M=192 144 -> 127 us; the 0.5B
            // width's few short panels lose, 13.5 against 24 us, and keep the
            // 128-row tiles, as does the interleaved layout, 95 against 107 us
            // at the 7B width)
            if (p.tiles_m == 2 && a.M <= 256 && p.tiles_n < p.cus && 2 * p.tiles_n >= p.cus) {
                swk::FusedArgs pa = a;
                pa.tiles_m = 1;
                pa.panels = 4 * p.tiles_n;
                const int g = std::min(pa.panels, p.cus);
                return launch_stream<256, false, true, IL, F8, false, false>(pa, g, g, s);
            }
        }
        if (p.panels > 0) {
            // the single-weight GEMM's units are half-panels (one weight half
            // each), as long as no workgroup gets more than its 4 waves
            swk::FusedArgs pa = a;
            pa.panels = GEMM ? 2 * p.panels : p.panels;
            if (pa.panels <= 4 * p.cus) {
                const int g = std::min(pa.panels, p.cus);
                return launch_stream<128, false, true, IL, F8, false, GEMM>(pa, g, g, s);
            }
        }
        return launch_stream<128, false, false, IL, F8, false, GEMM>(a, grid, grid, s);
    }
    // one workgroup per CU works through the 256-row tiles
    if (p.tail_ntiles == 0)
        return launch_stream<256, false, false, IL, F8, SEQ, GEMM>(a, grid, std::min(grid, p.cus), s);
    // one launch: the 256-row tiles of the first column tiles, then
    // the last tail_ntiles column tiles as 128-row tiles
    swk::FusedArgs big = a, tail = a;
    big.tiles_n = p.tiles_n - p.tail_ntiles;
    tail.tiles_m = (int)ceil_div(a.M, 128);
    tail.tiles_n = p.tail_ntiles;
    tail.n_tile0 = big.tiles_n;
    int n_big = big.tiles_m * big.tiles_n;
    int n_pers = std::min(n_big, p.cus);
    const int grid_all = n_pers + tail.tiles_m * tail.tiles_n;
    const bool ragged = (a.K % (F8 ? 128 : swk::BK)) != 0;
    const void* fn = ragged
                         ? reinterpret_cast<const void*>(&swk::stream_prefill_mixed_kernel<true, IL, F8, SEQ, GEMM>)
                         : reinterpret_cast<const void*>(&swk::stream_prefill_mixed_kernel<false, IL, F8, SEQ, GEMM>);
    void* kargs[] = {&big, &tail, &n_pers, &n_big};
    return hipLaunchKernel(fn, dim3(grid_all), dim3(256), kargs, 0, s);
}

// The data-parallel streaming plan (any M).
Plan stream_dp_plan(int64_t M, int64_t K, int64_t N, int cus) {
    return make_plan(M, K, N, SWIGLU_VARIANT_DATA_PARALLEL, cus);
}

// FP8 decode (M <= 32): groups of 32 output columns per workgroup (CG) and
// 128-k blocks in flight per wave (UNROLL).
constexpr int64_t kDecodeFp8MaxM = 32;

template <int CG, int UNROLL, bool LDSA = false>
hipError_t launch_decode_fp8_cfg(const swk::FusedArgs& a, hipStream_t s) {
    swk::FusedArgs args = a;
    void* kargs[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(&swk::decode_fp8_kernel<CG, UNROLL, LDSA>),
                           dim3((unsigned)ceil_div(a.N, 32 * CG)), dim3(256), kargs, 0, s);
}

// Measured (7B width M=1: <1,2> 26.1 us against 26.7-32.4 for the others;
// 72B width M=32: <4,1> 73.7 us against 78.6-112.8): four groups per
// workgroup when that grid still gives about one workgroup per CU, else one
// group and two blocks in flight (two workgroups per CU), its activations
// staged through LDS (L) from 9 rows on (7B width M=16 / 32: <1,2,L> 26.3 /
// 26.6 us against 27.0 / 31.3; M=1: 26.4 against 26.1; with <4,1> at 72B
// M=32 78.8 against 73.7).
hipError_t launch_decode_fp8(const swk::FusedArgs& a, int cus, hipStream_t s) {
    const int64_t wide = ceil_div(a.N, 128);
    if (wide <= cus && 4 * wide >= 3 * (int64_t)cus) return launch_decode_fp8_cfg<4, 1>(a, s);
    return a.M > 8 ? launch_decode_fp8_cfg<1, 2, true>(a, s) : launch_decode_fp8_cfg<1, 2>(a, s);
}

// The decode kernel's configuration for a plan: column groups per workgroup
// (CG) and K blocks in flight per wave (UNROLL), measured on this chip: wider
// groups read each activation fragment for more weight bytes and stream
// longer contiguous runs of the packed blocks; they pay off for long K (>= 96
// blocks), or from 17 tokens on, as long as the grid still gives about one
// workgroup per CU.  Measured (us, one call, inputs rotated past the
// last-level cache):
//   K=3584 N=18944 M=1 / 16: <1,1,8> 42.9 / 45.8, <1,1,4> 43.0 / 46.3, <1,2,4> 46.1 / 47.5
//   K=8192 N=29568 M=1 / 16: <1,8,2> 138.4 / 138.0, the same with L 142.3 / 142.0
//   K=8192 N=29568 M=32: <2,8,1> 140.2, <2,4,1> 147.3, <2,2,2> 170.4
//   K=3584 N=18944 M=32: <2,8,1> 52.2, <2,2,2> 54.7, <2,4,1> 61.8
//   K=896 N=4864 M=64: <4,2,1> 9.9, <4,2,2> 10.5, <4,1,1> 11.8
// With the activations staged through LDS (L = LDSA: one full-line load
// per 8 rows instead of a half-line per row and fragment), which pays once
// there are more than 8 distinct rows and the group is narrow:
//   K=3584 N=18944 M=16: <1,1,8,L> 44.1-44.4 against 45.9-46.3; M=1 / 4 / 8: no gain
//   K=896 N=4864 M=64: <4,2,1,L> 9.33-9.38 against 9.82-9.90; M=32 with 8 groups: 55.6 against 52.0
// n_tiled: the packed weights' output columns.
hipError_t launch_decode_cfg(const swk::DecodeArgs& d, int64_t n_tiled, const Plan& p, hipStream_t s) {
    const bool long_k = p.KB >= 96;
    const int64_t wg64 = ceil_div(n_tiled, 64), wg128 = ceil_div(n_tiled, 128);
    switch (p.decode_mt) {
        case 1:
            if (long_k && 4 * wg128 >= 3 * p.cus) return launch_decode<1, 8, 2>(d, n_tiled, s);
            return d.M > 8 ? launch_decode<1, 1, 8, false, false, true>(d, n_tiled, s)
                           : launch_decode<1, 1, 8>(d, n_tiled, s);
        case 2:
            if (2 * wg128 >= p.cus) return launch_decode<2, 8, 1>(d, n_tiled, s);
            return (long_k && 4 * wg64 >= 3 * p.cus) ? launch_decode<2, 4, 1>(d, n_tiled, s)
                                                    : launch_decode<2, 2, 2>(d, n_tiled, s);
        default:
            return (long_k && 4 * wg64 >= 3 * p.cus) ? launch_decode<4, 4, 1>(d, n_tiled, s)
                                                    : launch_decode<4, 2, 1, false, false, true>(d, n_tiled, s);
    }
}

// The same for the single-weight GEMM (n_tiled = 128 per 256-column packed
// tile), where a workgroup may take one weight half (HALF): half the bytes per
// workgroup and twice the grid.  Measured on this chip (us, one call, inputs
// rotated past the last-level cache):
//   K=3584 N=18944 M=1: <1,1,14,H> 22.6, <1,1,8,H> 23.2, <1,1,8> 23.9
//   K=3584 N=18944 M=16: <1,1,8> 26.7, <1,1,8,H> 29.7
//   K=8192 N=29568 M=1 / 16: <1,4,4,H> 79.5 / 78.6, <1,1,8> 93.7 / 99.0
//   K=18944 N=3584 M=1 / 16: <1,1,14,H> 23.3 / 31.3, <1,1,8,H> 23.6 / 30.8, <1,1,8> 30.6 / 42.6
//   K=8192 N=29568 M=32: <2,8,1,H> 73.3, <2,4,1> 76.1, <2,2,2,H> 113.4
//   K=29568 N=8192 M=32: <2,2,2,H> 92.8, <2,2,2> 129.3, <2,4,1,H> 123.9
//   K=896 N=4864 M=64: <4,2,1,H> 8.0, <4,2,1> 9.5
//   K=4864 N=896 M=64: <4,1,1,H> 21.8, <4,2,1,H> 24.4, <4,2,1> 31.8
// and with the activations staged through LDS (L, as for the fused product):
//   K=3584 N=18944 M=16: <1,1,8,H,L> 25.2, <1,1,8,L> 26.3, <1,1,8> 27.0
//   K=18944 N=3584 M=16: <1,1,8,H,L> 27.4, <1,1,8,H> 30.9; K=4864 N=896 M=16: 7.9 against 9.5
//   K=8192 N=29568 M=16: <1,4,4,H> 77.7, <1,4,4,H,L> 79.5
//   K=896 N=4864 M=64: <4,1,1,H,L> 6.8, <4,2,1,H,L> 7.1, <4,2,1,H> 8.0
//   K=4864 N=896 M=64: <4,1,1,H,L> 17.6, <4,1,1,H> 21.8
// i.e. halves whenever the whole-pair grid leaves CUs short of work, the
// deepest per-wave prefetch the registers allow at one or two tokens' rows,
// and staged activations for narrow groups from 9 rows on.
hipError_t launch_decode_gemm(const swk::DecodeArgs& d, int64_t n_tiled, const Plan& p, hipStream_t s) {
    const bool long_k = p.KB >= 96;
    const int64_t wg64 = ceil_div(n_tiled, 64);
    switch (p.decode_mt) {
        case 1:
            if (long_k && 2 * wg64 >= p.cus) return launch_decode<1, 4, 4, true, true>(d, n_tiled, s);
            if (d.M <= 8) return launch_decode<1, 1, 14, true, true>(d, n_tiled, s);
            return launch_decode<1, 1, 8, true, true, true>(d, n_tiled, s);
        case 2:
            if (long_k) {
                return 4 * wg64 >= 3 * p.cus ? launch_decode<2, 8, 1, true, true>(d, n_tiled, s)
                                             : launch_decode<2, 2, 2, true, true>(d, n_tiled, s);
            }
            return 2 * ceil_div(n_tiled, 128) >= p.cus ? launch_decode<2, 8, 1, true>(d, n_tiled, s)
                                                       : launch_decode<2, 2, 2, true>(d, n_tiled, s);
        default:
            if (long_k && 4 * wg64 >= 3 * p.cus) return launch_decode<4, 4, 1, true>(d, n_tiled, s);
            return launch_decode<4, 1, 1, true, true, true>(d, n_tiled, s);
    }
}

hipError_t launch_packed(const swk::FusedArgs& a, const Plan& p, hipStream_t s) {
    if (p.variant == SWIGLU_VARIANT_SEQUENTIAL) return launch_stream_dp<false, false, true>(a, p, s);
    if (p.variant == SWIGLU_VARIANT_DECODE) {
        swk::DecodeArgs d{};
        d.A = a.A; d.Wp = a.W1; d.Y = a.Y;
        d.M = a.M; d.K = a.K; d.N = a.N; d.KB = a.KB;
        return launch_decode_cfg(d, a.N, p, s);
    }
    const int grid = p.tiles * p.splits;
    const bool split = p.splits > 1;
    switch (p.t.BM) {
        case 32:
            return split ? launch_tile<32, 128, 1, 4, true, true, true>(a, grid, s)
                         : launch_tile<32, 128, 1, 4, true, true, false>(a, grid, s);
        case 64:
            return split ? launch_tile<64, 128, 2, 2, true, true, true>(a, grid, s)
                         : launch_tile<64, 128, 2, 2, true, true, false>(a, grid, s);
        case 128:
            if (split) return launch_stream<128, true>(a, grid, grid, s);
            return launch_stream_dp<false>(a, p, s);
        default:
            if (split) return launch_stream<256, true>(a, grid, grid, s);
            return launch_stream_dp<false>(a, p, s);
    }
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

int swiglu_abi_version(void) { return SWIGLU_ABI_VERSION; }

const char* swiglu_status_str(int s) {
    switch (s) {
        case SWIGLU_OK: return "ok";
        case SWIGLU_ERR_NULL_POINTER: return "null pointer";
        case SWIGLU_ERR_BAD_SHAPE: return "bad shape";
        case SWIGLU_ERR_UNSUPPORTED_SHAPE: return "unsupported shape (K and N must be multiples of 8)";
        case SWIGLU_ERR_MISALIGNED: return "pointer not 16-byte aligned";
        case SWIGLU_ERR_ALIASING: return "output overlaps another operand";
        case SWIGLU_ERR_WORKSPACE: return "workspace missing or too small";
        case SWIGLU_ERR_BAD_VARIANT: return "unknown variant";
        case SWIGLU_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

int swiglu_last_hip_error(void) { return g_last_hip_error; }

int swiglu_device_cu_count(void) { return cu_count_now(); }

size_t swiglu_packed_bytes(int64_t K, int64_t N) {
    if (check_shape(0, K, N) != SWIGLU_OK) return 0;
    return (size_t)packed_elems(K, N) * sizeof(swiglu_bf16);
}

}  // extern "C"

namespace {

template <bool IL>
swiglu_status pack_impl(const swiglu_bf16* W1, const swiglu_bf16* W2, swiglu_bf16* Wp, int64_t K, int64_t N,
                        void* stream) {
    swiglu_status st = check_shape(0, K, N);
    if (st != SWIGLU_OK) return st;
    if (!W1 || !W2 || !Wp) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(W1) || !aligned16(W2) || !aligned16(Wp)) return SWIGLU_ERR_MISALIGNED;
    const Range out = range_of(Wp, packed_elems(K, N) * 2);
    if (overlap(out, range_of(W1, K * N * 2)) || overlap(out, range_of(W2, K * N * 2)))
        return SWIGLU_ERR_ALIASING;
    const long long nchunks = (long long)packed_elems(K, N) / 8;
    const int KB = (int)ceil_div(K, swk::PACK_BK);
    int Ki = (int)K, Ni = (int)N;
    void* args[] = {(void*)&W1, (void*)&W2, (void*)&Wp, &Ki, &Ni, (void*)&KB, (void*)&nchunks};
    const dim3 grid((unsigned)ceil_div(nchunks, 256));
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&swk::pack_kernel<IL>), grid, dim3(256),
                                   args, 0, (hipStream_t)stream);
    return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
}

template <bool IL>
swiglu_status unpack_impl(const swiglu_bf16* Wp, swiglu_bf16* W1, swiglu_bf16* W2, int64_t K, int64_t N,
                          void* stream) {
    swiglu_status st = check_shape(0, K, N);
    if (st != SWIGLU_OK) return st;
    if (!W1 || !W2 || !Wp) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(W1) || !aligned16(W2) || !aligned16(Wp)) return SWIGLU_ERR_MISALIGNED;
    const Range in = range_of(Wp, packed_elems(K, N) * 2);
    const Range o1 = range_of(W1, K * N * 2), o2 = range_of(W2, K * N * 2);
    if (overlap(in, o1) || overlap(in, o2) || overlap(o1, o2)) return SWIGLU_ERR_ALIASING;
    const long long nchunks = (long long)packed_elems(K, N) / 8;
    const int KB = (int)ceil_div(K, swk::PACK_BK);
    int Ki = (int)K, Ni = (int)N;
    void* args[] = {(void*)&Wp, (void*)&W1, (void*)&W2, &Ki, &Ni, (void*)&KB, (void*)&nchunks};
    const dim3 grid((unsigned)ceil_div(nchunks, 256));
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&swk::unpack_kernel<IL>), grid, dim3(256),
                                   args, 0, (hipStream_t)stream);
    return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
}

}  // namespace

extern "C" {

swiglu_status swiglu_pack_weights(const swiglu_bf16* W1, const swiglu_bf16* W2, swiglu_bf16* Wp,
                                  int64_t K, int64_t N, void* stream) {
    return pack_impl<false>(W1, W2, Wp, K, N, stream);
}

swiglu_status swiglu_unpack_weights(const swiglu_bf16* Wp, swiglu_bf16* W1, swiglu_bf16* W2,
                                    int64_t K, int64_t N, void* stream) {
    return unpack_impl<false>(Wp, W1, W2, K, N, stream);
}

swiglu_status swiglu_pack_weights_interleaved(const swiglu_bf16* W1, const swiglu_bf16* W2, swiglu_bf16* Wp,
                                              int64_t K, int64_t N, void* stream) {
    return pack_impl<true>(W1, W2, Wp, K, N, stream);
}

swiglu_status swiglu_unpack_weights_interleaved(const swiglu_bf16* Wp, swiglu_bf16* W1, swiglu_bf16* W2,
                                                int64_t K, int64_t N, void* stream) {
    return unpack_impl<true>(Wp, W1, W2, K, N, stream);
}

swiglu_status swiglu_fused_packed_interleaved(const swiglu_bf16* A, const swiglu_bf16* Wp, swiglu_bf16* Y,
                                              int64_t M, int64_t K, int64_t N, void* stream) {
    swiglu_status st = check_shape(M, K, N);
    if (st != SWIGLU_OK) return st;
    if (M == 0) return SWIGLU_OK;
    if (!A || !Wp || !Y) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(A) || !aligned16(Wp) || !aligned16(Y)) return SWIGLU_ERR_MISALIGNED;
    const Range y = range_of(Y, M * N * 2);
    if (overlap(y, range_of(A, M * K * 2)) || overlap(y, range_of(Wp, packed_elems(K, N) * 2)))
        return SWIGLU_ERR_ALIASING;
    if (M > stream_rows_limit(K, 2)) {
        const int64_t rows = balanced_chunk(M, stream_rows_limit(K, 2));
        for (int64_t m0 = 0; m0 < M; m0 += rows) {
            st = swiglu_fused_packed_interleaved(A + m0 * K, Wp, Y + m0 * N, std::min(rows, M - m0), K, N, stream);
            if (st != SWIGLU_OK) return st;
        }
        return SWIGLU_OK;
    }
    const Plan p = stream_dp_plan(M, K, N, cu_count_now());
    swk::FusedArgs a{};
    a.A = A; a.W1 = Wp; a.W2 = nullptr; a.Y = Y;
    a.M = (int)M; a.K = (int)K; a.N = (int)N;
    a.tiles_m = p.tiles_m; a.tiles_n = p.tiles_n;
    a.splits = 1; a.kb_per_split = p.KB; a.KB = p.KB;
    const hipError_t e = launch_stream_dp<true>(a, p, (hipStream_t)stream);
    return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
}

size_t swiglu_packed_bytes_fp8(int64_t K, int64_t N) {
    if (check_shape_fp8(0, K, N) != SWIGLU_OK) return 0;
    return (size_t)packed_bytes_fp8(K, N);
}

swiglu_status swiglu_pack_weights_fp8(const uint8_t* W1, const uint8_t* W2, uint8_t* Wp, int64_t K, int64_t N,
                                      void* stream) {
    swiglu_status st = check_shape_fp8(0, K, N);
    if (st != SWIGLU_OK) return st;
    if (!W1 || !W2 || !Wp) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(W1) || !aligned16(W2) || !aligned16(Wp)) return SWIGLU_ERR_MISALIGNED;
    const Range out = range_of(Wp, packed_bytes_fp8(K, N));
    if (overlap(out, range_of(W1, K * N)) || overlap(out, range_of(W2, K * N))) return SWIGLU_ERR_ALIASING;
    const long long npieces = (long long)packed_bytes_fp8(K, N) / 16;
    const int KB = (int)ceil_div(K, 128);
    int Ki = (int)K, Ni = (int)N;
    void* args[] = {(void*)&W1, (void*)&W2, (void*)&Wp, &Ki, &Ni, (void*)&KB, (void*)&npieces};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&swk::pack_fp8_kernel),
                                   dim3((unsigned)ceil_div(npieces, 256)), dim3(256), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
}

swiglu_status swiglu_fused_packed_fp8(const uint8_t* A, const uint8_t* Wp, swiglu_bf16* Y, int64_t M, int64_t K,
                                      int64_t N, float sg, float su, void* stream) {
    swiglu_status st = check_shape_fp8(M, K, N);
    if (st != SWIGLU_OK) return st;
    if (M == 0) return SWIGLU_OK;
    if (!A || !Wp || !Y) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(A) || !aligned16(Wp) || !aligned16(Y)) return SWIGLU_ERR_MISALIGNED;
    const Range y = range_of(Y, M * N * 2);
    if (overlap(y, range_of(A, M * K)) || overlap(y, range_of(Wp, packed_bytes_fp8(K, N))))
        return SWIGLU_ERR_ALIASING;
    if (M > stream_rows_limit(K, 1)) {
        const int64_t rows = balanced_chunk(M, stream_rows_limit(K, 1));
        for (int64_t m0 = 0; m0 < M; m0 += rows) {
            st = swiglu_fused_packed_fp8(A + m0 * K, Wp, Y + m0 * N, std::min(rows, M - m0), K, N, sg, su, stream);
            if (st != SWIGLU_OK) return st;
        }
        return SWIGLU_OK;
    }
    swk::FusedArgs a{};
    a.A = reinterpret_cast<const uint16_t*>(A);
    a.W1 = reinterpret_cast<const uint16_t*>(Wp);
    a.W2 = nullptr; a.Y = Y;
    a.M = (int)M; a.K = (int)K; a.N = (int)N;
    a.KB = (int)ceil_div(K, 128);
    a.splits = 1; a.kb_per_split = a.KB;
    a.sg = sg; a.su = su;
    const int cus = cu_count_now();
    if (M <= kDecodeFp8MaxM) {
        const hipError_t e = launch_decode_fp8(a, cus, (hipStream_t)stream);
        return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
    }
    const Plan p = stream_dp_plan(M, K, N, cus);
    a.tiles_m = p.tiles_m; a.tiles_n = p.tiles_n;
    const hipError_t e = launch_stream_dp<false, true>(a, p, (hipStream_t)stream);
    return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
}

swiglu_status swiglu_fused(const swiglu_bf16* A, const swiglu_bf16* W1, const swiglu_bf16* W2,
                           swiglu_bf16* Y, int64_t M, int64_t K, int64_t N, void* stream) {
    swiglu_status st = check_shape(M, K, N);
    if (st != SWIGLU_OK) return st;
    if (M == 0) return SWIGLU_OK;
    if (!A || !W1 || !W2 || !Y) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(A) || !aligned16(W1) || !aligned16(W2) || !aligned16(Y)) return SWIGLU_ERR_MISALIGNED;
    const Range y = range_of(Y, M * N * 2);
    if (overlap(y, range_of(A, M * K * 2)) || overlap(y, range_of(W1, K * N * 2)) ||
        overlap(y, range_of(W2, K * N * 2)))
        return SWIGLU_ERR_ALIASING;

    swk::FusedArgs a{};
    a.A = A; a.W1 = W1; a.W2 = W2; a.Y = Y;
    a.M = (int)M; a.K = (int)K; a.N = (int)N;
    a.KB = (int)ceil_div(K, swk::BK);
    a.splits = 1; a.kb_per_split = a.KB;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    // small M: the row-major decode kernel (or, for 32 < M <= 64 when
    // 32-column workgroups would number more than the CUs, the
    // register-transposing tile kernel on 64-column tiles); above 64 rows:
    // direct loads of the row-major weight tiles, fragments through the
    // transposing LDS read
    const int cus = std::max(1, cu_count_now());
    // the weight-streaming row-major decode kernel: 64-column workgroups when
    // they are at least 1.5 per CU, else 32-column ones (measured:
    // 72B-width 195 -> 165 us at M=1 with 64 columns, 7B-width 80.6 -> 67.7 us
    // with 32 and two K blocks in flight); two 32-token tiles above 32 rows,
    // as long as the narrow grid stays within one workgroup per CU (every
    // workgroup reads all the activation rows: 7B-width M=64 keeps the tile
    // kernel, 91 against 111 us; the tiny point's M=64 21.9 -> 13.4 us)
    const bool wide = 2 * ceil_div(N, 64) >= 3 * (int64_t)cus;
    const bool two = M > 32;
    if (M <= 32 || (M <= 64 && (wide || ceil_div(N, 32) <= cus))) {
        const void* fn = wide ? (two ? reinterpret_cast<const void*>(&swk::rowmajor_decode_kernel<64, 1, 2>)
                                     : reinterpret_cast<const void*>(&swk::rowmajor_decode_kernel<64, 1, 1>))
                              : (two ? reinterpret_cast<const void*>(&swk::rowmajor_decode_kernel<32, 1, 2>)
                                     : reinterpret_cast<const void*>(&swk::rowmajor_decode_kernel<32, 2, 1>));
        swk::FusedArgs args = a;
        void* kargs[] = {&args};
        e = hipLaunchKernel(fn, dim3((unsigned)ceil_div(N, wide ? 64 : 32)), dim3(256), kargs, 0, s);
    } else if (M <= 64) {
        a.tiles_m = 1; a.tiles_n = (int)ceil_div(N, 64);
        e = launch_tile<64, 64, 2, 1, true, false, false>(a, a.tiles_m * a.tiles_n, s);
    } else if (M <= 512 && 4 * ceil_div(ceil_div(M, 256) * ceil_div(N, 128), (int64_t)cus) >=
                               3 * ceil_div(ceil_div(M, 128) * ceil_div(N, 128), (int64_t)cus)) {
        // 128-row tiles up to 512 rows unless 256-row ones need fewer rounds
        // of workgroups over the CUs by more than their 4/3 cost per tile
        // (7B-width M=192 177 -> 128 us, M=448 251 -> 242 us, 72B-width
        // M=256 408 -> 336 us, M=512 780 -> 589 us; 7B-width M=300 and the
        // 0.5B width up to 512 rows stay on 128 rows: 178 against 233 us and
        // 15.3 against 29.4 us at M=256).  128x64 tiles when 128x128 ones
        // leave CUs idle and the 64-column grid fits one round or fills at
        // least one and a half (72B-width M=128 298 -> 237 us, 0.5B-width
        // 29.2 -> 22.9 us; the 7B width's 296 tiles of 64 columns, a round
        // and a sixth, stay on 128 columns); 256-row tiles above 512 rows
        // (7B-width M=2048 899 -> 631 us, 72B-width M=1024 1742 -> 1199 us)
        a.tiles_m = (int)ceil_div(M, 128); a.tiles_n = (int)ceil_div(N, 128);
        const int64_t t64 = (int64_t)a.tiles_m * ceil_div(N, 64);
        if ((int64_t)a.tiles_m * a.tiles_n < cus && (t64 <= cus || 2 * t64 >= 3 * (int64_t)cus)) {
            a.tiles_n = (int)ceil_div(N, 64);
            e = launch_prefill<128, 64, 2, 2, false, swk::W_ROW_DUAL>(a, a.tiles_m * a.tiles_n, s);
        } else {
            e = launch_prefill<128, 128, 2, 2, false, swk::W_ROW_DUAL>(a, a.tiles_m * a.tiles_n, s);
        }
    } else {
        a.tiles_m = (int)ceil_div(M, 256); a.tiles_n = (int)ceil_div(N, 128);
        e = launch_prefill<256, 128, 2, 2, false, swk::W_ROW_DUAL>(a, a.tiles_m * a.tiles_n, s);
    }
    if (log_enabled()) std::fprintf(stderr, "[swiglu] fused M=%lld K=%lld N=%lld\n", (long long)M, (long long)K, (long long)N);
    return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
}

int swiglu_choose_variant(int64_t M, int64_t K, int64_t N) {
    if (check_shape(M, K, N) != SWIGLU_OK) return SWIGLU_VARIANT_AUTO;
    return make_plan(M, K, N, SWIGLU_VARIANT_AUTO, cu_count_now()).variant;
}

size_t swiglu_workspace_bytes(int64_t M, int64_t K, int64_t N, int variant) {
    if (check_shape(M, K, N) != SWIGLU_OK || M == 0) return 0;
    if (!variant_known(variant)) return 0;
    return split_workspace_bytes(make_plan(M, K, N, variant, cu_count_now()), M, N);
}

swiglu_status swiglu_fused_packed(const swiglu_bf16* A, const swiglu_bf16* Wp, swiglu_bf16* Y,
                                  int64_t M, int64_t K, int64_t N, void* workspace,
                                  size_t workspace_bytes, int variant, void* stream) {
    swiglu_status st = check_shape(M, K, N);
    if (st != SWIGLU_OK) return st;
    if (!variant_known(variant)) return SWIGLU_ERR_BAD_VARIANT;
    if (variant == SWIGLU_VARIANT_DECODE && M > kDecodeMaxM) return SWIGLU_ERR_BAD_VARIANT;
    if (M == 0) return SWIGLU_OK;
    if (!A || !Wp || !Y) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(A) || !aligned16(Wp) || !aligned16(Y)) return SWIGLU_ERR_MISALIGNED;
    const Range y = range_of(Y, M * N * 2);
    if (overlap(y, range_of(A, M * K * 2)) || overlap(y, range_of(Wp, packed_elems(K, N) * 2)))
        return SWIGLU_ERR_ALIASING;
    if (M > stream_rows_limit(K, 2)) {
        // chunks of at least half the limit: always the data-parallel
        // schedule, which needs no workspace
        const int64_t rows = balanced_chunk(M, stream_rows_limit(K, 2));
        for (int64_t m0 = 0; m0 < M; m0 += rows) {
            st = swiglu_fused_packed(A + m0 * K, Wp, Y + m0 * N, std::min(rows, M - m0), K, N, nullptr, 0,
                                     variant == SWIGLU_VARIANT_SEQUENTIAL ? SWIGLU_VARIANT_SEQUENTIAL
                                                                          : SWIGLU_VARIANT_DATA_PARALLEL,
                                     stream);
            if (st != SWIGLU_OK) return st;
        }
        return SWIGLU_OK;
    }

    const Plan p = make_plan(M, K, N, variant, cu_count_now());
    const size_t need = split_workspace_bytes(p, M, N);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return SWIGLU_ERR_WORKSPACE;
        if (!aligned16(workspace)) return SWIGLU_ERR_MISALIGNED;
        const Range w = range_of(workspace, (int64_t)need);
        if (overlap(w, y) || overlap(w, range_of(A, M * K * 2)) ||
            overlap(w, range_of(Wp, packed_elems(K, N) * 2)))
            return SWIGLU_ERR_ALIASING;
    }

    swk::FusedArgs a{};
    a.A = A; a.W1 = Wp; a.W2 = nullptr; a.Y = Y;
    a.M = (int)M; a.K = (int)K; a.N = (int)N;
    a.tiles_m = p.tiles_m; a.tiles_n = p.tiles_n;
    a.splits = p.splits; a.kb_per_split = p.kb_per_split; a.KB = p.KB;
    if (need > 0) a.part = reinterpret_cast<float*>(workspace);
    if (log_enabled())
        std::fprintf(stderr, "[swiglu] fused_packed M=%lld K=%lld N=%lld variant=%d tile=%dx%d tiles=%d splits=%d tail_ntiles=%d panels=%d\n",
                     (long long)M, (long long)K, (long long)N, p.variant, p.t.BM, p.t.BN, p.tiles, p.splits,
                     p.tail_ntiles, p.panels);
    hipError_t e = launch_packed(a, p, (hipStream_t)stream);
    if (e == hipSuccess && p.splits > 1) {
        const int cus = std::max(1, cu_count_now());
        const long long groups = (long long)M * (N / 4);
        const int grid = (int)std::max<long long>(1, std::min<long long>(ceil_div(groups, 256), (long long)cus * 8));
        int Mi = (int)M, Ni = (int)N, Si = p.splits;
        const float* part = a.part;
        uint16_t* yp = a.Y;
        void* args[] = {(void*)&part, (void*)&yp, &Mi, &Ni, &Si};
        e = hipLaunchKernel(reinterpret_cast<const void*>(&swk::splitk_reduce_kernel), dim3(grid), dim3(256),
                            args, 0, (hipStream_t)stream);
    }
    return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
}

// swiglu_fused_packed with the split-K partial sums in the library's own
// device scratch array instead of a caller's workspace: no allocation on any
// path.  The schedule is the one swiglu_fused_packed would run; a schedule
// whose partial sums exceed the array is rejected before any HIP call.
swiglu_status swiglu_fused_packed_noalloc(const swiglu_bf16* A, const swiglu_bf16* Wp, swiglu_bf16* Y,
                                          int64_t M, int64_t K, int64_t N, int variant, void* stream) {
    swiglu_status st = check_shape(M, K, N);
    if (st != SWIGLU_OK) return st;
    if (!variant_known(variant)) return SWIGLU_ERR_BAD_VARIANT;
    if (variant == SWIGLU_VARIANT_DECODE && M > kDecodeMaxM) return SWIGLU_ERR_BAD_VARIANT;
    if (M == 0) return SWIGLU_OK;
    if (!A || !Wp || !Y) return SWIGLU_ERR_NULL_POINTER;
    // products chunked by rows run on the data-parallel schedule, which
    // needs no partial sums; otherwise the plan swiglu_fused_packed makes
    size_t need = 0;
    if (M <= stream_rows_limit(K, 2)) need = split_workspace_bytes(make_plan(M, K, N, variant, cu_count_now()), M, N);
    if (need > (size_t)SWIGLU_NOALLOC_SCRATCH_BYTES) return SWIGLU_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        const hipError_t e = scratch_device_ptr(&ws);
        if (e != hipSuccess) return hip_fail(e);
    }
    return swiglu_fused_packed(A, Wp, Y, M, K, N, ws, need > 0 ? (size_t)SWIGLU_NOALLOC_SCRATCH_BYTES : 0, variant,
                               stream);
}

swiglu_status swiglu_gemm_bf16(const swiglu_bf16* A, const swiglu_bf16* W, swiglu_bf16* C,
                               int64_t M, int64_t K, int64_t N, void* stream) {
    swiglu_status st = check_shape(M, K, N);
    if (st != SWIGLU_OK) return st;
    if (M == 0) return SWIGLU_OK;
    if (!A || !W || !C) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(A) || !aligned16(W) || !aligned16(C)) return SWIGLU_ERR_MISALIGNED;
    const Range c = range_of(C, M * N * 2);
    if (overlap(c, range_of(A, M * K * 2)) || overlap(c, range_of(W, K * N * 2))) return SWIGLU_ERR_ALIASING;
    swk::FusedArgs a{};
    a.A = A; a.W1 = W; a.W2 = W; a.Y = C;
    a.M = (int)M; a.K = (int)K; a.N = (int)N;
    a.KB = (int)ceil_div(K, swk::BK);
    a.splits = 1; a.kb_per_split = a.KB;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (M <= 32) {
        a.tiles_m = (int)ceil_div(M, 32); a.tiles_n = (int)ceil_div(N, 128);
        e = launch_tile<32, 128, 1, 2, false, false, false>(a, a.tiles_m * a.tiles_n, s);
    } else if (M <= 64) {
        a.tiles_m = 1; a.tiles_n = (int)ceil_div(N, 128);
        e = launch_tile<64, 128, 2, 1, false, false, false>(a, a.tiles_m * a.tiles_n, s);
    } else if (M <= 2048) {
        a.tiles_m = (int)ceil_div(M, 128); a.tiles_n = (int)ceil_div(N, 256);
        e = launch_prefill<128, 256, 2, 2, false, swk::W_ROW_SINGLE>(a, a.tiles_m * a.tiles_n, s);
    } else {
        a.tiles_m = (int)ceil_div(M, 256); a.tiles_n = (int)ceil_div(N, 256);
        e = launch_prefill<256, 256, 2, 2, false, swk::W_ROW_SINGLE>(a, a.tiles_m * a.tiles_n, s);
    }
    return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
}

size_t swiglu_gemm_packed_bytes(int64_t K, int64_t N) {
    if (check_shape(0, K, N) != SWIGLU_OK) return 0;
    return (size_t)gemm_packed_elems(K, N) * sizeof(swiglu_bf16);
}

swiglu_status swiglu_gemm_pack_weight(const swiglu_bf16* W, swiglu_bf16* Wg, int64_t K, int64_t N, void* stream) {
    swiglu_status st = check_shape(0, K, N);
    if (st != SWIGLU_OK) return st;
    if (!W || !Wg) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(W) || !aligned16(Wg)) return SWIGLU_ERR_MISALIGNED;
    if (overlap(range_of(Wg, gemm_packed_elems(K, N) * 2), range_of(W, K * N * 2))) return SWIGLU_ERR_ALIASING;
    const long long nchunks = (long long)gemm_packed_elems(K, N) / 8;
    const int KB = (int)ceil_div(K, swk::PACK_BK);
    int Ki = (int)K, Ni = (int)N;
    void* args[] = {(void*)&W, (void*)&W, (void*)&Wg, &Ki, &Ni, (void*)&KB, (void*)&nchunks};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&swk::pack_kernel<false, true>),
                                   dim3((unsigned)ceil_div(nchunks, 256)), dim3(256), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
}

// The single-weight GEMM's plan: the fused product's AUTO rule on the pack's
// tiled width (128 columns per packed tile), whose split-K needs fp32
// partials over those tiled columns.  One addition: a compute-bound product
// (from 1024 rows on) whose data-parallel tiles leave over half the CUs idle
// -- a narrow output, like the MLP's down projection back to a small model
// width -- splits K as well: there the idle matrix cores cost more than the
// partial sums' traffic (measured: 0.5B-width down projection, M=4096
// K=4864 N=896, 86.6 us data-parallel on 64 tiles, 70 us in 4 splits).
Plan gemm_plan(int64_t M, int64_t K, int64_t N) {
    const int cus = cu_count_now();
    const int64_t nt = gemm_tiled_cols(N);
    Plan p = make_plan(M, K, nt, SWIGLU_VARIANT_AUTO, cus);
    if (p.variant == SWIGLU_VARIANT_DATA_PARALLEL && M >= 1024 && 2 * (int64_t)p.tiles < p.cus) {
        const Plan q = make_plan(M, K, nt, SWIGLU_VARIANT_SPLIT_K, cus);
        if (q.splits > 1) p = q;
    }
    return p;
}

size_t gemm_split_bytes(const Plan& p, int64_t M, int64_t N) {
    return split_workspace_bytes(p, M, gemm_tiled_cols(N));
}

size_t swiglu_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (check_shape(M, K, N) != SWIGLU_OK || M == 0) return 0;
    if (M > stream_rows_limit(K, 2)) return 0;   // row chunks run data-parallel
    return gemm_split_bytes(gemm_plan(M, K, N), M, N);
}

swiglu_status swiglu_gemm_packed(const swiglu_bf16* A, const swiglu_bf16* Wg, swiglu_bf16* C, int64_t M, int64_t K,
                                 int64_t N, void* workspace, size_t workspace_bytes, void* stream) {
    swiglu_status st = check_shape(M, K, N);
    if (st != SWIGLU_OK) return st;
    if (M == 0) return SWIGLU_OK;
    if (!A || !Wg || !C) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(A) || !aligned16(Wg) || !aligned16(C)) return SWIGLU_ERR_MISALIGNED;
    const Range c = range_of(C, M * N * 2);
    if (overlap(c, range_of(A, M * K * 2)) || overlap(c, range_of(Wg, gemm_packed_elems(K, N) * 2)))
        return SWIGLU_ERR_ALIASING;
    if (M > stream_rows_limit(K, 2)) {
        const int64_t rows = balanced_chunk(M, stream_rows_limit(K, 2));
        for (int64_t m0 = 0; m0 < M; m0 += rows) {
            st = swiglu_gemm_packed(A + m0 * K, Wg, C + m0 * N, std::min(rows, M - m0), K, N, nullptr, 0, stream);
            if (st != SWIGLU_OK) return st;
        }
        return SWIGLU_OK;
    }
    // the fused product's schedules on the packed tiles' width: decode for
    // small M, else the streaming grid, split over K when AUTO asks for it
    // and the workspace holds the partial sums
    const int64_t nt = gemm_tiled_cols(N);
    Plan p = gemm_plan(M, K, N);
    const size_t need = gemm_split_bytes(p, M, N);
    bool split = p.variant == SWIGLU_VARIANT_SPLIT_K && need > 0 && workspace && workspace_bytes >= need;
    if (split) {
        if (!aligned16(workspace)) return SWIGLU_ERR_MISALIGNED;
        const Range w = range_of(workspace, (int64_t)need);
        if (overlap(w, c) || overlap(w, range_of(A, M * K * 2)) ||
            overlap(w, range_of(Wg, gemm_packed_elems(K, N) * 2)))
            return SWIGLU_ERR_ALIASING;
    } else if (p.variant == SWIGLU_VARIANT_SPLIT_K) {
        p = make_plan(M, K, nt, SWIGLU_VARIANT_DATA_PARALLEL, p.cus);
    }
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (p.variant == SWIGLU_VARIANT_DECODE) {
        swk::DecodeArgs d{};
        d.A = A; d.Wp = Wg; d.Y = C;
        d.M = (int)M; d.K = (int)K; d.N = (int)N; d.KB = p.KB;
        e = launch_decode_gemm(d, nt, p, s);
    } else {
        swk::FusedArgs a{};
        a.A = A; a.W1 = Wg; a.W2 = nullptr; a.Y = C;
        a.M = (int)M; a.K = (int)K; a.N = (int)N;
        a.tiles_m = p.tiles_m; a.tiles_n = p.tiles_n;
        a.splits = p.splits; a.kb_per_split = p.kb_per_split; a.KB = p.KB;
        if (split) {
            a.part = reinterpret_cast<float*>(workspace);
            const int grid = p.tiles * p.splits;
            e = p.t.BM == 128 ? launch_stream<128, true, false, false, false, false, true>(a, grid, grid, s)
                              : launch_stream<256, true, false, false, false, false, true>(a, grid, grid, s);
            if (e == hipSuccess) {
                const long long groups = (long long)M * (nt / 4);
                const int rgrid = (int)std::max<long long>(
                    1, std::min<long long>(ceil_div(groups, 256), (long long)p.cus * 8));
                int Mi = (int)M, Ni = (int)N, NTi = (int)nt, Si = p.splits;
                const float* part = a.part;
                uint16_t* cp = C;
                void* args[] = {(void*)&part, (void*)&cp, &Mi, &Ni, &NTi, &Si};
                e = hipLaunchKernel(reinterpret_cast<const void*>(&swk::splitk_gemm_reduce_kernel), dim3(rgrid),
                                    dim3(256), args, 0, s);
            }
        } else {
            e = launch_stream_dp<false, false, false, true>(a, p, s);
        }
    }
    return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
}

swiglu_status swiglu_unfused_packed(const swiglu_bf16* A, const swiglu_bf16* W1g, const swiglu_bf16* W2g,
                                    swiglu_bf16* G_scratch, swiglu_bf16* U_scratch, swiglu_bf16* Y, int64_t M,
                                    int64_t K, int64_t N, void* stream) {
    swiglu_status st = check_shape(M, K, N);
    if (st != SWIGLU_OK) return st;
    if (M == 0) return SWIGLU_OK;
    if (!A || !W1g || !W2g || !G_scratch || !U_scratch || !Y) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(G_scratch) || !aligned16(U_scratch) || !aligned16(Y)) return SWIGLU_ERR_MISALIGNED;
    const Range g = range_of(G_scratch, M * N * 2), u = range_of(U_scratch, M * N * 2),
                y = range_of(Y, M * N * 2);
    const int64_t wb = gemm_packed_elems(K, N) * 2;
    const Range ins[3] = {range_of(A, M * K * 2), range_of(W1g, wb), range_of(W2g, wb)};
    for (const Range& r : ins)
        if (overlap(g, r) || overlap(u, r) || overlap(y, r)) return SWIGLU_ERR_ALIASING;
    if (overlap(g, u) || overlap(g, y) || overlap(u, y)) return SWIGLU_ERR_ALIASING;
    st = swiglu_gemm_packed(A, W1g, G_scratch, M, K, N, nullptr, 0, stream);
    if (st != SWIGLU_OK) return st;
    st = swiglu_gemm_packed(A, W2g, U_scratch, M, K, N, nullptr, 0, stream);
    if (st != SWIGLU_OK) return st;
    return swiglu_silu_mul(G_scratch, U_scratch, Y, M * N, stream);
}

swiglu_status swiglu_silu_mul(const swiglu_bf16* G, const swiglu_bf16* U, swiglu_bf16* Y,
                              int64_t count, void* stream) {
    if (count < 0) return SWIGLU_ERR_BAD_SHAPE;
    if (count == 0) return SWIGLU_OK;
    if (!G || !U || !Y) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(G) || !aligned16(U) || !aligned16(Y)) return SWIGLU_ERR_MISALIGNED;
    const Range y = range_of(Y, count * 2);
    if (overlap(y, range_of(G, count * 2)) || overlap(y, range_of(U, count * 2))) return SWIGLU_ERR_ALIASING;
    const int cus = std::max(1, cu_count_now());
    const long long nvec = (count + 7) / 8;
    const int grid = (int)std::max<long long>(1, std::min<long long>(ceil_div(nvec, 256), (long long)cus * 8));
    long long cnt = count;
    void* args[] = {(void*)&G, (void*)&U, (void*)&Y, &cnt};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&swk::silu_mul_kernel), dim3(grid),
                                   dim3(256), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
}

swiglu_status swiglu_unfused(const swiglu_bf16* A, const swiglu_bf16* W1, const swiglu_bf16* W2,
                             swiglu_bf16* G_scratch, swiglu_bf16* U_scratch, swiglu_bf16* Y,
                             int64_t M, int64_t K, int64_t N, void* stream) {
    swiglu_status st = check_shape(M, K, N);
    if (st != SWIGLU_OK) return st;
    if (M == 0) return SWIGLU_OK;
    if (!A || !W1 || !W2 || !G_scratch || !U_scratch || !Y) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(G_scratch) || !aligned16(U_scratch) || !aligned16(Y)) return SWIGLU_ERR_MISALIGNED;
    const Range g = range_of(G_scratch, M * N * 2), u = range_of(U_scratch, M * N * 2),
                y = range_of(Y, M * N * 2);
    const Range ins[3] = {range_of(A, M * K * 2), range_of(W1, K * N * 2), range_of(W2, K * N * 2)};
    for (const Range& r : ins)
        if (overlap(g, r) || overlap(u, r) || overlap(y, r)) return SWIGLU_ERR_ALIASING;
    if (overlap(g, u) || overlap(g, y) || overlap(u, y)) return SWIGLU_ERR_ALIASING;
    st = swiglu_gemm_bf16(A, W1, G_scratch, M, K, N, stream);
    if (st != SWIGLU_OK) return st;
    st = swiglu_gemm_bf16(A, W2, U_scratch, M, K, N, stream);
    if (st != SWIGLU_OK) return st;
    return swiglu_silu_mul(G_scratch, U_scratch, Y, M * N, stream);
}

// ---------------------------------------------------------------------------
// Down projection of the MLP block, Z[M,K] = bf16(Y[M,N] x W3[N,K]): a plain
// GEMM on this library's own kernels, Y as the activations (N deep) and W3 in
// the single-weight pack (swiglu_gemm_pack_weight of the [N,K] W3).
// ---------------------------------------------------------------------------
size_t swiglu_mlp_workspace_bytes(int64_t M, int64_t K, int64_t N, int variant) {
    if (check_shape(M, K, N) != SWIGLU_OK || M == 0 || !variant_known(variant)) return 0;
    return std::max(swiglu_workspace_bytes(M, K, N, variant), swiglu_gemm_workspace_bytes(M, N, K));
}

swiglu_status swiglu_mlp_down(const swiglu_bf16* Y, const swiglu_bf16* W3g, swiglu_bf16* Z, int64_t M, int64_t K,
                              int64_t N, void* workspace, size_t workspace_bytes, void* stream) {
    swiglu_status st = check_shape(M, K, N);
    if (st != SWIGLU_OK) return st;
    if (M == 0) return SWIGLU_OK;
    if (!Y || !W3g || !Z) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(Y) || !aligned16(W3g) || !aligned16(Z)) return SWIGLU_ERR_MISALIGNED;
    const Range z = range_of(Z, M * K * 2);
    if (overlap(z, range_of(Y, M * N * 2)) || overlap(z, range_of(W3g, gemm_packed_elems(N, K) * 2)))
        return SWIGLU_ERR_ALIASING;
    return swiglu_gemm_packed(Y, W3g, Z, M, N, K, workspace, workspace_bytes, stream);
}

swiglu_status swiglu_mlp_packed(const swiglu_bf16* A, const swiglu_bf16* Wp, const swiglu_bf16* W3g,
                                swiglu_bf16* Y, swiglu_bf16* Z, int64_t M, int64_t K, int64_t N,
                                void* workspace, size_t workspace_bytes, int variant, void* stream) {
    swiglu_status st = check_shape(M, K, N);
    if (st != SWIGLU_OK) return st;
    if (!variant_known(variant)) return SWIGLU_ERR_BAD_VARIANT;
    if (M == 0) return SWIGLU_OK;
    if (!A || !Wp || !W3g || !Y || !Z) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(W3g) || !aligned16(Z)) return SWIGLU_ERR_MISALIGNED;
    const Range z = range_of(Z, M * K * 2), w3 = range_of(W3g, gemm_packed_elems(N, K) * 2),
                y = range_of(Y, M * N * 2);
    if (overlap(z, range_of(A, M * K * 2)) || overlap(z, range_of(Wp, packed_elems(K, N) * 2)) ||
        overlap(z, w3) || overlap(z, y) || overlap(y, w3))
        return SWIGLU_ERR_ALIASING;
    if (workspace && workspace_bytes > 0 && overlap(z, range_of(workspace, (int64_t)workspace_bytes)))
        return SWIGLU_ERR_ALIASING;
    st = swiglu_fused_packed(A, Wp, Y, M, K, N, workspace, workspace_bytes, variant, stream);
    if (st != SWIGLU_OK) return st;
    // the same workspace then holds the down projection's partial sums (the
    // fused product's are consumed by then: both run in order on `stream`)
    return swiglu_gemm_packed(Y, W3g, Z, M, N, K, workspace, workspace_bytes, stream);
}

swiglu_status swiglu_mlp_unfused(const swiglu_bf16* A, const swiglu_bf16* W1g, const swiglu_bf16* W2g,
                                 const swiglu_bf16* W3g, swiglu_bf16* G_scratch, swiglu_bf16* U_scratch,
                                 swiglu_bf16* Y, swiglu_bf16* Z, int64_t M, int64_t K, int64_t N,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    swiglu_status st = check_shape(M, K, N);
    if (st != SWIGLU_OK) return st;
    if (M == 0) return SWIGLU_OK;
    if (!A || !W1g || !W2g || !W3g || !G_scratch || !U_scratch || !Y || !Z) return SWIGLU_ERR_NULL_POINTER;
    if (!aligned16(W3g) || !aligned16(Z)) return SWIGLU_ERR_MISALIGNED;
    const int64_t wb = gemm_packed_elems(K, N) * 2;
    const Range z = range_of(Z, M * K * 2), w3 = range_of(W3g, gemm_packed_elems(N, K) * 2);
    const Range others[7] = {range_of(A, M * K * 2), range_of(W1g, wb), range_of(W2g, wb), w3,
                             range_of(G_scratch, M * N * 2), range_of(U_scratch, M * N * 2),
                             range_of(Y, M * N * 2)};
    for (const Range& r : others)
        if (overlap(z, r)) return SWIGLU_ERR_ALIASING;
    for (int i = 4; i < 7; ++i)
        if (overlap(others[i], w3)) return SWIGLU_ERR_ALIASING;
    if (workspace && workspace_bytes > 0 && overlap(z, range_of(workspace, (int64_t)workspace_bytes)))
        return SWIGLU_ERR_ALIASING;
    st = swiglu_unfused_packed(A, W1g, W2g, G_scratch, U_scratch, Y, M, K, N, stream);
    if (st != SWIGLU_OK) return st;
    return swiglu_gemm_packed(Y, W3g, Z, M, N, K, workspace, workspace_bytes, stream);
}

swiglu_status swiglu_probe_mfma(float* sink, int blocks, int iters, void* stream) {
    if (!sink) return SWIGLU_ERR_NULL_POINTER;
    if (blocks < 1 || iters < 1) return SWIGLU_ERR_BAD_SHAPE;
    void* args[] = {(void*)&sink, &iters};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&swk::probe_mfma_kernel), dim3(blocks),
                                   dim3(256), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
}

swiglu_status swiglu_probe_read(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream) {
    if (!src || !sink) return SWIGLU_ERR_NULL_POINTER;
    if (blocks < 1 || bytes < 16 || (bytes % 16) != 0) return SWIGLU_ERR_BAD_SHAPE;
    if (!aligned16(src)) return SWIGLU_ERR_MISALIGNED;
    long long n16 = (long long)(bytes / 16);
    void* args[] = {(void*)&src, &n16, (void*)&sink};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&swk::probe_read_kernel), dim3(blocks),
                                   dim3(256), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? SWIGLU_OK : hip_fail(e);
}

}  // extern "C"
