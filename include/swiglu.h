/*
 * swiglu.h -- C ABI of libswiglu.so, the fused SwiGLU gated-MLP product for
 * AMD Instinct MI355X (gfx950).
 *
 * Citations name the pages about "Tile-Level Activation Overlap for Efficient
 * LLM Inference": [Abstract] is the paper's abstract (paper-with-me page);
 * [Summary: X] is section X of the gist.science technical summary.
 *
 * The operation ([Summary: Problem Statement]):
 *
 *     Y = SiLU(A x W1) (.) (A x W2),   SiLU(x) = x / (1 + e^-x)
 *
 * A [M,K], W1 [K,N], W2 [K,N], Y [M,N]; Gate = A x W1 is the operand SiLU is
 * applied to, Up = A x W2 multiplies it.  Gate and Up are accumulated in fp32
 * and never written to memory ([Abstract]; [Summary: Key Contributions],
 * tile-level fusion); SiLU and the product are fp32; Y is rounded once to bf16,
 * round-to-nearest-even.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Element type: swiglu_bf16 holds raw bf16 bit patterns.  Every matrix is
 *    row-major and contiguous (leading dimension = number of columns).
 *  - Pointers: all matrix pointers are DEVICE pointers (hipMalloc'd or torch
 *    CUDA tensors) of the current HIP device, 16-byte aligned.
 *  - Ownership: the caller owns every buffer.  The library allocates no memory
 *    on any path and keeps no pointer after a call returns.
 *  - Sizes: each buffer holds at least the elements its shape implies (A M*K,
 *    W1/W2 K*N, Y M*N, a packed weight buffer swiglu_packed_bytes(K, N)
 *    bytes).  The library receives bare pointers and cannot check this; a
 *    smaller buffer is read or written past its end.
 *  - Streams: `stream` is a hipStream_t (NULL = the default stream).  Work is
 *    enqueued and the call returns without synchronising; device-side faults
 *    surface at the caller's next synchronisation.
 *  - Shapes: M >= 0; K > 0 and N > 0 must be multiples of 8 (16-byte rows),
 *    K at most 4194304 (else SWIGLU_ERR_UNSUPPORTED_SHAPE); every dimension
 *    at most 2^30.  M == 0 is a valid empty call: SWIGLU_OK, nothing is
 *    launched.  Products whose activations reach 2 GiB are run as several
 *    equal row chunks on the same stream, each on the data-parallel schedule
 *    (the streaming kernel addresses each activation tile with 32-bit
 *    offsets).
 *  - Aliasing: inputs may alias each other (W1 == W2 is legal).  Outputs must
 *    not overlap any input or each other.
 *  - Errors: argument errors are detected on the host before any HIP call and
 *    leave every output untouched.  A failed launch returns SWIGLU_ERR_HIP and
 *    swiglu_last_hip_error() gives the hipError_t (per calling thread).
 *  - Thread safety: every entry point is re-entrant.  Calls on different
 *    streams may overlap as long as their outputs and workspaces differ.
 */
#ifndef SWIGLU_H_
#define SWIGLU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWIGLU_ABI_VERSION 3

typedef uint16_t swiglu_bf16;

typedef enum {
    SWIGLU_OK = 0,
    SWIGLU_ERR_NULL_POINTER = 1,      /* a required pointer is NULL (with M > 0)      */
    SWIGLU_ERR_BAD_SHAPE = 2,         /* M < 0, K <= 0, N <= 0, or sizes overflow     */
    SWIGLU_ERR_UNSUPPORTED_SHAPE = 3, /* K or N not a multiple of 8, or K > 2^22      */
    SWIGLU_ERR_MISALIGNED = 4,        /* a pointer is not 16-byte aligned             */
    SWIGLU_ERR_ALIASING = 5,          /* an output overlaps an input or other output  */
    SWIGLU_ERR_WORKSPACE = 6,         /* workspace missing or too small               */
    SWIGLU_ERR_BAD_VARIANT = 7,       /* unknown variant, or one the shape can't use  */
    SWIGLU_ERR_HIP = 8                /* a HIP call failed; see swiglu_last_hip_error */
} swiglu_status;

/* Schedules of the fused packed entry point.
 *  DATA_PARALLEL: the streaming kernel, full K per work item: 256- or
 *                 128-row tiles for large M (the pages' Kernel-1 regime,
 *                 [Summary: Methodology] Kernel-1); for one row of 128-row
 *                 tiles with fewer column tiles than CUs, the tiles' 32-column
 *                 weight panels spread over the CUs instead.
 *  SPLIT_K:       the K range is split across workgroups; each split writes
 *                 its fp32 Gate/Up partial sums to the workspace and a second
 *                 kernel adds them in fixed split order 0..S-1 BEFORE SiLU,
 *                 then applies the epilogue; for small M, where output tiles
 *                 alone cannot fill the GPU (the occupancy problem of
 *                 [Summary: Methodology] Kernel-2, "Optimization").
 *  DECODE:        M <= 64 only.  Weight streaming: one workgroup per 16 output
 *                 columns reads their Gate and Up weight rows once, its waves
 *                 split K and add their fp32 partials in LDS in fixed order
 *                 BEFORE SiLU; needs no workspace.  The product is then bound
 *                 by reading the weights from HBM.
 *  AUTO:          the library picks from M, K, N and the device's CU count:
 *                 DECODE up to 32 rows, and up to 64 rows while the weight
 *                 panels (4 per 128 columns) number fewer than the CUs;
 *                 otherwise DATA_PARALLEL, or SPLIT_K when the data-parallel
 *                 tiles would fill under half the CUs (and K >= 32 M).
 *  SEQUENTIAL:    the Gate-then-Up order ([Summary: Methodology] Kernel-1:
 *                 SiLU on the finished Gate accumulator while the Up
 *                 operands are still loading): on the data-parallel 128- or
 *                 256-row tiles,
 *                 each tile runs a K loop over the Gate half of the packed
 *                 weights, then computes SiLU(Gate) while the Up loop's first
 *                 stages load, then runs a second K loop over the activations
 *                 and the Up half.  Same result as DATA_PARALLEL, bit for bit;
 *                 any M; no workspace.  AUTO never picks it (it re-reads the
 *                 activation tiles and is slower on this chip at every
 *                 measured shape); it exists for comparison.
 * There is no stream-K schedule: the even share of work per CU it would give
 * comes from the column-split schedules (DECODE, the panel form of
 * DATA_PARALLEL) at small M and from the 128-row tail tiles of the last round
 * at large M, with no partial sums through memory. */
typedef enum {
    SWIGLU_VARIANT_AUTO = 0,
    SWIGLU_VARIANT_DATA_PARALLEL = 1,
    SWIGLU_VARIANT_SPLIT_K = 2,
    SWIGLU_VARIANT_DECODE = 3,
    SWIGLU_VARIANT_SEQUENTIAL = 4
} swiglu_variant;

/* Returns SWIGLU_ABI_VERSION. */
int swiglu_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *swiglu_status_str(int status);

/* hipError_t of the most recent SWIGLU_ERR_HIP on the calling thread (0 if none). */
int swiglu_last_hip_error(void);

/* Number of compute units of the current device as the library sees it
 * (0 if it cannot be queried).  Host call; used by the schedule heuristic. */
int swiglu_device_cu_count(void);

/* ------------------------------------------------------------------------
 * swiglu_fused -- Y = SiLU(A W1) (.) (A W2) from unpacked row-major weights.
 * [Summary: Problem Statement] (definition); [Abstract] (tile-level fusion:
 * Gate and Up stay in registers, only Y is written).
 *   A  [M,K] bf16, W1 [K,N] bf16, W2 [K,N] bf16 (inputs, device)
 *   Y  [M,N] bf16 (output, device; must not overlap A, W1, W2)
 * Needs no workspace; always uses the data-parallel schedule.  The weights are
 * transposed to K-contiguous order on the fly, tile by tile: their tiles are
 * loaded into LDS as they lie in memory and the transposing LDS read forms
 * the matrix-core fragments (for 32 < M <= 64 on products wider than the CU
 * count allows in 32-column workgroups, a tile kernel transposes them in
 * registers instead).
 * ---------------------------------------------------------------------- */
swiglu_status swiglu_fused(const swiglu_bf16 *A, const swiglu_bf16 *W1,
                           const swiglu_bf16 *W2, swiglu_bf16 *Y, int64_t M,
                           int64_t K, int64_t N, void *stream);

/* ------------------------------------------------------------------------
 * Packed weights.  The pages build one fused weight matrix holding W1 and W2
 * side by side before the GEMM runs ([Summary: Methodology] Kernel-2,
 * "Strategy": W_fused in R^{K x 2N}).  Here the two are interleaved per tile
 * of 128 output columns instead of per column, and stored K-contiguous in
 * the lane order of the matrix-core fragments:
 *
 *   Wp = for jt in 0 .. ceil(N/128)-1:            (output-column tile)
 *          for kb in 0 .. ceil(K/64)-1:           (64-deep K block, 32 KiB)
 *            for g in 0 .. 15:                    (16-row group: 0-7 W1, 8-15 W2)
 *              for h in 0 .. 1:                   (32-deep half of the block)
 *                for l in 0 .. 63:                (16 bytes each)
 *                  for e in 0 .. 7:
 *                    W[k][n] with  k = kb*64 + h*32 + (l/16)*8 + e,
 *                                  n = jt*128 + (g%8)*16 + l%16,
 *                                  W = W1 for g < 8, W2 for g >= 8
 *   Entries with k >= K or n >= N are zero.
 *
 * swiglu_packed_bytes: size of Wp in bytes for a K x N weight pair (0 if the
 *   shape is invalid).
 * swiglu_pack_weights: W1, W2 [K,N] -> Wp (device, swiglu_packed_bytes bytes).
 *   One-time transform (model-load time); not part of the fused call.
 * swiglu_unpack_weights: the inverse, Wp -> W1, W2 (for tests).
 * ---------------------------------------------------------------------- */
size_t swiglu_packed_bytes(int64_t K, int64_t N);
swiglu_status swiglu_pack_weights(const swiglu_bf16 *W1, const swiglu_bf16 *W2,
                                  swiglu_bf16 *Wp, int64_t K, int64_t N,
                                  void *stream);
swiglu_status swiglu_unpack_weights(const swiglu_bf16 *Wp, swiglu_bf16 *W1,
                                    swiglu_bf16 *W2, int64_t K, int64_t N,
                                    void *stream);

/* ------------------------------------------------------------------------
 * swiglu_fused_packed -- the same product from packed weights (the fast path).
 * [Summary: Problem Statement] (definition); [Summary: Methodology] Kernel-2
 * (one GEMM over the fused weight, SiLU(Gate) (.) Up applied to each pair of
 * accumulators before the store).
 *   A [M,K] bf16, Wp (swiglu_packed_bytes(K,N) bytes), Y [M,N] bf16 (device).
 *   workspace: device scratch for SWIGLU_VARIANT_SPLIT_K: fp32 partial sums,
 *     splits x M x 2N floats (Gate at column n, Up at column N + n of each
 *     split's [M, 2N] slab).  May be NULL when swiglu_workspace_bytes() returns
 *     0 for the chosen variant.  Its contents on entry do not matter (no
 *     clearing needed); calls that may run concurrently must not share one.
 *   variant: a swiglu_variant; AUTO lets the library choose.
 * swiglu_workspace_bytes: bytes of workspace the call needs for (M,K,N,variant)
 *   (for AUTO: the requirement of the variant AUTO would pick).
 * ---------------------------------------------------------------------- */
size_t swiglu_workspace_bytes(int64_t M, int64_t K, int64_t N, int variant);
swiglu_status swiglu_fused_packed(const swiglu_bf16 *A, const swiglu_bf16 *Wp,
                                  swiglu_bf16 *Y, int64_t M, int64_t K, int64_t N,
                                  void *workspace, size_t workspace_bytes,
                                  int variant, void *stream);

/* Variant AUTO resolves to for this shape on the current device. */
int swiglu_choose_variant(int64_t M, int64_t K, int64_t N);

/* ------------------------------------------------------------------------
 * swiglu_fused_packed_noalloc -- swiglu_fused_packed for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The caller passes the inputs and the
 * output only; the split-K schedule's fp32 partial sums go to a scratch
 * array the library keeps in device memory, SWIGLU_NOALLOC_SCRATCH_BYTES
 * bytes per device, held from the library's load until the process ends.
 * The call allocates nothing on any path (no hipMalloc, no hipFree, no
 * allocating library routine).
 *   A, Wp, Y, M, K, N, variant, stream: as swiglu_fused_packed; the schedule
 *     is the one swiglu_fused_packed runs for the same arguments, so the two
 *     give the same Y.
 *   Returns SWIGLU_ERR_WORKSPACE, before any HIP call, when that schedule's
 *     partial sums (swiglu_workspace_bytes(M, K, N, variant)) exceed
 *     SWIGLU_NOALLOC_SCRATCH_BYTES; AUTO, DATA_PARALLEL, DECODE and
 *     SEQUENTIAL need none at the Qwen-2.5 shapes.  Other validation codes as
 *     swiglu_fused_packed.
 * Every call on one device shares that device's array, which keeps the last
 * call's contents (nothing in it needs clearing: each split writes all of
 * its partial sums before the reduction reads them).  Calls that overlap in
 * time on one device race on it: issue them on one stream, or order them.
 * ---------------------------------------------------------------------- */
#define SWIGLU_NOALLOC_SCRATCH_BYTES (32u << 20)
swiglu_status swiglu_fused_packed_noalloc(const swiglu_bf16 *A,
                                          const swiglu_bf16 *Wp, swiglu_bf16 *Y,
                                          int64_t M, int64_t K, int64_t N,
                                          int variant, void *stream);

/* ------------------------------------------------------------------------
 * FP8 operands.  The pages note that quantised GEMMs (FP8, INT4) raise the
 * relative cost of SwiGLU's memory traffic ([Summary: Problem Statement]) but
 * give no scale convention; this library takes per-tensor scales:
 * A = sA * A8, W1 = s1 * W1_8, W2 = s2 * W2_8, with A8, W1_8, W2_8 in the
 * OCP FP8 E4M3 format (raw bytes, row-major), and computes
 *   Gate = fp32(sum_k a8 w1_8) * sg,  Up = fp32(sum_k a8 w2_8) * su,
 *   Y = bf16_RNE(SiLU(Gate) * Up)
 * with the caller's sg = fp32(sA * s1), su = fp32(sA * s2), on
 * v_mfma_f32_32x32x64_f8f6f4 (fp32 accumulation).
 *
 * swiglu_packed_bytes_fp8: bytes of the packed FP8 weights (0 for an invalid
 *   or unsupported shape): one 32 KiB block per 128 output columns and 128 k,
 *   [32-row block rb][64-k step][half h][lane][16 bytes] holding packed row
 *   rb*32 + (lane & 31) (rows 0-127 W1, 128-255 W2 columns of the tile) at
 *   k = 64*step + 32*(lane >> 5) + 16*h + 0..15; padding is zero.
 * swiglu_pack_weights_fp8: W1_8, W2_8 [K,N] bytes -> that layout.
 * swiglu_fused_packed_fp8: Y[M,N] bf16 from A8 [M,K] and the packed weights:
 *   a weight-streaming decode kernel for M <= 32, the data-parallel streaming
 *   schedule above (no workspace, any M >= 0).
 * Shapes: K a multiple of 16 and N a multiple of 8 (else
 * SWIGLU_ERR_UNSUPPORTED_SHAPE); pointers 16-byte aligned; Y must not
 * overlap A8 or the packed weights; validation codes return before any
 * launch; work is enqueued on `stream` with no synchronisation.
 * ---------------------------------------------------------------------- */
size_t swiglu_packed_bytes_fp8(int64_t K, int64_t N);
swiglu_status swiglu_pack_weights_fp8(const uint8_t *W1, const uint8_t *W2,
                                      uint8_t *Wp, int64_t K, int64_t N,
                                      void *stream);
swiglu_status swiglu_fused_packed_fp8(const uint8_t *A, const uint8_t *Wp,
                                      swiglu_bf16 *Y, int64_t M, int64_t K,
                                      int64_t N, float sg, float su,
                                      void *stream);

/* ------------------------------------------------------------------------
 * Column-granular interleaved weights: the pages' W_fused with Gate in the
 * even and Up in the odd columns ([Summary: Methodology], Kernel-2 "Fusion").
 * Same block structure and size as the per-tile pack above (one 32 KiB block
 * per 128 output columns and 64 k, 16-row groups of two 1 KiB halves in
 * fragment lane order, padding zero), but packed row 2c of column tile jt
 * holds W1 column jt*128 + c and row 2c + 1 holds W2 column jt*128 + c.
 * With the weights as the MFMA's first operand, each lane then holds a
 * column's Gate and Up in two adjacent accumulator registers, and the
 * epilogue pairs them without moving data between lanes.  This layout is an
 * ablation of the per-tile layout: the two compute bitwise-identical Y (the
 * same MFMA chain per output element).
 *
 * swiglu_pack_weights_interleaved / swiglu_unpack_weights_interleaved: as
 *   swiglu_pack_weights / swiglu_unpack_weights, in the interleaved layout;
 *   the buffer size is swiglu_packed_bytes(K, N).
 * swiglu_fused_packed_interleaved: Y = SiLU(A W1) * (A W2) from interleaved
 *   packed weights on the data-parallel streaming schedule (no workspace, any
 *   M >= 0); arguments, validation codes and stream semantics as
 *   swiglu_fused_packed.
 * ---------------------------------------------------------------------- */
swiglu_status swiglu_pack_weights_interleaved(const swiglu_bf16 *W1,
                                              const swiglu_bf16 *W2,
                                              swiglu_bf16 *Wp, int64_t K,
                                              int64_t N, void *stream);
swiglu_status swiglu_unpack_weights_interleaved(const swiglu_bf16 *Wp,
                                                swiglu_bf16 *W1, swiglu_bf16 *W2,
                                                int64_t K, int64_t N,
                                                void *stream);
swiglu_status swiglu_fused_packed_interleaved(const swiglu_bf16 *A,
                                              const swiglu_bf16 *Wp,
                                              swiglu_bf16 *Y, int64_t M,
                                              int64_t K, int64_t N, void *stream);

/* ------------------------------------------------------------------------
 * The unfused pipeline the pages measure against ([Summary: Problem
 * Statement]: two GEMMs materialise Gate and Up in memory, then a separate
 * element-wise activation reads them back; [Summary: Results]: "PyTorch
 * eager" baseline), built from this library's own kernels.
 *
 * swiglu_gemm_bf16: C[M,N] = bf16_RNE(A[M,K] x W[K,N]), fp32 accumulation,
 *   W row-major.  C must not overlap A or W.
 * swiglu_silu_mul:  Y[i] = bf16_RNE(SiLU(G[i]) * U[i]) for i < count, fp32 math
 *   from bf16 inputs; Y must not overlap G or U.  count >= 0, any value.
 * swiglu_unfused:   G = gemm(A, W1); U = gemm(A, W2); Y = silu_mul(G, U).
 *   G_scratch and U_scratch are caller-owned [M,N] bf16 device buffers.
 * ---------------------------------------------------------------------- */
swiglu_status swiglu_gemm_bf16(const swiglu_bf16 *A, const swiglu_bf16 *W,
                               swiglu_bf16 *C, int64_t M, int64_t K, int64_t N,
                               void *stream);
swiglu_status swiglu_silu_mul(const swiglu_bf16 *G, const swiglu_bf16 *U,
                              swiglu_bf16 *Y, int64_t count, void *stream);
swiglu_status swiglu_unfused(const swiglu_bf16 *A, const swiglu_bf16 *W1,
                             const swiglu_bf16 *W2, swiglu_bf16 *G_scratch,
                             swiglu_bf16 *U_scratch, swiglu_bf16 *Y, int64_t M,
                             int64_t K, int64_t N, void *stream);

/* ------------------------------------------------------------------------
 * The same unfused pipeline on this library's fastest GEMM: one weight
 * packed once (model-load time) into the fused pack's block layout, so the
 * plain GEMM runs on the fused product's own schedules (the weight-streaming
 * decode kernel for small M, the streaming MFMA grid otherwise) and the
 * fused-vs-unfused comparison measures the materialised Gate and Up, not a
 * slower GEMM ([Summary: Problem Statement]: two GEMMs, then the activation
 * reading them back; [Summary: Results]: the eager baseline).
 *
 * Single-weight pack of W [K,N]: tile jt (of ceil(N/256)) holds W's columns
 * jt*256 + 0..255 as its 256 packed rows, in the block layout of
 * swiglu_pack_weights (packed row p = g*16 + l%16 of 16-row group g):
 *   Wg = for jt, kb (64-deep block), g in 0..15, h in 0..1, l in 0..63,
 *        e in 0..7:  W[k][n], k = kb*64 + h*32 + (l/16)*8 + e,
 *                             n = jt*256 + g*16 + l%16;  zero past K or N.
 *
 * swiglu_gemm_packed_bytes: size of Wg in bytes (0 for an invalid shape).
 * swiglu_gemm_pack_weight:  W [K,N] -> Wg; Wg must not overlap W.
 * swiglu_gemm_workspace_bytes: bytes of fp32 partial sums swiglu_gemm_packed
 *   uses for (M,K,N) when given that much workspace: the fused product's AUTO
 *   rule on the pack's tiled width (ceil(N/256)*128 columns) asks for split-K
 *   when its data-parallel tiles would leave most CUs idle; then
 *   splits * M * 2 * ceil(N/256)*128 * 4 bytes, else 0.
 * swiglu_gemm_packed:       C[M,N] = bf16_RNE(A[M,K] x W), fp32 accumulation
 *   in the fused product's MFMA order; C must not overlap A or Wg.  With a
 *   workspace of at least swiglu_gemm_workspace_bytes(M,K,N) bytes (16-byte
 *   aligned device memory, not overlapping A, Wg or C; caller-owned, contents
 *   on entry irrelevant) a split-K plan runs split (the splits' fp32 partial
 *   sums of each output added in split order by a second launch, so results
 *   are deterministic); with less, or workspace NULL, the data-parallel
 *   schedule runs (no error).  Products whose activations reach 2 GiB run as
 *   row chunks, data-parallel.
 * swiglu_unfused_packed:    G = gemm_packed(A, W1g); U = gemm_packed(A, W2g);
 *   Y = silu_mul(G, U); G_scratch, U_scratch, Y as in swiglu_unfused (the two
 *   GEMMs without workspace, i.e. data-parallel).
 * All: K and N multiples of 8, pointers 16-byte aligned, M == 0 returns
 * SWIGLU_OK without a launch, validation before any launch, work enqueued
 * on `stream` with no synchronisation.
 * ---------------------------------------------------------------------- */
size_t swiglu_gemm_packed_bytes(int64_t K, int64_t N);
swiglu_status swiglu_gemm_pack_weight(const swiglu_bf16 *W, swiglu_bf16 *Wg,
                                      int64_t K, int64_t N, void *stream);
size_t swiglu_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N);
swiglu_status swiglu_gemm_packed(const swiglu_bf16 *A, const swiglu_bf16 *Wg,
                                 swiglu_bf16 *C, int64_t M, int64_t K, int64_t N,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);
swiglu_status swiglu_unfused_packed(const swiglu_bf16 *A, const swiglu_bf16 *W1g,
                                    const swiglu_bf16 *W2g,
                                    swiglu_bf16 *G_scratch,
                                    swiglu_bf16 *U_scratch, swiglu_bf16 *Y,
                                    int64_t M, int64_t K, int64_t N,
                                    void *stream);

/* ------------------------------------------------------------------------
 * The whole gated MLP block: the SwiGLU product followed by the down
 * projection back to the model width, Z[M,K] = bf16_RNE(Y[M,N] x W3[N,K])
 * with fp32 accumulation.  The pages give SwiGLU's cost as a share of MLP
 * execution time ([Summary: Problem Statement], 9-37 %; the speedup falling
 * with model size in [Summary: Results]); these entry points are that MLP,
 * fused and unfused, so the share can be measured.
 *
 * The down projection is a plain GEMM outside the fused product: W3 [N,K]
 * is passed in the single-weight pack (W3g = swiglu_gemm_pack_weight of the
 * [N,K] matrix, swiglu_gemm_packed_bytes(N, K) bytes) and Z =
 * swiglu_gemm_packed(Y, W3g, workspace) with N as the depth.
 *
 * swiglu_mlp_workspace_bytes: workspace for the fastest schedules of
 *   swiglu_mlp_packed / swiglu_mlp_unfused / swiglu_mlp_down: the larger of
 *   swiglu_workspace_bytes(M,K,N,variant) (the fused product) and
 *   swiglu_gemm_workspace_bytes(M,N,K) (the down projection).
 * swiglu_mlp_packed:  Y = swiglu_fused_packed(A, Wp, ...), then Z = Y x W3.
 *   Y is a caller-owned [M,N] bf16 device buffer and holds the SwiGLU
 *   product on return; workspace, workspace_bytes and variant are those of
 *   swiglu_fused_packed, and the same workspace then serves the down
 *   projection as in swiglu_gemm_packed (split-K only if it is large
 *   enough).  Z must not overlap A, Wp, W3g, Y or the workspace; Y must not
 *   overlap W3g (nor the inputs, as in swiglu_fused_packed).
 * swiglu_mlp_unfused: Y = swiglu_unfused_packed(A, W1g, W2g, G, U, ...), then
 *   Z = Y x W3 (W1g, W2g single-weight packs of W1, W2 [K,N]), the down
 *   projection with the workspace as in swiglu_gemm_packed (may be NULL); Z
 *   must not overlap any other buffer or the workspace, and no scratch may
 *   overlap W3g.
 * swiglu_mlp_down:    the down projection alone, Z = Y x W3 (the step both
 *   entry points above end with), the workspace as in swiglu_gemm_packed;
 *   Z must not overlap Y or W3g.
 * All: K and N multiples of 8, pointers 16-byte aligned; M == 0 returns
 * SWIGLU_OK without a launch; the validation codes return before any launch;
 * a launch failure returns SWIGLU_ERR_HIP; work is enqueued on `stream`
 * with no synchronisation.
 * ---------------------------------------------------------------------- */
size_t swiglu_mlp_workspace_bytes(int64_t M, int64_t K, int64_t N, int variant);
swiglu_status swiglu_mlp_packed(const swiglu_bf16 *A, const swiglu_bf16 *Wp,
                                const swiglu_bf16 *W3g, swiglu_bf16 *Y,
                                swiglu_bf16 *Z, int64_t M, int64_t K, int64_t N,
                                void *workspace, size_t workspace_bytes,
                                int variant, void *stream);
swiglu_status swiglu_mlp_down(const swiglu_bf16 *Y, const swiglu_bf16 *W3g,
                             swiglu_bf16 *Z, int64_t M, int64_t K, int64_t N,
                             void *workspace, size_t workspace_bytes,
                             void *stream);
swiglu_status swiglu_mlp_unfused(const swiglu_bf16 *A, const swiglu_bf16 *W1g,
                                 const swiglu_bf16 *W2g, const swiglu_bf16 *W3g,
                                 swiglu_bf16 *G_scratch, swiglu_bf16 *U_scratch,
                                 swiglu_bf16 *Y, swiglu_bf16 *Z, int64_t M,
                                 int64_t K, int64_t N, void *workspace,
                                 size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_H_ */
