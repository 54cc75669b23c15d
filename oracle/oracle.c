/*
 * CPU oracle for the SwiGLU gated-MLP product.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this file's library.  The GPU library never links, includes or calls it,
 * and it shares no source with the GPU library.
 *
 * What it computes (cited to the pages about "Tile-Level Activation Overlap for
 * Efficient LLM Inference"; "Summary" is the gist.science technical summary):
 *
 *   Y = SiLU(A x W1) (.) (A x W2)                Summary, "Problem Statement"
 *
 * A is [M,K], W1 and W2 are [K,N], all bf16 (raw 16-bit patterns, row-major,
 * contiguous).  Gate = A x W1 is the operand that goes through SiLU; Up = A x W2
 * is the multiplier (Summary, "Problem Statement"; Kernel-2 pairs SiLU of the
 * Gate column with the Up column, Summary, "Methodology", Kernel-2 "Fusion").
 * Precision: the pages compare against an FP32 reference (Summary, "Key
 * Contributions", numerical superiority), so this oracle accumulates in fp32:
 *
 *   1. decode bf16 -> fp32 exactly (the bf16 pattern is the top half of fp32);
 *   2. g = sum_k a[i,k] * w1[k,j], u = sum_k a[i,k] * w2[k,j], fp32, k increasing
 *      (each bf16*bf16 product is exact in fp32, so fused or separate
 *      multiply-add give the same sum);
 *   3. s = g / (1 + expf(-g))   -- SiLU(x) = x * sigmoid(x), fp32, libm expf;
 *   4. p = s * u                -- fp32 (the "FP32 reference" value);
 *   5. y = round-to-nearest-even of p to bf16 (IEEE 754 roundTiesToEven on the
 *      bf16 format; NaN stays a quiet NaN with its sign).
 *
 * The unfused pipeline (two GEMMs that write Gate and Up to memory, then a
 * separate elementwise SwiGLU; Summary, "Problem Statement" and "Results") is
 * also defined here: Gate and Up are rounded to bf16 when they are stored, and
 * the elementwise step reads them back as bf16.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- step 1: bf16 -> fp32 (exact) ------------------------------------- */
static inline float bf16_to_f32(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, sizeof f);
    return f;
}

/* ---- step 5: fp32 -> bf16, round to nearest, ties to even -------------- */
uint16_t oracle_bf16_rne(float p) {
    uint32_t b;
    memcpy(&b, &p, sizeof b);
    if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu) != 0u) {
        /* NaN: keep sign and top payload bits, force the quiet bit. */
        return (uint16_t)((b >> 16) | 0x0040u);
    }
    /* Add just under half an ulp of the kept part, plus one more if the kept
       part is odd, then truncate: exact ties go to the even neighbour, and a
       carry out of the exponent field turns the largest finite values into inf. */
    uint32_t lsb = (b >> 16) & 1u;
    b += 0x7FFFu + lsb;
    return (uint16_t)(b >> 16);
}

float oracle_bf16_to_f32(uint16_t h) { return bf16_to_f32(h); }

/* ---- step 3: SiLU in fp32 ---------------------------------------------- */
float oracle_silu(float g) { return g / (1.0f + expf(-g)); }

/* ---- step 2: fp32 GEMM, k increasing ------------------------------------
 * C[i,j] = sum_{k=0}^{K-1} a[i,k] * w[k,j], each partial sum rounded to fp32.
 * The loop nest i -> k -> j keeps, for every (i,j), the same sequence of
 * additions as i -> j -> k (k strictly increasing), so the result is the plain
 * triple-loop value; OpenMP splits rows, which does not touch any sum. */
void oracle_gemm_f32(const uint16_t *A, const uint16_t *W, int64_t M, int64_t K,
                     int64_t N, float *C) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        float *c = C + i * N;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float a = bf16_to_f32(A[i * K + k]);
            const uint16_t *w = W + k * N;
            for (int64_t j = 0; j < N; ++j) {
                const float prod = a * bf16_to_f32(w[j]);
                c[j] = c[j] + prod;
            }
        }
    }
}

/* ---- the fused product, steps 1-5 -----------------------------------------
 * Y  [M,N] bf16 bits (required).
 * P  [M,N] fp32 pre-rounding product s*u (optional, may be NULL).
 * G,U[M,N] fp32 Gate and Up accumulators (optional, may be NULL).
 * Rows are independent; each row uses a private [2,N] fp32 buffer. */
int oracle_swiglu(const uint16_t *A, const uint16_t *W1, const uint16_t *W2,
                  int64_t M, int64_t K, int64_t N, uint16_t *Y, float *P,
                  float *G, float *U) {
    if (M < 0 || K < 0 || N < 0) return 1;
    if (M == 0 || N == 0) return 0;
    int err = 0;
#pragma omp parallel
    {
        float *g = (float *)malloc(sizeof(float) * (size_t)N);
        float *u = (float *)malloc(sizeof(float) * (size_t)N);
        if (!g || !u) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(static)
            for (int64_t i = 0; i < M; ++i) {
                for (int64_t j = 0; j < N; ++j) { g[j] = 0.0f; u[j] = 0.0f; }
                for (int64_t k = 0; k < K; ++k) {
                    const float a = bf16_to_f32(A[i * K + k]);
                    const uint16_t *w1 = W1 + k * N;
                    const uint16_t *w2 = W2 + k * N;
                    for (int64_t j = 0; j < N; ++j) {
                        const float pg = a * bf16_to_f32(w1[j]);
                        const float pu = a * bf16_to_f32(w2[j]);
                        g[j] = g[j] + pg;
                        u[j] = u[j] + pu;
                    }
                }
                for (int64_t j = 0; j < N; ++j) {
                    const float s = oracle_silu(g[j]);
                    const float p = s * u[j];
                    Y[i * N + j] = oracle_bf16_rne(p);
                    if (P) P[i * N + j] = p;
                    if (G) G[i * N + j] = g[j];
                    if (U) U[i * N + j] = u[j];
                }
            }
        }
        free(g);
        free(u);
    }
    return err;
}

/* ---- the unfused pipeline ----------------------------------------------
 * Gate and Up are stored as bf16 (RNE) the way two separate bf16 GEMMs would
 * write them; the elementwise step decodes them, applies steps 3-5 in fp32 and
 * stores bf16.  Gb, Ub may be NULL. */
void oracle_silu_mul(const uint16_t *Gb, const uint16_t *Ub, uint16_t *Y,
                     int64_t count) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const float s = oracle_silu(bf16_to_f32(Gb[t]));
        Y[t] = oracle_bf16_rne(s * bf16_to_f32(Ub[t]));
    }
}

void oracle_gemm_bf16(const uint16_t *A, const uint16_t *W, int64_t M, int64_t K,
                      int64_t N, uint16_t *C) {
    float *acc = (float *)malloc(sizeof(float) * (size_t)(M * N > 0 ? M * N : 1));
    oracle_gemm_f32(A, W, M, K, N, acc);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < M * N; ++t) C[t] = oracle_bf16_rne(acc[t]);
    free(acc);
}

int oracle_unfused(const uint16_t *A, const uint16_t *W1, const uint16_t *W2,
                   int64_t M, int64_t K, int64_t N, uint16_t *Gb, uint16_t *Ub,
                   uint16_t *Y) {
    if (M < 0 || K < 0 || N < 0) return 1;
    if (M == 0 || N == 0) return 0;
    uint16_t *g = Gb ? Gb : (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(M * N));
    uint16_t *u = Ub ? Ub : (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(M * N));
    if (!g || !u) return 2;
    oracle_gemm_bf16(A, W1, M, K, N, g);
    oracle_gemm_bf16(A, W2, M, K, N, u);
    oracle_silu_mul(g, u, Y, M * N);
    if (!Gb) free(g);
    if (!Ub) free(u);
    return 0;
}

/* ---- FP8 (E4M3) variant -------------------------------------------------
 * The pages argue that quantised GEMMs (FP8) make SwiGLU's memory cost
 * relatively larger (Summary, "Problem Statement") but give no scale
 * convention.  This oracle takes the plainest reading: per-tensor scales,
 * A = sA * A8, W1 = s1 * W1_8, W2 = s2 * W2_8, with A8, W1_8, W2_8 in the
 * OCP FP8 E4M3 format (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent field 0 is subnormal, no infinities, S.1111.111 is NaN).
 *   1. decode each byte exactly to fp32;
 *   2. g = sum_k a8*w1_8, u = sum_k a8*w2_8 in fp32, k increasing (every
 *      product of two E4M3 values is exact in fp32);
 *   3. G = g * sg, U = u * su in fp32, with sg = fp32(sA*s1), su = fp32(sA*s2)
 *      computed by the caller;
 *   4.-5. Y = RNE_bf16(SiLU(G) * U) as in the bf16 product. */
float oracle_e4m3_to_f32(uint8_t b) {
    const int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
    float v;
    if (e == 15 && m == 7) {
        v = NAN;
    } else if (e == 0) {
        v = ldexpf((float)m, -9);                  /* m/8 * 2^(1-7) */
    } else {
        v = ldexpf((float)(8 + m), e - 7 - 3);     /* (1 + m/8) * 2^(e-7) */
    }
    return sign ? -v : v;
}

int oracle_swiglu_fp8(const uint8_t *A, const uint8_t *W1, const uint8_t *W2,
                      int64_t M, int64_t K, int64_t N, float sg, float su,
                      uint16_t *Y, float *P) {
    if (M < 0 || K < 0 || N < 0) return 1;
    if (M == 0 || N == 0) return 0;
    float table[256];
    for (int t = 0; t < 256; ++t) table[t] = oracle_e4m3_to_f32((uint8_t)t);
    int err = 0;
#pragma omp parallel
    {
        float *g = (float *)malloc(sizeof(float) * (size_t)N);
        float *u = (float *)malloc(sizeof(float) * (size_t)N);
        if (!g || !u) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(static)
            for (int64_t i = 0; i < M; ++i) {
                for (int64_t j = 0; j < N; ++j) { g[j] = 0.0f; u[j] = 0.0f; }
                for (int64_t k = 0; k < K; ++k) {
                    const float a = table[A[i * K + k]];
                    const uint8_t *w1 = W1 + k * N;
                    const uint8_t *w2 = W2 + k * N;
                    for (int64_t j = 0; j < N; ++j) {
                        const float pg = a * table[w1[j]];
                        const float pu = a * table[w2[j]];
                        g[j] = g[j] + pg;
                        u[j] = u[j] + pu;
                    }
                }
                for (int64_t j = 0; j < N; ++j) {
                    const float G = g[j] * sg;
                    const float U = u[j] * su;
                    const float p = oracle_silu(G) * U;
                    Y[i * N + j] = oracle_bf16_rne(p);
                    if (P) P[i * N + j] = p;
                }
            }
        }
        free(g);
        free(u);
    }
    return err;
}

/* ---- array forms of steps 3 and 5 (for the tests) ----------------------- */
void oracle_bf16_rne_array(const float *p, uint16_t *y, int64_t n) {
    for (int64_t t = 0; t < n; ++t) y[t] = oracle_bf16_rne(p[t]);
}

void oracle_silu_array(const float *x, float *s, int64_t n) {
    for (int64_t t = 0; t < n; ++t) s[t] = oracle_silu(x[t]);
}

/* ---- threading control -------------------------------------------------- */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
