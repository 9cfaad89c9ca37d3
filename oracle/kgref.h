/*
 * kgref.h -- CPU oracle for the K-grouped weight-gradient GEMM (host only).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may call this library. The product path never links it, and
 * this header shares nothing with the product's own header.
 *
 * What is computed (page "How to Use DeepGEMM Weight Gradient Kernels for
 * Training Backward Passes", sections "Understanding K-Grouped Weight Gradient
 * Kernels" and "FP8 Implementation Example"; GitHub issue "Is DeepGEMM directly
 * applicable to backward in training?", comment by qijiaxing of 2025-03-26 on
 * the token axis being the accumulation axis whose 128-element blocks share one
 * scale that is applied after accumulation):
 *
 *   expert g owns tokens [off[g], off[g+1]) of A [K_total, M] and B [K_total, N];
 *   D[g][m][n] = C[g][m][n] (or 0) + sum over the group's gran_k-token blocks kb of
 *                SA(g,kb,m) * SB(g,kb,n) * sum_{t in kb} dec(A[t][m]) * dec(B[t][n])
 *
 * All arithmetic is fp64. Every function returns one of the status codes below.
 */
#ifndef KGREF_H
#define KGREF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. Same numeric values as the GPU library's contract. */
#define KGREF_OK 0
#define KGREF_ERR_NULL (-1)
#define KGREF_ERR_SHAPE (-2)
#define KGREF_ERR_GRAN (-3)
#define KGREF_ERR_DTYPE (-4)
#define KGREF_ERR_KSUM (-9)

/* Input kinds. */
#define KGREF_E4M3_F32SCALE 0 /* fp8 e4m3fn data, fp32 scale per (block, channel) */
#define KGREF_E4M3_UE8M0 1    /* fp8 e4m3fn data, one-byte power-of-two scale     */
#define KGREF_BF16 2          /* bf16 data, no scales                             */

/* Decoders, from the format definitions. */
double kgref_e4m3(uint8_t byte);
double kgref_e8m0(uint8_t byte);
double kgref_bf16(uint16_t bits);

/* Rounding of the bf16 output variant: the nearest bf16 code to v (ties to the
 * even code, 2^128 and beyond to infinity, NaN to 0x7FC0), rounded once from
 * fp64. The array form rounds n values. */
uint16_t kgref_bf16_round(double v);
void kgref_bf16_round_array(const double* v, uint16_t* out, int64_t n);

/* Argument checks: shapes >= 0, known dtype, gran_k in {32,128} for fp8,
 * every ks[g] >= 0 and sum(ks) == K_total. */
int kgref_validate(const int32_t* ks, int G, int M, int N, int64_t K_total, int gran_k, int dtype);

/* Exclusive scans: off[g+1] = off[g] + ks[g]; boff[g+1] = boff[g] + ceil(ks[g]/gran_k). */
int kgref_offsets(const int32_t* ks, int G, int gran_k, int64_t* off, int32_t* boff);

/* Full reference over groups [g_lo,g_hi) and rows [m_lo,m_hi).
 * A: uint8 [K_total][M] (fp8) or uint16 [K_total][M] (bf16); B likewise with N.
 * sa: float [nblocks][M] or uint8 [nblocks][M]; sb likewise with N; NULL for bf16.
 * C: float [G][M][N] or NULL.
 * D_out, bound_out: double [(g_hi-g_lo)][(m_hi-m_lo)][N]; bound = sum_t |a(t,m)|*|b(t,n)|.
 * nthreads <= 0 means all host cores. */
int kgref_wgrad(const void* A, const void* sa, const void* B, const void* sb, const float* C,
                const int32_t* ks, int G, int M, int N, int64_t K_total, int gran_k, int dtype,
                int g_lo, int g_hi, int m_lo, int m_hi, double* D_out, double* bound_out,
                int nthreads);

/* The same value for single elements (sg[i], sm[i], sn[i]), i < ns. */
int kgref_wgrad_sampled(const void* A, const void* sa, const void* B, const void* sb,
                        const float* C, const int32_t* ks, int G, int M, int N, int64_t K_total,
                        int gran_k, int dtype, int64_t ns, const int32_t* sg, const int32_t* sm,
                        const int32_t* sn, double* out, double* bound_out, int nthreads);

/* Number of threads the last kgref_wgrad / kgref_wgrad_sampled call used. */
int kgref_last_threads(void);

/* ---- requantiser: the step that produces the GEMM's operands ----
 *
 * For expert g's token block kb (rows [t0, t1), gran_k tokens from the expert's first
 * token, the last block partial) and channel h, with x(t,h) the binary32 source value
 * (bf16 widened, or e4m3 decoded times the token's 1x128 scale as a binary32
 * product) and amax the largest |x| of the block:
 *   SCALE_F32:   s = amax / 448 (binary32; 1 if amax == 0), q = enc(x / s) (binary32 quotient)
 *   SCALE_UE8M0: e = 127 + smallest k with 2^k >= amax / 448 (binary32 quotient), clamped to
 *                [0, 254] (127 if amax == 0); q = enc(x * 2^(127 - e))
 * where enc rounds to the nearest e4m3fn value (ties to the even code, saturating at
 * +-448, sign kept). Scale rows are packed per expert as in the GEMM (boff). */
#define KGREF_SRC_BF16 0       /* X: uint16 bf16 [K_total][H]; xs NULL                       */
#define KGREF_SRC_E4M3_1X128 1 /* X: uint8 e4m3fn [K_total][H]; xs: float [K_total][H/128]   */
#define KGREF_SCALE_F32 0      /* S: float [nblocks][H]                                       */
#define KGREF_SCALE_UE8M0 1    /* S: uint8 [nblocks][H]                                       */

uint8_t kgref_e4m3_encode(double v);
int kgref_requant(const void* X, const float* xs, const int32_t* ks, int G, int H,
                  int64_t K_total, int gran_k, int src, int scale_kind, uint8_t* Q, void* S);

/* ---- M-grouped GEMM of the data gradient (dgrad), 1x128 x 128x128 scales ----
 *
 * Expert g owns the token rows [off[g], off[g+1]) (off from ms like the K-grouped
 * offsets). For such a token t and output column n:
 *   D[t][n] = sum over kb of SA[kb][t] * SW[g][kb][n/128] *
 *             sum_{k = 128 kb}^{128 kb + 127} dec(A[t][k]) * dec(W[g][k][n])
 * A: uint8 e4m3fn [M_total][K]; SA: float [K/128][M_total]; W: uint8 e4m3fn [G][K][N];
 * SW: float [G][K/128][N/128]; K and N multiples of 128 (KGREF_ERR_SHAPE otherwise),
 * ms[g] >= 0 adding up to M_total (KGREF_ERR_KSUM otherwise).
 * kgref_dgrad writes rows [t_lo, t_hi) of D and of the bound sum_k |a||w| (double
 * [(t_hi - t_lo)][N]); kgref_dgrad_sampled the elements (st[i], sn[i]). */
int kgref_dgrad_validate(const int32_t* ms, int G, int N, int K, int64_t M_total);
int kgref_dgrad(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                const int32_t* ms, int G, int N, int K, int64_t M_total, int64_t t_lo,
                int64_t t_hi, double* D_out, double* bound_out, int nthreads);
int kgref_dgrad_sampled(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                        const int32_t* ms, int G, int N, int K, int64_t M_total, int64_t ns,
                        const int64_t* st, const int32_t* sn, double* out, double* bound_out,
                        int nthreads);

#ifdef __cplusplus
}
#endif
#endif
