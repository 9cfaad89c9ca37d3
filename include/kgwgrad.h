/*
 * kgwgrad.h -- K-grouped weight-gradient GEMM for Mixture-of-Experts training on
 * AMD Instinct MI355X (gfx950). C ABI of libkgwgrad.so.
 *
 * Operation (page "How to Use DeepGEMM Weight Gradient Kernels for Training
 * Backward Passes": lede, "Understanding K-Grouped Weight Gradient Kernels",
 * "FP8 Implementation Example", "BF16 Alternative"; GitHub issue "Is DeepGEMM
 * directly applicable to backward in training?", qijiaxing's comment of
 * 2025-03-26 on per-128-token scales along the accumulation axis applied after
 * accumulation):
 *
 *   Expert g owns the contiguous token rows [off[g], off[g+1]) of
 *     A [K_total, M]  (activations, row-major, M contiguous) and
 *     B [K_total, N]  (output gradients, row-major, N contiguous),
 *   where off[0] = 0 and off[g+1] = off[g] + ks[g]. For every g:
 *
 *     D[g] = C[g] (or 0) + sum over token blocks kb of expert g of
 *            (sa[boff[g]+kb, :] outer sb[boff[g]+kb, :]) * (A_kb^T . B_kb)
 *
 *   with blocks of gran_k tokens that restart at each expert's first token (the
 *   last block of an expert may be partial) and boff[g+1] = boff[g] +
 *   ceil(ks[g] / gran_k). Empty experts (ks[g] == 0) are skipped: D[g] = C[g]
 *   bit for bit, or +0.0 without C ("Dispatch and Tensor-Map Handling").
 *
 * Memory: every pointer is a device pointer; the caller owns every buffer. The
 * library allocates no memory per call and never synchronises inside kg_wgrad.
 *
 * Thread safety: calls on different streams may run concurrently; they share
 * one per-device status word (see kg_status).
 *
 * Environment: with KG_VERBOSE set (to any value) the HIP runtime's errors go to
 * stderr; with KG_PRINT_CONFIG set, every kg_wgrad* launch's configuration (layout, kind,
 * tile and stage shape, whole tiles or stream-K, grid, tiles, LDS bytes) does, as the
 * knowledge-base index page's debugging article describes for the pages' own
 * kernel-configuration switch.
 */
#ifndef KGWGRAD_H
#define KGWGRAD_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input kinds (argument `dtype`). */
typedef enum {
  KG_E4M3_F32SCALE = 0, /* A, B: fp8 e4m3fn bytes; sa, sb: fp32 per (block, channel)      */
  KG_E4M3_UE8M0 = 1,    /* A, B: fp8 e4m3fn bytes; sa, sb: uint8 exponent e, scale 2^(e-127) */
  KG_BF16 = 2           /* A, B: bf16; sa, sb must be NULL; gran_k is ignored              */
} kg_dtype;

/*
 * Flag OR-ed into `dtype` for the fp8 kinds: contract with the fp8 MFMA instead of
 * widening the fp8 values to bf16 first. Twice the MFMA rate, but gfx950's fp8 MFMA
 * adds each group of 8 products aligned to the largest of them with about 13
 * bits, so the result is accurate to roughly 1e-4 of sum|a*b| rather than to
 * fp32 rounding (the default). Invalid with KG_BF16.
 */
#define KG_FLAG_FP8_MFMA 0x100

/*
 * Flag OR-ed into `dtype`: D (and C, when given) hold bf16 instead of fp32 (the
 * how-to page's FP8 example allocates a bf16 D; its FAQ describes accumulation into
 * a bf16 output). The sum C + sum_kb(...) is formed in fp32 as without the flag and
 * rounded once to the nearest bf16, ties to even. Empty experts copy C bit for bit
 * (or write +0.0). With a workspace, such calls never take the stream-K mode.
 */
#define KG_FLAG_D_BF16 0x200

/* Return codes. */
typedef enum {
  KG_OK = 0,
  KG_ERR_NULL = -1,        /* a required pointer is NULL, or sa/sb given for bf16          */
  KG_ERR_SHAPE = -2,       /* G, M, N or K_total negative                                  */
  KG_ERR_GRAN = -3,        /* fp8 with gran_k not in {32, 128}                             */
  KG_ERR_DTYPE = -4,       /* unknown dtype, or an invalid flag                            */
  KG_ERR_ALIGN = -5,       /* M or N not a multiple of 16, or a pointer not 16-byte aligned */
  KG_ERR_ALIAS = -6,       /* C and D overlap without being the same buffer                */
  KG_ERR_UNSUPPORTED = -7, /* a combination this build does not implement (see kg_wgrad)   */
  KG_ERR_HIP = -8,         /* the HIP runtime reported an error                            */
  KG_ERR_KSUM = -9,        /* some ks[g] < 0, or sum(ks) != K_total (reported by kg_status) */
  KG_ERR_SPLIT = -10,      /* reserved: the stream-K mode no longer waits for partial tiles,
                              so nothing reports this code any more                         */
  KG_ERR_SCALE_ROWS = -11, /* the scale tensors hold fewer rows than the experts' blocks need,
                              sum_g ceil(ks[g] / gran_k): returned when scale_rows <
                              ceil(K_total / gran_k), else found on the device (reported by
                              kg_status; nothing is written)                                */
  KG_ERR_SCALE_RANGE = -12 /* KG_E4M3_UE8M0 in the default mode: a block's scales lie outside
                              the accuracy envelope (see kg_wgrad); D is written, but the
                              block's terms may be inexact (reported by kg_status)          */
} kg_status_code;

/*
 * kg_wgrad -- enqueue D = C + K-grouped A^T B on `stream`.
 *
 *   A      [K_total, M]   fp8 e4m3fn bytes, or bf16
 *   sa     [nblk, M]      fp32 (KG_E4M3_F32SCALE) or uint8 E8M0 (KG_E4M3_UE8M0); NULL for bf16
 *   B      [K_total, N]   same element type as A
 *   sb     [nblk, N]      same type as sa; NULL for bf16
 *   C      [G, M, N] fp32 (bf16 with KG_FLAG_D_BF16), may be NULL (treated as 0) or
 *          equal to D (in-place accumulate)
 *   D      [G, M, N] fp32 (bf16 with KG_FLAG_D_BF16), output
 *   ks     [G] int32, device memory: tokens per expert, in expert order
 *   nblk   = sum_g ceil(ks[g] / gran_k), the scale rows the experts' blocks use
 *   K_total  rows of A and B; sum_g ks[g] must equal it
 *   scale_rows  rows that sa and sb each hold (>= nblk); ignored for bf16. The kernel
 *          never reads past row nblk - 1; scale_rows bounds that on the device.
 *   gran_k tokens per scale block: 128 or 32 (fp8); ignored for bf16
 *   stream a hipStream_t (NULL: the default stream)
 *
 * Implemented combinations: (KG_E4M3_F32SCALE, 128), (KG_E4M3_F32SCALE, 32),
 * (KG_E4M3_UE8M0, 32), (KG_E4M3_UE8M0, 128) and KG_BF16. G is limited to 1024
 * (kg_max_groups), M and N to 2^24, M * N to 2^29 and K_total to 2^31 - 1
 * (KG_ERR_UNSUPPORTED beyond).
 *
 * Accuracy (default mode): every product of two fp8 (or bf16) values is exact, sums
 * are fp32, and each block's partial sum is scaled once, so |D - D_exact| stays near
 * 2^-24 sum_t |a b| per term added; the tests hold it to 1e-5 sum_t |a b| + 1e-6 per
 * element and 1e-5 in Frobenius norm. That envelope assumes:
 *  - fp32 scales whose products sa * sb stay in fp32's normal range, and results
 *    (and single products) that fit fp32;
 *  - UE8M0 scales any exponent byte 0 .. 254 (2^-127 .. 2^127) such that, in every
 *    block and for every 64 channels of A and 128 of B that one wave handles, A's
 *    exponents span at most 236 and B's at most 236, and the block's products
 *    2^(ea + eb - 254) lie within 2^-234 .. 2^238. Outside that (or with a NaN scale,
 *    255) the block's terms may be inexact and kg_status reports KG_ERR_SCALE_RANGE.
 *    The fp8-MFMA mode's scaled MFMA takes every exponent 0 .. 254 directly;
 *  - experts of up to about 10^6 tokens: fp32 sums of K random-sign terms drift by
 *    about sqrt(K / 64) * 2^-24 of their norm (the Frobenius bound then nears 1e-5;
 *    sums of few-bit values, e.g. integers, stay exact to 2^24).
 *
 * Returns KG_OK after enqueueing, or an error code before enqueueing anything (D
 * untouched). G == 0, M == 0 or N == 0 return KG_OK without a launch. A ks that
 * does not add up to K_total or holds a negative count is detected on the device:
 * the kernel then writes nothing and records KG_ERR_KSUM for kg_status; so does an
 * nblk above scale_rows (KG_ERR_SCALE_ROWS).
 */
int kg_wgrad(const void* A, const void* sa, const void* B, const void* sb, const void* C,
             void* D, const int32_t* ks, int G, int M, int N, int64_t K_total,
             int64_t scale_rows, int gran_k, int dtype, void* stream);

/*
 * kg_wgrad_ws -- kg_wgrad with a caller-owned workspace that lets small bf16
 * problems use every compute unit.
 *
 * When G <= 64, D is fp32, and the problem's output tiles would occupy at most
 * half of the compute units, or whole rounds of tiles would leave more than 30%
 * of them idle, the token range of every tile is cut across all compute units
 * (stream-K): every workgroup that holds part of a cut tile writes its partial sum
 * to the workspace and counts its arrival; the one that arrives last adds C and the
 * partials in a fixed order, so results do not depend on timing, and no workgroup
 * waits for another (other kernels may run beside it). Other problems, or a NULL /
 * too small workspace, run exactly as kg_wgrad.
 *
 *   workspace        device memory, 256-byte aligned, at least
 *                    kg_wgrad_workspace_bytes() bytes. Its first
 *                    kg_wgrad_workspace_flag_bytes() bytes are arrival counters: they
 *                    must be zero before the first use, and every call that completes
 *                    leaves them zero again; the rest is scratch for partial tiles and
 *                    needs no initialisation. It must not overlap C or D. Calls that
 *                    share a workspace must not run concurrently.
 *   workspace_bytes  its size in bytes
 *
 * Returns and errors as kg_wgrad; KG_ERR_ALIGN for a workspace that is not 256-byte
 * aligned, KG_ERR_ALIAS for one that overlaps C or D.
 */
int kg_wgrad_ws(const void* A, const void* sa, const void* B, const void* sb, const void* C,
                void* D, const int32_t* ks, int G, int M, int N, int64_t K_total,
                int64_t scale_rows, int gran_k, int dtype, void* workspace,
                int64_t workspace_bytes, void* stream);

/*
 * kg_wgrad_noalloc -- kg_wgrad_ws for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid it): the
 * workspace is the library's own static device array (128 MiB + 1 KiB per device,
 * held from the library's first use on a device until the process ends), so the call
 * allocates and frees nothing. Arguments, results and errors as kg_wgrad_ws without
 * the workspace arguments; KG_ERR_UNSUPPORTED on a device with more than 256 compute
 * units (whose stream-K workspace would exceed the array). Before a stream-K launch a
 * small kernel zeroes the array's counters (no memset, so the call may be captured).
 * All calls on one device share the array: calls that overlap in time on one device
 * (other streams, other threads) race and must not be made.
 */
int kg_wgrad_noalloc(const void* A, const void* sa, const void* B, const void* sb, const void* C,
                     void* D, const int32_t* ks, int G, int M, int N, int64_t K_total,
                     int64_t scale_rows, int gran_k, int dtype, void* stream);

/*
 * kg_wgrad_nt, kg_wgrad_nt_ws -- kg_wgrad and kg_wgrad_ws with K-major (NT)
 * operands: the token index is the contiguous one. The GitHub issue page
 * (qijiaxing, 2025-04-03) writes dw = dy^t x as a GEMM of dy^t [h_out, tokens] and
 * x^t [h_in, tokens]; the how-to page's SM90 entry point k_grouped_fp8_gemm_nt_contiguous
 * takes this layout ("API Entry Points", FAQ on the NT and TN variants).
 *
 *   A    [M, lda]  element (t, m) of kg_wgrad's A at A[m * lda + t]; expert g's tokens
 *                  are columns [off[g], off[g+1]) of every row; columns >= K_total
 *                  are never read (padding)
 *   lda  row stride of A in elements: >= K_total, lda * element size a multiple of
 *        16 bytes, and 256 * lda * element size at most 2^32 - 256
 *   B    [N, ldb]  the same for B
 *   ldb  row stride of B in elements, as lda
 *
 * Everything else (scales sa [nblk, M] and sb [nblk, N] with scale_rows, C, D, ks,
 * gran_k, dtype and flags, workspace) is as for kg_wgrad / kg_wgrad_ws, and so is the result: with
 * whole tiles (no stream-K), bit for bit what kg_wgrad returns on the token-major
 * operands.
 * Expert starts need no alignment. Extra errors, returned before anything is
 * enqueued: KG_ERR_SHAPE if lda or ldb < K_total, KG_ERR_ALIGN if a row is not a
 * whole number of 16-byte units, KG_ERR_UNSUPPORTED for a stride beyond the limit.
 */
int kg_wgrad_nt(const void* A, int64_t lda, const void* sa, const void* B, int64_t ldb,
                const void* sb, const void* C, void* D, const int32_t* ks, int G, int M, int N,
                int64_t K_total, int64_t scale_rows, int gran_k, int dtype, void* stream);
int kg_wgrad_nt_ws(const void* A, int64_t lda, const void* sa, const void* B, int64_t ldb,
                   const void* sb, const void* C, void* D, const int32_t* ks, int G, int M,
                   int N, int64_t K_total, int64_t scale_rows, int gran_k, int dtype,
                   void* workspace, int64_t workspace_bytes, void* stream);

/*
 * kg_wgrad_workspace_bytes -- workspace size that kg_wgrad_ws needs on the current
 * device (two 256 KB partial tiles per compute unit plus counters), or -1 if the HIP
 * runtime reports an error.
 */
int64_t kg_wgrad_workspace_bytes(void);

/*
 * kg_wgrad_workspace_flag_bytes -- size of the arrival-counter area at the start of
 * the workspace (zero before first use, kept zero by every call), or -1 if the HIP
 * runtime reports an error.
 */
int64_t kg_wgrad_workspace_flag_bytes(void);

/*
 * kg_status -- synchronise `stream`, then return and clear the device status word of
 * the current device: KG_OK, or the last asynchronous error a call since the previous
 * kg_status recorded (KG_ERR_KSUM, KG_ERR_SCALE_ROWS, KG_ERR_SCALE_RANGE). The how-to
 * page ("Dispatch and Tensor-Map Handling") has the host check the per-expert counts
 * against the operands before any work; with the counts in device memory that check
 * runs in the kernel, which writes nothing on a mismatch and leaves its result here.
 * Returns KG_ERR_HIP if the stream reports an error.
 */
int kg_status(void* stream);

/*
 * kg_debug_offsets -- run the device prefix scan that kg_wgrad's kernels use and
 * write off[G+1] (int64 token offsets) and boff[G+1] (int32 scale-row offsets)
 * to device memory: the expert boundaries that the how-to page's "FP8 Implementation
 * Example" builds from its per-expert counts (its counts 32, 45 and 27 start the
 * experts at tokens 0, 32 and 77 of 104), and the first scale row of each expert.
 * Test hook. Errors: KG_ERR_NULL, KG_ERR_SHAPE (G < 0 or G > 1024), KG_ERR_GRAN
 * (gran_k <= 0), KG_ERR_HIP.
 */
int kg_debug_offsets(const int32_t* ks, int G, int gran_k, int64_t* off, int32_t* boff,
                     void* stream);

/* Largest G accepted by kg_wgrad and kg_debug_offsets. */
int kg_max_groups(void);

/* Source kinds of kg_requant (argument `src`). */
#define KG_SRC_BF16 0       /* X: bf16 [K_total, H]; xs must be NULL                       */
#define KG_SRC_E4M3_1X128 1 /* X: e4m3fn bytes [K_total, H] with xs: fp32 [K_total, H/128],
                               one scale per token per 128 channels (the forward pass's
                               1x128 tiles)                                                */

/*
 * kg_requant -- enqueue the requantisation that produces kg_wgrad's fp8 operands
 * (GitHub issue "Is DeepGEMM directly applicable to backward in training?",
 * soundOfDestiny's comments of 2025-03-12: the weight-gradient GEMM needs scales per
 * channel per 128 tokens, the forward pass keeps fp8 with per-token 1x128 scales, so
 * a requantisation is inevitable).
 *
 *   Q [K_total, H] fp8 e4m3fn bytes and S [nblk, H] (fp32 for KG_E4M3_F32SCALE,
 *   uint8 E8M0 for KG_E4M3_UE8M0), nblk = sum_g ceil(ks[g] / gran_k), such that
 *   kg_wgrad(Q, S, ...) reads them as A (or B) and sa (or sb). For expert g's token
 *   block kb (gran_k tokens from the expert's first token, the last one partial)
 *   and channel h, with x the binary32 source value (bf16 widened, or the e4m3 value
 *   times its token's 1x128 scale as one binary32 product) and amax the block's
 *   largest |x|:
 *     KG_E4M3_F32SCALE: s = amax / 448 (1 if amax == 0), q = e4m3(x / s), binary32
 *                       quotients rounded to nearest;
 *     KG_E4M3_UE8M0:    e = 127 + the smallest k with 2^k >= amax / 448, clamped to
 *                       [0, 254] (127 if amax == 0), q = e4m3(x * 2^(127 - e));
 *   e4m3() rounds to the nearest e4m3fn value, ties to the even code, saturating at
 *   +-448 and keeping the sign; NaN becomes 0x7F. Special values: amax skips NaNs;
 *   an infinite amax gives s = inf (finite x -> signed zero codes, infinite x -> NaN
 *   0x7F) or the E8M0 byte 254 (infinite x -> +-448); a nonzero amax of at most
 *   224 * 2^-149 makes amax / 448 = 0: s = 0 (x != 0 -> +-448, x == 0 -> 0x7F) or
 *   the E8M0 byte 0.
 *
 *   scale_kind  KG_E4M3_F32SCALE or KG_E4M3_UE8M0; gran_k 32 or 128
 *   H           a multiple of 128; X, Q, S 16-byte aligned
 *   s_rows      rows that S holds (>= nblk); no row past nblk - 1 is written
 *
 * Errors (before any launch): KG_ERR_DTYPE, KG_ERR_SHAPE, KG_ERR_GRAN, KG_ERR_NULL,
 * KG_ERR_ALIGN, KG_ERR_ALIAS (outputs overlapping each other or an input),
 * KG_ERR_UNSUPPORTED (G > 1024, H > 2^23, or H * K_total > 2^46), KG_ERR_SCALE_ROWS
 * (s_rows < ceil(K_total / gran_k)),
 * KG_ERR_HIP. A ks that does not add up to K_total (KG_ERR_KSUM), or whose nblk
 * exceeds s_rows (KG_ERR_SCALE_ROWS), is reported by kg_status and nothing is
 * written. G == 0 or H == 0: KG_OK, no launch.
 */
int kg_requant(const void* X, const float* xs, const int32_t* ks, int G, int H, int64_t K_total,
               int gran_k, int src, int scale_kind, void* Q, void* S, int64_t s_rows,
               void* stream);

/*
 * kg_dgrad -- enqueue the M-grouped GEMM of the data gradient, dx = dy . w per expert
 * (GitHub issue "Is DeepGEMM directly applicable to backward in training?": the
 * backward pass of a GEMM is two GEMMs, YouJiacheng 2025-02-26; activations carry
 * 1x128 scales and only weights carry 128x128 block scales, soundOfDestiny
 * 2025-02-28). Expert g owns the contiguous token rows [off[g], off[g+1]) of A,
 * off[g+1] = off[g] + ms[g]; for such a row t and output column n
 *
 *   D[t][n] = sum over kb of sa[kb][t] * sw[g][kb][n/128] *
 *             sum_{k = 128 kb}^{128 kb + 127} A[t][k] * W[g][k][n]
 *
 *   A   [M_total, K]      fp8 e4m3fn bytes (dy, K contiguous)
 *   sa  [K/128, M_total]  fp32, one scale per token per 128 channels
 *   W   [G, K, N]         fp8 e4m3fn bytes (each expert's w as the forward pass
 *                         stores it, N contiguous)
 *   sw  [G, K/128, N/128] fp32, one scale per 128 x 128 block of W
 *   D   [M_total, N]      fp32 output (bf16 with KG_FLAG_D_BF16, rounded to
 *                         nearest even from the fp32 sum)
 *   ms  [G] int32, device memory: tokens per expert, in expert order
 *   flags  KG_FLAG_FP8_MFMA (contract with the fp8 MFMA, accuracy as for kg_wgrad)
 *          and/or KG_FLAG_D_BF16
 *
 * Each block's partial sum is formed exactly from the fp8 products (bf16 MFMA on
 * widened values; see KG_FLAG_FP8_MFMA for the fast mode) and multiplied by its two
 * scales before it is added in fp32. K and N must be multiples of 128 and every
 * pointer 16-byte aligned except sw and ms (4 bytes) (KG_ERR_ALIGN). Errors before
 * any launch: KG_ERR_DTYPE (unknown flag), KG_ERR_SHAPE (negative sizes), KG_ERR_NULL,
 * KG_ERR_ALIGN, KG_ERR_ALIAS (D overlapping an input), KG_ERR_UNSUPPORTED (G > 1024,
 * M_total > 2^31 - 1, or byte offsets within a 256-row tile past 2^31: N > 2097024
 * or K > 8388480), KG_ERR_HIP.
 * A ms that holds a negative count or does not add up to M_total is reported by
 * kg_status (KG_ERR_KSUM) and nothing is written. G, N or M_total == 0: KG_OK, no
 * launch. Rows of D are written exactly once (by the tile that owns them).
 */
int kg_dgrad(const void* A, const float* sa, const void* W, const float* sw, void* D,
             const int32_t* ms, int G, int N, int K, int64_t M_total, int flags, void* stream);

#ifdef __cplusplus
}
#endif
#endif
