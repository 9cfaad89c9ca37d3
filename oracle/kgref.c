/*
 * kgref.c -- CPU oracle for the K-grouped weight-gradient GEMM.
 *
 * TEST INFRASTRUCTURE, not the product: only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load this library. It shares no code with
 * the GPU library. Plain C11 + pthreads, fp64 throughout.
 *
 * Method (the pages' wording restated):
 *  - Page "How to Use DeepGEMM Weight Gradient Kernels for Training Backward
 *    Passes", "Understanding K-Grouped Weight Gradient Kernels": every expert keeps
 *    the two output dimensions fixed and owns a variable number of tokens; the
 *    tokens of expert g are a contiguous slice of A [sum K, M] and B [sum K, N]
 *    ("FP8 Implementation Example"). The weight gradient of expert g is the
 *    contraction of its two slices over the token axis.
 *  - GitHub issue "Is DeepGEMM directly applicable to backward in training?",
 *    comments by qijiaxing (2025-03-26, 2025-05-12) and hxdtest (2025-05-09): the
 *    token axis is the accumulation axis; each run of gran_k tokens shares one scale
 *    per channel, and the scale is applied to the block's partial sum after that
 *    block has been accumulated.
 *  - Same how-to page, "Dispatch and Tensor-Map Handling": the group sizes must add
 *    up to the rows of A and B; zero-size groups are skipped. The recipe text under
 *    the FP8 example restricts gran_k to 32 or 128.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - Scale blocks restart at each group start; group g's blocks occupy scale rows
 *    [boff[g], boff[g+1]) with boff[g+1] = boff[g] + ceil(K_g / gran_k). The last
 *    block of a group may be partial and uses its own scale row.
 *  - sa is [nblocks][M], sb is [nblocks][N], row-major.
 *  - The output is fp32 [G][M][N] on the GPU; here it is fp64. An empty group
 *    yields C[g] unchanged, or +0.0 without C.
 *
 * Exactness: every e4m3fn value is an integer multiple of 2^-9 below 2^9 in
 * magnitude, so each product is a multiple of 2^-18 below 2^18 and a sum of at
 * most 128 of them is below 2^25 with 2^-18 resolution: 43 bits, exact in fp64.
 * The block partial is therefore exact; the only roundings are the multiply by the
 * scale product and the fp64 accumulation over blocks.
 */
#include "kgref.h"

#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ---------------------------------------------------------------- decoders */

static double g_e4m3[256];
static pthread_once_t g_once = PTHREAD_ONCE_INIT;

/* OCP e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
 * is subnormal (m/8 * 2^-6); no infinities; 0x7F and 0xFF are NaN; max 448. */
static void build_tables(void) {
  for (int x = 0; x < 256; ++x) {
    int s = (x >> 7) & 1, e = (x >> 3) & 15, m = x & 7;
    double mag;
    if (e == 15 && m == 7)
      mag = NAN;
    else if (e == 0)
      mag = ldexp((double)m, -9); /* (m/8) * 2^-6 */
    else
      mag = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    g_e4m3[x] = s ? -mag : mag;
  }
}

double kgref_e4m3(uint8_t byte) {
  pthread_once(&g_once, build_tables);
  return g_e4m3[byte];
}

/* UE8M0: an unsigned biased exponent, value 2^(e-127); 255 is NaN. */
double kgref_e8m0(uint8_t byte) { return byte == 255 ? NAN : ldexp(1.0, (int)byte - 127); }

/* bf16: the upper 16 bits of an IEEE binary32. */
double kgref_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Nearest bf16 to v, from the format's definition (binary32's exponent range,
 * 8 significant bits): with q the spacing of bf16 values at |v| (2^(e-7) for
 * 2^e <= |v| < 2^(e+1), e >= -126; 2^-133 below 2^-126), |v| / q is rounded to
 * the nearest integer, ties to the even one; results of 2^128 or more become
 * infinity; the sign follows v; NaN gives the quiet NaN code 0x7FC0. This is
 * the rounding of the bf16 output variant of the GEMM (the how-to page's FP8
 * example allocates a bf16 D). The rounding is done once, from fp64, not through
 * binary32. */
uint16_t kgref_bf16_round(double v) {
  if (isnan(v)) return 0x7FC0;
  const uint16_t sign = signbit(v) ? 0x8000 : 0;
  const double a = fabs(v);
  if (a == 0.0) return sign;
  int x;
  frexp(a, &x); /* a = f * 2^x, f in [0.5, 1): 2^(x-1) <= a < 2^x */
  const int e = x - 1;
  const double q = e < -126 ? ldexp(1.0, -133) : ldexp(1.0, e - 7);
  const double n = a / q; /* exact: q is a power of two */
  double r = floor(n);
  const double frac = n - r;
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  const double val = r * q;
  if (val >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
  /* val has at most 8 significant bits inside binary32's range: the binary32
   * conversion is exact and its low 16 bits are zero */
  const float f = (float)val;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (u >> 16));
}

void kgref_bf16_round_array(const double* v, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = kgref_bf16_round(v[i]);
}

/* ---------------------------------------------------------------- checks */

int kgref_validate(const int32_t* ks, int G, int M, int N, int64_t K_total, int gran_k, int dtype) {
  if (G < 0 || M < 0 || N < 0 || K_total < 0) return KGREF_ERR_SHAPE;
  if (dtype != KGREF_E4M3_F32SCALE && dtype != KGREF_E4M3_UE8M0 && dtype != KGREF_BF16)
    return KGREF_ERR_DTYPE;
  if (dtype != KGREF_BF16 && gran_k != 32 && gran_k != 128) return KGREF_ERR_GRAN;
  if (G > 0 && ks == NULL) return KGREF_ERR_NULL;
  int64_t sum = 0;
  for (int g = 0; g < G; ++g) {
    if (ks[g] < 0) return KGREF_ERR_KSUM;
    sum += ks[g];
  }
  if (sum != K_total) return KGREF_ERR_KSUM;
  return KGREF_OK;
}

int kgref_offsets(const int32_t* ks, int G, int gran_k, int64_t* off, int32_t* boff) {
  if (G < 0 || gran_k <= 0) return KGREF_ERR_SHAPE;
  off[0] = 0;
  boff[0] = 0;
  for (int g = 0; g < G; ++g) {
    if (ks[g] < 0) return KGREF_ERR_KSUM;
    off[g + 1] = off[g] + ks[g];
    boff[g + 1] = boff[g] + (ks[g] + gran_k - 1) / gran_k;
  }
  return KGREF_OK;
}

/* ---------------------------------------------------------------- element access */

typedef struct {
  const void *A, *sa, *B, *sb;
  const float* C;
  const int64_t* off;
  const int32_t* boff;
  int M, N, gran_k, dtype;
} problem_t;

static inline double dec_a(const problem_t* p, int64_t t, int m) {
  if (p->dtype == KGREF_BF16) return kgref_bf16(((const uint16_t*)p->A)[t * p->M + m]);
  return g_e4m3[((const uint8_t*)p->A)[t * p->M + m]];
}

static inline double dec_b(const problem_t* p, int64_t t, int n) {
  if (p->dtype == KGREF_BF16) return kgref_bf16(((const uint16_t*)p->B)[t * p->N + n]);
  return g_e4m3[((const uint8_t*)p->B)[t * p->N + n]];
}

/* Scale of scale-row r for channel c of an operand with `width` channels. */
static inline double scale_of(const problem_t* p, const void* s, int64_t r, int c, int width) {
  if (p->dtype == KGREF_BF16) return 1.0;
  if (p->dtype == KGREF_E4M3_F32SCALE) return (double)((const float*)s)[r * width + c];
  return kgref_e8m0(((const uint8_t*)s)[r * width + c]);
}

static inline int block_len(const problem_t* p) {
  /* Tokens per block partial. bf16 carries no scales (every scale is 1), so its runs
   * of gran_k tokens only split the fp64 sum of exact products: the same sum up to
   * fp64 rounding. */
  return p->gran_k;
}

/* ---------------------------------------------------------------- one row of D */

/* D[g][m][:] and its bound, using caller-provided scratch of 4*N doubles. */
static void row_of_d(const problem_t* p, int g, int m, double* d_row, double* bnd_row,
                     double* scratch) {
  const int N = p->N;
  double* part = scratch;           /* block partial, exact for fp8 */
  double* part_abs = scratch + N;   /* block partial of |a||b|      */
  double* acc = scratch + 2 * N;
  double* acc_abs = scratch + 3 * N;
  for (int n = 0; n < N; ++n) acc[n] = acc_abs[n] = 0.0;

  const int64_t t_begin = p->off[g], t_end = p->off[g + 1];
  if (t_end > t_begin) {
    const int L = block_len(p);
    int64_t kb = 0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += L, ++kb) {
      const int64_t t1 = (t0 + L < t_end) ? t0 + L : t_end;
      for (int n = 0; n < N; ++n) part[n] = part_abs[n] = 0.0;
      for (int64_t t = t0; t < t1; ++t) {
        const double a = dec_a(p, t, m);
        const double aa = fabs(a);
        for (int n = 0; n < N; ++n) {
          const double b = dec_b(p, t, n);
          part[n] += a * b;
          part_abs[n] += aa * fabs(b);
        }
      }
      /* scales are applied to the finished block partial */
      const int64_t srow = (int64_t)p->boff[g] + kb;
      const double s_a = scale_of(p, p->sa, srow, m, p->M);
      for (int n = 0; n < N; ++n) {
        const double s = s_a * scale_of(p, p->sb, srow, n, p->N);
        acc[n] += s * part[n];
        acc_abs[n] += fabs(s) * part_abs[n];
      }
    }
  }
  for (int n = 0; n < N; ++n) {
    const double c = p->C ? (double)p->C[((int64_t)g * p->M + m) * N + n] : 0.0;
    /* empty group: D = C exactly (or +0.0) */
    d_row[n] = (t_end > t_begin) ? c + acc[n] : c;
    bnd_row[n] = acc_abs[n];
  }
}

/* One element, same arithmetic as row_of_d. */
static void elem_of_d(const problem_t* p, int g, int m, int n, double* d, double* bnd) {
  double acc = 0.0, acc_abs = 0.0;
  const int64_t t_begin = p->off[g], t_end = p->off[g + 1];
  const int L = block_len(p);
  int64_t kb = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += L, ++kb) {
    const int64_t t1 = (t0 + L < t_end) ? t0 + L : t_end;
    double part = 0.0, part_abs = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
      const double a = dec_a(p, t, m), b = dec_b(p, t, n);
      part += a * b;
      part_abs += fabs(a) * fabs(b);
    }
    const int64_t srow = (int64_t)p->boff[g] + kb;
    const double s = scale_of(p, p->sa, srow, m, p->M) * scale_of(p, p->sb, srow, n, p->N);
    acc += s * part;
    acc_abs += fabs(s) * part_abs;
  }
  const double c = p->C ? (double)p->C[((int64_t)g * p->M + m) * p->N + n] : 0.0;
  *d = (t_end > t_begin) ? c + acc : c;
  *bnd = acc_abs;
}

/* ---------------------------------------------------------------- threading */

static int g_last_threads = 0;
int kgref_last_threads(void) { return g_last_threads; }

static int pick_threads(int requested) {
  if (requested > 0) return requested;
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

typedef struct {
  const problem_t* p;
  int g_lo, g_hi, m_lo, m_hi;
  double *D, *bound;
  atomic_long next;
  long nitems;
  /* sampled mode */
  int64_t ns;
  const int32_t *sg, *sm, *sn;
  int err;
} job_t;

static void* full_worker(void* arg) {
  job_t* j = (job_t*)arg;
  const int N = j->p->N, rows = j->m_hi - j->m_lo;
  double* scratch = (double*)malloc(sizeof(double) * 4 * (size_t)(N > 0 ? N : 1));
  if (!scratch) {
    j->err = 1;
    return NULL;
  }
  for (;;) {
    long it = atomic_fetch_add(&j->next, 1);
    if (it >= j->nitems) break;
    int g = j->g_lo + (int)(it / rows), mm = (int)(it % rows);
    size_t o = ((size_t)(g - j->g_lo) * rows + mm) * N;
    row_of_d(j->p, g, j->m_lo + mm, j->D + o, j->bound + o, scratch);
  }
  free(scratch);
  return NULL;
}

static void* sampled_worker(void* arg) {
  job_t* j = (job_t*)arg;
  for (;;) {
    long it = atomic_fetch_add(&j->next, 1);
    if (it >= j->ns) break;
    elem_of_d(j->p, j->sg[it], j->sm[it], j->sn[it], j->D + it, j->bound + it);
  }
  return NULL;
}

static int run_threads(job_t* job, void* (*fn)(void*), int nthreads) {
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return KGREF_ERR_SHAPE;
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, fn, job) != 0) break;
    ++started;
  }
  if (started == 0) fn(job);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  g_last_threads = started > 0 ? started : 1;
  return job->err ? KGREF_ERR_SHAPE : KGREF_OK;
}

/* ---------------------------------------------------------------- entry points */

static int setup(problem_t* p, int64_t** off, int32_t** boff, const void* A, const void* sa,
                 const void* B, const void* sb, const float* C, const int32_t* ks, int G, int M,
                 int N, int64_t K_total, int gran_k, int dtype) {
  pthread_once(&g_once, build_tables);
  int rc = kgref_validate(ks, G, M, N, K_total, gran_k, dtype);
  if (rc != KGREF_OK) return rc;
  if (K_total > 0 && (A == NULL || B == NULL)) return KGREF_ERR_NULL;
  if (dtype != KGREF_BF16 && K_total > 0 && (sa == NULL || sb == NULL)) return KGREF_ERR_NULL;
  *off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G + 1));
  *boff = (int32_t*)malloc(sizeof(int32_t) * (size_t)(G + 1));
  if (!*off || !*boff) return KGREF_ERR_SHAPE;
  /* bf16 has no scale blocks: one accumulation per group (gran_k only sizes the
   * summation runs, which does not change the exact-product sum beyond rounding). */
  int gk = (dtype == KGREF_BF16) ? (gran_k > 0 ? gran_k : 128) : gran_k;
  kgref_offsets(ks, G, gk, *off, *boff);
  p->A = A;
  p->sa = sa;
  p->B = B;
  p->sb = sb;
  p->C = C;
  p->off = *off;
  p->boff = *boff;
  p->M = M;
  p->N = N;
  p->gran_k = gk;
  p->dtype = dtype;
  return KGREF_OK;
}

int kgref_wgrad(const void* A, const void* sa, const void* B, const void* sb, const float* C,
                const int32_t* ks, int G, int M, int N, int64_t K_total, int gran_k, int dtype,
                int g_lo, int g_hi, int m_lo, int m_hi, double* D_out, double* bound_out,
                int nthreads) {
  problem_t p;
  int64_t* off = NULL;
  int32_t* boff = NULL;
  int rc = setup(&p, &off, &boff, A, sa, B, sb, C, ks, G, M, N, K_total, gran_k, dtype);
  if (rc == KGREF_OK && (g_lo < 0 || g_hi > G || g_lo > g_hi || m_lo < 0 || m_hi > M || m_lo > m_hi))
    rc = KGREF_ERR_SHAPE;
  if (rc == KGREF_OK && (long)(g_hi - g_lo) * (m_hi - m_lo) > 0 && N > 0) {
    if (!D_out || !bound_out) {
      rc = KGREF_ERR_NULL;
    } else {
      job_t job;
      memset(&job, 0, sizeof job);
      job.p = &p;
      job.g_lo = g_lo;
      job.g_hi = g_hi;
      job.m_lo = m_lo;
      job.m_hi = m_hi;
      job.D = D_out;
      job.bound = bound_out;
      atomic_init(&job.next, 0);
      job.nitems = (long)(g_hi - g_lo) * (m_hi - m_lo);
      int nt = pick_threads(nthreads);
      if (nt > job.nitems) nt = (int)job.nitems;
      rc = run_threads(&job, full_worker, nt);
    }
  }
  free(off);
  free(boff);
  return rc;
}

int kgref_wgrad_sampled(const void* A, const void* sa, const void* B, const void* sb,
                        const float* C, const int32_t* ks, int G, int M, int N, int64_t K_total,
                        int gran_k, int dtype, int64_t ns, const int32_t* sg, const int32_t* sm,
                        const int32_t* sn, double* out, double* bound_out, int nthreads) {
  problem_t p;
  int64_t* off = NULL;
  int32_t* boff = NULL;
  int rc = setup(&p, &off, &boff, A, sa, B, sb, C, ks, G, M, N, K_total, gran_k, dtype);
  if (rc == KGREF_OK && ns > 0) {
    if (!sg || !sm || !sn || !out || !bound_out) rc = KGREF_ERR_NULL;
    for (int64_t i = 0; rc == KGREF_OK && i < ns; ++i)
      if (sg[i] < 0 || sg[i] >= G || sm[i] < 0 || sm[i] >= M || sn[i] < 0 || sn[i] >= N)
        rc = KGREF_ERR_SHAPE;
    if (rc == KGREF_OK) {
      job_t job;
      memset(&job, 0, sizeof job);
      job.p = &p;
      job.D = out;
      job.bound = bound_out;
      atomic_init(&job.next, 0);
      job.ns = ns;
      job.sg = sg;
      job.sm = sm;
      job.sn = sn;
      int nt = pick_threads(nthreads);
      if (nt > ns) nt = (int)ns;
      rc = run_threads(&job, sampled_worker, nt);
    }
  }
  free(off);
  free(boff);
  return rc;
}

/* ---------------------------------------------------------------- requantiser
 *
 * The step before the GEMM that the issue page's discussion calls inevitable
 * (soundOfDestiny, 2025-03-12): activations or output gradients, stored as bf16 or
 * as the forward pass's fp8 copy with one fp32 scale per token per 128 channels,
 * become fp8 e4m3fn operands with one scale per channel per gran_k tokens of an
 * expert. Every step is done in the precision the kernels use (fp32 values and
 * divisions), so that the fp8 bytes and the scales are compared bit for bit.
 */

/* Nearest e4m3fn code to v, ties to the even code, magnitudes at or above 448
 * saturating to 448; the sign bit follows v (also for zero); NaN -> 0x7F. The
 * positive codes 0..126 decode to increasing magnitudes, so a binary search over
 * the decode table finds the two neighbours. */
uint8_t kgref_e4m3_encode(double v) {
  pthread_once(&g_once, build_tables);
  if (isnan(v)) return 0x7F;
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  const double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  int lo = 0, hi = 126; /* g_e4m3[lo] <= a < g_e4m3[hi] */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (g_e4m3[mid] <= a)
      lo = mid;
    else
      hi = mid;
  }
  const double dlo = a - g_e4m3[lo], dhi = g_e4m3[hi] - a;
  int c;
  if (dlo < dhi)
    c = lo;
  else if (dhi < dlo)
    c = hi;
  else
    c = (lo % 2 == 0) ? lo : hi;
  return sign | (uint8_t)c;
}

/* Smallest power-of-two exponent k with 2^k >= r (r > 0, a normal or subnormal
 * binary32 value), as the E8M0 byte k + 127 clamped to [0, 254]. An infinite r (a
 * block holding an infinity) has no such k: it takes the clamp's upper end, 254. A
 * zero r (a nonzero amax whose quotient by 448 underflows) is met by every k: the
 * clamp's lower end, 0. */
static uint8_t e8m0_ceil(float r) {
  if (isinf(r)) return 254;
  if (r == 0.0f) return 0;
  int k;
  const double f = frexp((double)r, &k); /* r = f * 2^k, f in [0.5, 1) */
  if (f == 0.5) k -= 1;                   /* r is a power of two */
  int e = k + 127;
  if (e < 0) e = 0;
  if (e > 254) e = 254;
  return (uint8_t)e;
}

int kgref_requant(const void* X, const float* xs, const int32_t* ks, int G, int H,
                  int64_t K_total, int gran_k, int src, int scale_kind, uint8_t* Q, void* S) {
  if (G < 0 || H < 0 || K_total < 0) return KGREF_ERR_SHAPE;
  if (gran_k != 32 && gran_k != 128) return KGREF_ERR_GRAN;
  if ((src != KGREF_SRC_BF16 && src != KGREF_SRC_E4M3_1X128) ||
      (scale_kind != KGREF_SCALE_F32 && scale_kind != KGREF_SCALE_UE8M0))
    return KGREF_ERR_DTYPE;
  if (src == KGREF_SRC_E4M3_1X128 && H % 128 != 0) return KGREF_ERR_SHAPE;
  if (G > 0 && ks == NULL) return KGREF_ERR_NULL;
  int64_t sum = 0;
  for (int g = 0; g < G; ++g) {
    if (ks[g] < 0) return KGREF_ERR_KSUM;
    sum += ks[g];
  }
  if (sum != K_total) return KGREF_ERR_KSUM;
  if (K_total > 0 && H > 0 && (X == NULL || Q == NULL || S == NULL)) return KGREF_ERR_NULL;
  if (src == KGREF_SRC_E4M3_1X128 && K_total > 0 && H > 0 && xs == NULL) return KGREF_ERR_NULL;
  pthread_once(&g_once, build_tables);

  float* col = (float*)malloc(sizeof(float) * (size_t)(gran_k > 0 ? gran_k : 1));
  if (!col) return KGREF_ERR_SHAPE;
  int64_t t_first = 0, brow = 0;
  for (int g = 0; g < G; ++g) {
    for (int64_t t0 = t_first; t0 < t_first + ks[g]; t0 += gran_k, ++brow) {
      const int64_t t1 = t0 + gran_k < t_first + ks[g] ? t0 + gran_k : t_first + ks[g];
      for (int h = 0; h < H; ++h) {
        /* the block's values of channel h, in fp32, and their largest magnitude
         * (NaNs are skipped: the comparison below is false for them) */
        float amax = 0.0f;
        for (int64_t t = t0; t < t1; ++t) {
          float x;
          if (src == KGREF_SRC_BF16) {
            x = (float)kgref_bf16(((const uint16_t*)X)[t * H + h]);
          } else {
            const float d = (float)g_e4m3[((const uint8_t*)X)[t * H + h]];
            x = d * xs[t * (H / 128) + h / 128]; /* binary32 product */
          }
          col[t - t0] = x;
          if (fabsf(x) > amax) amax = fabsf(x);
        }
        if (scale_kind == KGREF_SCALE_F32) {
          const float s = amax == 0.0f ? 1.0f : amax / 448.0f; /* binary32 quotient */
          ((float*)S)[brow * H + h] = s;
          for (int64_t t = t0; t < t1; ++t) {
            const float y = col[t - t0] / s; /* binary32 quotient */
            Q[t * H + h] = kgref_e4m3_encode((double)y);
          }
        } else {
          const uint8_t e = amax == 0.0f ? 127 : e8m0_ceil(amax / 448.0f);
          ((uint8_t*)S)[brow * H + h] = e;
          for (int64_t t = t0; t < t1; ++t)
            Q[t * H + h] = kgref_e4m3_encode(ldexp((double)col[t - t0], 127 - (int)e));
        }
      }
    }
    t_first += ks[g];
  }
  free(col);
  return KGREF_OK;
}

/* ---------------------------------------------------------------- M-grouped dgrad
 *
 * The other backward GEMM (GitHub issue "Is DeepGEMM directly applicable to
 * backward in training?": the backward pass of a GEMM is two GEMMs, YouJiacheng
 * 2025-02-26; the library shipped this one first, LyricZhao 2025-02-26; activations
 * carry 1x128 scales and only weights carry 128x128 block scales, soundOfDestiny
 * 2025-02-28). With y = x w^T in the forward pass, the data gradient is
 * dx = dy w. Per expert g (token rows [off[g], off[g+1]) of dy, contiguous):
 *
 *   D[t][n] = sum over 128-channel blocks kb of the contraction axis of
 *             SA[kb][t] * SW[g][kb][n/128] * sum_{k in kb} dec(A[t][k]) * dec(W[g][k][n])
 *
 * A = dy [M_total][K] (K contiguous), SA [K/128][M_total] fp32 (one scale per token
 * per 128 channels, stored channel-block-major), W [G][K][N] (the expert's weight
 * as the forward pass stores it, N contiguous), SW [G][K/128][N/128] fp32 (one scale
 * per 128x128 block). K and N are multiples of 128. Each block partial is exact in
 * fp64 (as for the K-grouped GEMM); the scales are applied to it once it is formed.
 */

typedef struct {
  const uint8_t *A, *W;
  const float *sa, *sw;
  const int64_t* off;
  int G, N, K;
  int64_t M_total;
} dgrad_t;

static int dgrad_group_of(const dgrad_t* p, int64_t t) {
  int lo = 0, hi = p->G; /* off[lo] <= t < off[hi] */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (p->off[mid] <= t) lo = mid; else hi = mid;
  }
  while (lo < p->G && p->off[lo + 1] <= t) ++lo; /* skip empty experts */
  return lo;
}

static void dgrad_elem(const dgrad_t* p, int64_t t, int n, double* d, double* bnd) {
  const int g = dgrad_group_of(p, t);
  const int nkb = p->K / 128;
  const uint8_t* a = p->A + t * (int64_t)p->K;
  const uint8_t* w = p->W + (int64_t)g * p->K * p->N;
  double acc = 0.0, acc_abs = 0.0;
  for (int kb = 0; kb < nkb; ++kb) {
    double part = 0.0, part_abs = 0.0;
    for (int k = 128 * kb; k < 128 * kb + 128; ++k) {
      const double x = g_e4m3[a[k]], y = g_e4m3[w[(int64_t)k * p->N + n]];
      part += x * y;
      part_abs += fabs(x) * fabs(y);
    }
    const double s = (double)p->sa[(int64_t)kb * p->M_total + t] *
                     (double)p->sw[((int64_t)g * nkb + kb) * (p->N / 128) + n / 128];
    acc += s * part;
    acc_abs += fabs(s) * part_abs;
  }
  *d = acc;
  *bnd = acc_abs;
}

typedef struct {
  const dgrad_t* p;
  int64_t t_lo, ns;
  const int64_t* st;
  const int32_t* sn;
  double *D, *bound;
  atomic_long next;
  long nitems;
} dgrad_job_t;

static void* dgrad_rows_worker(void* arg) {
  dgrad_job_t* j = (dgrad_job_t*)arg;
  const int N = j->p->N;
  for (;;) {
    const long it = atomic_fetch_add(&j->next, 1);
    if (it >= j->nitems) break;
    for (int n = 0; n < N; ++n)
      dgrad_elem(j->p, j->t_lo + it, n, j->D + (size_t)it * N + n, j->bound + (size_t)it * N + n);
  }
  return NULL;
}

static void* dgrad_sampled_worker(void* arg) {
  dgrad_job_t* j = (dgrad_job_t*)arg;
  for (;;) {
    const long it = atomic_fetch_add(&j->next, 1);
    if (it >= j->nitems) break;
    dgrad_elem(j->p, j->st[it], j->sn[it], j->D + it, j->bound + it);
  }
  return NULL;
}

static int dgrad_run(dgrad_job_t* job, void* (*fn)(void*), int nthreads) {
  int nt = pick_threads(nthreads);
  if (nt > job->nitems) nt = (int)job->nitems;
  if (nt < 1) nt = 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
  if (!th) return KGREF_ERR_SHAPE;
  int started = 0;
  for (int i = 0; i < nt; ++i) {
    if (pthread_create(&th[i], NULL, fn, job) != 0) break;
    ++started;
  }
  if (started == 0) fn(job);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  g_last_threads = started > 0 ? started : 1;
  return KGREF_OK;
}

int kgref_dgrad_validate(const int32_t* ms, int G, int N, int K, int64_t M_total) {
  if (G < 0 || N < 0 || K < 0 || M_total < 0) return KGREF_ERR_SHAPE;
  if (K % 128 != 0 || N % 128 != 0) return KGREF_ERR_SHAPE;
  if (G > 0 && ms == NULL) return KGREF_ERR_NULL;
  int64_t sum = 0;
  for (int g = 0; g < G; ++g) {
    if (ms[g] < 0) return KGREF_ERR_KSUM;
    sum += ms[g];
  }
  return sum == M_total ? KGREF_OK : KGREF_ERR_KSUM;
}

static int dgrad_setup(dgrad_t* p, int64_t** off, const uint8_t* A, const float* sa,
                       const uint8_t* W, const float* sw, const int32_t* ms, int G, int N, int K,
                       int64_t M_total) {
  pthread_once(&g_once, build_tables);
  int rc = kgref_dgrad_validate(ms, G, N, K, M_total);
  if (rc != KGREF_OK) return rc;
  if (M_total > 0 && K > 0 && (!A || !sa || !W || !sw)) return KGREF_ERR_NULL;
  *off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G + 1));
  if (!*off) return KGREF_ERR_SHAPE;
  (*off)[0] = 0;
  for (int g = 0; g < G; ++g) (*off)[g + 1] = (*off)[g] + ms[g];
  p->A = A;
  p->W = W;
  p->sa = sa;
  p->sw = sw;
  p->off = *off;
  p->G = G;
  p->N = N;
  p->K = K;
  p->M_total = M_total;
  return KGREF_OK;
}

int kgref_dgrad(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                const int32_t* ms, int G, int N, int K, int64_t M_total, int64_t t_lo,
                int64_t t_hi, double* D_out, double* bound_out, int nthreads) {
  dgrad_t p;
  int64_t* off = NULL;
  int rc = dgrad_setup(&p, &off, A, sa, W, sw, ms, G, N, K, M_total);
  if (rc == KGREF_OK && (t_lo < 0 || t_hi > M_total || t_lo > t_hi)) rc = KGREF_ERR_SHAPE;
  if (rc == KGREF_OK && t_hi > t_lo && N > 0) {
    if (!D_out || !bound_out) {
      rc = KGREF_ERR_NULL;
    } else {
      dgrad_job_t job;
      memset(&job, 0, sizeof job);
      job.p = &p;
      job.t_lo = t_lo;
      job.D = D_out;
      job.bound = bound_out;
      atomic_init(&job.next, 0);
      job.nitems = (long)(t_hi - t_lo);
      rc = dgrad_run(&job, dgrad_rows_worker, nthreads);
    }
  }
  free(off);
  return rc;
}

int kgref_dgrad_sampled(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                        const int32_t* ms, int G, int N, int K, int64_t M_total, int64_t ns,
                        const int64_t* st, const int32_t* sn, double* out, double* bound_out,
                        int nthreads) {
  dgrad_t p;
  int64_t* off = NULL;
  int rc = dgrad_setup(&p, &off, A, sa, W, sw, ms, G, N, K, M_total);
  if (rc == KGREF_OK && ns > 0) {
    if (!st || !sn || !out || !bound_out) rc = KGREF_ERR_NULL;
    for (int64_t i = 0; rc == KGREF_OK && i < ns; ++i)
      if (st[i] < 0 || st[i] >= M_total || sn[i] < 0 || sn[i] >= N) rc = KGREF_ERR_SHAPE;
    if (rc == KGREF_OK) {
      dgrad_job_t job;
      memset(&job, 0, sizeof job);
      job.p = &p;
      job.st = st;
      job.sn = sn;
      job.D = out;
      job.bound = bound_out;
      atomic_init(&job.next, 0);
      job.nitems = (long)ns;
      rc = dgrad_run(&job, dgrad_sampled_worker, nthreads);
    }
  }
  free(off);
  return rc;
}
