/*
 * CPU oracle for the tiled GEMM  C = epi(alpha * sa*sb * op(A) op(B) + beta * C_in [+ bias]).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct definition that
 * the HIP library is checked against.  It shares no code with the HIP library: its decoders,
 * its loops and its GELU are its own.  Only tests, the smoke check and the CPU-baseline leg of
 * the benchmark may load it.
 *
 * What it computes (the textbook product that every page's tiling only reorganises:
 * "Case Study: The Tiled GEMM" ends in the BLAS form alpha*AB + beta*C; "Case Study: Steel's
 * BlockMMA" applies bias / activation / scaling per element after the product; "Rigel"
 * (arXiv 2606.12765) section 3 builds its reference in float64 from the exact quantised
 * bytes the GPU consumes):
 *
 *   a(i,k) = transA ? A[k*lda + i] : A[i*lda + k]      decoded exactly to double
 *   b(k,j) = transB ? B[j*ldb + k] : B[k*ldb + j]      decoded exactly to double
 *   S(i,j) = sum_k a(i,k) b(k,j)                        double, k ascending
 *   D(i,j) = sa*sb * sum_k |a(i,k) b(k,j)|             double (denominator of the gate)
 *   t      = alpha*(sa*sb)*S + (beta != 0 ? beta*C_in(i,j) : 0) + (BIAS ? bias[j] : 0)
 *   Cref   = GELU ? 0.5*t*erfc(-t/sqrt(2)) : t          double, libm erfc
 *
 * Block-scaled (OCP microscaling, "MX") inputs: each run of 32 consecutive k of a row of op(A)
 * and of a column of op(B) shares one E8M0 scale 2^(e - 127) (e = 255 is NaN), so
 *   a(i,k) = dec(A ...) * 2^(sa[i*ldsa + k/32] - 127),  b(k,j) = dec(B ...) * 2^(sb[j*ldsb + k/32] - 127)
 * with the per-tensor scales then 1.  This is the plain reading of the MX formats that
 * "Rigel" (arXiv 2606.12765) lists next to fp8 (section 1: fp4 and block-scaled MXFP4); the
 * 6-bit element types E2M3 and E3M2 of the same MX family are decoded as the OCP MX v1.0
 * specification defines them (the pages name no 6-bit type).
 *
 * Every product of two decoded inputs is exact in double (at most 24+24 significant bits; a
 * power-of-two block scale only moves the exponent, and 2^(+-127) products stay inside the
 * double range), so the only roundings are the k-ordered sums and the epilogue, each at 2^-53.
 * Build: gcc -O3 -fopenmp -ffp-contract=off (no fast-math: no reassociation, no FMA).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_E4M3 = 3, OR_E5M2 = 4, OR_E2M1 = 5, OR_E2M3 = 6,
       OR_E3M2 = 7 };
enum { OR_EPI_BIAS = 1u, OR_EPI_GELU = 2u };

/* Storage bits per element (E2M1 packs two elements per byte, the 6-bit types four per three
 * bytes). */
static int ebits_of(int t) {
  switch (t) {
    case OR_F32: return 32;
    case OR_F16: return 16;
    case OR_BF16: return 16;
    case OR_E4M3: return 8;
    case OR_E5M2: return 8;
    case OR_E2M1: return 4;
    case OR_E2M3: return 6;
    case OR_E3M2: return 6;
    default: return 0;
  }
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits; subnormals m * 2^-24. */
static double dec_f16(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32 word. */
static double dec_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP 8-bit E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities, NaN only at
 * S.1111.111, largest finite 448, subnormals m * 2^-9. */
static double dec_e4m3(uint8_t q) {
  int s = q >> 7, e = (q >> 3) & 15, m = q & 7;
  double v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

/* OCP 8-bit E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa bits, IEEE-style: exponent 31 is
 * infinity (mantissa 0) or NaN, largest finite 57344, subnormals m * 2^-16. */
static double dec_e5m2(uint8_t q) {
  int s = q >> 7, e = (q >> 2) & 31, m = q & 3;
  double v;
  if (e == 31) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -16);
  else v = ldexp((double)(4 + m), e - 17);
  return s ? -v : v;
}

/* OCP 4-bit E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit, no infinities or NaN:
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (exponent 0 is the subnormal m * 2^-1). */
static double dec_e2m1(uint8_t q) {
  int s = (q >> 3) & 1, e = (q >> 1) & 3, m = q & 1;
  double v = (e == 0) ? 0.5 * m : ldexp((double)(2 + m), e - 2);
  return s ? -v : v;
}

/* The 6-bit element types of the OCP Microscaling Formats (MX) v1.0 specification, neither with
 * infinities or NaN:
 *   E2M3: 1 sign, 2 exponent (bias 1), 3 mantissa bits; largest 7.5, subnormals m * 2^-3;
 *   E3M2: 1 sign, 3 exponent (bias 3), 2 mantissa bits; largest 28, subnormals m * 2^-4. */
static double dec_e2m3(uint8_t q) {
  int s = (q >> 5) & 1, e = (q >> 3) & 3, m = q & 7;
  double v = (e == 0) ? ldexp((double)m, -3) : ldexp((double)(8 + m), e - 4);
  return s ? -v : v;
}
static double dec_e3m2(uint8_t q) {
  int s = (q >> 5) & 1, e = (q >> 2) & 7, m = q & 3;
  double v = (e == 0) ? ldexp((double)m, -4) : ldexp((double)(4 + m), e - 5);
  return s ? -v : v;
}

/* Packed 6-bit storage: element idx occupies bits 6 idx .. 6 idx + 5 of the byte string read
 * as one little-endian integer (four elements per three bytes).  The second byte is read only
 * when the element reaches into it. */
static uint8_t get6(const uint8_t* base, int64_t idx) {
  const int64_t bit = 6 * idx, by = bit >> 3;
  const int sh = (int)(bit & 7);
  unsigned v = (unsigned)base[by] >> sh;
  if (sh > 2) v |= (unsigned)base[by + 1] << (8 - sh);
  return (uint8_t)(v & 63u);
}

/* OCP E8M0 block scale: 2^(e - 127); e = 255 is NaN. */
static double dec_e8m0(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

static double dec_f32(const void* p) {
  float f;
  memcpy(&f, p, 4);
  return (double)f;
}

static double dec_one(int t, const uint8_t* base, int64_t idx) {
  switch (t) {
    case OR_F32: return dec_f32(base + 4 * idx);
    case OR_F16: { uint16_t h; memcpy(&h, base + 2 * idx, 2); return dec_f16(h); }
    case OR_BF16: { uint16_t h; memcpy(&h, base + 2 * idx, 2); return dec_bf16(h); }
    case OR_E4M3: return dec_e4m3(base[idx]);
    case OR_E5M2: return dec_e5m2(base[idx]);
    /* element idx sits in byte idx/2: the low nibble for even idx, the high one for odd */
    case OR_E2M1: return dec_e2m1((uint8_t)((base[idx >> 1] >> (4 * (idx & 1))) & 15));
    case OR_E2M3: return dec_e2m3(get6(base, idx));
    case OR_E3M2: return dec_e3m2(get6(base, idx));
    default: return NAN;
  }
}

/* Decode n E8M0 scale bytes to doubles. */
int oracle_decode_e8m0(const void* src, int64_t n, double* dst) {
  const uint8_t* p = (const uint8_t*)src;
  for (int64_t i = 0; i < n; ++i) dst[i] = dec_e8m0(p[i]);
  return 0;
}

/* Decode n consecutive stored values of type t into doubles. Returns 0, or -1 on bad type. */
int oracle_decode(int t, const void* src, int64_t n, double* dst) {
  if (ebits_of(t) == 0) return -1;
  const uint8_t* p = (const uint8_t*)src;
  for (int64_t i = 0; i < n; ++i) dst[i] = dec_one(t, p, i);
  return 0;
}

/* GELU with the Gauss error function: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), evaluated as
 * 0.5 x erfc(-x / sqrt 2) (the same function; erfc avoids the cancellation of 1 + erf for
 * negative x). */
double oracle_gelu(double t) { return 0.5 * t * erfc(-t / sqrt(2.0)); }

typedef struct {
  int64_t M, N, K;
  int transA, transB;
  double alpha, sa, sb, beta;
  const uint8_t *A, *B, *Cin;
  int64_t lda, ldb, ldc;
  int at, bt, ct;
  unsigned epi;
  const float* bias;
  const uint8_t *sa_blk, *sb_blk; /* E8M0 block scales, or NULL */
  int64_t ldsa, ldsb;
} problem_t;

static int check(const problem_t* p) {
  if (p->M < 0 || p->N < 0 || p->K < 0) return -1;
  if (!ebits_of(p->at) || !ebits_of(p->bt) || !ebits_of(p->ct)) return -1;
  if (p->ct == OR_E2M1 || p->ct == OR_E2M3 || p->ct == OR_E3M2) return -1;
  if ((p->sa_blk != NULL) != (p->sb_blk != NULL)) return -1;
  if (p->sa_blk && (p->K % 32 != 0 || p->ldsa < p->K / 32 || p->ldsb < p->K / 32)) return -1;
  if (p->K > 0 && (!p->A || !p->B)) return -1;
  if (p->beta != 0.0 && !p->Cin) return -1;
  if ((p->epi & OR_EPI_BIAS) && !p->bias) return -1;
  return 0;
}

/* op(A)[i][k] and op(B)[k][j], decoded exactly, block scale applied. */
static double opA(const problem_t* p, int64_t i, int64_t k) {
  double a = dec_one(p->at, p->A, p->transA ? k * p->lda + i : i * p->lda + k);
  if (p->sa_blk) a *= dec_e8m0(p->sa_blk[i * p->ldsa + k / 32]);
  return a;
}
static double opB(const problem_t* p, int64_t k, int64_t j) {
  double b = dec_one(p->bt, p->B, p->transB ? j * p->ldb + k : k * p->ldb + j);
  if (p->sb_blk) b *= dec_e8m0(p->sb_blk[j * p->ldsb + k / 32]);
  return b;
}

/* op(B) as a K x N row-major double matrix. */
static double* decode_opB(const problem_t* p) {
  double* b = (double*)malloc(sizeof(double) * (size_t)(p->K > 0 ? p->K : 1) *
                              (size_t)(p->N > 0 ? p->N : 1));
  if (!b) return NULL;
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < p->K; ++k)
    for (int64_t j = 0; j < p->N; ++j)
      b[k * p->N + j] = opB(p, k, j);
  return b;
}

static double apply_epilogue(const problem_t* p, int64_t i, int64_t j, double s) {
  double t = p->alpha * (p->sa * p->sb) * s;
  if (p->beta != 0.0) t += p->beta * dec_one(p->ct, p->Cin, i * p->ldc + j);
  if (p->epi & OR_EPI_BIAS) t += (double)p->bias[j];
  if (p->epi & OR_EPI_GELU) t = oracle_gelu(t);
  return t;
}

/* Rows [row0, row0 + nrows) of Cref and D (each nrows x N, row-major). */
static int run_rows(const problem_t* p, int64_t row0, int64_t nrows, double* Cref, double* D) {
  if (check(p)) return -1;
  if (row0 < 0 || nrows < 0 || row0 + nrows > p->M) return -1;
  if (nrows == 0 || p->N == 0) return 0;
  double* b = decode_opB(p);
  if (!b) return -2;
  int fail = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)p->N);
    double* d = (double*)malloc(sizeof(double) * (size_t)p->N);
    if (!s || !d) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = row0 + r;
        for (int64_t j = 0; j < p->N; ++j) { s[j] = 0.0; d[j] = 0.0; }
        for (int64_t k = 0; k < p->K; ++k) {
          const double a = opA(p, i, k);
          const double* brow = b + k * p->N;
          for (int64_t j = 0; j < p->N; ++j) {
            const double prod = a * brow[j];
            s[j] += prod;
            d[j] += fabs(prod);
          }
        }
        for (int64_t j = 0; j < p->N; ++j) {
          Cref[r * p->N + j] = apply_epilogue(p, i, j, s[j]);
          D[r * p->N + j] = (p->sa * p->sb) * d[j];
        }
      }
    }
    free(s);
    free(d);
  }
  free(b);
  return fail ? -2 : 0;
}

#define PROBLEM_ARGS                                                                       \
  int64_t M, int64_t N, int64_t K, int transA, int transB, double alpha, const void* A,   \
      int64_t lda, double scale_a, const void* B, int64_t ldb, double scale_b, double beta, \
      const void* Cin, int64_t ldc, int a_type, int b_type, int c_type, unsigned epilogue,  \
      const float* bias

#define FILL_PROBLEM(p)                                                                     \
  problem_t p = {M, N, K, transA, transB, alpha, scale_a, scale_b, beta,                    \
                 (const uint8_t*)A, (const uint8_t*)B, (const uint8_t*)Cin, lda, ldb, ldc,  \
                 a_type, b_type, c_type, epilogue, bias, NULL, NULL, 0, 0}

#define MX_ARGS const void *sa_blk, int64_t ldsa, const void *sb_blk, int64_t ldsb
#define FILL_MX(p)                          \
  p.sa_blk = (const uint8_t*)sa_blk;        \
  p.sb_blk = (const uint8_t*)sb_blk;        \
  p.ldsa = ldsa;                            \
  p.ldsb = ldsb

/* Full M x N result: Cref and D are caller-owned M*N double arrays.  Returns 0 on success. */
int oracle_gemm(PROBLEM_ARGS, double* Cref, double* D) {
  FILL_PROBLEM(p);
  return run_rows(&p, 0, M, Cref, D);
}

/* Rows [row0, row0+nrows): a bounded slice of the full result (used to time the oracle). */
int oracle_gemm_rows(PROBLEM_ARGS, int64_t row0, int64_t nrows, double* Cref, double* D) {
  FILL_PROBLEM(p);
  return run_rows(&p, row0, nrows, Cref, D);
}

/* Selected entries (rows[t], cols[t]), t < npts, each computed on its own with k ascending. */
static int run_points(const problem_t* p, int64_t npts, const int64_t* rows, const int64_t* cols,
                      double* Cref, double* D) {
  if (check(p)) return -1;
  for (int64_t t = 0; t < npts; ++t)
    if (rows[t] < 0 || rows[t] >= p->M || cols[t] < 0 || cols[t] >= p->N) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < npts; ++t) {
    const int64_t i = rows[t], j = cols[t];
    double s = 0.0, d = 0.0;
    for (int64_t k = 0; k < p->K; ++k) {
      const double prod = opA(p, i, k) * opB(p, k, j);
      s += prod;
      d += fabs(prod);
    }
    Cref[t] = apply_epilogue(p, i, j, s);
    D[t] = (p->sa * p->sb) * d;
  }
  return 0;
}

int oracle_gemm_points(PROBLEM_ARGS, int64_t npts, const int64_t* rows, const int64_t* cols,
                       double* Cref, double* D) {
  FILL_PROBLEM(p);
  return run_points(&p, npts, rows, cols, Cref, D);
}

/* Block-scaled variants: the same with E8M0 scales sa_blk (row i of op(A), block k/32 at
 * sa_blk[i*ldsa + k/32]) and sb_blk (column j of op(B) at sb_blk[j*ldsb + k/32]); K % 32 == 0. */
int oracle_gemm_mx(PROBLEM_ARGS, MX_ARGS, double* Cref, double* D) {
  FILL_PROBLEM(p);
  FILL_MX(p);
  return run_rows(&p, 0, M, Cref, D);
}

int oracle_gemm_mx_points(PROBLEM_ARGS, MX_ARGS, int64_t npts, const int64_t* rows,
                          const int64_t* cols, double* Cref, double* D) {
  FILL_PROBLEM(p);
  FILL_MX(p);
  return run_points(&p, npts, rows, cols, Cref, D);
}

/* ---------------------------------------------------------------------------------------
 * Affine group-quantized weights (the quantized matmul the "X3" page names as the main LLM
 * workload: a memory-bound matrix-vector product for decode and a matrix product for prefill,
 * with dequantisation fused into the multiply-add, section 7).  The page fixes no format; the
 * reading taken here:
 *
 *   x(i,k) = dec(X[i*ldx + k])                                  activations, f16 or bf16
 *   q(j,k) = bits == 8 ? Wq[j*ldw + k]                          unsigned codes, row j of W,
 *                      : (Wq[j*ldw + k/2] >> 4*(k%2)) & 15      low nibble first
 *   w(j,k) = s(j, k/G) * q(j,k) + o(j, k/G)                     s, o: f16 or bf16, one per
 *                                                               G consecutive k of a row
 *   S(i,j) = sum_k x(i,k) w(j,k),  D(i,j) = sum_k |x(i,k) w(j,k)|   double, k ascending
 *   Cref   = epi(alpha*S + beta*C_in + bias)                    as for the plain product
 *
 * that is C = X W^T with W (N x K) dequantised.  s*q is exact in double (at most 11 + 8
 * significant bits) and so is s*q + o whenever the two terms are within 2^34 of each other in
 * magnitude, which holds for every generated input; the products with x are then exact too.
 */
typedef struct {
  const uint8_t* W;
  int64_t ldw; /* bytes per row of W */
  int bits;
  int64_t G;
  const uint8_t *S, *O;
  int64_t ldg; /* scales / offsets per row */
  int st;
} qweights_t;

static int qcheck(const problem_t* p, const qweights_t* q) {
  if (check(p)) return -1;
  if (p->at != OR_F16 && p->at != OR_BF16) return -1;
  if (q->st != OR_F16 && q->st != OR_BF16) return -1;
  if (q->bits != 4 && q->bits != 8) return -1;
  if (q->G <= 0 || p->K % q->G != 0) return -1;
  if (p->K > 0 && (!q->W || !q->S || !q->O)) return -1;
  if (q->ldw * 8 < p->K * q->bits || q->ldg < p->K / q->G) return -1;
  return 0;
}

static double q_weight(const qweights_t* q, int64_t j, int64_t k) {
  const uint8_t* row = q->W + j * q->ldw;
  const unsigned v = q->bits == 8 ? row[k] : (unsigned)((row[k >> 1] >> (4 * (k & 1))) & 15);
  const int64_t g = j * q->ldg + k / q->G;
  return dec_one(q->st, q->S, g) * (double)v + dec_one(q->st, q->O, g);
}

static int run_q(const problem_t* p, const qweights_t* q, int64_t npts, const int64_t* rows,
                 const int64_t* cols, double* Cref, double* D) {
  if (qcheck(p, q)) return -1;
  if (!rows) { /* every entry: W^T decoded once as a K x N matrix, then i-k-j */
    if (p->M == 0 || p->N == 0) return 0;
    double* w = (double*)malloc(sizeof(double) * (size_t)(p->K > 0 ? p->K : 1) * (size_t)p->N);
    if (!w) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < p->N; ++j)
      for (int64_t k = 0; k < p->K; ++k) w[k * p->N + j] = q_weight(q, j, k);
    int fail = 0;
#pragma omp parallel
    {
      double* sv = (double*)malloc(sizeof(double) * (size_t)p->N);
      double* dv = (double*)malloc(sizeof(double) * (size_t)p->N);
      if (!sv || !dv) {
#pragma omp atomic write
        fail = 1;
      } else {
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < p->M; ++i) {
          for (int64_t j = 0; j < p->N; ++j) { sv[j] = 0.0; dv[j] = 0.0; }
          for (int64_t k = 0; k < p->K; ++k) {
            const double x = dec_one(p->at, p->A, i * p->lda + k);
            const double* wr = w + k * p->N;
            for (int64_t j = 0; j < p->N; ++j) {
              const double prod = x * wr[j];
              sv[j] += prod;
              dv[j] += fabs(prod);
            }
          }
          for (int64_t j = 0; j < p->N; ++j) {
            Cref[i * p->N + j] = apply_epilogue(p, i, j, sv[j]);
            D[i * p->N + j] = dv[j];
          }
        }
      }
      free(sv);
      free(dv);
    }
    free(w);
    return fail ? -2 : 0;
  }
  for (int64_t t = 0; t < npts; ++t)
    if (rows[t] < 0 || rows[t] >= p->M || cols[t] < 0 || cols[t] >= p->N) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < npts; ++t) {
    const int64_t i = rows[t], j = cols[t];
    double sv = 0.0, dv = 0.0;
    for (int64_t k = 0; k < p->K; ++k) {
      const double prod = dec_one(p->at, p->A, i * p->lda + k) * q_weight(q, j, k);
      sv += prod;
      dv += fabs(prod);
    }
    Cref[t] = apply_epilogue(p, i, j, sv);
    D[t] = dv;
  }
  return 0;
}

#define Q_ARGS                                                                           \
  int64_t M, int64_t N, int64_t K, double alpha, const void* X, int64_t ldx, int x_type, \
      const void* Wq, int64_t ldw, int bits, int64_t group, const void* scales,          \
      const void* offsets, int64_t ldg, int s_type, double beta, const void* Cin,        \
      int64_t ldc, int c_type, unsigned epilogue, const float* bias

#define FILL_Q(p, q)                                                                          \
  problem_t p = {M, N, K, 0, 0, alpha, 1.0, 1.0, beta, (const uint8_t*)X, NULL,              \
                 (const uint8_t*)Cin, ldx, 0, ldc, x_type, x_type, c_type, epilogue, bias,   \
                 NULL, NULL, 0, 0};                                                          \
  qweights_t q = {(const uint8_t*)Wq, ldw, bits, group, (const uint8_t*)scales,              \
                  (const uint8_t*)offsets, ldg, s_type}

/* C = epi(alpha * X W^T + beta * C_in + bias) with W group-quantized (above): full M x N. */
int oracle_qgemm(Q_ARGS, double* Cref, double* D) {
  FILL_Q(p, q);
  p.B = q.W; /* only so that check() sees a non-null B when K > 0 */
  return run_q(&p, &q, 0, NULL, NULL, Cref, D);
}

/* The same at selected entries (rows[t], cols[t]). */
int oracle_qgemm_points(Q_ARGS, int64_t npts, const int64_t* rows, const int64_t* cols,
                        double* Cref, double* D) {
  FILL_Q(p, q);
  p.B = q.W;
  return run_q(&p, &q, npts, rows, cols, Cref, D);
}

/* Number of OpenMP threads a parallel region of the oracle uses. */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}
