/*
 * oracle.c -- plain, slow, obviously-correct fp64 CPU oracle for BLAS GEMM and
 * the fused SwiGLU-GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this file; only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or helper with the HIP library.
 *
 * Sources (page title, section):
 *   [GEMM]    "GEMM o Coração Matemático", §1 (classical product, transpose, the
 *             BLAS update C = alpha*op(A)*op(B) + beta*C_old element by element),
 *             §2 (row-major linearisation), §2.1 (the i-p-j loop order, which gives
 *             the same C as the dot-product order in exact arithmetic).
 *   [SWIGLU]  "Resumo Técnico: Sobreposição de Ativação em Nível de Tile para
 *             Inferência Eficiente de LLM", Definição do Problema (Y = SiLU(A W1) ⊙
 *             (A W2)) and Metodologia / Kernel-2 (W_fused in R^{K x 2N}: even columns
 *             gate, odd columns up; the epilogue pairs D[m,2n] with D[m,2n+1]).
 *   [QUANT]   "GEMM o Coração Matemático", §12.4 (per-tensor scale, zero point 0):
 *             the real value of a stored code q is s*q.
 *
 * Precision: every input is first decoded exactly into fp64.  All storage types
 * here have at most 24 significant bits, so each product is exact in fp64 (at most
 * 48 bits); the only error is fp64 summation in a fixed order (p ascending).
 *
 * Parity pins: every function here is pinned by a CPU test against something
 * other than itself (the worked 2x3x2 example of §1, brute force in exact rational
 * arithmetic, numpy's fp64 matmul, closed forms of SiLU, torch's dtype casts for
 * the decoders).  None of them is "parity unpinned".
 *
 * Built with plain gcc -O2 (no -ffast-math, no vector intrinsics, no blocking);
 * rows of C are independent and run in parallel threads (OpenMP).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* Exact decoders of the storage formats.                                      */
/* ------------------------------------------------------------------------- */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);               /* subnormal: f * 2^(1-15-10) */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);   /* (1 + f/2^10) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16: the upper half of an IEEE binary32 (1 sign, 8 exponent bits with bias
 * 127, 7 fraction bits). */
double oracle_bf16_to_f64(uint16_t b) {
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133);              /* f * 2^(1-127-7) */
    } else if (e == 255) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + f), e - 134);   /* (1 + f/2^7) * 2^(e-127) */
    }
    return sign ? -v : v;
}

/* OCP 8-bit E4M3 ("fn" variant): 1 sign, 4 exponent bits (bias 7), 3 fraction
 * bits; no infinities; S.1111.111 is NaN; largest finite magnitude 448. */
double oracle_e4m3_to_f64(uint8_t q) {
    int sign = (q >> 7) & 1;
    int e = (q >> 3) & 0xf;
    int f = q & 0x7;
    double v;
    if (e == 15 && f == 7) {
        v = NAN;
    } else if (e == 0) {
        v = ldexp((double)f, -9);                /* f * 2^(1-7-3) */
    } else {
        v = ldexp((double)(8 + f), e - 10);      /* (1 + f/8) * 2^(e-7) */
    }
    return sign ? -v : v;
}

void oracle_decode_f16(const uint16_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(in[i]);
}
void oracle_decode_bf16(const uint16_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f64(in[i]);
}
void oracle_decode_e4m3(const uint8_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_to_f64(in[i]);
}
void oracle_decode_f32(const float* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = (double)in[i];
}

/* ------------------------------------------------------------------------- */
/* op(X) element access, row-major with a leading dimension ([GEMM] §1, §2).  */
/* ------------------------------------------------------------------------- */

static int is_trans(char t) { return t == 'T' || t == 't'; }

/* op(A) is M x K.  'N': A is stored M rows of lda; 'T': A is stored K rows of lda
 * and op(A)(i,p) = A(p,i). */
static double opA_at(const double* A, int64_t lda, int ta, int64_t i, int64_t p) {
    return ta ? A[p * lda + i] : A[i * lda + p];
}
/* op(B) is K x N.  'N': B is stored K rows of ldb; 'T': B is stored N rows. */
static double opB_at(const double* B, int64_t ldb, int tb, int64_t p, int64_t j) {
    return tb ? B[j * ldb + p] : B[p * ldb + j];
}

static int check_trans(char t) {
    return t == 'N' || t == 'n' || t == 'T' || t == 't';
}

/*
 * C = alpha * op(A) * op(B) + beta * C_old, in place on C ([GEMM] §1).
 * i-p-j order: for a fixed row i, each term a = op(A)(i,p) is multiplied into the
 * whole row p of op(B) and accumulated into a per-row fp64 accumulator ([GEMM]
 * §2.1, outer-product / AXPY form).  When beta == 0 the old C is never read (BLAS
 * convention), so NaN in C_old cannot propagate.  alpha == 0 or K == 0 leaves
 * C = beta * C_old.
 * Returns 0, or a negative value for an invalid transpose flag or negative size.
 */
int oracle_gemm_f64(char transA, char transB, int64_t M, int64_t N, int64_t K,
                    double alpha, const double* A, int64_t lda,
                    const double* B, int64_t ldb,
                    double beta, double* C, int64_t ldc, int nthreads) {
    if (!check_trans(transA)) return -1;
    if (!check_trans(transB)) return -2;
    if (M < 0) return -3;
    if (N < 0) return -4;
    if (K < 0) return -5;
    int ta = is_trans(transA), tb = is_trans(transB);
    if (nthreads < 1) nthreads = 1;
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (i = 0; i < M; ++i) {
        double* acc = (double*)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
        for (int64_t p = 0; p < K; ++p) {
            double a = opA_at(A, lda, ta, i, p);
            for (int64_t j = 0; j < N; ++j) acc[j] += a * opB_at(B, ldb, tb, p, j);
        }
        for (int64_t j = 0; j < N; ++j) {
            double old = (beta == 0.0) ? 0.0 : beta * C[i * ldc + j];
            C[i * ldc + j] = alpha * acc[j] + old;
        }
        free(acc);
    }
    return 0;
}

/*
 * The same GEMM in the i-j-p (dot-product) order of [GEMM] §2: each C(i,j) is the
 * dot product of row i of op(A) with column j of op(B).  Kept only so the tests can
 * show that the two loop orders agree (exactly on integer inputs).
 */
int oracle_gemm_dot_f64(char transA, char transB, int64_t M, int64_t N, int64_t K,
                        double alpha, const double* A, int64_t lda,
                        const double* B, int64_t ldb,
                        double beta, double* C, int64_t ldc) {
    if (!check_trans(transA) || !check_trans(transB)) return -1;
    if (M < 0 || N < 0 || K < 0) return -3;
    int ta = is_trans(transA), tb = is_trans(transB);
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0;
            for (int64_t p = 0; p < K; ++p)
                s += opA_at(A, lda, ta, i, p) * opB_at(B, ldb, tb, p, j);
            double old = (beta == 0.0) ? 0.0 : beta * C[i * ldc + j];
            C[i * ldc + j] = alpha * s + old;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* SwiGLU ([SWIGLU]).                                                          */
/* ------------------------------------------------------------------------- */

/* SiLU(x) = x * sigmoid(x) = x / (1 + e^{-x}) (Swish with unit slope; the pages
 * name the function but never write it out). */
double oracle_silu_f64(double x) {
    return x / (1.0 + exp(-x));
}

/*
 * Y[m,n] = SiLU(g) * u with g = s * sum_p A[m,p] Wf[p,2n], u = s * sum_p A[m,p]
 * Wf[p,2n+1], s = scale_a * scale_w ([SWIGLU] Definição do Problema; Kernel-2
 * column pairs; [QUANT] dequantisation s*q applied to the accumulated sum).
 * A is M x K (ld K), Wf is K x 2N (ld 2N), Y is M x N (ld N); all fp64.
 */
int oracle_swiglu_f64(int64_t M, int64_t N, int64_t K,
                      const double* A, const double* Wf,
                      double scale_a, double scale_w, double* Y, int nthreads) {
    if (M < 0 || N < 0 || K < 0) return -1;
    const double s = scale_a * scale_w;
    const int64_t N2 = 2 * N;
    if (nthreads < 1) nthreads = 1;
    int64_t m;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (m = 0; m < M; ++m) {
        double* acc = (double*)calloc((size_t)(N2 > 0 ? N2 : 1), sizeof(double));
        for (int64_t p = 0; p < K; ++p) {
            double a = A[m * K + p];
            const double* w = Wf + p * N2;
            for (int64_t j = 0; j < N2; ++j) acc[j] += a * w[j];
        }
        for (int64_t n = 0; n < N; ++n) {
            double g = s * acc[2 * n];
            double u = s * acc[2 * n + 1];
            Y[m * N + n] = oracle_silu_f64(g) * u;
        }
        free(acc);
    }
    return 0;
}

/*
 * W_fused[k, 2n] = W1[k, n], W_fused[k, 2n+1] = W2[k, n] ([SWIGLU] Kernel-2).
 * Byte-level copy of elements of `esize` bytes; W1, W2 are K x N, Wf is K x 2N.
 */
void oracle_interleave(const void* W1, const void* W2, void* Wf,
                       int64_t K, int64_t N, int esize) {
    const char* a = (const char*)W1;
    const char* b = (const char*)W2;
    char* o = (char*)Wf;
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t n = 0; n < N; ++n) {
            memcpy(o + ((k * 2 * N) + 2 * n) * esize, a + (k * N + n) * esize, (size_t)esize);
            memcpy(o + ((k * 2 * N) + 2 * n + 1) * esize, b + (k * N + n) * esize, (size_t)esize);
        }
    }
}

/* The exact inverse of oracle_interleave. */
void oracle_deinterleave(const void* Wf, void* W1, void* W2,
                         int64_t K, int64_t N, int esize) {
    const char* f = (const char*)Wf;
    char* a = (char*)W1;
    char* b = (char*)W2;
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t n = 0; n < N; ++n) {
            memcpy(a + (k * N + n) * esize, f + ((k * 2 * N) + 2 * n) * esize, (size_t)esize);
            memcpy(b + (k * N + n) * esize, f + ((k * 2 * N) + 2 * n + 1) * esize, (size_t)esize);
        }
    }
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
