/*
 * Exercises the fp64 oracle (oracle/oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host: every entry point, every transpose pair,
 * padded leading dimensions, empty and one-element shapes, many threads.  Values
 * are checked where they are exact (the 2x3x2 worked example of "GEMM o Coração
 * Matemático" §1 and integer inputs, on which the i-p-j and dot-product orders of
 * §2 / §2.1 agree exactly).  Exit status 0: no finding and every check held.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemm_f64(char, char, int64_t, int64_t, int64_t, double, const double*, int64_t,
                    const double*, int64_t, double, double*, int64_t, int);
int oracle_gemm_dot_f64(char, char, int64_t, int64_t, int64_t, double, const double*, int64_t,
                        const double*, int64_t, double, double*, int64_t);
int oracle_swiglu_f64(int64_t, int64_t, int64_t, const double*, const double*, double, double,
                      double*, int);
double oracle_silu_f64(double);
double oracle_f16_to_f64(uint16_t);
double oracle_bf16_to_f64(uint16_t);
double oracle_e4m3_to_f64(uint8_t);
void oracle_decode_f16(const uint16_t*, double*, int64_t);
void oracle_decode_bf16(const uint16_t*, double*, int64_t);
void oracle_decode_e4m3(const uint8_t*, double*, int64_t);
void oracle_interleave(const void*, const void*, void*, int64_t, int64_t, int);
void oracle_deinterleave(const void*, void*, void*, int64_t, int64_t, int);
int oracle_max_threads(void);

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);   \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

/* exact-size heap blocks, so any read or write past them is reported */
static double* dalloc(int64_t n) { return (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double)); }

static void worked_example(void) {
    /* A = [[1,2,0],[0,1,3]], B = [[4,1],[2,0],[1,5]]; alpha 2, beta 1, C_old = I */
    const double a[6] = {1, 2, 0, 0, 1, 3}, b[6] = {4, 1, 2, 0, 1, 5};
    double* A = dalloc(6);
    double* B = dalloc(6);
    double* C = dalloc(4);
    memcpy(A, a, sizeof a);
    memcpy(B, b, sizeof b);
    const double c0[4] = {1, 0, 0, 1}, want[4] = {17, 2, 10, 31};
    memcpy(C, c0, sizeof c0);
    CHECK(oracle_gemm_f64('N', 'N', 2, 2, 3, 2.0, A, 3, B, 2, 1.0, C, 2, 2) == 0);
    for (int i = 0; i < 4; ++i) CHECK(C[i] == want[i]);
    for (int i = 0; i < 4; ++i) C[i] = NAN;       /* beta = 0 never reads C_old */
    CHECK(oracle_gemm_f64('N', 'N', 2, 2, 3, 1.0, A, 3, B, 2, 0.0, C, 2, 1) == 0);
    CHECK(C[0] == 8 && C[1] == 1 && C[2] == 5 && C[3] == 15);
    CHECK(oracle_gemm_f64('X', 'N', 2, 2, 3, 1.0, A, 3, B, 2, 0.0, C, 2, 1) < 0);
    CHECK(oracle_gemm_f64('N', 'N', -1, 2, 3, 1.0, A, 3, B, 2, 0.0, C, 2, 1) < 0);
    free(A);
    free(B);
    free(C);
}

/* every transpose pair, padded ld, integer values: both loop orders agree exactly */
static void transposes(int64_t M, int64_t N, int64_t K, int pad, int threads) {
    const char tr[2] = {'N', 'T'};
    for (int ta = 0; ta < 2; ++ta)
        for (int tb = 0; tb < 2; ++tb) {
            const int64_t ar = ta ? K : M, ac = ta ? M : K, br = tb ? N : K, bc = tb ? K : N;
            const int64_t lda = (ac > 0 ? ac : 1) + pad, ldb = (bc > 0 ? bc : 1) + pad;
            const int64_t ldc = (N > 0 ? N : 1) + pad;
            const int64_t na = ar > 0 ? (ar - 1) * lda + ac : 0;
            const int64_t nb = br > 0 ? (br - 1) * ldb + bc : 0;
            const int64_t nc = M > 0 ? (M - 1) * ldc + N : 0;
            double* A = dalloc(na);
            double* B = dalloc(nb);
            double* C1 = dalloc(nc);
            double* C2 = dalloc(nc);
            for (int64_t i = 0; i < na; ++i) A[i] = (double)((i * 7 + 3) % 9) - 4.0;
            for (int64_t i = 0; i < nb; ++i) B[i] = (double)((i * 5 + 1) % 7) - 3.0;
            for (int64_t i = 0; i < nc; ++i) C1[i] = C2[i] = (double)(i % 5);
            CHECK(oracle_gemm_f64(tr[ta], tr[tb], M, N, K, 2.0, A, lda, B, ldb, 0.5, C1, ldc,
                                  threads) == 0);
            CHECK(oracle_gemm_dot_f64(tr[ta], tr[tb], M, N, K, 2.0, A, lda, B, ldb, 0.5, C2,
                                      ldc) == 0);
            for (int64_t i = 0; i < nc; ++i) CHECK(C1[i] == C2[i]);
            free(A);
            free(B);
            free(C1);
            free(C2);
        }
}

static void swiglu_and_layout(int threads) {
    const int64_t M = 5, N = 7, K = 9;
    double* A = dalloc(M * K);
    double* Wf = dalloc(K * 2 * N);
    double* Y = dalloc(M * N);
    for (int64_t i = 0; i < M * K; ++i) A[i] = (double)(i % 5) - 2.0;
    for (int64_t i = 0; i < K * 2 * N; ++i) Wf[i] = (double)(i % 3) - 1.0;
    CHECK(oracle_swiglu_f64(M, N, K, A, Wf, 1.0, 1.0, Y, threads) == 0);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double g = 0, u = 0;
            for (int64_t p = 0; p < K; ++p) {
                g += A[m * K + p] * Wf[p * 2 * N + 2 * n];
                u += A[m * K + p] * Wf[p * 2 * N + 2 * n + 1];
            }
            CHECK(Y[m * N + n] == oracle_silu_f64(g) * u);
        }
    CHECK(oracle_swiglu_f64(0, N, K, A, Wf, 1.0, 1.0, Y, threads) == 0);
    CHECK(oracle_silu_f64(0.0) == 0.0);
    CHECK(oracle_silu_f64(-1000.0) == -0.0);
    free(A);
    free(Wf);
    free(Y);

    /* interleave / de-interleave round trip for every element size */
    const int sizes[3] = {1, 2, 4};
    for (int s = 0; s < 3; ++s) {
        const int es = sizes[s];
        const int64_t k = 3, n = 5, bytes = k * n * es;
        unsigned char* w1 = (unsigned char*)malloc((size_t)bytes);
        unsigned char* w2 = (unsigned char*)malloc((size_t)bytes);
        unsigned char* wf = (unsigned char*)malloc((size_t)(2 * bytes));
        unsigned char* r1 = (unsigned char*)malloc((size_t)bytes);
        unsigned char* r2 = (unsigned char*)malloc((size_t)bytes);
        for (int64_t i = 0; i < bytes; ++i) {
            w1[i] = (unsigned char)(i * 3 + 1);
            w2[i] = (unsigned char)(i * 5 + 2);
        }
        oracle_interleave(w1, w2, wf, k, n, es);
        oracle_deinterleave(wf, r1, r2, k, n, es);
        CHECK(memcmp(w1, r1, (size_t)bytes) == 0 && memcmp(w2, r2, (size_t)bytes) == 0);
        CHECK(memcmp(wf, w1, (size_t)es) == 0 && memcmp(wf + es, w2, (size_t)es) == 0);
        free(w1);
        free(w2);
        free(wf);
        free(r1);
        free(r2);
    }
}

static void decoders(void) {
    uint16_t* h = (uint16_t*)malloc(65536 * sizeof(uint16_t));
    double* d = dalloc(65536);
    for (int i = 0; i < 65536; ++i) h[i] = (uint16_t)i;
    oracle_decode_f16(h, d, 65536);
    CHECK(d[0x3c00] == 1.0 && d[0xc000] == -2.0 && d[0x0001] == ldexp(1.0, -24));
    CHECK(isinf(d[0x7c00]) && isnan(d[0x7e00]));
    oracle_decode_bf16(h, d, 65536);
    CHECK(d[0x3f80] == 1.0 && d[0x0001] == ldexp(1.0, -133));
    uint8_t q[256];
    for (int i = 0; i < 256; ++i) q[i] = (uint8_t)i;
    oracle_decode_e4m3(q, d, 256);
    CHECK(d[0x7e] == 448.0 && isnan(d[0x7f]) && d[0x01] == ldexp(1.0, -9) && d[0x38] == 1.0);
    free(h);
    free(d);
}

int main(void) {
    const int threads = oracle_max_threads() > 4 ? 4 : oracle_max_threads();
    worked_example();
    static const int64_t shapes[][3] = {{0, 3, 4}, {3, 0, 4}, {3, 4, 0}, {1, 1, 1},
                                        {2, 3, 2}, {7, 5, 11}, {33, 17, 9}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
        transposes(shapes[i][0], shapes[i][1], shapes[i][2], 0, threads);
        transposes(shapes[i][0], shapes[i][1], shapes[i][2], 3, threads);
    }
    swiglu_and_layout(threads);
    decoders();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
