/*
 * Exercises the argument checking of the C ABI (include/swiglu_gemm.h) on the host
 * under AddressSanitizer and UndefinedBehaviorSanitizer: every entry point with
 * each invalid argument (which must return -i before any HIP call), the quick
 * returns that enqueue nothing, sg_status_string over its whole range,
 * sg_last_config into short buffers, and sg_release with nothing allocated.  It
 * needs no GPU.  Exit status 0: no finding and every status as documented.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "swiglu_gemm.h"

static int failures = 0;
#define EXPECT(call, want)                                                         \
    do {                                                                           \
        const int got_ = (call);                                                   \
        if (got_ != (want)) {                                                      \
            fprintf(stderr, "line %d: %s returned %d, want %d\n", __LINE__, #call,  \
                    got_, (want));                                                 \
            ++failures;                                                            \
        }                                                                          \
    } while (0)

int main(void) {
    static char buf[64];
    void* P = buf;     /* never dereferenced: every call below returns before a launch */
    void* Z = NULL;
    const int F16 = SG_F16, BF = SG_BF16, F8 = SG_F8E4M3;

    /* sg_gemm: arguments in order */
    EXPECT(sg_gemm('X', 'N', 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, F16, Z), -1);
    EXPECT(sg_gemm('N', 'x', 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, F16, Z), -2);
    EXPECT(sg_gemm('N', 'N', -1, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, F16, Z), -3);
    EXPECT(sg_gemm('N', 'N', 4, -1, 4, 1.f, P, 4, P, 4, 0.f, P, 4, F16, Z), -4);
    EXPECT(sg_gemm('N', 'N', 4, 4, -1, 1.f, P, 4, P, 4, 0.f, P, 4, F16, Z), -5);
    EXPECT(sg_gemm('N', 'N', 4, 4, 4, 1.f, Z, 4, P, 4, 0.f, P, 4, F16, Z), -7);
    EXPECT(sg_gemm('N', 'N', 4, 4, 8, 1.f, P, 7, P, 4, 0.f, P, 4, F16, Z), -8);
    EXPECT(sg_gemm('T', 'N', 9, 4, 8, 1.f, P, 8, P, 4, 0.f, P, 4, F16, Z), -8);
    EXPECT(sg_gemm('N', 'N', 4, 4, 4, 1.f, P, 4, Z, 4, 0.f, P, 4, F16, Z), -9);
    EXPECT(sg_gemm('N', 'N', 4, 6, 4, 1.f, P, 4, P, 5, 0.f, P, 6, F16, Z), -10);
    EXPECT(sg_gemm('N', 'T', 4, 6, 9, 1.f, P, 9, P, 8, 0.f, P, 6, F16, Z), -10);
    EXPECT(sg_gemm('N', 'N', 4, 4, 4, 1.f, P, 4, P, 4, 0.f, Z, 4, F16, Z), -12);
    EXPECT(sg_gemm('N', 'N', 4, 6, 4, 1.f, P, 4, P, 6, 0.f, P, 5, F16, Z), -13);
    EXPECT(sg_gemm('N', 'N', 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, 7, Z), -14);
    EXPECT(sg_gemm('N', 'N', 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, -1, Z), -14);
    /* quick returns: nothing to write */
    EXPECT(sg_gemm('N', 'N', 0, 4, 4, 1.f, Z, 4, Z, 4, 0.f, Z, 4, F16, Z), 0);
    EXPECT(sg_gemm('T', 'T', 4, 0, 4, 1.f, Z, 4, Z, 4, 0.f, Z, 1, BF, Z), 0);

    /* sg_gemm_ex: the epilogue (-15) and its conflict with beta (-11) */
    sg_epilogue e = {NULL, SG_F32, SG_ACT_NONE, -1, 1.0f};
    EXPECT(sg_gemm_ex('N', 'N', 0, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, F16, &e, Z), 0);
    e.activation = 99;
    EXPECT(sg_gemm_ex('N', 'N', 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, F16, &e, Z), -15);
    e.activation = SG_ACT_GELU;
    e.out_dtype = SG_BF16;
    EXPECT(sg_gemm_ex('N', 'N', 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, F16, &e, Z), -15);
    e.out_dtype = F8;
    e.out_scale = 0.0f;
    EXPECT(sg_gemm_ex('N', 'N', 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, F16, &e, Z), -15);
    e.out_scale = INFINITY;
    EXPECT(sg_gemm_ex('N', 'N', 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, F16, &e, Z), -15);
    e.out_scale = 0.5f;
    EXPECT(sg_gemm_ex('N', 'N', 4, 4, 4, 1.f, P, 4, P, 4, 0.5f, P, 4, F16, &e, Z), -11);
    e.out_dtype = -1;
    e.bias = P;
    e.bias_dtype = F8;
    EXPECT(sg_gemm_ex('N', 'N', 4, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, F16, &e, Z), -15);
    EXPECT(sg_gemm_ex('N', 'N', 4, 4, 4, 1.f, P, 4, P, 3, 0.f, P, 4, F16, &e, Z), -10);
    EXPECT(sg_gemm_ex('N', 'N', 0, 4, 4, 1.f, P, 4, P, 4, 0.f, P, 4, F16, NULL, Z), 0);

    /* sg_gemm_strided_batched */
    EXPECT(sg_gemm_strided_batched('N', 'N', 4, 4, 4, 1.f, P, 4, -1, P, 4, 0, 0.f, P, 4, 16,
                                   2, BF, Z), -9);
    EXPECT(sg_gemm_strided_batched('N', 'N', 4, 4, 4, 1.f, P, 4, 0, P, 4, -1, 0.f, P, 4, 16,
                                   2, BF, Z), -12);
    EXPECT(sg_gemm_strided_batched('N', 'N', 4, 4, 4, 1.f, P, 4, 0, P, 4, 0, 0.f, P, 4, 15,
                                   2, BF, Z), -16);
    EXPECT(sg_gemm_strided_batched('N', 'N', 4, 4, 4, 1.f, P, 4, 0, P, 4, 0, 0.f, P, 4, 16,
                                   -1, BF, Z), -17);
    EXPECT(sg_gemm_strided_batched('N', 'N', 4, 4, 4, 1.f, P, 4, 0, P, 4, 0, 0.f, P, 4, 16,
                                   70000, BF, Z), -17);
    EXPECT(sg_gemm_strided_batched('N', 'N', 4, 4, 4, 1.f, P, 4, 0, P, 4, 0, 0.f, P, 4, 16,
                                   2, 9, Z), -18);
    EXPECT(sg_gemm_strided_batched('N', 'N', 4, 4, 4, 1.f, P, 4, 0, P, 4, 0, 0.f, P, 4, 16,
                                   0, BF, Z), 0);

    /* sg_swiglu_gemm */
    EXPECT(sg_swiglu_gemm(Z, P, P, 4, 4, 4, BF, 1.f, 1.f, Z), -1);
    EXPECT(sg_swiglu_gemm(P, Z, P, 4, 4, 4, BF, 1.f, 1.f, Z), -2);
    EXPECT(sg_swiglu_gemm(P, P, Z, 4, 4, 4, BF, 1.f, 1.f, Z), -3);
    EXPECT(sg_swiglu_gemm(P, P, P, -4, 4, 4, BF, 1.f, 1.f, Z), -4);
    EXPECT(sg_swiglu_gemm(P, P, P, 4, -4, 4, BF, 1.f, 1.f, Z), -5);
    EXPECT(sg_swiglu_gemm(P, P, P, 4, 4, -4, BF, 1.f, 1.f, Z), -6);
    EXPECT(sg_swiglu_gemm(P, P, P, 4, 4, 4, SG_F32, 1.f, 1.f, Z), -7);
    EXPECT(sg_swiglu_gemm(P, P, P, 4, 4, 4, F8, NAN, 1.f, Z), -8);
    EXPECT(sg_swiglu_gemm(P, P, P, 4, 4, 4, F8, 1.f, -2.f, Z), -9);
    EXPECT(sg_swiglu_gemm(P, P, P, 4, 4, 4, BF, 2.f, 1.f, Z), -8);
    EXPECT(sg_swiglu_gemm(P, P, P, 4, 4, 4, BF, 1.f, 0.5f, Z), -9);
    EXPECT(sg_swiglu_gemm(P, P, P, 0, 4, 4, BF, 1.f, 1.f, Z), 0);

    /* sg_swiglu_gemm_w12 */
    EXPECT(sg_swiglu_gemm_w12(P, Z, P, P, 4, 4, 4, BF, 1.f, 1.f, Z), -2);
    EXPECT(sg_swiglu_gemm_w12(P, P, Z, P, 4, 4, 4, BF, 1.f, 1.f, Z), -3);
    EXPECT(sg_swiglu_gemm_w12(P, P, P, Z, 4, 4, 4, BF, 1.f, 1.f, Z), -4);
    EXPECT(sg_swiglu_gemm_w12(P, P, P, P, 4, 4, 4, F8, 1.f, 0.f, Z), -10);
    EXPECT(sg_swiglu_gemm_w12(P, P, P, P, 4, 0, 4, BF, 1.f, 1.f, Z), 0);

    /* helpers */
    EXPECT(sg_interleave_gate_up(Z, P, P, 1, 1, BF, Z), -1);
    EXPECT(sg_interleave_gate_up(P, P, P, 1, -1, BF, Z), -5);
    EXPECT(sg_interleave_gate_up(P, P, P, 0, 5, BF, Z), 0);
    EXPECT(sg_silu_mul(P, P, P, 1, 1, SG_F32, Z), -6);
    EXPECT(sg_silu_mul(P, P, P, 0, 3, BF, Z), 0);

    for (int s = -20; s <= 0; ++s) {
        const char* t = sg_status_string(s);
        if (!t || !*t) {
            fprintf(stderr, "empty status string for %d\n", s);
            ++failures;
        }
    }
    char small[4];
    const int n = sg_last_config(small, (int)sizeof small);
    if (n < 0 || small[sizeof small - 1] != '\0') ++failures;
    EXPECT(sg_last_config(NULL, 0) >= 0, 1);
    sg_release();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ABI sanitizer driver: ok\n");
    return 0;
}
