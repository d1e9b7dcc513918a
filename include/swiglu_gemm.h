/*
 * swiglu_gemm.h -- C ABI of the MI355X (gfx950) GEMM / fused SwiGLU-GEMM library
 * (libswiglu_gemm.so).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All matrix pointers are DEVICE pointers owned by the caller; the library keeps
 *   no pointer after the enqueued work has finished.  Matrices are row-major with
 *   a leading dimension (the distance, in elements, between the starts of two
 *   consecutive stored rows).
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *   call is asynchronous: it enqueues kernels on `stream` and returns without
 *   synchronising.
 * - Return value: 0 on success; -i when argument i (1-based) is invalid, checked
 *   before any HIP call; a positive hipError_t when a HIP call failed.  Nothing is
 *   printed and nothing aborts.
 * - Output buffers must not overlap input buffers.
 * - dtype codes: SG_F32 = 0, SG_F16 = 1, SG_BF16 = 2, SG_F8E4M3 = 3 (OCP e4m3fn:
 *   bias 7, largest magnitude 448, no infinities).  Every product is accumulated
 *   in fp32 and rounded to the output type (nearest-even) once, at the end.
 * - Split-K workspace (fp32 partial sums) is owned by the library: one buffer per
 *   device, grown on first need (to a power of two, at least 1 MiB), released by
 *   sg_release().  A call fetches it once and passes that address to each of its
 *   kernels.  Growth never synchronises the device: the smaller buffer, which work
 *   enqueued earlier may still read, is kept until sg_release().  Calls that need
 *   the workspace and run concurrently on different streams of one device are
 *   serialised by the caller (the library does not order streams).
 * - Problems with 1..32 rows of A ('N') may run on the decode kernels: a persistent
 *   stream-K pass over the weight and, when a column tile is shared by several
 *   work-groups, a second fix-up launch that adds their partial sums (a fixed
 *   order: results are run-to-run identical).  Its partial sums live in the same
 *   kind of library-owned workspace, with the same rule for concurrent streams.
 */
#ifndef SWIGLU_GEMM_H
#define SWIGLU_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SG_F32 = 0,
    SG_F16 = 1,
    SG_BF16 = 2,
    SG_F8E4M3 = 3
} sg_dtype;

/*
 * sg_gemm: C = alpha * op(A) * op(B) + beta * C_old.
 *
 * The BLAS update of "GEMM o Coração Matemático" §1 (op is the identity or the
 * transpose; alpha and beta scalars), row-major as in its §2.
 *
 *  1 transA  'N'/'n': op(A) = A, A stored M x K (lda >= max(1,K));
 *            'T'/'t': op(A) = A^T, A stored K x M (lda >= max(1,M)).
 *  2 transB  'N'/'n': op(B) = B, B stored K x N (ldb >= max(1,N));
 *            'T'/'t': op(B) = B^T, B stored N x K (ldb >= max(1,K)).
 *  3 M, 4 N, 5 K   sizes of op(A) (M x K), op(B) (K x N) and C (M x N); >= 0.
 *  6 alpha   fp32 scalar.
 *  7 A, 8 lda, 9 B, 10 ldb   operands (see above).
 *  11 beta   fp32 scalar.  beta == 0: C is write-only (C_old is never read, so
 *            NaN/Inf there cannot propagate).
 *  12 C, 13 ldc   M x N output, ldc >= max(1,N).  Elements outside the logical
 *            M x N block (the ld padding) are never written.
 *  14 dtype  SG_F32: A, B, C fp32.  SG_F16 / SG_BF16: A, B, C in that type.
 *            SG_F8E4M3: A, B e4m3 codes, C bf16; per-tensor scales are folded
 *            into alpha by the caller (alpha = s_A * s_B * alpha').
 *  15 stream hipStream_t (void*).
 * Quick returns: M == 0 or N == 0 does nothing; K == 0 or alpha == 0 computes
 * C = beta * C_old without reading A or B.
 * Alignment: any element-aligned pointers and leading dimensions are accepted.
 * For fp16, bf16 and e4m3 the direct-to-LDS kernels run when A and B are 16-byte
 * aligned and lda, ldb times the element size are multiples of 16 (any M, N, K);
 * other fp16 / bf16 problems run on a register-staged kernel, other e4m3 problems
 * on a kernel with one thread per output.
 * Invalid: trans flag (-1/-2), negative size (-3/-4/-5), NULL A/B when they are
 * read (-7/-9), ld too small (-8/-10/-13), NULL C (-12), unknown dtype (-14).
 */
int sg_gemm(char transA, char transB, int64_t M, int64_t N, int64_t K,
            float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
            float beta, void* C, int64_t ldc, int dtype, void* stream);

/* Activations of the GEMM epilogue (sg_epilogue.activation). */
typedef enum {
    SG_ACT_NONE = 0,
    SG_ACT_RELU = 1,      /* max(x, 0) */
    SG_ACT_GELU = 2,      /* x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)) */
    SG_ACT_GELU_TANH = 3, /* x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3))) */
    SG_ACT_SILU = 4       /* x / (1 + e^-x) */
} sg_activation;

/* Extra steps of the GEMM epilogue, applied before the single store. */
typedef struct {
    const void* bias;   /* NULL, or N values (device memory), one per column of C */
    int bias_dtype;     /* SG_F32, SG_F16 or SG_BF16 (ignored when bias is NULL) */
    int activation;     /* sg_activation, applied after the bias */
    int out_dtype;      /* -1: C has sg_gemm's output type; SG_F8E4M3: C holds e4m3 codes */
    float out_scale;    /* SG_F8E4M3 output: per-tensor scale s_C > 0 (finite; its fp32
                           reciprocal must be finite too) */
} sg_epilogue;

/*
 * sg_gemm_noalloc: sg_gemm for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, semantics, kernels and results are those of sg_gemm (bit-identical
 * output for the same problem, with one exception below).  The split-K partial
 * sums, the decode path's partial sums and the 16-byte-row copies of e4m3 operands
 * whose rows are not 16-byte multiples, which sg_gemm keeps in library-allocated
 * workspace, live here in a fixed device array of SG_NOALLOC_SCRATCH_BYTES built
 * into the library: every GPU the library runs on holds one copy until the process
 * ends.  No call allocates or frees device memory (its device address is looked up
 * once per device, on the first call there).
 * - A problem whose chosen kernels need more scratch than that returns
 *   SG_STATUS_SCRATCH_LIMIT before enqueuing anything (C is untouched).
 * - The exception: e4m3 operands whose copies would not fit run the one-thread-
 *   per-output kernel instead of the tile kernels (same tolerance, different
 *   summation order, so not the same bits as sg_gemm).
 * - Every call on one GPU shares that GPU's array, which keeps the last call's
 *   contents; nothing in it needs to start at zero (each partial sum is written
 *   before it is read).  Calls that overlap in time on one GPU (different streams,
 *   or host threads enqueuing concurrently) race on it: order them.
 */
#define SG_NOALLOC_SCRATCH_BYTES (32u << 20)
#define SG_STATUS_SCRATCH_LIMIT (-100)
int sg_gemm_noalloc(char transA, char transB, int64_t M, int64_t N, int64_t K, float alpha,
                    const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                    int64_t ldc, int dtype, void* stream);

/*
 * sg_gemm_ex: sg_gemm with the steps a fused GEMM epilogue folds in before the
 * accumulator is stored ("GEMM o Coração Matemático" §1, closing paragraph, and
 * §13.3, closing paragraph: bias and activations in the epilogue; "为什么 GEMM 是
 * CUDA 的必修课", list of optimisations, epilogue fusion of bias, activation,
 * scale and quantisation):
 *     v = alpha * op(A) * op(B) + beta * C_old
 *     y = act(v + bias[n])
 *     C[m, n] = y rounded once to the output type, or, with out_dtype SG_F8E4M3,
 *               the OCP e4m3fn code of y * r, r = 1/out_scale rounded to fp32
 *               (round to nearest, ties to even, saturating at +-448, NaN to 0x7F;
 *               the per-tensor scale of §12.4; exact division for power-of-two
 *               scales).
 * Attention scores QK^T / sqrt(d_h) are the plain call with transB = 'T' and
 * alpha = 1/sqrt(d_h) (§1); the fused Q, K, V projection is one call on the
 * concatenated weight [W_Q W_K W_V] (N = 3d, §13.1).
 *
 * Arguments 1-14 and 16 as sg_gemm (15 there is the stream):
 *  15 epi    NULL or the steps above; NULL, or no bias, SG_ACT_NONE and
 *            out_dtype -1, is exactly sg_gemm.
 *  16 stream hipStream_t (void*).
 * With an e4m3 output C is M x N bytes (ldc in elements = bytes) and beta must
 * be 0.  Quick returns as sg_gemm: K == 0 or alpha == 0 gives
 * C = out(act(beta * C_old + bias)).
 * Invalid: as sg_gemm; beta != 0 with an e4m3 output (-11); an unknown
 * activation, bias dtype or out_dtype, or out_scale not finite and > 0 (-15).
 */
int sg_gemm_ex(char transA, char transB, int64_t M, int64_t N, int64_t K, float alpha,
               const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C,
               int64_t ldc, int dtype, const sg_epilogue* epi, void* stream);

/*
 * sg_gemm_strided_batched: for b in [0, batch): C_b = alpha * op(A_b) * op(B_b)
 * + beta * C_b, with X_b = X + b * strideX elements -- the same BLAS update as
 * sg_gemm ("GEMM o Coração Matemático" §1, §2) over a batch of equally shaped
 * problems in one launch: the batched products of the same page's §13.2, where
 * attention's score and context steps are one GEMM per (sequence, head).
 *
 * Arguments 1-8 and 10, 11, 13-15, 18, 19 as sg_gemm (transA, transB, M, N, K,
 * alpha, A, lda, B, ldb, beta, C, ldc, dtype, stream); 9 strideA, 12 strideB,
 * 16 strideC: element distance between consecutive problems (>= 0; 0 repeats
 * the operand for every problem; strideC must keep the outputs disjoint:
 * >= (M-1)*ldc + N when batch > 1); 17 batch: number of problems, 0..65535.
 * Split-K is not used inside a batch.  Quick returns as sg_gemm, per problem;
 * batch == 0 does nothing.
 * Invalid: as sg_gemm at the shifted positions (-1..-5, -7, -8, -10, -11, -14,
 * -15, -18), negative stride (-9/-12), overlapping outputs (-16), batch (-17).
 */
int sg_gemm_strided_batched(char transA, char transB, int64_t M, int64_t N, int64_t K,
                            float alpha, const void* A, int64_t lda, int64_t strideA,
                            const void* B, int64_t ldb, int64_t strideB, float beta, void* C,
                            int64_t ldc, int64_t strideC, int64_t batch, int dtype,
                            void* stream);

/*
 * sg_swiglu_gemm: Y = SiLU(s * A * W1) ⊙ (s * A * W2), s = scale_a * scale_w.
 *
 * The gated MLP of "Resumo Técnico: Sobreposição de Ativação em Nível de Tile para
 * Inferência Eficiente de LLM" (Definição do Problema), computed as ONE GEMM over
 * [M, 2N, K] on the column-interleaved W_fused of its Metodologia / Kernel-2 (even
 * columns gate = W1, odd columns up = W2); the epilogue pairs columns (2n, 2n+1)
 * in registers, so the gate and up intermediates never reach memory.
 * SiLU(x) = x / (1 + e^-x).  The scales are the per-tensor dequantisation factors
 * (value = s * code, zero point 0) of "GEMM o Coração Matemático" §12.4, applied
 * to the fp32 sums before SiLU.
 *
 *  1 A       M x K, contiguous (ld = K).
 *  2 Wfused  K x 2N, contiguous (ld = 2N).
 *  3 Y       M x N, contiguous (ld = N).
 *  4 M, 5 N, 6 K   >= 0.
 *  7 dtype   SG_BF16: A, W bf16, Y bf16.  SG_F16: A, W fp16, Y fp16.
 *            SG_F8E4M3: A, W e4m3 codes, Y bf16.
 *  8 scale_a, 9 scale_w   fp32 per-tensor scales; finite and > 0; must be 1.0
 *            unless dtype is SG_F8E4M3.
 *  10 stream hipStream_t (void*).
 * Quick returns: M == 0 or N == 0 does nothing; K == 0 writes Y = 0.
 * Invalid: NULL pointer (-1/-2/-3), negative size (-4/-5/-6), unsupported dtype
 * (-7), bad scale (-8/-9).
 */
int sg_swiglu_gemm(const void* A, const void* Wfused, void* Y,
                   int64_t M, int64_t N, int64_t K, int dtype,
                   float scale_a, float scale_w, void* stream);

/*
 * sg_swiglu_gemm_w12: the same Y = SiLU(s * A * W1) ⊙ (s * A * W2) from separate,
 * non-interleaved W1 and W2 -- the weight layout of Kernel-1 in "Resumo Técnico:
 * Sobreposição de Ativação em Nível de Tile para Inferência Eficiente de LLM"
 * (Metodologia).  One work-group tile loads BN/2 columns of W1 and the same BN/2
 * columns of W2 side by side, so gate and up of every output still meet in
 * registers and never reach memory.  Results equal sg_swiglu_gemm on the
 * interleaved W_fused to the same tolerance (and, for the same tile configuration,
 * bit for bit).
 *
 *  1 A       M x K, contiguous (ld = K).
 *  2 W1, 3 W2   K x N each, contiguous (ld = N).
 *  4 Y       M x N, contiguous (ld = N).
 *  5 M, 6 N, 7 K   >= 0.
 *  8 dtype   as sg_swiglu_gemm.   9 scale_a, 10 scale_w   as sg_swiglu_gemm.
 *  11 stream hipStream_t (void*).
 * Shapes the direct kernel cannot take (rows of A, W1 or W2 that are not 16-byte
 * multiples, unaligned pointers) are run by interleaving W1, W2 into a
 * library-owned buffer (grown on demand, freed by sg_release) and calling
 * sg_swiglu_gemm; calls on several streams of one device must not overlap then.
 * Quick returns: M == 0 or N == 0 does nothing; K == 0 writes Y = 0.
 * Invalid: NULL pointer (-1/-2/-3/-4), negative size (-5/-6/-7), unsupported dtype
 * (-8), bad scale (-9/-10).
 */
int sg_swiglu_gemm_w12(const void* A, const void* W1, const void* W2, void* Y,
                       int64_t M, int64_t N, int64_t K, int dtype,
                       float scale_a, float scale_w, void* stream);

/*
 * sg_interleave_gate_up: Wfused[k, 2n] = W1[k, n], Wfused[k, 2n+1] = W2[k, n]
 * (the W_fused layout of the same page's Kernel-2).  Bit-exact copy.
 *  1 W1, 2 W2   K x N contiguous; 3 Wfused  K x 2N contiguous;
 *  4 K, 5 N >= 0; 6 dtype any sg_dtype (element size 4, 2, 2 or 1 bytes);
 *  7 stream.
 * Invalid: NULL pointer (-1/-2/-3), negative size (-4/-5), unknown dtype (-6).
 */
int sg_interleave_gate_up(const void* W1, const void* W2, void* Wfused,
                          int64_t K, int64_t N, int dtype, void* stream);

/*
 * sg_silu_mul: Y = SiLU(G) ⊙ U, elementwise over M x N contiguous matrices (the
 * separate activation step of the unfused MLP that the same page's Definição do
 * Problema describes: two GEMMs write Gate and Up to memory, then this reads them).
 *  1 G, 2 U, 3 Y   M x N contiguous, dtype SG_BF16 or SG_F16 (all three);
 *  4 M, 5 N >= 0; 6 dtype; 7 stream.
 * Invalid: NULL pointer (-1/-2/-3), negative size (-4/-5), unsupported dtype (-6).
 */
int sg_silu_mul(const void* G, const void* U, void* Y, int64_t M, int64_t N,
                int dtype, void* stream);

/* Text for a status code returned by any sg_* call (static storage). */
const char* sg_status_string(int status);

/* Identifies the build (static storage): "swiglu_gemm source <hash> gfx950", where
 * <hash> is 16 hex digits of the SHA-256 over the library's kernel and ABI sources
 * (swiglu_gemm_amd/build.py, source_hash).  The Python binding compares it with the
 * sources beside the library and refuses a library built from other sources. */
const char* sg_build_info(void);

/*
 * Describes the kernel configuration chosen by the most recent successful
 * sg_gemm / sg_swiglu_gemm call on the calling thread (tile, split count; for a
 * problem run as two launches over column ranges, "columns 0..n1" and the tail's
 * configuration; for the decode kernels their grid and units) as a NUL-terminated
 * string copied into buf (at most len bytes).  Returns the full length of the
 * description.  Meant for logs and tests; the format is not a stable interface.
 */
int sg_last_config(char* buf, int len);

/* Frees the library-owned workspace buffers (current and outgrown) on every device,
 * after synchronising each device that holds one. */
void sg_release(void);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_GEMM_H */
