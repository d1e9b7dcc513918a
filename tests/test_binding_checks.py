"""The Python binding refuses, before any library call, tensors that do not hold
what the C ABI would read or write: wrong shapes, dtypes, strides or storage too
short for the sizes and leading dimensions given.  CPU tensors reach every check
(the device is checked last), so a call that passes all of them ends in the
"must be on the GPU" error here."""
import pytest

torch = pytest.importorskip("torch")

import swiglu_gemm_amd as sg

ON_GPU = "on the GPU"


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def raises(exc, match, fn, *a, **k):
    with pytest.raises(exc, match=match):
        fn(*a, **k)


# ------------------------------------------------------------------ gemm
def test_gemm_well_formed_reaches_the_device_check():
    raises(ValueError, ON_GPU, sg.gemm, t(8, 16), t(16, 4), t(8, 4))
    raises(ValueError, ON_GPU, sg.gemm, t(16, 8), t(4, 16), t(8, 4), transA="T", transB="T")
    # e4m3 operands write a bf16 C
    raises(ValueError, ON_GPU, sg.gemm, t(8, 16, dtype=torch.float8_e4m3fn),
           t(16, 4, dtype=torch.float8_e4m3fn), t(8, 4))


def test_gemm_noalloc_checks_like_gemm():
    raises(ValueError, ON_GPU, sg.gemm_noalloc, t(8, 16), t(16, 4), t(8, 4))
    raises(ValueError, "rows", sg.gemm_noalloc, t(8, 16), t(15, 4), t(8, 4))
    raises(ValueError, "C holds", sg.gemm_noalloc, t(8, 16), t(16, 4), t(7, 4))
    raises(TypeError, "C has dtype", sg.gemm_noalloc, t(8, 16), t(16, 4),
           t(8, 4, dtype=torch.float16))


def test_gemm_inner_dimensions_must_agree():
    raises(ValueError, "rows", sg.gemm, t(8, 16), t(15, 4), t(8, 4))
    raises(ValueError, "rows", sg.gemm, t(8, 16), t(4, 15), t(8, 4), transB="T")


def test_gemm_output_too_small_or_wrong_type():
    raises(ValueError, "C holds", sg.gemm, t(8, 16), t(16, 4), t(7, 4))
    raises(ValueError, "C holds", sg.gemm, t(8, 16), t(16, 4), t(31), M=8, N=4, K=16,
           lda=16, ldb=4, ldc=4)
    raises(TypeError, "C has dtype", sg.gemm, t(8, 16), t(16, 4), t(8, 4, dtype=torch.float16))
    raises(TypeError, "C has dtype", sg.gemm, t(8, 16), t(16, 4), t(8, 4, dtype=torch.uint8))
    raises(TypeError, "C has dtype", sg.gemm, t(8, 16, dtype=torch.float8_e4m3fn),
           t(16, 4, dtype=torch.float8_e4m3fn), t(8, 4, dtype=torch.uint8))


def test_gemm_operand_dtypes_must_match():
    raises(TypeError, "B has", sg.gemm, t(8, 16), t(16, 4, dtype=torch.float32), t(8, 4))
    raises(TypeError, "A has", sg.gemm, t(8, 16, dtype=torch.uint8), t(16, 4), t(8, 4),
           dtype=sg.SG_BF16)


def test_gemm_explicit_sizes_checked_against_storage():
    A, B, C = t(8, 16), t(16, 4), t(8, 4)
    raises(ValueError, "A holds", sg.gemm, A, B, C, M=9, N=4, K=16, lda=16, ldb=4, ldc=4)
    raises(ValueError, "A holds", sg.gemm, A, B, C, M=8, N=4, K=16, lda=17, ldb=4, ldc=4)
    raises(ValueError, "B holds", sg.gemm, A, B, C, M=8, N=4, K=16, lda=16, ldb=5, ldc=4)
    raises(ValueError, "C holds", sg.gemm, A, B, C, M=8, N=4, K=16, lda=16, ldb=4, ldc=5)
    raises(ValueError, ON_GPU, sg.gemm, A, B, C, M=8, N=4, K=16, lda=16, ldb=4, ldc=4)
    # a view that starts late in its storage has fewer elements ahead of it
    flat = t(8 * 16)
    raises(ValueError, "A holds", sg.gemm, flat[1:], B, C, M=8, N=4, K=16, lda=16, ldb=4, ldc=4)
    # K = 0 reads neither operand
    raises(ValueError, ON_GPU, sg.gemm, t(1), t(1), C, M=8, N=4, K=0, lda=1, ldb=4, ldc=4)


def test_gemm_strided_last_dimension_rejected():
    raises(ValueError, "contiguous", sg.gemm, t(16, 8).t(), t(16, 4), t(8, 4))
    raises(ValueError, "transA", sg.gemm, t(8, 16), t(16, 4), t(8, 4), transA="X")


def test_gemm_ex_checks():
    A, B = t(8, 16), t(16, 4)
    raises(ValueError, ON_GPU, sg.gemm_ex, A, B, t(8, 4, dtype=torch.uint8), out_scale=0.5)
    raises(TypeError, "C has dtype", sg.gemm_ex, A, B, t(8, 4), out_scale=0.5)
    raises(ValueError, "bias", sg.gemm_ex, A, B, t(8, 4), bias=t(3, dtype=torch.float32))
    raises(TypeError, "bias", sg.gemm_ex, A, B, t(8, 4), bias=t(4, dtype=torch.uint8))
    raises(ValueError, "activation", sg.gemm_ex, A, B, t(8, 4), activation="tanh")
    raises(ValueError, ON_GPU, sg.gemm_ex, A, B, t(8, 4), bias=t(4, dtype=torch.float32),
           activation="gelu")


def test_gemm_strided_batched_checks_every_problem():
    M, N, K, batch = 4, 8, 16, 3
    A, B, C = t(batch * M * K), t(batch * K * N), t(batch * M * N)
    kw = dict(M=M, N=N, K=K, lda=K, ldb=N, ldc=N)
    raises(ValueError, ON_GPU, sg.gemm_strided_batched, A, B, C, batch, M * K, K * N, M * N, **kw)
    raises(ValueError, ON_GPU, sg.gemm_strided_batched, A, B[: K * N], C, batch, M * K, 0,
           M * N, **kw)
    raises(ValueError, "A holds", sg.gemm_strided_batched, A, B, C, batch + 1, M * K, K * N,
           M * N, **kw)
    raises(ValueError, "C holds", sg.gemm_strided_batched, A, B, t(batch * M * N - 1), batch,
           M * K, K * N, M * N, **kw)
    raises(ValueError, ">= 0", sg.gemm_strided_batched, A, B, C, batch, -1, K * N, M * N, **kw)


# ------------------------------------------------------------------ SwiGLU
def test_swiglu_well_formed_reaches_the_device_check():
    raises(ValueError, ON_GPU, sg.swiglu_gemm, t(8, 16), t(16, 10), t(8, 5))
    raises(ValueError, ON_GPU, sg.swiglu_gemm, t(8, 16, dtype=torch.float16),
           t(16, 10, dtype=torch.float16), t(8, 5, dtype=torch.float16))
    raises(ValueError, ON_GPU, sg.swiglu_gemm, t(8, 16, dtype=torch.float8_e4m3fn),
           t(16, 10, dtype=torch.float8_e4m3fn), t(8, 5), 0.5, 0.25)
    raises(ValueError, ON_GPU, sg.swiglu_gemm_w12, t(8, 16), t(16, 5), t(16, 5), t(8, 5))


def test_swiglu_shapes_and_types():
    raises(ValueError, "weight 0", sg.swiglu_gemm, t(8, 16), t(15, 10), t(8, 5))
    raises(ValueError, "even", sg.swiglu_gemm, t(8, 16), t(16, 9), t(8, 4))
    raises(ValueError, "Y has shape", sg.swiglu_gemm, t(8, 16), t(16, 10), t(8, 4))
    raises(ValueError, "Y has shape", sg.swiglu_gemm, t(8, 16), t(16, 10), t(7, 5))
    raises(TypeError, "Y has dtype", sg.swiglu_gemm, t(8, 16), t(16, 10),
           t(8, 5, dtype=torch.float16))
    raises(TypeError, "Y has dtype", sg.swiglu_gemm, t(8, 16, dtype=torch.float8_e4m3fn),
           t(16, 10, dtype=torch.float8_e4m3fn), t(8, 5, dtype=torch.uint8))
    raises(TypeError, "A's dtype", sg.swiglu_gemm, t(8, 16), t(16, 10, dtype=torch.float16),
           t(8, 5))
    raises(TypeError, "SwiGLU takes", sg.swiglu_gemm, t(8, 16, dtype=torch.float32),
           t(16, 10, dtype=torch.float32), t(8, 5, dtype=torch.float32))
    raises(ValueError, "weight 1", sg.swiglu_gemm_w12, t(8, 16), t(16, 5), t(16, 6), t(8, 5))


def test_swiglu_views_must_be_contiguous():
    raises(ValueError, "A must be contiguous", sg.swiglu_gemm, t(16, 8).t(), t(16, 10), t(8, 5))
    raises(ValueError, "must be contiguous", sg.swiglu_gemm, t(8, 16), t(16, 20)[:, :10],
           t(8, 5))
    raises(ValueError, "Y must be contiguous", sg.swiglu_gemm, t(8, 16), t(16, 10),
           t(8, 6)[:, :5])


# ------------------------------------------------------------------ helpers
def test_interleave_and_silu_mul_checks():
    raises(ValueError, ON_GPU, sg.interleave_gate_up, t(4, 6), t(4, 6))
    raises(ValueError, "W2 has shape", sg.interleave_gate_up, t(4, 6), t(4, 5))
    raises(TypeError, "one dtype", sg.interleave_gate_up, t(4, 6), t(4, 6, dtype=torch.float16))
    raises(ValueError, "out has shape", sg.interleave_gate_up, t(4, 6), t(4, 6), t(4, 11))
    raises(ValueError, ON_GPU, sg.silu_mul, t(4, 6), t(4, 6), t(4, 6))
    raises(ValueError, "Y has shape", sg.silu_mul, t(4, 6), t(4, 6), t(4, 5))
    raises(TypeError, "one dtype", sg.silu_mul, t(4, 6), t(4, 6, dtype=torch.float16), t(4, 6))
    raises(TypeError, "bf16 or fp16", sg.silu_mul, t(4, 6, dtype=torch.float32),
           t(4, 6, dtype=torch.float32), t(4, 6, dtype=torch.float32))
