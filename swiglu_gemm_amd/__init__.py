"""MI355X (gfx950) BLAS GEMM and fused SwiGLU-GEMM: thin Python binding.

Every function here only marshals arguments (torch tensors -> device pointers,
leading dimensions, the current HIP stream) and calls the C ABI of
``libswiglu_gemm.so`` (declared in ``include/swiglu_gemm.h``); all arithmetic runs
in the library's HIP kernels.  There is no fallback: if the library is missing or
fails to load, every call raises.

    gemm(A, B, C, alpha=1, beta=0, transA='N', transB='N')   # C updated in place
    gemm_ex(A, B, C, ..., bias=None, activation='gelu', out_scale=None)  # + epilogue
    swiglu_gemm(A, Wfused, Y, scale_a=1, scale_w=1)          # Y written in place
    interleave_gate_up(W1, W2, out=None) -> Wfused
    silu_mul(G, U, Y)                                        # unfused activation
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libswiglu_gemm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "swiglu_gemm.h")

SG_F32, SG_F16, SG_BF16, SG_F8E4M3 = 0, 1, 2, 3
ACTIVATIONS = {"none": 0, "relu": 1, "gelu": 2, "gelu_tanh": 3, "silu": 4}


class Epilogue(ctypes.Structure):
    """sg_epilogue of include/swiglu_gemm.h."""
    _fields_ = [("bias", ctypes.c_void_p), ("bias_dtype", ctypes.c_int),
                ("activation", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("out_scale", ctypes.c_float)]

_lib = None
_lock = threading.Lock()


class SwigluGemmError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libswiglu_gemm.so (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise SwigluGemmError(
                "libswiglu_gemm.so is not built (run __graft_entry__.build() or "
                "python -m swiglu_gemm_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, f32, c = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_char
        L.sg_gemm.argtypes = [c, c, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64,
                              ctypes.c_int, vp]
        L.sg_gemm.restype = ctypes.c_int
        L.sg_gemm_ex.argtypes = [c, c, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64,
                                 ctypes.c_int, ctypes.POINTER(Epilogue), vp]
        L.sg_gemm_ex.restype = ctypes.c_int
        L.sg_gemm_strided_batched.argtypes = [c, c, i64, i64, i64, f32, vp, i64, i64, vp, i64,
                                              i64, f32, vp, i64, i64, i64, ctypes.c_int, vp]
        L.sg_gemm_strided_batched.restype = ctypes.c_int
        L.sg_swiglu_gemm.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int, f32, f32, vp]
        L.sg_swiglu_gemm.restype = ctypes.c_int
        L.sg_swiglu_gemm_w12.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, f32, f32,
                                         vp]
        L.sg_swiglu_gemm_w12.restype = ctypes.c_int
        L.sg_interleave_gate_up.argtypes = [vp, vp, vp, i64, i64, ctypes.c_int, vp]
        L.sg_interleave_gate_up.restype = ctypes.c_int
        L.sg_silu_mul.argtypes = [vp, vp, vp, i64, i64, ctypes.c_int, vp]
        L.sg_silu_mul.restype = ctypes.c_int
        L.sg_status_string.argtypes = [ctypes.c_int]
        L.sg_status_string.restype = ctypes.c_char_p
        L.sg_last_config.argtypes = [ctypes.c_char_p, ctypes.c_int]
        L.sg_last_config.restype = ctypes.c_int
        L.sg_release.argtypes = []
        L.sg_release.restype = None
        _lib = L
        return L


def declared_symbols() -> list:
    """Names of the functions include/swiglu_gemm.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sg_\w+)\s*\(", text, re.M)))


def status_string(status: int) -> str:
    return lib().sg_status_string(int(status)).decode()


def last_config() -> str:
    buf = ctypes.create_string_buffer(256)
    lib().sg_last_config(buf, 256)
    return buf.value.decode()


def release() -> None:
    lib().sg_release()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise SwigluGemmError("%s failed: %s (status %d)" % (what, status_string(status), status))


# ---------------------------------------------------------------- torch glue
def _dtype_code(t) -> int:
    import torch
    m = {torch.float32: SG_F32, torch.float16: SG_F16, torch.bfloat16: SG_BF16,
         torch.float8_e4m3fn: SG_F8E4M3, torch.uint8: SG_F8E4M3}
    if t.dtype not in m:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return m[t.dtype]


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ld(t) -> int:
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.stride(1) != 1 and t.size(1) > 1:
        raise ValueError("the last dimension must be contiguous (stride 1)")
    return max(int(t.stride(0)), 1) if t.size(0) > 1 else max(int(t.size(1)), 1)


def gemm(A, B, C, alpha: float = 1.0, beta: float = 0.0, transA: str = "N", transB: str = "N",
         dtype: int | None = None, M=None, N=None, K=None, lda=None, ldb=None, ldc=None):
    """C = alpha * op(A) @ op(B) + beta * C, in place on C (2-D row-major tensors on the
    GPU; the leading dimension is each tensor's row stride).  For e4m3 operands C is
    bf16 and alpha should carry the product of the two per-tensor scales."""
    code = _dtype_code(A) if dtype is None else dtype
    ta, tb = transA.upper(), transB.upper()
    if M is None:
        M = A.size(1) if ta == "T" else A.size(0)
        K = A.size(0) if ta == "T" else A.size(1)
        N = B.size(0) if tb == "T" else B.size(1)
    lda = _ld(A) if lda is None else lda
    ldb = _ld(B) if ldb is None else ldb
    ldc = _ld(C) if ldc is None else ldc
    st = lib().sg_gemm(ta.encode(), tb.encode(), int(M), int(N), int(K), float(alpha),
                       ctypes.c_void_p(A.data_ptr()), int(lda), ctypes.c_void_p(B.data_ptr()),
                       int(ldb), float(beta), ctypes.c_void_p(C.data_ptr()), int(ldc), code,
                       _stream(C))
    _check(st, "sg_gemm")
    return C


def gemm_ex(A, B, C, alpha: float = 1.0, beta: float = 0.0, transA: str = "N",
            transB: str = "N", bias=None, activation: str = "none", out_scale=None,
            dtype: int | None = None, M=None, N=None, K=None, lda=None, ldb=None, ldc=None):
    """C = out(act(alpha * op(A) @ op(B) + beta * C_old + bias[n])), in place on C.
    bias: None or a device vector of N values (fp32 / fp16 / bf16).  activation:
    'none', 'relu', 'gelu', 'gelu_tanh' or 'silu'.  out_scale: None (C has gemm's
    output type) or the per-tensor scale of an e4m3 output (C an e4m3 / uint8
    tensor holding the codes of y / out_scale; beta must be 0)."""
    code = _dtype_code(A) if dtype is None else dtype
    ta, tb = transA.upper(), transB.upper()
    if M is None:
        M = A.size(1) if ta == "T" else A.size(0)
        K = A.size(0) if ta == "T" else A.size(1)
        N = B.size(0) if tb == "T" else B.size(1)
    lda = _ld(A) if lda is None else lda
    ldb = _ld(B) if ldb is None else ldb
    ldc = _ld(C) if ldc is None else ldc
    if activation not in ACTIVATIONS:
        raise ValueError("unknown activation %r" % activation)
    epi = Epilogue(ctypes.c_void_p(bias.data_ptr()) if bias is not None else None,
                   _dtype_code(bias) if bias is not None else SG_F32, ACTIVATIONS[activation],
                   SG_F8E4M3 if out_scale is not None else -1,
                   float(out_scale) if out_scale is not None else 1.0)
    st = lib().sg_gemm_ex(ta.encode(), tb.encode(), int(M), int(N), int(K), float(alpha),
                          ctypes.c_void_p(A.data_ptr()), int(lda), ctypes.c_void_p(B.data_ptr()),
                          int(ldb), float(beta), ctypes.c_void_p(C.data_ptr()), int(ldc), code,
                          ctypes.byref(epi), _stream(C))
    _check(st, "sg_gemm_ex")
    return C


def gemm_strided_batched(A, B, C, batch, strideA, strideB, strideC, alpha: float = 1.0,
                         beta: float = 0.0, transA: str = "N", transB: str = "N",
                         dtype: int | None = None, M=None, N=None, K=None, lda=None, ldb=None,
                         ldc=None):
    """C_b = alpha * op(A_b) @ op(B_b) + beta * C_b for b < batch, X_b = X + b*strideX
    elements (A, B, C: device tensors whose storage holds every problem; sizes and
    leading dimensions default to those of the 2-D views given)."""
    code = _dtype_code(A) if dtype is None else dtype
    ta, tb = transA.upper(), transB.upper()
    if M is None:
        M = A.size(-1) if ta == "T" else A.size(-2)
        K = A.size(-2) if ta == "T" else A.size(-1)
        N = B.size(-2) if tb == "T" else B.size(-1)
    lda = A.stride(-2) if lda is None else lda
    ldb = B.stride(-2) if ldb is None else ldb
    ldc = C.stride(-2) if ldc is None else ldc
    st = lib().sg_gemm_strided_batched(ta.encode(), tb.encode(), int(M), int(N), int(K),
                                       float(alpha), ctypes.c_void_p(A.data_ptr()), int(lda),
                                       int(strideA), ctypes.c_void_p(B.data_ptr()), int(ldb),
                                       int(strideB), float(beta), ctypes.c_void_p(C.data_ptr()),
                                       int(ldc), int(strideC), int(batch), code, _stream(C))
    _check(st, "sg_gemm_strided_batched")
    return C


def swiglu_gemm(A, Wfused, Y, scale_a: float = 1.0, scale_w: float = 1.0):
    """Y = SiLU(s*A@W1) * (s*A@W2) from the column-interleaved Wfused [K, 2N]
    (s = scale_a*scale_w); A [M, K], Y [M, N], all contiguous."""
    M, K = A.shape
    N = Wfused.shape[1] // 2
    st = lib().sg_swiglu_gemm(ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(Wfused.data_ptr()),
                              ctypes.c_void_p(Y.data_ptr()), int(M), int(N), int(K),
                              _dtype_code(A), float(scale_a), float(scale_w), _stream(Y))
    _check(st, "sg_swiglu_gemm")
    return Y


def swiglu_gemm_w12(A, W1, W2, Y, scale_a: float = 1.0, scale_w: float = 1.0):
    """Y = SiLU(s*A@W1) * (s*A@W2) from separate W1, W2 [K, N] (s = scale_a*scale_w);
    A [M, K], Y [M, N], all contiguous."""
    M, K = A.shape
    N = W1.shape[1]
    st = lib().sg_swiglu_gemm_w12(ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(W1.data_ptr()),
                                  ctypes.c_void_p(W2.data_ptr()), ctypes.c_void_p(Y.data_ptr()),
                                  int(M), int(N), int(K), _dtype_code(A), float(scale_a),
                                  float(scale_w), _stream(Y))
    _check(st, "sg_swiglu_gemm_w12")
    return Y


def interleave_gate_up(W1, W2, out=None):
    """Wfused[:, 0::2] = W1, Wfused[:, 1::2] = W2 (bit-exact), on the GPU."""
    import torch
    K, N = W1.shape
    if out is None:
        out = torch.empty((K, 2 * N), dtype=W1.dtype, device=W1.device)
    st = lib().sg_interleave_gate_up(ctypes.c_void_p(W1.data_ptr()), ctypes.c_void_p(W2.data_ptr()),
                                     ctypes.c_void_p(out.data_ptr()), int(K), int(N),
                                     _dtype_code(W1), _stream(out))
    _check(st, "sg_interleave_gate_up")
    return out


def silu_mul(G, U, Y):
    """Y = SiLU(G) * U elementwise (contiguous, bf16 or fp16)."""
    M, N = G.shape
    st = lib().sg_silu_mul(ctypes.c_void_p(G.data_ptr()), ctypes.c_void_p(U.data_ptr()),
                           ctypes.c_void_p(Y.data_ptr()), int(M), int(N), _dtype_code(G),
                           _stream(Y))
    _check(st, "sg_silu_mul")
    return Y
