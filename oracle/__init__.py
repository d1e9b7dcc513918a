"""fp64 CPU oracle for BLAS GEMM and the fused SwiGLU-GEMM (ctypes binding).

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(``swiglu_gemm_amd``) never imports this package, and this package never imports
the product: the two share no code.

What is computed, with sources (page title, section):

* ``gemm``: C = alpha*op(A)*op(B) + beta*C_old, row-major with leading dimensions
  ("GEMM o Coração Matemático", §1 and §2), fp64 accumulation in i-p-j order
  (§2.1).  beta == 0 never reads C_old (BLAS convention).
* ``swiglu``: Y = SiLU(s*A*W1) ⊙ (s*A*W2), read from the column-interleaved
  W_fused (even columns gate, odd columns up) ("Resumo Técnico: Sobreposição de
  Ativação em Nível de Tile para Inferência Eficiente de LLM", Definição do
  Problema and Metodologia/Kernel-2); s = scale_a*scale_w is the per-tensor
  dequantisation of §12.4 of the first page.
* ``interleave`` / ``deinterleave``: the W_fused layout of Kernel-2, bit-exact.
* ``decode``: exact decoders of fp16, bf16 and OCP e4m3fn storage.
* ``activation`` / ``gemm_epilogue``: the GEMM followed by the steps a fused
  epilogue folds in before the accumulator is stored -- per-column bias, then an
  activation (ReLU, GELU, SiLU) -- ("GEMM o Coração Matemático" §1, last
  paragraph, and §13.3, last paragraph; "为什么 GEMM 是 CUDA 的必修课", the
  optimisation list, item on epilogue fusion: bias, activation, scale, quantise).
  GELU is x*Phi(x) with the normal CDF written through erf; the tanh form is the
  common approximation of it.
* ``quantize_e4m3``: a value to the OCP e4m3fn code of value/scale (per-tensor
  scale with zero point 0, §12.4), nearest code, ties to the even code,
  saturating at +-448; found by search over the decoded code table.

Inputs are raw storage arrays (numpy ``uint16`` for fp16/bf16, ``uint8`` for
e4m3, ``float32`` for fp32); outputs are float64.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

DTYPES = ("f32", "f16", "bf16", "e4m3")


def build(force: bool = True) -> str:
    """Compile oracle.c with plain gcc (-O2, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or \
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.oracle_gemm_f64.argtypes = [ctypes.c_char, ctypes.c_char, i64, i64, i64,
                                        ctypes.c_double, dp, i64, dp, i64,
                                        ctypes.c_double, dp, i64, ctypes.c_int]
        lib.oracle_gemm_f64.restype = ctypes.c_int
        lib.oracle_gemm_dot_f64.argtypes = [ctypes.c_char, ctypes.c_char, i64, i64, i64,
                                            ctypes.c_double, dp, i64, dp, i64,
                                            ctypes.c_double, dp, i64]
        lib.oracle_gemm_dot_f64.restype = ctypes.c_int
        lib.oracle_swiglu_f64.argtypes = [i64, i64, i64, dp, dp, ctypes.c_double,
                                          ctypes.c_double, dp, ctypes.c_int]
        lib.oracle_swiglu_f64.restype = ctypes.c_int
        lib.oracle_silu_f64.argtypes = [ctypes.c_double]
        lib.oracle_silu_f64.restype = ctypes.c_double
        for name in ("oracle_decode_f16", "oracle_decode_bf16"):
            getattr(lib, name).argtypes = [ctypes.c_void_p, dp, i64]
        lib.oracle_decode_e4m3.argtypes = [ctypes.c_void_p, dp, i64]
        lib.oracle_decode_f32.argtypes = [ctypes.c_void_p, dp, i64]
        lib.oracle_interleave.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          i64, i64, ctypes.c_int]
        lib.oracle_deinterleave.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            i64, i64, ctypes.c_int]
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def _dptr(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


_STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8}


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of every element of a raw storage array."""
    lib = _load()
    bits = np.ascontiguousarray(bits)
    want = _STORAGE[dtype]
    if bits.dtype != want:
        raise TypeError("decode(%s) expects %s storage, got %s" % (dtype, want, bits.dtype))
    out = np.empty(bits.shape, dtype=np.float64)
    n = bits.size
    fn = {"f32": lib.oracle_decode_f32, "f16": lib.oracle_decode_f16,
          "bf16": lib.oracle_decode_bf16, "e4m3": lib.oracle_decode_e4m3}[dtype]
    if n:
        fn(bits.ctypes.data, _dptr(out), n)
    return out


def silu(x: float) -> float:
    return float(_load().oracle_silu_f64(float(x)))


def as_f32(x: float) -> float:
    """Scalars (alpha, beta, scales) are passed by value as fp32."""
    return float(np.float32(x))


def gemm_f64(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
             nthreads=None, order="ipj"):
    """GEMM on fp64 arrays; C (flat or 2-D fp64, contiguous) is updated in place."""
    lib = _load()
    if nthreads is None:
        nthreads = max_threads()
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    assert C.dtype == np.float64 and C.flags.c_contiguous
    # bounds of the storage the routine will touch
    if M and K:
        need_a = ((K - 1) * lda + M) if transA in "Tt" else ((M - 1) * lda + K)
        assert A.size >= need_a, "A storage too small"
    if N and K:
        need_b = ((N - 1) * ldb + K) if transB in "Tt" else ((K - 1) * ldb + N)
        assert B.size >= need_b, "B storage too small"
    if M and N:
        assert C.size >= (M - 1) * ldc + N, "C storage too small"
    ta = transA.encode() if isinstance(transA, str) else transA
    tb = transB.encode() if isinstance(transB, str) else transB
    if order == "ipj":
        rc = lib.oracle_gemm_f64(ta, tb, M, N, K, float(alpha), _dptr(A), lda, _dptr(B), ldb,
                                 float(beta), _dptr(C), ldc, int(nthreads))
    elif order == "dot":
        rc = lib.oracle_gemm_dot_f64(ta, tb, M, N, K, float(alpha), _dptr(A), lda, _dptr(B),
                                     ldb, float(beta), _dptr(C), ldc)
    else:
        raise ValueError(order)
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments (%d)" % rc)
    return C


def gemm(transA, transB, M, N, K, alpha, A_bits, lda, B_bits, ldb, beta, C_bits, ldc,
         dtype, c_dtype=None, nthreads=None):
    """GEMM on raw storage: decodes A, B (dtype) and C_old (c_dtype), returns fp64 C
    with the shape of C's storage.  alpha and beta are taken as fp32 values."""
    c_dtype = c_dtype or dtype
    A = decode(A_bits, dtype).ravel()
    B = decode(B_bits, dtype).ravel()
    C = decode(C_bits, c_dtype)
    shape = C.shape
    C = np.ascontiguousarray(C.ravel())
    gemm_f64(transA, transB, M, N, K, as_f32(alpha), A, lda, B, ldb, as_f32(beta), C, ldc,
             nthreads=nthreads)
    return C.reshape(shape)


def swiglu_f64(M, N, K, A, Wf, scale_a=1.0, scale_w=1.0, nthreads=None):
    lib = _load()
    if nthreads is None:
        nthreads = max_threads()
    A = np.ascontiguousarray(A, dtype=np.float64).ravel()
    Wf = np.ascontiguousarray(Wf, dtype=np.float64).ravel()
    assert A.size >= M * K and Wf.size >= K * 2 * N
    Y = np.zeros(M * N, dtype=np.float64)
    rc = lib.oracle_swiglu_f64(M, N, K, _dptr(A), _dptr(Wf), float(scale_a), float(scale_w),
                               _dptr(Y), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_swiglu rejected its arguments")
    return Y.reshape(M, N)


def swiglu(M, N, K, A_bits, Wf_bits, dtype, scale_a=1.0, scale_w=1.0, nthreads=None):
    """SwiGLU on raw storage (A M x K, W_fused K x 2N), fp64 result M x N.  The scales
    are taken as fp32 values; their product is formed in fp64 (exact)."""
    A = decode(np.ascontiguousarray(A_bits).ravel()[: M * K], dtype)
    Wf = decode(np.ascontiguousarray(Wf_bits).ravel()[: K * 2 * N], dtype)
    return swiglu_f64(M, N, K, A, Wf, as_f32(scale_a), as_f32(scale_w), nthreads=nthreads)


def interleave(W1: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """W_fused[k,2n] = W1[k,n], W_fused[k,2n+1] = W2[k,n], bit-exact."""
    lib = _load()
    W1 = np.ascontiguousarray(W1)
    W2 = np.ascontiguousarray(W2)
    assert W1.shape == W2.shape and W1.dtype == W2.dtype and W1.ndim == 2
    K, N = W1.shape
    out = np.empty((K, 2 * N), dtype=W1.dtype)
    if out.size:
        lib.oracle_interleave(W1.ctypes.data, W2.ctypes.data, out.ctypes.data, K, N,
                              W1.dtype.itemsize)
    return out


def deinterleave(Wf: np.ndarray):
    lib = _load()
    Wf = np.ascontiguousarray(Wf)
    K, N2 = Wf.shape
    assert N2 % 2 == 0
    N = N2 // 2
    W1 = np.empty((K, N), dtype=Wf.dtype)
    W2 = np.empty((K, N), dtype=Wf.dtype)
    if W1.size:
        lib.oracle_deinterleave(Wf.ctypes.data, W1.ctypes.data, W2.ctypes.data, K, N,
                                Wf.dtype.itemsize)
    return W1, W2


ACTIVATIONS = ("none", "relu", "gelu", "gelu_tanh", "silu")


def activation(x, act: str) -> np.ndarray:
    """Elementwise activation in fp64 (see the module docstring for the sources).

    relu(x) = max(x, 0); gelu(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2));
    gelu_tanh(x) = x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3)));
    silu(x) = x / (1 + e^-x)."""
    x = np.asarray(x, dtype=np.float64)
    if act == "none":
        return x.copy()
    if act == "relu":
        return np.where(x > 0, x, 0.0)
    if act == "gelu":
        # Phi(x) = (1 + erf(x/sqrt 2))/2 = erfc(-x/sqrt 2)/2; the erfc form keeps full
        # relative accuracy in the negative tail, where 1 + erf cancels
        erfc = np.frompyfunc(math.erfc, 1, 1)
        return 0.5 * x * erfc(-x / math.sqrt(2.0)).astype(np.float64)
    if act == "gelu_tanh":
        c = math.sqrt(2.0 / math.pi)
        return 0.5 * x * (1.0 + np.tanh(c * (x + 0.044715 * x ** 3)))
    if act == "silu":
        with np.errstate(over="ignore"):
            return x / (1.0 + np.exp(-x))
    raise ValueError("unknown activation %r" % act)


def gemm_epilogue(transA, transB, M, N, K, alpha, A_bits, lda, B_bits, ldb, beta, C_bits, ldc,
                  dtype, c_dtype=None, bias_bits=None, bias_dtype=None, act="none",
                  nthreads=None):
    """fp64 value of act(alpha*op(A)*op(B) + beta*C_old + bias[n]) for every (m, n),
    shape (M, N): the GEMM of ``gemm`` followed by the per-column bias and the
    activation, before any output rounding or quantisation."""
    V = gemm(transA, transB, M, N, K, alpha, A_bits, lda, B_bits, ldb, beta, C_bits, ldc,
             dtype, c_dtype=c_dtype, nthreads=nthreads)
    V = np.ascontiguousarray(V.reshape(-1)[: M * ldc].reshape(M, ldc)[:, :N]) if M else \
        np.zeros((0, N))
    if bias_bits is not None:
        V = V + decode(np.ascontiguousarray(bias_bits).ravel()[:N], bias_dtype)[None, :]
    return activation(V, act)


def _e4m3_table():
    """Decoded values of the non-negative finite e4m3fn codes 0x00..0x7E (0x7F is NaN)."""
    return decode(np.arange(0x7F, dtype=np.uint8), "e4m3")


def quantize_e4m3(values, scale: float) -> np.ndarray:
    """OCP e4m3fn codes of values/scale (division in fp64): the nearest finite code,
    ties to the code with an even mantissa (even code number), magnitudes past 448
    saturate to 448, NaN gives 0x7F; the sign goes to bit 7 (also for zero)."""
    v = np.asarray(values, dtype=np.float64) / float(scale)
    table = _e4m3_table()                       # increasing, 127 entries
    a = np.abs(v)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    d_hi = np.abs(table[hi] - a)
    d_lo = np.abs(a - table[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = np.where(a >= table[-1], np.uint8(0x7E), code)
    code = code | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))
    code = np.where(np.isnan(v), np.uint8(0x7F), code)
    return code.astype(np.uint8)
