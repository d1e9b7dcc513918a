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
    if _lib is not None:
        return _lib
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
        L.sg_gemm_noalloc.argtypes = L.sg_gemm.argtypes
        L.sg_gemm_noalloc.restype = ctypes.c_int
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
        L.sg_build_info.argtypes = []
        L.sg_build_info.restype = ctypes.c_char_p
        _check_build(L)
        _lib = L
        return L


def _check_build(L) -> None:
    """Refuse a library built from sources other than the ones beside it (a stale
    build would run kernels that the sources and tests no longer describe)."""
    from . import build
    if not os.path.isdir(build.CSRC):
        return                      # a library shipped without its sources
    info = L.sg_build_info().decode()
    want = build.source_hash()
    if want not in info.split():
        raise SwigluGemmError(
            "libswiglu_gemm.so (%s) was built from other sources than %s (source %s); "
            "rebuild with __graft_entry__.build() or python -m swiglu_gemm_amd.build"
            % (info, build.CSRC, want))


def build_info() -> str:
    """The loaded library's build identity (see sg_build_info)."""
    return lib().sg_build_info().decode()


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
# Every wrapper checks, before the library is called, that the tensors it passes
# hold what the C ABI will read and write (shapes, dtypes, row strides, storage
# extent): the library sees bare pointers, so a short or mistyped tensor would
# otherwise send the kernels past its allocation.  The device is checked last,
# so that every other check can be exercised without a GPU.
_TABLES = None


def _tables():
    """dtype -> code and code -> accepted output dtypes (built once: these checks run
    on every call, so they avoid per-call allocations)."""
    global _TABLES
    if _TABLES is None:
        import torch
        code = {torch.float32: SG_F32, torch.float16: SG_F16, torch.bfloat16: SG_BF16,
                torch.float8_e4m3fn: SG_F8E4M3, torch.uint8: SG_F8E4M3}
        out = {SG_F32: (torch.float32,), SG_F16: (torch.float16,), SG_BF16: (torch.bfloat16,),
               SG_F8E4M3: (torch.bfloat16,)}
        _TABLES = (code, out, (torch.float8_e4m3fn, torch.uint8),
                   (torch.float32, torch.float16, torch.bfloat16))
    return _TABLES


def _dtype_code(t) -> int:
    code = _tables()[0].get(t.dtype)
    if code is None:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return code


# bytes per element of the operands and of the output, per dtype code
_IN_SIZE = {SG_F32: 4, SG_F16: 2, SG_BF16: 2, SG_F8E4M3: 1}


def _out_dtypes(code: int):
    """torch dtypes accepted for C / Y when the operands have dtype code `code`."""
    return _tables()[1][code]


_RAW_STREAM = None


def _stream(t):
    """Handle (an int) of torch's current HIP stream on t's device.  torch's raw-stream
    query skips building a Stream object (about 2 us a call); older builds without it
    take the public route."""
    global _RAW_STREAM
    if _RAW_STREAM is None:
        import torch
        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None) or \
            (lambda d: torch.cuda.current_stream(d).cuda_stream)
    return _RAW_STREAM(t.get_device())


def _ld(t) -> int:
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.stride(1) != 1 and t.size(1) > 1:
        raise ValueError("the last dimension must be contiguous (stride 1)")
    return max(int(t.stride(0)), 1) if t.size(0) > 1 else max(int(t.size(1)), 1)


def _span(rows: int, cols: int, ld: int) -> int:
    """Elements from the first to one past the last of a rows x cols row-major view
    with row stride ld (0 for an empty view)."""
    return 0 if rows <= 0 or cols <= 0 else (rows - 1) * ld + cols


def _avail(t) -> int:
    """Elements of t's storage from t's first element to the end of the storage."""
    return t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()


def _need(t, name: str, elems: int) -> None:
    if elems <= t.numel() and t.is_contiguous():
        return                    # the view itself covers the span
    if elems > _avail(t):
        raise ValueError("%s holds %d elements from its first one, the call needs %d"
                         % (name, _avail(t), elems))


def _same_size(t, name: str, code: int, what: str) -> None:
    if t.element_size() != _IN_SIZE[code]:
        raise TypeError("%s has %d-byte elements, %s needs %d" % (name, t.element_size(), what,
                                                                   _IN_SIZE[code]))


def _on_gpu(*ts) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("every tensor must be on the GPU")


def _contig(t, name: str, shape) -> None:
    if t.shape != shape:
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _view_ld(sh, st) -> int:
    """Leading dimension of a 2-D (or batched) row-major view from its shape and strides."""
    if len(sh) == 2 and sh[0] <= 1:
        return max(sh[1], 1)
    return max(st[-2], 1)


def _need_span(t, sh, name: str, elems: int) -> None:
    n = 1
    for d in sh:
        n *= d
    if elems <= n and t.is_contiguous():
        return                    # the view itself covers the span
    if elems > _avail(t):
        raise ValueError("%s holds %d elements from its first one, the call needs %d"
                         % (name, _avail(t), elems))


def _gemm_args(A, B, C, ta, tb, code, M, N, K, lda, ldb, ldc, c_dtypes, batch=1,
               strides=(0, 0, 0)):
    """Sizes and leading dimensions of a GEMM call, checked against the tensors (each
    tensor's shape and strides are read once: these checks run on every call)."""
    if ta not in ("N", "T") or tb not in ("N", "T"):
        raise ValueError("transA and transB must be 'N' or 'T'")
    ash, bsh, csh = A.shape, B.shape, C.shape
    ast, bst, cst = A.stride(), B.stride(), C.stride()
    if M is None:
        if len(ash) < 2 or len(bsh) < 2:
            raise ValueError("A and B must have at least 2 dimensions")
        M = ash[-1] if ta == "T" else ash[-2]
        K = ash[-2] if ta == "T" else ash[-1]
        N = bsh[-2] if tb == "T" else bsh[-1]
        kb = bsh[-1] if tb == "T" else bsh[-2]
        if kb != K:
            raise ValueError("op(A) is %d x %d but op(B) has %d rows" % (M, K, kb))
    elif N is None or K is None:
        raise ValueError("give M, N and K together")
    M, N, K = int(M), int(N), int(K)
    if M < 0 or N < 0 or K < 0:
        raise ValueError("M, N and K must be >= 0")
    for sh, st, name in ((ash, ast, "A"), (bsh, bst, "B"), (csh, cst, "C")):
        if len(sh) >= 2 and sh[-1] > 1 and st[-1] != 1:
            raise ValueError("%s: the last dimension must be contiguous (stride 1)" % name)
    lda = (_view_ld(ash, ast) if len(ash) >= 2 else 1) if lda is None else int(lda)
    ldb = (_view_ld(bsh, bst) if len(bsh) >= 2 else 1) if ldb is None else int(ldb)
    ldc = (_view_ld(csh, cst) if len(csh) >= 2 else 1) if ldc is None else int(ldc)
    want = _IN_SIZE[code]
    if A.element_size() != want:
        raise TypeError("A has %d-byte elements, the operand dtype needs %d"
                        % (A.element_size(), want))
    if B.element_size() != want:
        raise TypeError("B has %d-byte elements, the operand dtype needs %d"
                        % (B.element_size(), want))
    if C.dtype not in c_dtypes:
        raise TypeError("C has dtype %s, expected one of %s" % (C.dtype, c_dtypes))
    sA, sB, sC = strides
    last = max(int(batch) - 1, 0)
    if M and K:
        _need_span(A, ash, "A",
                   last * sA + (_span(K, M, lda) if ta == "T" else _span(M, K, lda)))
    if N and K:
        _need_span(B, bsh, "B",
                   last * sB + (_span(N, K, ldb) if tb == "T" else _span(K, N, ldb)))
    if M and N:
        _need_span(C, csh, "C", last * sC + _span(M, N, ldc))
    return M, N, K, lda, ldb, ldc


def gemm(A, B, C, alpha: float = 1.0, beta: float = 0.0, transA: str = "N", transB: str = "N",
         dtype: int | None = None, M=None, N=None, K=None, lda=None, ldb=None, ldc=None):
    """C = alpha * op(A) @ op(B) + beta * C, in place on C (2-D row-major tensors on the
    GPU; the leading dimension is each tensor's row stride).  For e4m3 operands C is
    bf16 and alpha should carry the product of the two per-tensor scales."""
    code = _dtype_code(A) if dtype is None else dtype
    ta, tb = transA.upper(), transB.upper()
    M, N, K, lda, ldb, ldc = _gemm_args(A, B, C, ta, tb, code, M, N, K, lda, ldb, ldc,
                                        _out_dtypes(code))
    _on_gpu(A, B, C)
    st = lib().sg_gemm(ta.encode(), tb.encode(), M, N, K, float(alpha),
                       A.data_ptr(), lda, B.data_ptr(),
                       ldb, float(beta), C.data_ptr(), ldc, code, _stream(C))
    _check(st, "sg_gemm")
    return C


def gemm_noalloc(A, B, C, alpha: float = 1.0, beta: float = 0.0, transA: str = "N",
                 transB: str = "N", dtype: int | None = None, M=None, N=None, K=None, lda=None,
                 ldb=None, ldc=None):
    """gemm() through sg_gemm_noalloc: the same result with no device allocation (its
    scratch is a fixed array of the library), for code under HIP graph capture.  A
    problem that needs more scratch raises (SG_STATUS_SCRATCH_LIMIT) with C untouched."""
    code = _dtype_code(A) if dtype is None else dtype
    ta, tb = transA.upper(), transB.upper()
    M, N, K, lda, ldb, ldc = _gemm_args(A, B, C, ta, tb, code, M, N, K, lda, ldb, ldc,
                                        _out_dtypes(code))
    _on_gpu(A, B, C)
    st = lib().sg_gemm_noalloc(ta.encode(), tb.encode(), M, N, K, float(alpha),
                               A.data_ptr(), lda, B.data_ptr(),
                               ldb, float(beta), C.data_ptr(), ldc, code,
                               _stream(C))
    _check(st, "sg_gemm_noalloc")
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
    c_dtypes = _tables()[2] if out_scale is not None else _out_dtypes(code)
    M, N, K, lda, ldb, ldc = _gemm_args(A, B, C, ta, tb, code, M, N, K, lda, ldb, ldc, c_dtypes)
    if activation not in ACTIVATIONS:
        raise ValueError("unknown activation %r" % activation)
    if bias is not None:
        if bias.dtype not in _tables()[3]:
            raise TypeError("bias must be fp32, fp16 or bf16")
        if bias.dim() != 1 or not bias.is_contiguous() or bias.numel() < N:
            raise ValueError("bias must be a contiguous vector of at least N = %d values" % N)
    _on_gpu(A, B, C, bias)
    epi = Epilogue(ctypes.c_void_p(bias.data_ptr()) if bias is not None else None,
                   _dtype_code(bias) if bias is not None else SG_F32, ACTIVATIONS[activation],
                   SG_F8E4M3 if out_scale is not None else -1,
                   float(out_scale) if out_scale is not None else 1.0)
    st = lib().sg_gemm_ex(ta.encode(), tb.encode(), M, N, K, float(alpha),
                          A.data_ptr(), lda, B.data_ptr(),
                          ldb, float(beta), C.data_ptr(), ldc, code,
                          ctypes.byref(epi), _stream(C))
    _check(st, "sg_gemm_ex")
    return C


def gemm_strided_batched(A, B, C, batch, strideA, strideB, strideC, alpha: float = 1.0,
                         beta: float = 0.0, transA: str = "N", transB: str = "N",
                         dtype: int | None = None, M=None, N=None, K=None, lda=None, ldb=None,
                         ldc=None):
    """C_b = alpha * op(A_b) @ op(B_b) + beta * C_b for b < batch, X_b = X + b*strideX
    elements (A, B, C: device tensors whose storage holds every problem; sizes and
    leading dimensions default to those of the last two dimensions given)."""
    code = _dtype_code(A) if dtype is None else dtype
    ta, tb = transA.upper(), transB.upper()
    if int(batch) < 0 or min(int(strideA), int(strideB), int(strideC)) < 0:
        raise ValueError("batch and strides must be >= 0")
    M, N, K, lda, ldb, ldc = _gemm_args(A, B, C, ta, tb, code, M, N, K, lda, ldb, ldc,
                                        _out_dtypes(code), batch=int(batch),
                                        strides=(int(strideA), int(strideB), int(strideC)))
    _on_gpu(A, B, C)
    st = lib().sg_gemm_strided_batched(ta.encode(), tb.encode(), M, N, K,
                                       float(alpha), A.data_ptr(), lda,
                                       int(strideA), B.data_ptr(), ldb,
                                       int(strideB), float(beta), C.data_ptr(),
                                       ldc, int(strideC), int(batch), code, _stream(C))
    _check(st, "sg_gemm_strided_batched")
    return C


def _swiglu_args(A, W_list, Y, two_n: bool):
    """M, N, K of a SwiGLU call, with A [M, K], each weight [K, 2N] (two_n) or [K, N]
    and Y [M, N] contiguous; operands of one dtype, Y bf16 (fp16 for fp16 inputs).
    Each tensor attribute is read once (these checks run on every call)."""
    ash = A.shape
    wshapes = [w.shape for w in W_list]
    if len(ash) != 2 or any(len(sh) != 2 for sh in wshapes):
        raise ValueError("A and the weights must be 2-D")
    M, K = ash
    ncols = wshapes[0][1]
    if two_n and ncols % 2:
        raise ValueError("Wfused must have an even number of columns (gate, up pairs)")
    N = ncols // 2 if two_n else ncols
    codes = _tables()[0]
    code = codes.get(A.dtype)
    if code is None:
        raise TypeError("unsupported dtype %s" % A.dtype)
    if code == SG_F32:
        raise TypeError("SwiGLU takes bf16, fp16 or e4m3 operands")
    if not A.is_contiguous():
        raise ValueError("A must be contiguous")
    want = (K, ncols)
    for i, (w, sh) in enumerate(zip(W_list, wshapes)):
        if sh != want:
            raise ValueError("weight %d has shape %s, expected %s" % (i, tuple(sh), want))
        if not w.is_contiguous():
            raise ValueError("weight %d must be contiguous" % i)
        if codes.get(w.dtype) != code:
            raise TypeError("the weights must have A's dtype")
    outs = _tables()[1][code]
    if Y.dtype not in outs:
        raise TypeError("Y has dtype %s, expected %s" % (Y.dtype, outs[0]))
    _contig(Y, "Y", (M, N))
    return M, N, K, code


def swiglu_gemm(A, Wfused, Y, scale_a: float = 1.0, scale_w: float = 1.0):
    """Y = SiLU(s*A@W1) * (s*A@W2) from the column-interleaved Wfused [K, 2N]
    (s = scale_a*scale_w); A [M, K], Y [M, N], all contiguous."""
    M, N, K, code = _swiglu_args(A, [Wfused], Y, True)
    _on_gpu(A, Wfused, Y)
    st = lib().sg_swiglu_gemm(A.data_ptr(), Wfused.data_ptr(),
                              Y.data_ptr(), M, N, K, code, float(scale_a),
                              float(scale_w), _stream(Y))
    _check(st, "sg_swiglu_gemm")
    return Y


def swiglu_gemm_w12(A, W1, W2, Y, scale_a: float = 1.0, scale_w: float = 1.0):
    """Y = SiLU(s*A@W1) * (s*A@W2) from separate W1, W2 [K, N] (s = scale_a*scale_w);
    A [M, K], Y [M, N], all contiguous."""
    M, N, K, code = _swiglu_args(A, [W1, W2], Y, False)
    _on_gpu(A, W1, W2, Y)
    st = lib().sg_swiglu_gemm_w12(A.data_ptr(), W1.data_ptr(),
                                  W2.data_ptr(), Y.data_ptr(),
                                  M, N, K, code, float(scale_a), float(scale_w), _stream(Y))
    _check(st, "sg_swiglu_gemm_w12")
    return Y


def interleave_gate_up(W1, W2, out=None):
    """Wfused[:, 0::2] = W1, Wfused[:, 1::2] = W2 (bit-exact), on the GPU."""
    import torch
    if W1.dim() != 2:
        raise ValueError("W1 must be 2-D")
    K, N = int(W1.shape[0]), int(W1.shape[1])
    _contig(W1, "W1", (K, N))
    _contig(W2, "W2", (K, N))
    if W2.dtype != W1.dtype:
        raise TypeError("W1 and W2 must have one dtype")
    if out is None:
        out = torch.empty((K, 2 * N), dtype=W1.dtype, device=W1.device)
    _contig(out, "out", (K, 2 * N))
    if out.element_size() != W1.element_size():
        raise TypeError("out must have W1's element size")
    _on_gpu(W1, W2, out)
    st = lib().sg_interleave_gate_up(W1.data_ptr(), W2.data_ptr(),
                                     out.data_ptr(), K, N,
                                     _dtype_code(W1), _stream(out))
    _check(st, "sg_interleave_gate_up")
    return out


def silu_mul(G, U, Y):
    """Y = SiLU(G) * U elementwise (contiguous, bf16 or fp16)."""
    import torch
    if G.dim() != 2:
        raise ValueError("G must be 2-D")
    M, N = int(G.shape[0]), int(G.shape[1])
    if G.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("silu_mul takes bf16 or fp16")
    for t, name in ((G, "G"), (U, "U"), (Y, "Y")):
        _contig(t, name, (M, N))
        if t.dtype != G.dtype:
            raise TypeError("G, U and Y must have one dtype")
    _on_gpu(G, U, Y)
    st = lib().sg_silu_mul(G.data_ptr(), U.data_ptr(),
                           Y.data_ptr(), M, N, _dtype_code(G), _stream(Y))
    _check(st, "sg_silu_mul")
    return Y
