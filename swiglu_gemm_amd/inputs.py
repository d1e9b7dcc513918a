"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and rounds them to the storage formats; it holds
none of the GEMM / SwiGLU arithmetic.  Both the HIP path and the CPU oracle read
the identical bits it produces.

Recipe
------
* Generator: ``numpy.random.default_rng(SeedSequence([workload, tensor_id, M]))``
  (PCG64).  ``tensor_id`` 0 = A, 1 = B or W1, 2 = C or W2; ``workload`` is a small
  integer naming the workload family (1: fp32 GEMM, 2: fp16 square GEMM, 3: bf16
  ragged GEMM, 4: bf16 SwiGLU, 5: fp8 SwiGLU; other values for test-only shapes).
* Values are drawn in fp64, scaled, then rounded to nearest-even into the storage
  dtype.
* fp8 (OCP e4m3fn) tensors are quantised per tensor: s = amax/448 (fp32), code =
  round-to-nearest-even(x/s) saturated to +-448 (zero point 0), so the real value
  of a code q is s*q.
* Leading-dimension padding of A/B holds NaN (it must never be read); padding of
  C/Y holds a fixed sentinel bit pattern (it must never be written).
"""
from __future__ import annotations

import numpy as np

STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8}
ESIZE = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}

# sentinels for C/Y padding (quiet-NaN payloads that no arithmetic produces)
SENTINEL = {"f32": np.uint32(0x7FC01234), "f16": np.uint16(0x7E55),
            "bf16": np.uint16(0x7FA5), "e4m3": np.uint8(0x7F)}
NAN_BITS = {"f32": np.uint32(0x7FC00000), "f16": np.uint16(0x7E00),
            "bf16": np.uint16(0x7FC0), "e4m3": np.uint8(0x7F)}

E4M3_MAX = 448.0


def rng(workload: int, tensor_id: int, m: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(workload), int(tensor_id), int(m)]))


def _f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even); NaN stays a quiet NaN."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        r[nan] = NAN_BITS["bf16"]
    return r


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the storage dtype (nearest-even); returns raw storage."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        # fp64 -> fp32 is exact for every value drawn here at the magnitudes used
        # (the draws are then rounded once more, to bf16).
        return _f32_to_bf16_bits(x.astype(np.float32))
    if dtype == "e4m3":
        import torch
        t = torch.from_numpy(np.clip(x, -E4M3_MAX, E4M3_MAX).astype(np.float32))
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    raise ValueError(dtype)


def quantize_e4m3(x: np.ndarray):
    """Per-tensor e4m3 quantisation: returns (codes uint8, scale as an fp32 float)."""
    x = np.asarray(x, dtype=np.float64)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    s = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
    return to_storage(x / s, "e4m3"), s


def draw(gen: np.random.Generator, shape, dist: str, scale: float = 1.0) -> np.ndarray:
    if dist == "uniform":          # U[-scale, scale]
        return gen.uniform(-1.0, 1.0, size=shape) * scale
    if dist == "normal":           # N(0, scale^2): scale is the standard deviation
        return gen.standard_normal(size=shape) * scale
    if dist == "int":              # small integers in [-scale, scale]
        return gen.integers(-int(scale), int(scale) + 1, size=shape).astype(np.float64)
    raise ValueError(dist)


def padded(values_storage: np.ndarray, ld: int, fill) -> np.ndarray:
    """Place a rows x cols storage array into rows x ld storage, padding with `fill` bits."""
    rows, cols = values_storage.shape
    assert ld >= cols
    out = np.empty((rows, ld), dtype=values_storage.dtype)
    out.view(np.uint8)[...] = 0
    if ld > cols:
        pad = np.array(fill).astype(values_storage.dtype) if values_storage.dtype != np.float32 \
            else np.array(fill, dtype=np.uint32).view(np.float32)
        out[:, cols:] = pad
    out[:, :cols] = values_storage
    return out


def matrix(workload, tensor_id, m_key, rows, cols, ld, dtype, dist, scale=1.0, pad="nan"):
    """Seeded rows x cols matrix stored row-major with leading dimension ld."""
    gen = rng(workload, tensor_id, m_key)
    vals = to_storage(draw(gen, (rows, cols), dist, scale), dtype)
    fill = NAN_BITS[dtype] if pad == "nan" else SENTINEL[dtype]
    return padded(vals, ld, fill)


def stored_shape(trans: str, rows_op: int, cols_op: int):
    """Storage shape (rows, cols) of X such that op(X) is rows_op x cols_op."""
    return (cols_op, rows_op) if trans in "Tt" else (rows_op, cols_op)


def ld_padded(cols: int) -> int:
    """Leading dimension rounded up to a multiple of 64, plus 8."""
    return ((cols + 63) // 64) * 64 + 8


def gemm_problem(workload, transA, transB, M, N, K, dtype, dist, scale=1.0,
                 ld_mode="tight", beta_zero=False, c_dtype=None):
    """A, B, C storage for one GEMM problem.  C_old is NaN everywhere when beta == 0
    (beta_zero=True) since it must not be read; C padding holds the sentinel."""
    c_dtype = c_dtype or dtype
    ar, ac = stored_shape(transA, M, K)
    br, bc = stored_shape(transB, K, N)
    lda = ac if ld_mode == "tight" else ld_padded(ac)
    ldb = bc if ld_mode == "tight" else ld_padded(bc)
    ldc = N if ld_mode == "tight" else ld_padded(N)
    lda, ldb, ldc = max(lda, 1), max(ldb, 1), max(ldc, 1)
    if dtype == "e4m3":
        A_vals, sa = quantize_e4m3(draw(rng(workload, 0, M), (ar, ac), dist, scale))
        B_vals, sb = quantize_e4m3(draw(rng(workload, 1, M), (br, bc), dist, scale))
        A = padded(A_vals, lda, NAN_BITS[dtype])
        B = padded(B_vals, ldb, NAN_BITS[dtype])
    else:
        A = matrix(workload, 0, M, ar, ac, lda, dtype, dist, scale)
        B = matrix(workload, 1, M, br, bc, ldb, dtype, dist, scale)
        sa = sb = 1.0
    if beta_zero:
        nanv = NAN_BITS[c_dtype]
        cvals = np.full((M, N), nanv, dtype=STORAGE[c_dtype]) if c_dtype != "f32" else \
            np.full((M, N), nanv, dtype=np.uint32).view(np.float32)
        C = padded(cvals, ldc, SENTINEL[c_dtype])
    else:
        C = matrix(workload, 2, M, M, N, ldc, c_dtype, dist, scale, pad="sentinel")
    return dict(A=A, B=B, C=C, lda=lda, ldb=ldb, ldc=ldc, scale_a=sa, scale_b=sb)


def swiglu_problem(workload, M, N, K, dtype, a_std=1.0, w_std=0.02):
    """A (M x K), W1, W2 (K x N) storage for a SwiGLU problem.  For e4m3 the two
    weight matrices share one per-tensor scale (they form one W_fused tensor)."""
    a = draw(rng(workload, 0, M), (M, K), "normal", a_std)
    w1 = draw(rng(workload, 1, 0), (K, N), "normal", w_std)
    w2 = draw(rng(workload, 2, 0), (K, N), "normal", w_std)
    if dtype == "e4m3":
        A, sa = quantize_e4m3(a)
        amax = max(float(np.max(np.abs(w1))), float(np.max(np.abs(w2))))
        sw = float(np.float32(amax / E4M3_MAX))
        W1 = to_storage(w1 / sw, "e4m3")
        W2 = to_storage(w2 / sw, "e4m3")
        return dict(A=A, W1=W1, W2=W2, scale_a=sa, scale_w=sw)
    return dict(A=to_storage(a, dtype), W1=to_storage(w1, dtype), W2=to_storage(w2, dtype),
                scale_a=1.0, scale_w=1.0)
