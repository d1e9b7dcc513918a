"""Shared helpers for the GPU parity tests: device transfer of raw storage and the
comparison rule |y - yhat| <= atol + rtol*|yhat| (the tolerance form of
"为什么 GEMM 是 CUDA 的必修课", 精度不是数据类型名称这么简单)."""
import re

import numpy as np

import oracle

# Tolerances per output precision (fp32 atol scales with sqrt(K)).
TOL = {
    "f32": lambda K: (1e-5 * max(K, 1) ** 0.5, 1e-5),
    "f16": lambda K: (1e-3, 1e-2),
    "bf16": lambda K: (1e-2, 2e-2),
    "e4m3": lambda K: (1e-2, 6e-2),
}


def out_dtype(dtype):
    return "bf16" if dtype == "e4m3" else dtype


def to_dev(bits, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits))
    if dtype == "f16":
        t = t.view(torch.int16).view(torch.float16)
    elif dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    elif dtype == "e4m3":
        t = t.view(torch.float8_e4m3fn)
    return t.to("cuda:0")


def from_dev(t):
    import torch
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def assert_close(y, yhat, dtype, K, what=""):
    """y: fp64 values decoded from the GPU output; yhat: fp64 oracle values."""
    atol, rtol = TOL[dtype](K)
    assert y.shape == yhat.shape
    assert np.all(np.isfinite(y)), "%s: non-finite output" % what
    excess = np.abs(y - yhat) - (atol + rtol * np.abs(yhat))
    if np.any(excess > 0):
        i = np.unravel_index(np.argmax(excess), excess.shape)
        raise AssertionError("%s: %d/%d elements outside tolerance (atol %g rtol %g); worst at %s: "
                             "got %r want %r" % (what, int(np.sum(excess > 0)), excess.size, atol,
                                                 rtol, i, y[i], yhat[i]))


def bits_equal(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


def gemm_oracle_rows(rows, p, transA, transB, M, N, K, alpha, beta, dtype):
    """Oracle for a subset of rows of C: returns fp64 [len(rows), N]."""
    rows = np.asarray(rows)
    A = oracle.decode(p["A"], dtype)
    B = oracle.decode(p["B"], dtype).ravel()
    C = oracle.decode(p["C"], out_dtype(dtype))
    if transA in "Tt":     # A stored K x M: take columns
        Asub = np.ascontiguousarray(A[:, rows])
        lda = len(rows)
    else:
        Asub = np.ascontiguousarray(A[rows, :])
        lda = p["lda"]
    Csub = np.ascontiguousarray(C[rows, :]).ravel()
    oracle.gemm_f64(transA, transB, len(rows), N, K, oracle.as_f32(alpha), Asub.ravel(), lda, B,
                    p["ldb"], oracle.as_f32(beta), Csub, p["ldc"])
    return Csub.reshape(len(rows), p["ldc"])[:, :N]


def split_count(cfg: str) -> int:
    """The split-K count from a sg_last_config() description."""
    m = re.search(r"splits=(\d+)", cfg)
    return int(m.group(1)) if m else 1
