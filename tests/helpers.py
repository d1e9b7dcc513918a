"""Shared helpers for the GPU parity tests: device transfer of raw storage and the
comparison rule |y - yhat| <= atol + rtol*|yhat| (the tolerance form of
"为什么 GEMM 是 CUDA 的必修课", 精度不是数据类型名称这么简单)."""
import json
import os
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


def error_stats(y, yhat, dtype, K):
    """Error of the GPU values y against the oracle's yhat, beside the pass/fail rule:
    largest absolute and relative error, the largest error over max|yhat|, the share of
    elements more than 1 % off (the mismatch measure of "Resumo Técnico: Sobreposição
    de Ativação em Nível de Tile ...", Resultados), and the worst |y - yhat| as a
    fraction of the tolerance atol + rtol*|yhat| (pass iff <= 1)."""
    atol, rtol = TOL[dtype](K)
    d = np.abs(y - yhat)
    a = np.abs(yhat)
    n = int(d.size)
    if n == 0:
        return dict(n=0)
    nz = a > 0
    rel = d[nz] / a[nz]
    amax = float(a.max())
    return dict(n=n, K=int(K), dtype=dtype,
                max_abs=float(d.max()),
                max_rel=float(rel.max()) if rel.size else 0.0,
                max_abs_over_max_ref=float(d.max() / amax) if amax > 0 else 0.0,
                share_rel_gt_1pct=float(np.count_nonzero(d > 0.01 * a)) / n,
                worst_over_tol=float(np.max(d / (atol + rtol * a))))


def record(what, stats):
    """Append one comparison's statistics to the JSON-lines file named by
    SG_NUMERICS_REPORT (no-op when unset)."""
    path = os.environ.get("SG_NUMERICS_REPORT")
    if not path:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "a") as f:
        f.write(json.dumps(dict(case=what, **stats)) + "\n")


def assert_close(y, yhat, dtype, K, what="", report=False):
    """y: fp64 values decoded from the GPU output; yhat: fp64 oracle values.  Every
    element must satisfy |y - yhat| <= atol + rtol*|yhat|; with report=True the error
    statistics of the comparison are also recorded."""
    atol, rtol = TOL[dtype](K)
    assert y.shape == yhat.shape
    assert np.all(np.isfinite(y)), "%s: non-finite output" % what
    if report:
        record(what, error_stats(y, yhat, dtype, K))
    excess = np.abs(y - yhat) - (atol + rtol * np.abs(yhat))
    if np.any(excess > 0):
        i = np.unravel_index(np.argmax(excess), excess.shape)
        raise AssertionError("%s: %d/%d elements outside tolerance (atol %g rtol %g); worst at %s: "
                             "got %r want %r" % (what, int(np.sum(excess > 0)), excess.size, atol,
                                                 rtol, i, y[i], yhat[i]))


def bits_equal(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


def split_count(cfg: str) -> int:
    """The split-K count from a sg_last_config() description."""
    m = re.search(r"splits=(\d+)", cfg)
    return int(m.group(1)) if m else 1
