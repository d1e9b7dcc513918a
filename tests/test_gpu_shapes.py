"""Default-path GEMMs over a seeded spread of shapes against the fp64 oracle, through
the C ABI: multi-round grids with ragged edges (row-staged stores on full tiles,
register stores on edge tiles), beta != 0, every transpose pair, the 16-bit cost model
(64-row tiles, split-K) and the e4m3 rules (32-row, 8-wave 128 x 256 and 256 x 256
tiles, the column split).  Every output is compared."""
import os

import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import assert_close, from_dev, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# (dtype, transposes, M, N, K, beta)
CASES = [
    ("bf16", "NN", 4608, 4200, 128, 0.0),     # 18 x 17 tiles of 256: staged + edge tiles
    ("f16", "NT", 4608, 4200, 192, 0.0),
    ("bf16", "TN", 4608, 4104, 128, 0.0),
    ("f16", "TT", 2304, 4104, 256, 0.0),
    ("bf16", "NN", 4608, 4200, 128, 0.5),     # beta: register stores everywhere
    ("f16", "NN", 8192, 4096, 64, 0.0),       # exact multiple of every tile
    ("bf16", "NT", 384, 4096, 4096, 0.0),     # 64-row tiles, no split
    ("bf16", "NT", 96, 4096, 4096, 0.25),     # split-K with its reduction
    ("f16", "NN", 200, 3000, 2048, 0.0),
    ("e4m3", "NT", 384, 4096, 4096, 0.0),     # 32-row tiles, two per CU
    ("e4m3", "NN", 200, 22016, 1024, 0.0),    # 8-wave 128 x 256
    ("e4m3", "NN", 1536, 4608, 512, 0.0),     # 256 x 256, one round
    ("e4m3", "NT", 4096, 8704, 256, 0.0),     # 256 x 256, column split
    ("e4m3", "TN", 1024, 2048, 512, 0.3),     # transposed A: 128 x 128 (32-row rows too short)
]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()
    yield


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-%s-%dx%dx%d-b%g" % c)
def test_default_path_shape(case):
    import swiglu_gemm_amd as sg
    dtype, tr, M, N, K, beta = case
    ta, tb = tr
    od = "bf16" if dtype == "e4m3" else dtype
    seed = 1000 + M + N + K
    p = inputs.gemm_problem(seed, ta, tb, M, N, K, dtype, "normal", ld_mode="tight",
                            c_dtype=od)
    alpha = 0.7 * (p["scale_a"] * p["scale_b"] if dtype == "e4m3" else 1.0)
    A, B, C = to_dev(p["A"], dtype), to_dev(p["B"], dtype), to_dev(p["C"], od)
    print("shape %s %s %dx%dx%d beta %g" % (dtype, tr, M, N, K, beta), flush=True)
    sg.gemm(A, B, C, alpha=alpha, beta=beta, transA=ta, transB=tb, M=M, N=N, K=K,
            lda=p["lda"], ldb=p["ldb"], ldc=p["ldc"],
            dtype={"f16": 1, "bf16": 2, "e4m3": 3}[dtype])
    torch.cuda.synchronize()
    desc = sg.last_config()
    assert "generic" not in desc, desc
    got = oracle.decode(from_dev(C), od)
    ref = oracle.gemm(ta, tb, M, N, K, alpha, p["A"], p["lda"], p["B"], p["ldb"], beta,
                      p["C"], p["ldc"], dtype, c_dtype=od)
    assert_close(got, ref, dtype, K, desc)
