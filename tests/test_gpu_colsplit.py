"""The column split: a problem whose 256-row tiles take more than one round of the
CUs and leave the last round at most half full runs as two launches -- the chosen
tile over the leading columns that fill whole rounds, a smaller tile over the
remaining column strip (16-bit: 128 x 128; e4m3: 128 x 192, configuration 47, when
its tiles fit one round, which they do here: 32 x 2 tiles over a 256-column strip,
the second one ragged).  GEMM (B stored K x N and N x K, 16-bit and e4m3 operands,
alpha and beta) and the fused SwiGLU against the fp64 oracle on every output (both
launches and the seam between them), the routing itself, and no split under a
forced configuration."""
import os

import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import assert_close, from_dev, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# (dtype, M, N, K): 256-row tiles fill the last pass over the CUs to 1/16 (e4m3, 256 x 256 tiles:
# 16 x 33 = 528) or to 3/8 (bf16, 256 x 320 tiles: 32 x 27 = 864)
SHAPES = {"bf16": (8192, 8448, 256), "e4m3": (4096, 8448, 256)}
SEAM = {"bf16": 7680, "e4m3": 8192}     # first column of the tail launch
TAIL = {"bf16": 13, "e4m3": 47}         # configuration of the tail launch


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()
    yield
    os.environ.pop("SG_FORCE_CONFIG", None)


def run_gemm(dtype, tb, forced=None):
    import swiglu_gemm_amd as sg
    M, N, K = SHAPES[dtype]
    od = "bf16"
    p = inputs.gemm_problem(300, "N", tb, M, N, K, dtype, "normal", ld_mode="tight", c_dtype=od)
    alpha = 0.7 * (p["scale_a"] * p["scale_b"] if dtype == "e4m3" else 1.0)
    A, B, C = to_dev(p["A"], dtype), to_dev(p["B"], dtype), to_dev(p["C"], od)
    if forced:
        os.environ["SG_FORCE_CONFIG"] = forced
    print("colsplit gemm %s N%s M=%d N=%d K=%d forced=%s" % (dtype, tb, M, N, K, forced),
          flush=True)
    try:
        sg.gemm(A, B, C, alpha=alpha, beta=0.3, transA="N", transB=tb,
                dtype={"bf16": 2, "e4m3": 3}[dtype])
        torch.cuda.synchronize()
        desc = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    ref = oracle.gemm("N", tb, M, N, K, alpha, p["A"], p["lda"], p["B"], p["ldb"], 0.3, p["C"],
                      p["ldc"], dtype, c_dtype=od)
    got = oracle.decode(from_dev(C), od)
    assert_close(got[:, :N], ref[:, :N], dtype, K, desc)
    return desc


@pytest.mark.parametrize("tb", ["N", "T"])
@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_gemm_column_split(dtype, tb):
    desc = run_gemm(dtype, tb)
    assert ("tail cfg=%d " % TAIL[dtype]) in desc and "columns 0..%d," % SEAM[dtype] in desc, desc


def test_forced_config_is_not_split():
    desc = run_gemm("bf16", "N", forced="24,1")
    assert "tail" not in desc and "cfg=24 " in desc, desc


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_swiglu_column_split(dtype):
    import swiglu_gemm_amd as sg
    M, N2, K = SHAPES[dtype]
    N = N2 // 2
    pb = inputs.swiglu_problem(310, M, N, K, dtype)
    Wf = oracle.interleave(pb["W1"], pb["W2"])
    A, W = to_dev(pb["A"], dtype), to_dev(Wf, dtype)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    sa, sw = pb.get("scale_a", 1.0), pb.get("scale_w", 1.0)
    print("colsplit swiglu %s M=%d N=%d K=%d" % (dtype, M, N, K), flush=True)
    sg.swiglu_gemm(A, W, Y, sa, sw)
    torch.cuda.synchronize()
    desc = sg.last_config()
    assert ("tail cfg=%d " % TAIL[dtype]) in desc and "columns 0..%d," % SEAM[dtype] in desc, desc
    got = oracle.decode(from_dev(Y), "bf16")
    assert np.all(np.isfinite(got)), desc           # every output written
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, dtype, sa, sw)
    assert_close(got, ref, dtype, K, desc)


@pytest.mark.parametrize("dtype,M,N,K,seam,tail", [("bf16", 2048, 4864, 896, 8192, 7),
                                                  ("e4m3", 4096, 11008, 4096, 20480, 45)])
def test_swiglu_w12_column_split(dtype, M, N, K, seam, tail):
    """Split-weight SwiGLU: the seam is a fused column, W1, W2 and Y continue at half of
    it in the tail launch (bf16: 256 x 256 tiles, 8 x 38 = 304; e4m3: 16 x 86 = 1376)."""
    import swiglu_gemm_amd as sg
    pb = inputs.swiglu_problem(320, M, N, K, dtype)
    sa, sw = pb.get("scale_a", 1.0), pb.get("scale_w", 1.0)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    print("colsplit swiglu_w12 %s M=%d N=%d K=%d" % (dtype, M, N, K), flush=True)
    sg.swiglu_gemm_w12(to_dev(pb["A"], dtype), to_dev(pb["W1"], dtype), to_dev(pb["W2"], dtype),
                       Y, sa, sw)
    torch.cuda.synchronize()
    desc = sg.last_config()
    assert ("tail cfg=%d " % tail) in desc and "columns 0..%d," % seam in desc, desc
    got = oracle.decode(from_dev(Y), "bf16")
    assert np.all(np.isfinite(got)), desc
    Wf = oracle.interleave(pb["W1"], pb["W2"])
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, dtype, sa, sw)
    assert_close(got, ref, dtype, K, desc)
