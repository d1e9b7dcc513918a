"""The L2 warm-up of the direct-to-LDS tile kernel (warm_l2 in gemm16_dma.hpp): where
one partial round of tiles leaves CUs idle, B is row-major and each XCD's share of
B fits its L2, the idle CUs read that share ahead of the tiles.  It only loads, so
these tests check that the default launch takes it where it should ("l2warm=" in
the configuration string) and nowhere else, that it changes no output bit
(SG_NO_WARM=1 gives the same bits), and that the outputs match the oracle on the
SwiGLU workload at 256 tokens, ragged GEMMs with padded leading dimensions (both
orientations of A) and a fused-epilogue and an e4m3 SwiGLU case."""
import os

import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import assert_close, bits_equal, from_dev, out_dtype, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()
    yield


def twice(fn, force=None):
    """fn() with the warm-up allowed, then with SG_NO_WARM=1: (bits, config) each."""
    import swiglu_gemm_amd as sg
    out = []
    saved = {k: os.environ.get(k) for k in ("SG_NO_WARM", "SG_FORCE_CONFIG")}
    try:
        if force is not None:
            os.environ["SG_FORCE_CONFIG"] = force
        for off in (False, True):
            if off:
                os.environ["SG_NO_WARM"] = "1"
            else:
                os.environ.pop("SG_NO_WARM", None)
            bits = fn()
            torch.cuda.synchronize()
            out.append((bits, sg.last_config()))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    (warm, dw), (cold, dc) = out
    assert "l2warm=" not in dc, dc
    assert bits_equal(warm, cold), "the warm-up changed outputs: %s / %s" % (dw, dc)
    return warm, dw


def swiglu_call(A_bits, Wf_bits, M, N, dtype, sa=1.0, sw=1.0):
    import swiglu_gemm_amd as sg
    A, W = to_dev(A_bits, dtype), to_dev(Wf_bits, dtype)

    def fn():
        Y = torch.full((M, N), float("nan"), device="cuda:0", dtype=torch.bfloat16)
        print("swiglu %s M=%d N=%d K=%d warm=%s" % (dtype, M, N, A.shape[1],
                                                      os.environ.get("SG_NO_WARM") != "1"),
              flush=True)
        sg.swiglu_gemm(A, W, Y, sa, sw)
        return from_dev(Y)
    return fn


@pytest.mark.parametrize("M", [128, 256, 512])
def test_swiglu_workload_warm(M):
    """The bf16 SwiGLU workload (K = 896, N = 4864) at 128-512 tokens runs with the
    warm-up by default, bit-identical to the launch without it; at 256 tokens (not
    one of the workload's sizes, so not in the full-size parity test) every output
    is compared with the oracle as well."""
    N, K = 4864, 896
    pb = inputs.swiglu_problem(4, M, N, K, "bf16")
    Wf = oracle.interleave(pb["W1"], pb["W2"])
    y, desc = twice(swiglu_call(pb["A"], Wf, M, N, "bf16"))
    assert "l2warm=" in desc, desc
    if M == 256:
        ref = oracle.swiglu(M, N, K, pb["A"], Wf, "bf16")
        assert_close(oracle.decode(y, "bf16"), ref, "bf16", K, "swiglu warm " + desc)


def gemm_call(p, ta, tb, M, N, K, alpha, beta, dtype):
    import swiglu_gemm_amd as sg
    A, B = to_dev(p["A"], dtype), to_dev(p["B"], dtype)

    def fn():
        C = to_dev(p["C"], out_dtype(dtype))
        print("gemm %s %s%s M=%d N=%d K=%d warm=%s" % (dtype, ta, tb, M, N, K,
                                                       os.environ.get("SG_NO_WARM") != "1"),
              flush=True)
        sg.gemm(A, B, C, alpha=alpha, beta=beta, transA=ta, transB=tb, M=M, N=N, K=K,
                lda=p["lda"], ldb=p["ldb"], ldc=p["ldc"],
                dtype={"f16": 1, "bf16": 2}[dtype])
        return from_dev(C)
    return fn


@pytest.mark.parametrize("ta", ["N", "T"])
@pytest.mark.parametrize("shape", [(300, 1000, 640), (130, 2050, 448)])
def test_gemm_ragged_warm(ta, shape):
    """Ragged bf16 GEMMs (last row and column tiles partial, padded leading
    dimensions, alpha 0.7, beta 0.3) on the 128 x 128 direct-to-LDS tile: every
    output against the oracle, with and without the warm-up."""
    M, N, K = shape
    p = inputs.gemm_problem(31, ta, "N", M, N, K, "bf16", "normal", ld_mode="padded")
    cbits, desc = twice(gemm_call(p, ta, "N", M, N, K, 0.7, 0.3, "bf16"), force="13")
    assert "cfg=13 " in desc and "l2warm=" in desc, desc
    ref = oracle.gemm(ta, "N", M, N, K, 0.7, p["A"], p["lda"], p["B"], p["ldb"], 0.3, p["C"],
                      p["ldc"], "bf16", c_dtype="bf16")
    assert_close(oracle.decode(cbits, "bf16")[:, :N], ref[:, :N], "bf16", K, "warm " + desc)
    assert bits_equal(cbits[:, N:], p["C"][:, N:]), "ld padding of C was written"


def test_gemm_ex_warm():
    """fp16 GEMM + bias + GELU (the fused epilogue) under the warm-up: against the
    oracle's epilogue, and bit-identical without it."""
    import swiglu_gemm_amd as sg
    M, N, K = 200, 1536, 512
    p = inputs.gemm_problem(32, "N", "N", M, N, K, "f16", "normal", beta_zero=True)
    bias_bits = inputs.to_storage(np.random.default_rng(5).standard_normal(N) * 2.0, "f32")
    A, B, bias = to_dev(p["A"], "f16"), to_dev(p["B"], "f16"), to_dev(bias_bits, "f32")

    def fn():
        C = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
        print("gemm_ex f16 M=%d N=%d K=%d warm=%s" % (M, N, K,
                                                      os.environ.get("SG_NO_WARM") != "1"),
              flush=True)
        sg.gemm_ex(A, B, C, bias=bias, activation="gelu")
        return from_dev(C)
    cbits, desc = twice(fn, force="13")
    assert "l2warm=" in desc, desc
    y = oracle.gemm_epilogue("N", "N", M, N, K, 1.0, p["A"], p["lda"], p["B"], p["ldb"], 0.0,
                             p["C"], p["ldc"], "f16", c_dtype="f16", bias_bits=bias_bits,
                             bias_dtype="f32", act="gelu")
    assert_close(oracle.decode(cbits, "f16"), y, "f16", K, "gemm_ex warm " + desc)


def test_swiglu_e4m3_warm():
    """An e4m3 SwiGLU whose weights fit the XCDs' L2 (K = 1024, fused width 2000):
    against the oracle with the per-tensor scales, and bit-identical without the
    warm-up."""
    M, N, K = 64, 1000, 1024
    pb = inputs.swiglu_problem(5, M, N, K, "e4m3")
    Wf = oracle.interleave(pb["W1"], pb["W2"])
    sa, sw = pb["scale_a"], pb["scale_w"]
    y, desc = twice(swiglu_call(pb["A"], Wf, M, N, "e4m3", sa, sw), force="15,1")
    assert "l2warm=" in desc, desc
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, "e4m3", sa, sw)
    assert_close(oracle.decode(y, "bf16"), ref, "e4m3", K, "swiglu e4m3 warm " + desc)


def test_warm_not_taken():
    """No warm-up where it would not pay or does not apply: weights larger than the
    XCDs' L2 (the skinny e4m3 SwiGLU workload, K = 4096, fused width 22016), B
    stored N x K, and more tile rows than one group (each XCD's columns would not be
    one range)."""
    import swiglu_gemm_amd as sg
    M, N, K = 16, 11008, 4096
    A = torch.zeros((M, K), dtype=torch.uint8, device="cuda:0")
    W = torch.zeros((K, 2 * N), dtype=torch.uint8, device="cuda:0")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    sg.swiglu_gemm(A, W, Y, 1.0, 1.0)
    torch.cuda.synchronize()
    assert "l2warm" not in sg.last_config(), sg.last_config()
    assert float(Y.float().abs().max()) == 0.0
    Ab = torch.ones((300, 640), dtype=torch.bfloat16, device="cuda:0")
    Bt = torch.ones((1000, 640), dtype=torch.bfloat16, device="cuda:0")
    C = torch.empty((300, 1000), dtype=torch.bfloat16, device="cuda:0")
    old = os.environ.get("SG_FORCE_CONFIG")
    os.environ["SG_FORCE_CONFIG"] = "13"
    try:
        sg.gemm(Ab, Bt, C, transB="T")
        torch.cuda.synchronize()
        desc = sg.last_config()
        assert "cfg=13 " in desc and "l2warm" not in desc, desc
        assert float((C.float() - 640.0).abs().max()) == 0.0
        Am = torch.ones((1000, 640), dtype=torch.bfloat16, device="cuda:0")
        B = torch.ones((640, 1000), dtype=torch.bfloat16, device="cuda:0")
        C2 = torch.empty((1000, 1000), dtype=torch.bfloat16, device="cuda:0")
        sg.gemm(Am, B, C2)
        torch.cuda.synchronize()
        desc = sg.last_config()
        assert "cfg=13 " in desc and "l2warm" not in desc, desc
        assert float((C2.float() - 640.0).abs().max()) == 0.0
    finally:
        if old is None:
            os.environ.pop("SG_FORCE_CONFIG", None)
        else:
            os.environ["SG_FORCE_CONFIG"] = old
