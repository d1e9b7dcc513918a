"""GPU parity of the decode-shaped path (M <= 32 token rows: a persistent stream-K
kernel that streams the weight once, and a fix-up kernel that finishes the column
tiles several runs share) against the fp64 oracle, through the C ABI.

Covers the GEMM with the weight stored K x N ('N') or N x K ('T') including
alpha/beta and ld padding, the interleaved fused SwiGLU-GEMM and the split-weight
form, in fp16, bf16 and e4m3; every decode configuration; ragged column tails;
tiles split among up to 40 work-groups; the full-size 1- and 16-token SwiGLU
shapes; run-to-run identity across configurations and problems; which shapes the
library routes to the path by default; and the shapes that must not take it."""
import contextlib
import os

import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import assert_close, bits_equal, from_dev, out_dtype, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DT_CODE = {"f16": 1, "bf16": 2, "e4m3": 3}
DEC_CFGS = [0, 1, 2, 3, 4, 5, 6]
W12_DEC_CFGS = [1, 4]          # two fragments per wave: gate and up halves


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()
    yield
    os.environ.pop("SG_FORCE_DECODE", None)


@contextlib.contextmanager
def decode_cfg(cfg):
    if cfg is None:
        yield
        return
    os.environ["SG_FORCE_DECODE"] = str(cfg)
    try:
        yield
    finally:
        os.environ.pop("SG_FORCE_DECODE", None)


def run_gemm(p, tb, M, N, K, alpha, beta, dtype, cfg=None):
    import swiglu_gemm_amd as sg
    A, B, C = to_dev(p["A"], dtype), to_dev(p["B"], dtype), to_dev(p["C"], out_dtype(dtype))
    print("decode gemm %s N%s M=%d N=%d K=%d cfg=%s" % (dtype, tb, M, N, K, cfg), flush=True)
    with decode_cfg(cfg):
        sg.gemm(A, B, C, alpha=alpha, beta=beta, transA="N", transB=tb, M=M, N=N, K=K,
                lda=p["lda"], ldb=p["ldb"], ldc=p["ldc"], dtype=DT_CODE[dtype])
        torch.cuda.synchronize()
        desc = sg.last_config()
    return from_dev(C), desc


def gemm_case(dtype, tb, M, N, K, seed, ld_mode):
    p = inputs.gemm_problem(seed, "N", tb, M, N, K, dtype, "normal", ld_mode=ld_mode,
                            c_dtype=out_dtype(dtype))
    scale = p["scale_a"] * p["scale_b"] if dtype == "e4m3" else 1.0
    return p, 0.7 * scale, 0.3


def check_gemm(p, tb, M, N, K, alpha, beta, dtype, cfg=None):
    bits, desc = run_gemm(p, tb, M, N, K, alpha, beta, dtype, cfg)
    assert desc.startswith("decode"), desc
    od = out_dtype(dtype)
    ref = oracle.gemm("N", tb, M, N, K, alpha, p["A"], p["lda"], p["B"], p["ldb"], beta, p["C"],
                      p["ldc"], dtype, c_dtype=od)
    assert_close(oracle.decode(bits, od)[:, :N], ref[:, :N], od, K, desc)
    assert bits_equal(bits[:, N:], p["C"][:, N:]), "ld padding of C was written"
    return bits, desc


def run_swiglu(pb, M, N, K, dtype, cfg=None, w12=False):
    import swiglu_gemm_amd as sg
    A = to_dev(pb["A"], dtype)
    out = torch.float16 if dtype == "f16" else torch.bfloat16
    Y = torch.full((M, N), float("nan"), dtype=out, device="cuda:0")
    sa, sw = pb.get("scale_a", 1.0), pb.get("scale_w", 1.0)
    print("decode swiglu%s %s M=%d N=%d K=%d cfg=%s" % ("_w12" if w12 else "", dtype, M, N, K,
                                                         cfg), flush=True)
    with decode_cfg(cfg):
        if w12:
            sg.swiglu_gemm_w12(A, to_dev(pb["W1"], dtype), to_dev(pb["W2"], dtype), Y, sa, sw)
        else:
            sg.swiglu_gemm(A, to_dev(oracle.interleave(pb["W1"], pb["W2"]), dtype), Y, sa, sw)
        torch.cuda.synchronize()
        desc = sg.last_config()
    return from_dev(Y), desc


def check_swiglu(pb, M, N, K, dtype, cfg=None, w12=False):
    y, desc = run_swiglu(pb, M, N, K, dtype, cfg, w12)
    assert desc.startswith("decode"), desc
    ref = oracle.swiglu(M, N, K, pb["A"], oracle.interleave(pb["W1"], pb["W2"]), dtype,
                        pb.get("scale_a", 1.0), pb.get("scale_w", 1.0))
    assert_close(oracle.decode(y, out_dtype(dtype)), ref, dtype, K, desc)
    return y, desc


@pytest.mark.parametrize("cfg", DEC_CFGS)
@pytest.mark.parametrize("M", [1, 7, 32])
@pytest.mark.parametrize("tb", ["N", "T"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "e4m3"])
def test_decode_gemm(dtype, tb, M, cfg):
    """alpha/beta GEMM, ragged column tail (1040 = 8 tiles of 128 + 16)."""
    N, K = 1040, 640
    ld_mode = "tight" if dtype == "e4m3" else "padded"
    p, alpha, beta = gemm_case(dtype, tb, M, N, K, 300 + M + cfg, ld_mode)
    check_gemm(p, tb, M, N, K, alpha, beta, dtype, cfg)


@pytest.mark.parametrize("cfg", DEC_CFGS)
@pytest.mark.parametrize("M", [1, 16, 29])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "e4m3"])
def test_decode_swiglu(dtype, M, cfg):
    N, K = 1000, 1024                     # fused width 2000: a ragged last tile
    pb = inputs.swiglu_problem(320 + M + cfg, M, N, K, dtype)
    check_swiglu(pb, M, N, K, dtype, cfg)


@pytest.mark.parametrize("cfg", W12_DEC_CFGS)
@pytest.mark.parametrize("M", [1, 16, 32])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "e4m3"])
def test_decode_swiglu_w12_bit_equal_to_interleaved(dtype, M, cfg):
    """Split weights: same tile columns and K order as the interleaved form, so the
    outputs are identical bits; both meet the oracle."""
    N, K = 1040, 1024
    pb = inputs.swiglu_problem(340 + M + cfg, M, N, K, dtype)
    y1, d1 = check_swiglu(pb, M, N, K, dtype, cfg, w12=True)
    y2, d2 = check_swiglu(pb, M, N, K, dtype, cfg, w12=False)
    assert "cfg=%d " % cfg in d1 and "cfg=%d " % cfg in d2, (d1, d2)


@pytest.mark.parametrize("cfg", DEC_CFGS)
@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_decode_many_contributors(dtype, cfg):
    """Fewer units than work-groups: every unit is its own run, so each column tile
    is summed from up to 40 partials by the fix-up kernel."""
    M, N = 9, 384
    K = 40 * (128 if dtype == "e4m3" else 64)
    p, alpha, beta = gemm_case(dtype, "N", M, N, K, 360 + cfg, "tight")
    check_gemm(p, "N", M, N, K, alpha, beta, dtype, cfg)
    pb = inputs.swiglu_problem(361 + cfg, M, N // 2, K, dtype)
    check_swiglu(pb, M, N // 2, K, dtype, cfg)


@pytest.mark.parametrize("M", [1, 16])
def test_decode_e4m3_swiglu_full_size(M):
    """The 1- and 16-token e4m3 SwiGLU at full size (K 4096, N 11008), every row."""
    N, K = 11008, 4096
    pb = inputs.swiglu_problem(370 + M, M, N, K, "e4m3")
    check_swiglu(pb, M, N, K, "e4m3", cfg=5)


def test_decode_default_routing():
    """By default the path replaces the large-tile kernels exactly where those would
    split K: a 1 x 4096 x 4096 bf16 projection goes to it, the e4m3 SwiGLU at
    1 x 4096 x 2*11008 (one large-tile launch) does not."""
    import swiglu_gemm_amd as sg
    p, alpha, beta = gemm_case("bf16", "T", 1, 4096, 4096, 375, "tight")
    _, desc = check_gemm(p, "T", 1, 4096, 4096, alpha, beta, "bf16")
    assert "cfg=5 " in desc, desc
    pb = inputs.swiglu_problem(376, 1, 11008, 4096, "e4m3")
    y, desc = run_swiglu(pb, 1, 11008, 4096, "e4m3")
    assert not desc.startswith("decode"), desc


def test_decode_bf16_gemm_full_size_nt():
    """A 4096 x 4096 bf16 projection with the weight stored N x K (row-major [out, in])."""
    M, N, K = 4, 4096, 4096
    p, alpha, beta = gemm_case("bf16", "T", M, N, K, 380, "tight")
    check_gemm(p, "T", M, N, K, alpha, 0.0, "bf16")


def test_decode_deterministic_across_problems():
    """Run X, then a problem Y with a different tile count (workspace reused), then X
    again: X's bits are unchanged; every configuration is run-to-run identical."""
    M, N, K = 16, 2048, 2048
    pX, aX, bX = gemm_case("bf16", "N", M, N, K, 390, "tight")
    x1, _ = check_gemm(pX, "N", M, N, K, aX, bX, "bf16")
    pb = inputs.swiglu_problem(391, 3, 3000, 1536, "e4m3")
    check_swiglu(pb, 3, 3000, 1536, "e4m3")
    x2, _ = run_gemm(pX, "N", M, N, K, aX, bX, "bf16")
    assert bits_equal(x1, x2)
    for cfg in DEC_CFGS:
        xa, _ = run_gemm(pX, "N", M, N, K, aX, bX, "bf16", cfg)
        xb, _ = run_gemm(pX, "N", M, N, K, aX, bX, "bf16", cfg)
        assert bits_equal(xa, xb), cfg


def test_decode_not_taken():
    """33 rows, a K that is not a whole number of 128-byte tiles, a pinned large-tile
    configuration, or a transposed A: the large-tile paths run instead."""
    import swiglu_gemm_amd as sg
    cases = [(33, 256, 256, "N", None), (4, 256, 200, "N", None), (4, 256, 256, "N", "2,1"),
             (4, 256, 256, "T", None)]
    for M, N, K, ta, force in cases:
        p = inputs.gemm_problem(395, ta, "N", M, N, K, "bf16", "normal")
        A, B, C = to_dev(p["A"], "bf16"), to_dev(p["B"], "bf16"), to_dev(p["C"], "bf16")
        if force:
            os.environ["SG_FORCE_CONFIG"] = force
        try:
            sg.gemm(A, B, C, alpha=1.0, beta=0.5, transA=ta, M=M, N=N, K=K, lda=p["lda"],
                    ldb=p["ldb"], ldc=p["ldc"], dtype=2)
            torch.cuda.synchronize()
            desc = sg.last_config()
        finally:
            os.environ.pop("SG_FORCE_CONFIG", None)
        assert not desc.startswith("decode"), (M, N, K, ta, force, desc)
        ref = oracle.gemm(ta, "N", M, N, K, 1.0, p["A"], p["lda"], p["B"], p["ldb"], 0.5, p["C"],
                          p["ldc"], "bf16")
        assert_close(oracle.decode(from_dev(C), "bf16")[:, :N], ref[:, :N], "bf16", K, desc)
