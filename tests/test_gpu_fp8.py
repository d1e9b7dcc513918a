"""GPU parity of the OCP e4m3 path (fused SwiGLU-GEMM and GEMM) against the fp64
oracle, through the C ABI.

Workload: A[M x 4096] ~ N(0,1), W1, W2 [4096 x 11008] ~ N(0, 0.02^2), each tensor
quantised per tensor (s = amax/448, W1 and W2 share one scale as they form one
W_fused), W_fused [4096 x 22016], Y bf16, M in {1, 16, 256, 4096}.  The oracle
reads the same codes and scales ("GEMM o Coração Matemático" §12.4: value =
s * code)."""
import os

import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import assert_close, bits_equal, from_dev, split_count, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

E4M3_CFGS = [14, 15, 16, 17, 33, 45, 47]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()
    yield
    os.environ.pop("SG_FORCE_CONFIG", None)


def run_swiglu8(pb, Wf, M, N, K):
    import swiglu_gemm_amd as sg
    A = to_dev(pb["A"], "e4m3")
    W = to_dev(Wf, "e4m3")
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    print("swiglu e4m3 M=%d N=%d K=%d" % (M, N, K), flush=True)
    sg.swiglu_gemm(A, W, Y, pb["scale_a"], pb["scale_w"])
    torch.cuda.synchronize()
    return from_dev(Y), sg.last_config()


@pytest.fixture(scope="module")
def weights():
    N, K = 11008, 4096
    pb = inputs.swiglu_problem(5, 1, N, K, "e4m3")
    return pb, oracle.interleave(pb["W1"], pb["W2"])


@pytest.mark.parametrize("M", [1, 16, 256, 4096])
def test_swiglu_e4m3_full(M, weights):
    """Every output of the e4m3 SwiGLU workload (K = 4096, N = 11008, per-tensor
    scales) at each of its token counts, in the default launch configuration."""
    N, K = 11008, 4096
    wb, Wf = weights
    pb = inputs.swiglu_problem(5, M, N, K, "e4m3")
    assert pb["scale_w"] == wb["scale_w"]
    y, cfg = run_swiglu8(pb, Wf, M, N, K)
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, "e4m3", pb["scale_a"], pb["scale_w"])
    assert_close(oracle.decode(y, "bf16"), ref, "e4m3", K, "swiglu e4m3 M=%d %s" % (M, cfg),
                 report=True)


@pytest.mark.parametrize("force", [("SG_FORCE_CONFIG", "17,2"), ("SG_FORCE_CONFIG", "17,4"),
                                   ("SG_FORCE_CONFIG", "16,2"), ("SG_FORCE_DECODE", "5")])
@pytest.mark.parametrize("M", [1, 16])
def test_swiglu_e4m3_skinny_split_paths(M, force, weights):
    """The skinny rows of the e4m3 SwiGLU workload (K = 4096, N = 11008) on the paths
    that split K -- split-K with the fp32 reduction, and the stream-K decode kernel
    with its fix-up -- every output against the oracle."""
    N, K = 11008, 4096
    wb, Wf = weights
    pb = inputs.swiglu_problem(5, M, N, K, "e4m3")
    var, val = force
    os.environ[var] = val
    try:
        y, desc = run_swiglu8(pb, Wf, M, N, K)
    finally:
        os.environ.pop(var, None)
    if var == "SG_FORCE_DECODE":
        assert "decode" in desc and "fixup" in desc, desc
    else:
        assert split_count(desc) == int(val.split(",")[1]), desc
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, "e4m3", pb["scale_a"], pb["scale_w"])
    assert_close(oracle.decode(y, "bf16"), ref, "e4m3", K, desc)


@pytest.mark.parametrize("splits", [1, 2])
@pytest.mark.parametrize("cfg", E4M3_CFGS)
def test_swiglu_e4m3_every_config(cfg, splits):
    import swiglu_gemm_amd as sg
    M, N, K = 96, 640, 1024            # ragged M for every tile height
    pb = inputs.swiglu_problem(80 + cfg, M, N, K, "e4m3")
    Wf = oracle.interleave(pb["W1"], pb["W2"])
    os.environ["SG_FORCE_CONFIG"] = "%d,%d" % (cfg, splits)
    try:
        y1, desc = run_swiglu8(pb, Wf, M, N, K)
        y2, _ = run_swiglu8(pb, Wf, M, N, K)
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    assert "cfg=%d " % cfg in desc, desc
    assert split_count(desc) == splits, desc
    assert bits_equal(y1, y2)
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, "e4m3", pb["scale_a"], pb["scale_w"])
    assert_close(oracle.decode(y1, "bf16"), ref, "e4m3", K, desc)


@pytest.mark.parametrize("tr", ["NN", "NT", "TN", "TT"])
@pytest.mark.parametrize("cfg", E4M3_CFGS + [None])
def test_gemm_e4m3_configs_and_transposes(cfg, tr):
    import swiglu_gemm_amd as sg
    M, N, K = 160, 384, 1024
    ta, tb = tr
    p = inputs.gemm_problem(90, ta, tb, M, N, K, "e4m3", "normal", ld_mode="tight",
                            c_dtype="bf16")
    alpha = p["scale_a"] * p["scale_b"] * 0.5
    A, B, C = to_dev(p["A"], "e4m3"), to_dev(p["B"], "e4m3"), to_dev(p["C"], "bf16")
    if cfg is not None:
        os.environ["SG_FORCE_CONFIG"] = "%d,0" % cfg
    try:
        sg.gemm(A, B, C, alpha=alpha, beta=0.25, transA=ta, transB=tb, M=M, N=N, K=K,
                lda=p["lda"], ldb=p["ldb"], ldc=p["ldc"], dtype=3)
        torch.cuda.synchronize()
        desc = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    if cfg is not None:
        # a transposed A has 32-byte rows in a 32-row tile: the 128 x 128 tile runs it
        assert "cfg=%d " % (15 if ta == "T" and cfg in (16, 17) else cfg) in desc, desc
    ref = oracle.gemm(ta, tb, M, N, K, alpha, p["A"], p["lda"], p["B"], p["ldb"], 0.25, p["C"],
                      p["ldc"], "e4m3", c_dtype="bf16")
    assert_close(oracle.decode(from_dev(C), "bf16"), ref, "e4m3", K, desc)


@pytest.mark.parametrize("shape", [(37, 50, 70), (1, 1, 1), (5, 300, 130), (300, 1001, 1000)])
def test_e4m3_odd_rows_relaid(shape):
    """Rows that are not 16-byte multiples (odd K or N, tight leading dimensions):
    the operands are copied with 16-byte rows and the tile kernels run, GEMM and
    SwiGLU (whose W_fused rows of 2N bytes are then not 16-byte multiples either)."""
    import swiglu_gemm_amd as sg
    M, N, K = shape
    p = inputs.gemm_problem(91, "N", "N", M, N, K, "e4m3", "normal", c_dtype="bf16")
    A, B, C = to_dev(p["A"], "e4m3"), to_dev(p["B"], "e4m3"), to_dev(p["C"], "bf16")
    alpha = p["scale_a"] * p["scale_b"]          # the per-tensor scales: O(1) outputs
    print("gemm e4m3 relaid M=%d N=%d K=%d" % (M, N, K), flush=True)
    sg.gemm(A, B, C, alpha=alpha, beta=0.0, M=M, N=N, K=K, lda=p["lda"], ldb=p["ldb"],
            ldc=p["ldc"], dtype=3)
    torch.cuda.synchronize()
    desc = sg.last_config()
    assert "generic" not in desc, desc
    ref = oracle.gemm("N", "N", M, N, K, alpha, p["A"], p["lda"], p["B"], p["ldb"], 0.0, p["C"],
                      p["ldc"], "e4m3", c_dtype="bf16")
    assert_close(oracle.decode(from_dev(C), "bf16"), ref, "e4m3", K, desc)
    pb = inputs.swiglu_problem(92, M, N, K, "e4m3")
    Wf = oracle.interleave(pb["W1"], pb["W2"])
    y, desc = run_swiglu8(pb, Wf, M, N, K)
    assert "generic" not in desc, desc
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, "e4m3", pb["scale_a"], pb["scale_w"])
    assert_close(oracle.decode(y, "bf16"), ref, "e4m3", K, desc)


@pytest.mark.parametrize("tr", ["NN", "NT", "TN", "TT"])
def test_e4m3_padded_ld_relaid(tr):
    """Leading dimensions padded to 64k + 8 bytes (8 bytes off the 16-byte grid),
    several tiles and a ragged edge: the re-laid copies feed the tile kernels;
    every output against the oracle and the ld padding of C untouched."""
    import swiglu_gemm_amd as sg
    ta, tb = tr
    M, N, K = 700, 900, 1000
    p = inputs.gemm_problem(93, ta, tb, M, N, K, "e4m3", "normal", ld_mode="padded",
                            c_dtype="bf16")
    A, B, C = to_dev(p["A"], "e4m3"), to_dev(p["B"], "e4m3"), to_dev(p["C"], "bf16")
    alpha = 0.7 * p["scale_a"] * p["scale_b"]
    print("gemm e4m3 padded ld %s M=%d N=%d K=%d" % (tr, M, N, K), flush=True)
    sg.gemm(A, B, C, alpha=alpha, beta=0.3, transA=ta, transB=tb, M=M, N=N, K=K, lda=p["lda"],
            ldb=p["ldb"], ldc=p["ldc"], dtype=3)
    torch.cuda.synchronize()
    desc = sg.last_config()
    assert "gemm8 cfg=" in desc, desc
    got = from_dev(C)
    ref = oracle.gemm(ta, tb, M, N, K, alpha, p["A"], p["lda"], p["B"], p["ldb"], 0.3, p["C"],
                      p["ldc"], "e4m3", c_dtype="bf16")
    assert_close(oracle.decode(got, "bf16")[:, :N], ref[:, :N], "e4m3", K, desc)
    assert bits_equal(got[:, N:], p["C"][:, N:]), "ld padding of C was written"


@pytest.mark.parametrize("M", [1, 16, 256])
def test_swiglu_e4m3_one_hot_bit_exact(M):
    """Unit scales; W1, W2 select columns of A.  Gate sources are powers of two
    in [32, 256] (exact in e4m3; SiLU(g) rounds to g in fp32), up sources are
    integers in [-3, 3]: Y = g*u exactly in bf16."""
    N, K = 512, 1024
    gen = np.random.default_rng(M + 7)
    half = K // 2
    A = np.zeros((M, K))
    A[:, :half] = 2.0 ** gen.integers(5, 9, size=(M, half))
    A[:, half:] = gen.integers(-3, 4, size=(M, K - half))
    pi1 = gen.integers(0, half, size=N)
    pi2 = half + gen.integers(0, K - half, size=N)
    W1 = np.zeros((K, N))
    W2 = np.zeros((K, N))
    W1[pi1, np.arange(N)] = 1.0
    W2[pi2, np.arange(N)] = 1.0
    pb = dict(A=inputs.to_storage(A, "e4m3"), scale_a=1.0, scale_w=1.0)
    Wf = oracle.interleave(inputs.to_storage(W1, "e4m3"), inputs.to_storage(W2, "e4m3"))
    y, cfg = run_swiglu8(pb, Wf, M, N, K)
    assert np.array_equal(oracle.decode(y, "bf16"), A[:, pi1] * A[:, pi2]), cfg
