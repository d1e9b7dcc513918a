"""GPU parity of the split-weight fused SwiGLU-GEMM (separate W1, W2; the
non-interleaved weight layout of Kernel-1 in "Resumo Técnico: Sobreposição de
Ativação em Nível de Tile ...", Metodologia) against the fp64 oracle, through the
C ABI.  The oracle takes W_fused, so the reference interleaves W1, W2 on the CPU
(oracle.interleave) -- a layout step with no arithmetic."""
import os

import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import assert_close, bits_equal, from_dev, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W12_CFGS16 = [10, 8, 32, 6, 43]  # configurations that can take separate weights
W12_CFGS8 = [14, 16, 33, 45]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()
    yield
    os.environ.pop("SG_FORCE_CONFIG", None)


def run_w12(pb, M, N, K, dtype):
    import swiglu_gemm_amd as sg
    A = to_dev(pb["A"], dtype)
    W1, W2 = to_dev(pb["W1"], dtype), to_dev(pb["W2"], dtype)
    out = torch.bfloat16 if dtype in ("bf16", "e4m3") else torch.float16
    Y = torch.full((M, N), float("nan"), dtype=out, device="cuda:0")
    print("swiglu_w12 %s M=%d N=%d K=%d" % (dtype, M, N, K), flush=True)
    sg.swiglu_gemm_w12(A, W1, W2, Y, pb.get("scale_a", 1.0), pb.get("scale_w", 1.0))
    torch.cuda.synchronize()
    return from_dev(Y), sg.last_config()


def reference(pb, M, N, K, dtype):
    Wf = oracle.interleave(pb["W1"], pb["W2"])
    return oracle.swiglu(M, N, K, pb["A"], Wf, dtype, pb.get("scale_a", 1.0),
                         pb.get("scale_w", 1.0))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(256, 512, 512), (300, 1000, 640), (2048, 4864, 128)])
def test_w12_16bit(dtype, shape):
    M, N, K = shape
    pb = inputs.swiglu_problem(130, M, N, K, dtype)
    y, cfg = run_w12(pb, M, N, K, dtype)
    assert "swiglu_w12 cfg=" in cfg, cfg                  # the direct kernel, not the fallback
    out = "f16" if dtype == "f16" else "bf16"
    assert_close(oracle.decode(y, out), reference(pb, M, N, K, dtype), dtype, K, cfg)


@pytest.mark.parametrize("cfg", W12_CFGS16)
def test_w12_every_config_bit_equal_to_interleaved(cfg):
    """Same tile configuration, same K order: the split-weight kernel and the
    interleaved kernel produce identical bits; both meet the oracle."""
    import swiglu_gemm_amd as sg
    M, N, K = 384, 1280, 512
    pb = inputs.swiglu_problem(140 + cfg, M, N, K, "bf16")
    os.environ["SG_FORCE_CONFIG"] = "%d,1" % cfg
    try:
        y1, desc = run_w12(pb, M, N, K, "bf16")
        A = to_dev(pb["A"], "bf16")
        Wf = to_dev(oracle.interleave(pb["W1"], pb["W2"]), "bf16")
        Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        sg.swiglu_gemm(A, Wf, Y)
        torch.cuda.synchronize()
        desc2 = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    assert "swiglu_w12 cfg=%d " % cfg in desc, desc
    assert "cfg=%d " % cfg in desc2, desc2
    assert bits_equal(y1, from_dev(Y)), (desc, desc2)
    assert_close(oracle.decode(y1, "bf16"), reference(pb, M, N, K, "bf16"), "bf16", K, desc)


@pytest.mark.parametrize("cfg", W12_CFGS8)
@pytest.mark.parametrize("M", [16, 300])
def test_w12_e4m3(cfg, M):
    N, K = 1536, 1024
    pb = inputs.swiglu_problem(150 + cfg, M, N, K, "e4m3")
    os.environ["SG_FORCE_CONFIG"] = "%d,1" % cfg
    try:
        y, desc = run_w12(pb, M, N, K, "e4m3")
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    assert "swiglu_w12 cfg=%d " % cfg in desc, desc
    assert_close(oracle.decode(y, "bf16"), reference(pb, M, N, K, "e4m3"), "e4m3", K, desc)


@pytest.mark.parametrize("shape", [(37, 50, 70), (64, 101, 256), (5, 60, 8)])
def test_w12_fallback_shapes(shape):
    """Rows of A or of the weights that are not whole 16-byte chunks go through
    W_fused."""
    M, N, K = shape
    pb = inputs.swiglu_problem(160, M, N, K, "bf16")
    y, cfg = run_w12(pb, M, N, K, "bf16")
    assert "via W_fused" in cfg, cfg
    assert_close(oracle.decode(y, "bf16"), reference(pb, M, N, K, "bf16"), "bf16", K, cfg)


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_w12_one_hot_bit_exact(dtype):
    """W1, W2 select columns of A: gate sources powers of two in [32, 256], up
    sources integers in [-3, 3], so Y = g*u exactly."""
    M, N, K = 128, 512, 1024
    gen = np.random.default_rng(7)
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
    pb = dict(A=inputs.to_storage(A, dtype), W1=inputs.to_storage(W1, dtype),
              W2=inputs.to_storage(W2, dtype), scale_a=1.0, scale_w=1.0)
    y, cfg = run_w12(pb, M, N, K, dtype)
    assert np.array_equal(oracle.decode(y, "bf16"), A[:, pi1] * A[:, pi2]), cfg


# --------------------------------------------------------------------------
# Gate then Up (Kernel-1 of the SwiGLU page): SiLU(Gate) computed between the two
# K loops while the first Up tiles load
# --------------------------------------------------------------------------
SEQ_CFGS16 = [49, 50, 53]        # 53: loads in 4 producer waves beside 4 consumer waves
SEQ_CFGS8 = [51, 52, 54]


def run_forced(pb, M, N, K, dtype, cfg):
    os.environ["SG_FORCE_CONFIG"] = "%d,1" % cfg
    try:
        return run_w12(pb, M, N, K, dtype)
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)


@pytest.mark.parametrize("cfg", SEQ_CFGS16)
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_seq_16bit_bit_equal_to_side_by_side(cfg, dtype):
    """Gate and Up accumulate the same products in the same K order as the kernel
    that computes them side by side, and SiLU(s*g)*(s*u) is evaluated with the same
    operations: identical bits.  Ragged M and N, several work-group rows."""
    M, N, K = 300, 1000, 640
    pb = inputs.swiglu_problem(170 + cfg, M, N, K, dtype)
    y, desc = run_forced(pb, M, N, K, dtype, cfg)
    assert "swiglu_seq cfg=%d " % cfg in desc, desc
    y2, desc2 = run_forced(pb, M, N, K, dtype, 10)
    assert "swiglu_w12 cfg=10 " in desc2, desc2
    assert bits_equal(y, y2), (desc, desc2)
    out = "f16" if dtype == "f16" else "bf16"
    assert_close(oracle.decode(y, out), reference(pb, M, N, K, dtype), dtype, K, desc)


@pytest.mark.parametrize("cfg", SEQ_CFGS8)
@pytest.mark.parametrize("M", [16, 300])
def test_seq_e4m3(cfg, M):
    N, K = 1536, 1024
    pb = inputs.swiglu_problem(180 + cfg, M, N, K, "e4m3")
    y, desc = run_forced(pb, M, N, K, "e4m3", cfg)
    assert "swiglu_seq cfg=%d " % cfg in desc, desc
    y2, desc2 = run_forced(pb, M, N, K, "e4m3", 14)
    assert bits_equal(y, y2), (desc, desc2)
    assert_close(oracle.decode(y, "bf16"), reference(pb, M, N, K, "e4m3"), "e4m3", K, desc)


@pytest.mark.parametrize("dtype,cfg", [("bf16", 49), ("e4m3", 51), ("bf16", 53), ("e4m3", 54)])
def test_seq_one_hot_bit_exact(dtype, cfg):
    M, N, K = 256, 512, 1024
    gen = np.random.default_rng(8)
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
    pb = dict(A=inputs.to_storage(A, dtype), W1=inputs.to_storage(W1, dtype),
              W2=inputs.to_storage(W2, dtype), scale_a=1.0, scale_w=1.0)
    y, desc = run_forced(pb, M, N, K, dtype, cfg)
    assert "swiglu_seq cfg=%d " % cfg in desc, desc
    assert np.array_equal(oracle.decode(y, "bf16"), A[:, pi1] * A[:, pi2]), desc


@pytest.mark.parametrize("dtype,M", [("bf16", 128), ("bf16", 512), ("bf16", 2048), ("bf16", 8192),
                                     ("e4m3", 1), ("e4m3", 16), ("e4m3", 256), ("e4m3", 4096)])
def test_split_weight_default_path_full(dtype, M):
    """The split-weight entry point at the SwiGLU workloads' full sizes, in its
    default choice between the two schedules: every output against the oracle."""
    N, K = (4864, 896) if dtype == "bf16" else (11008, 4096)
    pb = inputs.swiglu_problem(4 if dtype == "bf16" else 5, M, N, K, dtype)
    y, desc = run_w12(pb, M, N, K, dtype)
    assert_close(oracle.decode(y, "bf16"), reference(pb, M, N, K, dtype), dtype, K,
                 "split-weight %s M=%d %s" % (dtype, M, desc), report=True)


@pytest.mark.parametrize("dtype,M,cfg", [("bf16", 2048, 49), ("bf16", 8192, 49),
                                         ("e4m3", 4096, 51), ("e4m3", 256, 52),
                                         ("bf16", 2048, 53), ("e4m3", 16, 54)])
def test_seq_workload_sizes_full(dtype, M, cfg):
    """Gate then Up forced at the SwiGLU workloads' full sizes: every output."""
    N, K = (4864, 896) if dtype == "bf16" else (11008, 4096)
    pb = inputs.swiglu_problem(4 if dtype == "bf16" else 5, M, N, K, dtype)
    y, desc = run_forced(pb, M, N, K, dtype, cfg)
    assert "swiglu_seq cfg=%d " % cfg in desc, desc
    assert_close(oracle.decode(y, "bf16"), reference(pb, M, N, K, dtype), dtype, K,
                 "seq %s M=%d %s" % (dtype, M, desc), report=True)
